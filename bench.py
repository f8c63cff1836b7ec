#!/usr/bin/env python3
"""Throughput of the CSA2 decode hot path on one MI355X.

One step = one csa2_decode call (indexer scoring -> top-512 selection ->
sparse attention over 512 FP4 latents + 128 SWA rows) over one batch of
synthetic input already resident in HBM. Steps rotate over device replicas of
the batch so that consecutive steps cannot be served from the 256 MB
memory-side cache.

Prints one JSON line: queries/s (value), entries scored/s, per-stage times
from HIP events recorded by the library on its stream, the roofline of the
dominant kernel (indexer scoring, HBM-bound: 68 B per scored entry) and the
CPU oracle timed on the host as a baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFLOPS = 10100.0
METRIC = "CSA2 decode queries/s + indexer entries scored/s; % HBM / FP4-MFMA roofline"
IQ_BYTES = 32 * 64 + 32 * 4 + 32 * 4  # indexer query codes + scales + head weights
FIXED_BYTES = IQ_BYTES + 65536 + 131072 + 512 * 288 + 65536  # + q, SWA, selected latents, output


class HipEvents:
    """hipEvent_t handles via the HIP runtime (created once, reused)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev.append(h.value)

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(self.ev[b])) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[a]),
                                            ctypes.c_void_p(self.ev[b])) == 0
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def replicate(db, R):
    import dataclasses

    import torch
    reps = [db]
    for _ in range(R - 1):
        reps.append(dataclasses.replace(db, main_cache=db.main_cache.clone(), key_codes=db.key_codes.clone(),
                                        key_scales=db.key_scales.clone()))
    torch.cuda.synchronize()
    return reps


def cpu_baseline(wl, gpu_out=None):
    import oracle
    threads = oracle.get_threads()
    t0 = time.perf_counter()
    ref = oracle.decode(wl)
    dt = time.perf_counter() - t0
    return ref, dict(value=wl.Q / dt, unit="queries/s", cores=min(threads, wl.Q), kind="oracle",
                     sample=f"one full batch of the same workload ({wl.Q} queries x {wl.n_cand} candidates), "
                            f"fp64 CPU oracle, {dt:.2f} s wall")


def parity_summary(wl, ref, out_bf16, idx):
    """Band-rule ids + attention tolerance of the first timed batch (reported)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    try:
        from gpu_util import check_attn, check_topk_band
        check_topk_band(idx, ref["scores"], ref["idx"], wl, wl.k, "bench")
        rel = check_attn(out_bf16, ref["out_f32"], "bench")
        return dict(ok=True, attn_max_err_rel=rel)
    except AssertionError as e:
        return dict(ok=False, error=str(e)[:300])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload shape 0..4 (default 1: batch 16 x 65,536)")
    ap.add_argument("--replicas", type=int, default=0, help="device copies rotated per step (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported on this single-GPU build "
              "(the decode batch shards by sequence with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import compressed_sparse_attention_score_amd as csa
    import synth
    from synth.device import to_device

    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    wl = synth.make_config(args.config, dense_rows=False)
    gen_s = time.perf_counter() - t_gen
    db = to_device(wl)
    Q, n_cand = wl.Q, wl.n_cand
    step_bytes = Q * (FIXED_BYTES + 68 * n_cand + (4 * n_cand // 8 if wl.cand_blocks is not None else 0))
    score_bytes = Q * (68 * n_cand + IQ_BYTES + (4 * n_cand // 8 if wl.cand_blocks is not None else 0))
    if wl.n_valid is not None:  # causal prefill: only visible entries are scored
        pairs = int(np.minimum(wl.n_valid, wl.n_entries).astype(np.int64).sum())
    else:
        pairs = Q * n_cand
    resident = sum(t.numel() * t.element_size() for t in (db.main_cache, db.key_codes, db.key_scales))
    R = args.replicas or int(min(8, max(1, math.ceil(768e6 / max(1, resident)))))
    reps = replicate(db, R)

    out, lse, idx = db.new_outputs()
    probe = db.decode_args(out, lse, idx)
    ws = torch.empty(max(1, csa.csa2_workspace_size(csa.CSA2_WS_DECODE, probe)), dtype=torch.uint8, device="cuda")
    K, W = args.steps, args.warmup
    # Stage events are recorded on every EVERY-th timed step only: an event
    # between two kernels costs a few microseconds of idle time.
    EVERY = 10
    sampled = list(range(0, K, EVERY))
    ev = HipEvents(4 * len(sampled) + 2)
    stream = torch.cuda.current_stream()

    for i in range(W):
        csa.csa2_decode(reps[i % R].decode_args(out, lse, idx), ws, stream)
    torch.cuda.synchronize()
    # first batch outputs (replica 0) for the parity report
    csa.csa2_decode(reps[0].decode_args(out, lse, idx), ws, stream)
    torch.cuda.synchronize()
    first_out = out.cpu().numpy().view(np.uint16).copy()
    first_idx = idx.cpu().numpy().copy()

    timed_args = []
    for i in range(K):
        if i % EVERY == 0:
            j = i // EVERY
            timed_args.append(reps[i % R].decode_args(out, lse, idx, stage_events=tuple(ev.ev[4 * j:4 * j + 4])))
        else:
            timed_args.append(reps[i % R].decode_args(out, lse, idx))
    start_ev, end_ev = len(ev.ev) - 2, len(ev.ev) - 1
    hip_record = ev.hip.hipEventRecord
    hip_record.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip_record(ctypes.c_void_p(ev.ev[start_ev]), ctypes.c_void_p(stream.cuda_stream))
    for i in range(K):
        csa.csa2_decode(timed_args[i], ws, stream)
    hip_record(ctypes.c_void_p(ev.ev[end_ev]), ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_elapsed_ms = ev.ms(start_ev, end_ev)

    st = np.array([[ev.ms(4 * j, 4 * j + 1), ev.ms(4 * j + 1, 4 * j + 2), ev.ms(4 * j + 2, 4 * j + 3)]
                   for j in range(len(sampled))])
    ev.close()
    score_ms, select_ms, attn_ms = st.mean(axis=0)
    ms_per_step = 1e3 * elapsed / K
    value = Q * K / elapsed
    achieved = score_bytes / (score_ms * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4(mx)+bf16",
        "data": "synthetic (seeded N(0,1) latents/keys/queries quantised to FP4 per the pages' formats)",
        "config": {"workload": synth.CONFIG_NAMES[args.config], "config_index": args.config, "queries": Q,
                   "candidates_per_query": n_cand, "top_k": wl.k, "swa_rows": wl.n_swa, "replicas": R},
        "entries_scored_per_s": round(pairs * K / elapsed, 1),
        "gpu_ms_per_step": round(gpu_elapsed_ms / K, 5),
        "stage_us": {"index_score": round(1e3 * score_ms, 2), "select": round(1e3 * select_ms, 2),
                     "attention": round(1e3 * attn_ms, 2), "sampled_steps": len(sampled)},
        "path_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "k_index_score", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": score_bytes},
    }
    if args.config == 3:
        tflops = pairs * 8192 / (score_ms * 1e-3) / 1e12
        res["roofline"] = {"kernel": "k_index_score", "bound": "mfma", "achieved": round(tflops, 2),
                           "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / FP4_PEAK_TFLOPS, 4),
                           "traffic": None, "algorithmic_flops_per_launch": pairs * 8192}
    if not args.no_cpu_baseline:
        if wl.extra.get("dense_rows", True) and args.config != 3:
            ref, cb = cpu_baseline(wl)
            res["cpu_baseline"] = cb
            res["parity"] = parity_summary(wl, ref, first_out, first_idx)
        else:
            res["cpu_baseline"] = None
    res["gen_s"] = round(gen_s, 2)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
