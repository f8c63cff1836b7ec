#!/usr/bin/env python3
"""Throughput of the CSA2 hot path on one MI355X, over the five workload shapes.

One step = one csa2_decode call (indexer scoring -> top-512 selection ->
sparse attention over 512 FP4 latents + 128 SWA rows) over one batch of
synthetic input already resident in HBM. Steps rotate over device replicas of
the batch (enough that one rotation's key reads exceed three times the 256 MB
memory-side cache) so that consecutive steps cannot be served from it.

The headline (`value`, `config`, `roofline`, `cpu_baseline`) is the largest
single-GPU workload, decode of 4 sequences x 1,048,576 entries; `workloads`
holds the same figures for all five. Per workload (all on one stream):
  1. warm-up, then K timed decode steps bracketed by synchronisation and two
     HIP events (no other event inside the timed region);
  2. per-stage times: up to 50 more steps with the library's stage events;
  3. isolated kernel timing: K back-to-back launches of csa2_index_score (the
     scan kernel) and of csa2_sparse_attn over the decode's ids, each
     bracketed by two HIP events on the launch stream; the roofline is that
     of whichever takes longer, the kernel with the larger share of the step;
  4. the CPU oracle on all host threads over a bounded sample, then one query
     per call on a single thread for half that time.
The headline workload also times the kernels of the rows beside the path
(FP8 window + RoPE attention, pool construction, Reuse gather, cache writes);
at the end, the box's streaming bandwidth (torch row sums and copy, 1 GiB).

Prints one JSON line. `python bench.py --pmc-summary DIR` instead summarises
the counter CSVs of `rocprofv3 --pmc ... --output-format csv -d DIR` runs of
this script (with --copy-calibration) into per-launch HBM bytes, and
`--trace-summary DIR` the kernel-trace CSVs of a `--kernel-trace` run.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import dataclasses
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
FP4_PEAK_TFLOPS = 10100.0    # MI355X dense MXFP4 MFMA, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
METRIC = "CSA2 decode queries/s + indexer entries scored/s; % HBM / FP4-MFMA roofline"
IQ_BYTES = 32 * 64 + 32 * 4 + 32 * 4   # indexer query codes + E8M0 scales + head weights
ENTRY_BYTES_INDEX = 68                 # 64 B codes + 4 B scales per scored entry
ENTRY_BYTES_MAIN = 288
FLOP_PER_PAIR = 2 * 32 * 128
# Kernel families whose roofline a workload may report, with the sources a
# counter summary of them depends on (a summary taken on other sources is stale).
KERNEL_SOURCES = {
    "k_index_score": ("index_score.hip", "csa2_device.h"),
    "k_index_score_qtile": ("index_score.hip", "csa2_device.h"),
    "k_sparse_attn": ("sparse_attn.hip", "csa2_device.h", "select_device.h"),
}
CSRC = os.path.join(ROOT, "compressed_sparse_attention_score_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_MIB = 512
POOL_BLOCKS = 2048                  # Reindex pool: 16,384 entries in blocks of 8
CACHE_WRITE_ROWS = 131072           # new entries quantised per cache-write launch (a long prefill chunk)


# ------------------------------------------------------------------ helpers

class HipEvents:
    """hipEvent_t handles via the HIP runtime (created once, reused)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev.append(h.value)

    def record(self, i, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(self.ev[i]), ctypes.c_void_p(stream.cuda_stream)) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(self.ev[b])) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[a]),
                                            ctypes.c_void_p(self.ev[b])) == 0
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def replica_count(work, resident, requested):
    """Device replicas rotated per step: enough that the keys the scan reads
    over one rotation exceed three times the 256 MB memory-side cache, at most
    64, and at most 16 GB of copies."""
    if requested:
        return requested
    per_step = max(1, work["score_bytes"])
    R = -(-768_000_000 // per_step)
    return int(max(1, min(64, R, 16_000_000_000 // max(1, resident))))


def replicate(db, wl, R):
    """R device replicas of the batch. Caches are cloned; a Reindex batch whose
    cache holds only its pool rows (the rest poison) instead gets, per further
    replica, a fresh random pool of the same size drawn from blocks no earlier
    replica uses, over the same cache tensors, with replica 0's pool rows
    copied there (so every replica scores real entries)."""
    import torch
    reps = [db]
    pool_rows = wl.extra.get("pool_rows") if wl.cand_blocks is not None else None
    if pool_rows is None:
        for _ in range(R - 1):
            reps.append(dataclasses.replace(db, main_cache=db.main_cache.clone(), key_codes=db.key_codes.clone(),
                                            key_scales=db.key_scales.clone()))
    else:
        Q, nb, N = wl.Q, wl.n_blocks, wl.cache_q_stride
        n_blk = wl.n_entries // 8
        used = np.zeros((Q, n_blk), bool)
        for i in range(Q):
            used[i, wl.cand_blocks[i]] = True
        src = torch.from_numpy(pool_rows).to(db.main_cache.device)
        for r in range(1, R):
            rng = np.random.default_rng(7919 + r)
            blocks = np.empty((Q, nb), np.int32)
            for i in range(Q):
                b = np.sort(rng.choice(np.flatnonzero(~used[i]), nb, replace=False))
                used[i, b] = True
                blocks[i] = b
            rows = (np.arange(Q)[:, None, None] * N + 8 * blocks[:, :, None].astype(np.int64)
                    + np.arange(8)[None, None, :]).reshape(-1)
            dst = torch.from_numpy(rows).to(db.main_cache.device)
            db.main_cache[dst] = db.main_cache[src]
            db.key_codes[dst] = db.key_codes[src]
            db.key_scales[dst] = db.key_scales[src]
            reps.append(dataclasses.replace(db, cand_blocks=torch.from_numpy(blocks).to(db.main_cache.device)))
    torch.cuda.synchronize()
    return reps


def work_of(wl):
    """Algorithmic bytes / FLOP of one batch (inputs read once, outputs written once)."""
    Q = wl.Q
    if wl.n_valid is not None:
        per_q = np.minimum(wl.n_valid.astype(np.int64), wl.n_entries)
    else:
        per_q = np.full(Q, wl.n_cand, np.int64)
    pairs = int(per_q.sum())
    block_ids = 4 * wl.n_blocks if wl.cand_blocks is not None else 0
    # keys: a shared prefill cache is read once, independent decode caches once per query
    if wl.cache_q_stride == 0:
        key_bytes = ENTRY_BYTES_INDEX * int(per_q.max(initial=0))
    else:
        key_bytes = ENTRY_BYTES_INDEX * pairs
    score_bytes = key_bytes + Q * (IQ_BYTES + block_ids)
    k_sel = np.minimum(per_q, wl.k)
    swa_rows = (Q - 1) * wl.swa_q_stride + wl.n_swa if Q else 0
    swa_rows = min(swa_rows, Q * wl.n_swa)
    attn_bytes = Q * 65536 * 2 + ENTRY_BYTES_MAIN * int(k_sel.sum()) + 1024 * swa_rows
    attn_flops = int(2 * 2 * 64 * 512 * (k_sel + wl.n_swa).sum())
    # FP8 window rows (528 B) and the (cos, sin) table instead of bf16 rows
    attn_fp8_bytes = attn_bytes - (1024 - 528) * swa_rows + Q * 32 * 2 * 4
    return dict(pairs=pairs, score_bytes=score_bytes, score_flops=pairs * FLOP_PER_PAIR, attn_bytes=attn_bytes,
                attn_flops=attn_flops, step_bytes=score_bytes + attn_bytes, attn_fp8_bytes=attn_fp8_bytes)


def stream_bandwidth(reps=20):
    """The box's own streaming bandwidth, for comparison with the scan
    kernel, over 1 GiB of fp32 (four times the 256 MB memory-side cache):
    torch's row sums over 16 KB rows (the fastest read-only torch pattern
    measured here; a whole-tensor sum reaches about two thirds of it), bytes
    read per mean launch time, and torch's copy, bytes read + written per
    mean launch time. GB/s."""
    import torch
    x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    rows = x.view(-1, 4096)
    out = []
    for op, nbytes in ((lambda: rows.sum(1), 1 << 30), (lambda: y.copy_(x), 2 << 30)):
        for _ in range(3):
            op()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            op()
        b.record()
        torch.cuda.synchronize()
        out.append(nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9)
    del x, y
    return out


def source_digest(kernel):
    h = hashlib.sha256()
    for n in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload_name):
    """HBM bytes per launch of `kernel` on `workload_name` from the committed
    counter summaries (profiles/*hbm_traffic*.md), or None if absent or taken
    on different kernel sources."""
    digest = source_digest(kernel)
    for path in sorted(glob.glob(os.path.join(PROFILES, "*hbm_traffic*.md"))):
        for line in open(path):
            # machine-readable lines: "traffic: <digest> <kernel> <bytes_per_launch> <workload name>"
            if line.startswith("traffic: "):
                parts = line[len("traffic: "):].strip().split(" ", 3)
                if len(parts) == 4 and parts[0] == digest and parts[1] == kernel and parts[3] == workload_name:
                    return float(parts[2])
    return None


def _time_oracle(wl, view, per_call, seconds):
    """Oracle decode calls on `per_call` queries each (strided subsets when
    fewer than the batch) until `seconds` of wall time have passed."""
    import oracle
    done, calls = 0, 0
    t0 = time.perf_counter()
    first = None
    while True:
        if per_call == wl.Q:
            qs = None
        else:
            stride = wl.Q // per_call
            qs = [(calls + stride * j) % wl.Q for j in range(per_call)]
        ref = oracle.decode(view, queries=qs)
        if first is None:
            first = (qs, ref)
        done += per_call
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or calls >= 100000:
            return first, done, calls, dt


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, seconds):
    """The oracle as it stands, timed over a bounded sample of the workload:
    whole batches (or, when one batch is too long, strided query subsets) on
    all host threads until `seconds` of wall time have passed; then one query
    per call on a single thread for half that time."""
    import oracle
    import synth
    view = synth.compact_pool_view(wl) if (wl.cand_blocks is not None and not wl.extra.get("dense_rows", True)) \
        else wl
    threads = oracle.get_threads()
    per_call = wl.Q
    if wl.n_valid is not None and wl.Q > 2 * threads:   # prefill: strided subsets of `threads` queries
        per_call = threads
    first, done, calls, dt = _time_oracle(wl, view, per_call, seconds)
    what = "the whole batch" if per_call == wl.Q else f"strided subsets of {per_call} queries"
    res = dict(value=round(done / dt, 3), unit="queries/s", cores=int(min(threads, per_call)), kind="oracle",
               sample=f"{calls} oracle decode call(s) on {what} of this workload ({wl.Q} queries, "
                      f"{wl.n_cand} candidates each; {done} queries in all), fp64, {dt:.1f} s wall",
               cpu_model=_cpu_model(), host_threads=int(threads))
    oracle.set_threads(1)
    try:
        _, done1, calls1, dt1 = _time_oracle(wl, view, 1, max(1.0, seconds / 2))
    finally:
        oracle.set_threads(threads)
    res["one_thread"] = dict(value=round(done1 / dt1, 3), unit="queries/s", cores=1,
                             sample=f"{calls1} oracle decode call(s) of one query each (strided), fp64, "
                                    f"{dt1:.1f} s wall")
    return first, res


def parity_summary(wl, first, out_bf16, idx):
    """Band-rule ids + attention tolerance of the first timed batch on the
    queries the CPU baseline computed (reported, not asserted)."""
    import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import QueryView, check_attn, check_topk_band
    qs, ref = first
    sel = np.arange(wl.Q) if qs is None else np.asarray(qs)
    try:
        if wl.cand_blocks is not None and not wl.extra.get("dense_rows", True):
            comp = synth.compact_pool_view(wl)
            gidx = np.stack([np.searchsorted(synth.pool_ids(wl, i), idx[i]) for i in sel]).astype(np.int32)
            check_topk_band(gidx, ref["scores"], ref["idx"], QueryView(comp, sel), wl.k, "bench")
        else:
            check_topk_band(idx[sel], ref["scores"], ref["idx"], QueryView(wl, sel), wl.k, "bench")
        rel = check_attn(out_bf16[sel], ref["out_f32"], "bench")
        return dict(ok=True, queries_checked=int(len(sel)), attn_max_err_rel=round(float(rel), 6))
    except AssertionError as e:
        return dict(ok=False, error=str(e)[:300])


# ------------------------------------------------------- counter summaries

def pmc_summary(root):
    """Per-kernel mean counter values (KiB per dispatch for FETCH_SIZE /
    WRITE_SIZE) over every counter_collection CSV under `root`."""
    acc = {}
    for path in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name", "")
                cn, cv = row.get("Counter_Name"), row.get("Counter_Value")
                did = row.get("Dispatch_Id")
                if cn is None or cv is None:
                    continue
                d = acc.setdefault(name, {}).setdefault(cn, {})
                d[did] = d.get(did, 0.0) + float(cv)
    out = {}
    for name, counters in acc.items():
        out[name] = {cn: (sum(v.values()) / len(v), len(v)) for cn, v in counters.items()}
    return out


def print_pmc_summary(root):
    s = pmc_summary(root)
    copy_bytes = COPY_MIB << 20
    fetch_f = write_f = None
    for name, cs in s.items():
        if "neg" in name.lower():   # the calibration kernel: reads and writes COPY_MIB MiB
            if "FETCH_SIZE" in cs:
                fetch_f = cs["FETCH_SIZE"][0] * 1024 / copy_bytes
            if "WRITE_SIZE" in cs:
                write_f = cs["WRITE_SIZE"][0] * 1024 / copy_bytes
    print(f"calibration kernel (elementwise negation, {COPY_MIB} MiB in + {COPY_MIB} MiB out): "
          f"FETCH_SIZE factor {fetch_f}, WRITE_SIZE factor {write_f}")
    print(f"{'kernel':70s} {'counter':12s} {'mean KiB/dispatch':>18s} {'dispatches':>10s} {'calibrated MB':>14s}")
    for name, cs in sorted(s.items()):
        for cn, (v, n) in sorted(cs.items()):
            f = fetch_f if cn == "FETCH_SIZE" else write_f if cn == "WRITE_SIZE" else None
            cal = f"{v * 1024 / f / 1e6:14.3f}" if f else f"{'':14s}"
            print(f"{name[:70]:70s} {cn:12s} {v:18.1f} {n:10d} {cal}")
    for kern, srcs in KERNEL_SOURCES.items():
        print(f"kernel source digest of {kern} ({', '.join(srcs)}): {source_digest(kern)}")


def print_trace_summary(root):
    """Per-kernel durations from `rocprofv3 --kernel-trace --output-format csv`
    (as in its kernel_stats file), plus the scan kernel split into launches
    inside decode steps and the isolated back-to-back launches bench.py times."""
    rows = []
    for path in glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"],
                             r["Grid_Size_X"], r["Grid_Size_Y"], r["Workgroup_Size_X"], r["LDS_Block_Size"],
                             r["VGPR_Count"], r["Accum_VGPR_Count"], r["Scratch_Size"]))
    rows.sort()
    stats, meta = {}, {}
    for st, en, name, *m in rows:
        stats.setdefault(name, []).append((en - st) / 1e3)
        meta.setdefault(name, m)
    print(f"{'kernel':72s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}")
    for name, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        print(f"{name[:72]:72s} {len(v):6d} {sum(v) / len(v):9.2f} {min(v):9.2f} {max(v):9.2f}")
    print("launch shapes (grid threads x, y; workgroup; LDS B; VGPR; AGPR; scratch):")
    for name, m in meta.items():
        if "csa2" in name:
            print(f"  {name[:60]:60s} grid {m[0]}x{m[1]} wg {m[2]} lds {m[3]} vgpr {m[4]} agpr {m[5]} scratch {m[6]}")
    # each library kernel split into launches inside decode steps (a neighbour
    # is another kernel) and the back-to-back launches bench.py times alone
    lib = [r for r in rows if "csa2" in r[2]]
    split = {}
    for i, (st, en, name, *_) in enumerate(lib):
        nb = [lib[j][2] for j in (i - 1, i + 1) if 0 <= j < len(lib)]
        iso = all(n == name for n in nb)
        split.setdefault(name, ([], []))[1 if iso else 0].append((en - st) / 1e3)
    for name, (dec, iso) in split.items():
        for label, v in (("inside decode steps", dec), ("isolated back-to-back", iso)):
            if v:
                print(f"{name[:60]} {label}: {len(v)} launches, avg {sum(v) / len(v):.2f} us")


# -------------------------------------------------------------------- main

HEADLINE = 4   # the largest single-GPU workload: decode of 4 sequences x 1,048,576 entries


def _timed(ev, i0, stream, K, launch):
    """Mean ms of K back-to-back launches of `launch(i)`, by two HIP events on
    the launch stream (after 3 untimed launches)."""
    import torch
    for i in range(3):
        launch(i)
    torch.cuda.synchronize()
    ev.record(i0, stream)
    for i in range(K):
        launch(i)
    ev.record(i0 + 1, stream)
    torch.cuda.synchronize()
    return ev.ms(i0, i0 + 1) / K


def run_workload(wi, args, extras, cpu_seconds):
    """Every figure of one workload: decode steps, stage times, isolated
    kernels and their rooflines, the oracle's CPU baseline and a parity
    report. Frees its device memory before returning."""
    import torch

    import compressed_sparse_attention_score_amd as csa
    import synth
    from synth.device import to_device

    name = synth.WORKLOAD_NAMES[wi]
    print(f"[bench] workload {wi}: {name}", file=sys.stderr, flush=True)
    t_gen = time.perf_counter()
    wl = synth.make_workload(wi, dense_rows=False)
    gen_s = time.perf_counter() - t_gen
    db = to_device(wl)
    Q = wl.Q
    work = work_of(wl)
    if wl.cand_blocks is not None and "pool_rows" in wl.extra:
        resident = len(wl.extra["pool_rows"]) * (ENTRY_BYTES_MAIN + ENTRY_BYTES_INDEX)  # pool rows copied per replica
    else:
        resident = sum(t.numel() * t.element_size() for t in (db.main_cache, db.key_codes, db.key_scales))
    R = replica_count(work, resident, args.replicas)
    reps = replicate(db, wl, R)
    stream = torch.cuda.current_stream()
    out, lse, idx = db.new_outputs()
    ws = torch.empty(max(1, csa.csa2_workspace_size(csa.CSA2_WS_DECODE, db.decode_args(out, lse, idx))),
                     dtype=torch.uint8, device="cuda")
    K, W = args.steps, args.warmup
    S = min(K, 50)
    ev = HipEvents(2 + 4 * S + 24)

    # ---- timed decode steps
    dec_args = [reps[i % R].decode_args(out, lse, idx) for i in range(R)]
    for i in range(W):
        csa.csa2_decode(dec_args[i % R], ws, stream)
    csa.csa2_decode(dec_args[0], ws, stream)   # replica 0's outputs for the parity report
    torch.cuda.synchronize()
    first_out = out.cpu().numpy().view(np.uint16).copy()
    first_idx = idx.cpu().numpy().copy()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(0, stream)
    for i in range(K):
        csa.csa2_decode(dec_args[i % R], ws, stream)
    ev.record(1, stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_ms = ev.ms(0, 1)

    # ---- per-stage times (events between the kernels cost a few us each)
    st_args = [reps[i % R].decode_args(out, lse, idx, stage_events=tuple(ev.ev[2 + 4 * i:6 + 4 * i]))
               for i in range(S)]
    for i in range(S):
        csa.csa2_decode(st_args[i], ws, stream)
    torch.cuda.synchronize()
    st = np.array([[ev.ms(2 + 4 * i + j, 3 + 4 * i + j) for j in range(3)] for i in range(S)])
    stage_ms = st.mean(axis=0)

    # ---- isolated kernels: the scan and the attention (ids of the decode)
    e0 = 2 + 4 * S
    scores = torch.empty((Q, max(1, wl.n_cand)), dtype=torch.float32, device="cuda")
    sc_args = [reps[i % R].index_args() for i in range(R)]
    score_ms = _timed(ev, e0, stream, K, lambda i: csa.csa2_index_score(sc_args[i % R], scores, stream))
    at_out, at_lse = torch.empty_like(out), torch.empty_like(lse)
    at_args = [reps[i % R].attn_args(idx, at_out, at_lse) for i in range(R)]
    at_ws = torch.empty(max(1, csa.csa2_workspace_size(csa.CSA2_WS_ATTN, at_args[0])), dtype=torch.uint8,
                        device="cuda")
    attn_ms = _timed(ev, e0 + 2, stream, K, lambda i: csa.csa2_sparse_attn(at_args[i % R], at_ws, stream))

    prefill = wl.n_valid is not None
    scan_kernel = "k_index_score_qtile" if (wl.cache_q_stride == 0 and Q >= 32) else "k_index_score"
    score_gbs = work["score_bytes"] / (score_ms * 1e-3) / 1e9
    score_tfs = work["score_flops"] / (score_ms * 1e-3) / 1e12
    attn_gbs = work["attn_bytes"] / (attn_ms * 1e-3) / 1e9
    attn_tfs = work["attn_flops"] / (attn_ms * 1e-3) / 1e12
    kernels = {
        "index_score": {"kernels": [scan_kernel], "us_per_launch": round(1e3 * score_ms, 3),
                        "algorithmic_bytes": work["score_bytes"], "GB_s": round(score_gbs, 1),
                        "hbm_frac": round(score_gbs / HBM_PEAK_GBS, 4), "TFLOP_s": round(score_tfs, 2),
                        "fp4_mfma_frac": round(score_tfs / FP4_PEAK_TFLOPS, 4)},
        "sparse_attn": {"kernels": ["k_sparse_attn"], "us_per_launch": round(1e3 * attn_ms, 3),
                        "algorithmic_bytes": work["attn_bytes"], "GB_s": round(attn_gbs, 1),
                        "hbm_frac": round(attn_gbs / HBM_PEAK_GBS, 4), "TFLOP_s": round(attn_tfs, 2),
                        "bf16_mfma_frac": round(attn_tfs / BF16_PEAK_TFLOPS, 4)},
    }
    if extras:
        kernels.update(extra_kernels(wl, reps, R, idx, out, lse, scores, at_ws, ev, e0 + 4, stream, K))

    # ---- roofline of the kernel with the larger share of the step
    if score_ms >= attn_ms:
        kern = scan_kernel
        if prefill:
            roof = {"bound": "mfma", "achieved": round(score_tfs, 2), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(score_tfs / FP4_PEAK_TFLOPS, 4),
                    "algorithmic_flops_per_launch": work["score_flops"]}
        else:
            roof = {"bound": "hbm", "achieved": round(score_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(score_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": work["score_bytes"]}
        launch_ms = score_ms
    else:
        kern = "k_sparse_attn"
        roof = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": work["attn_bytes"],
                "bf16_mfma_frac": round(attn_tfs / BF16_PEAK_TFLOPS, 4)}
        launch_ms = attn_ms
    roof["traffic"] = recorded_traffic(kern, name)
    roof["kernel"] = kern
    roof["launch_us"] = round(1e3 * launch_ms, 3)
    roof["share_of_step"] = round(launch_ms / (gpu_ms / K), 4)

    ms_per_step = 1e3 * elapsed / K
    res = {
        "workload": name,
        "workload_index": wi,
        "queries": Q,
        "candidates_per_query": wl.n_cand,
        "top_k": wl.k,
        "swa_rows": wl.n_swa,
        "replicas": R,
        "queries_per_s": round(Q * K / elapsed, 1),
        "entries_scored_per_s": round(work["pairs"] * K / elapsed, 1),
        "ms_per_step": round(ms_per_step, 5),
        "gpu_ms_per_step": round(gpu_ms / K, 5),
        "algorithmic_bytes_per_step": work["step_bytes"],
        "path_hbm_frac": round(work["step_bytes"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "stage_us": {"index_score": round(1e3 * stage_ms[0], 2), "select": round(1e3 * stage_ms[1], 2),
                     "attention": round(1e3 * stage_ms[2], 2), "steps": S},
        "roofline": roof,
        "kernels": kernels,
        "gen_s": round(gen_s, 2),
    }
    if prefill:
        res["indexer_pairs_per_s"] = round(work["pairs"] / (score_ms * 1e-3), 1)
    ev.close()
    del reps, db, scores, ws, at_ws, at_out, at_lse, dec_args, st_args, sc_args, at_args
    out, lse, idx = None, None, None
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu_seconds > 0:
        first, cb = cpu_baseline(wl, cpu_seconds)
        res["cpu_baseline"] = cb
        res["parity"] = parity_summary(wl, first, first_out, first_idx)
    return res


def extra_kernels(wl, reps, R, idx, out, lse, scores, at_ws, ev, e0, stream, K):
    """The kernels of the rows built beside the hot path, timed on this
    workload: attention with FP8 window rows and the RoPE epilogue, Reindex
    pool construction from these scores, the Reuse-layer gather and attention
    over the gathered list, and the cache writes (131,072 new rows; 65,536
    m=2 pooled entries)."""
    import torch

    import compressed_sparse_attention_score_amd as csa
    import synth
    Q = wl.Q
    work = work_of(wl)
    res = {}
    at_out, at_lse = torch.empty_like(out), torch.empty_like(lse)
    if wl.extra.get("shared_swa"):
        rows8 = synth.fp8_rows(0, synth.TID_SWA, 0, 0, wl.swa.shape[0])
    else:
        rows8 = np.concatenate([synth.fp8_rows(0, synth.TID_SWA, i, 0, wl.n_swa) for i in range(Q)])
    pos = wl.extra["t0"] + np.arange(Q) if "t0" in wl.extra else wl.n_entries + 7 * np.arange(Q)
    swa8 = torch.from_numpy(np.ascontiguousarray(rows8)).cuda()
    rope_t = torch.from_numpy(synth.rope_table(pos)).cuda()
    a8 = [dataclasses.replace(reps[i % R], swa=swa8, swa_format=csa.CSA2_SWA_FP8, rope=rope_t)
          .attn_args(idx, at_out, at_lse) for i in range(R)]
    ms = _timed(ev, e0, stream, K, lambda i: csa.csa2_sparse_attn(a8[i % R], at_ws, stream))
    res["sparse_attn_fp8_window_rope"] = {"kernels": ["k_sparse_attn<fp8 window>"], "us_per_launch": round(1e3 * ms, 3),
                                          "algorithmic_bytes": work["attn_fp8_bytes"],
                                          "GB_s": round(work["attn_fp8_bytes"] / (ms * 1e-3) / 1e9, 1)}
    del swa8, rope_t, a8
    if wl.cand_blocks is None and wl.n_valid is None:
        n_pool = int(min(POOL_BLOCKS, (wl.n_cand + 7) // 8))
        pool_out = torch.empty((Q, n_pool), dtype=torch.int32, device="cuda")
        pa = csa.pool_args(scores, n_pool, pool_out)
        pool_ws = torch.empty(max(1, csa.csa2_workspace_size(csa.CSA2_WS_POOL, pa)), dtype=torch.uint8, device="cuda")
        ms = _timed(ev, e0 + 2, stream, K, lambda i: csa.csa2_build_pool(pa, pool_ws, stream))
        pb = Q * (4 * wl.n_cand + 4 * n_pool)  # scores read once, pool ids written
        res["build_pool"] = {"kernels": ["k_block_max", "k_score_maxima", "k_select_*"], "blocks_kept": n_pool,
                             "us_per_launch": round(1e3 * ms, 3), "algorithmic_bytes": pb,
                             "GB_s": round(pb / (ms * 1e-3) / 1e9, 1)}
        del pool_out, pool_ws
    kk = int(idx.shape[1])
    g_out = torch.empty((Q, kk, ENTRY_BYTES_MAIN), dtype=torch.uint8, device="cuda")
    g_dense = torch.empty((Q, kk), dtype=torch.int32, device="cuda")
    ms_g = _timed(ev, e0 + 4, stream, K, lambda i: csa.csa2_gather_selected(
        reps[i % R].main_cache, wl.n_entries, wl.cache_q_stride, idx, g_out, g_dense, stream))
    ad = dataclasses.replace(reps[0], main_cache=g_out.view(-1, ENTRY_BYTES_MAIN), n_entries=kk,
                             cache_q_stride=kk).attn_args(g_dense, at_out, at_lse)
    ms_d = _timed(ev, e0 + 6, stream, K, lambda i: csa.csa2_sparse_attn(ad, at_ws, stream))
    res["reuse_layer"] = {"kernels": ["k_gather_selected", "k_sparse_attn"], "gather_us": round(1e3 * ms_g, 3),
                          "gather_GB_s": round(2 * Q * kk * ENTRY_BYTES_MAIN / (ms_g * 1e-3) / 1e9, 1),
                          "attn_over_dense_list_us": round(1e3 * ms_d, 3)}
    del g_out, g_dense
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    xm = torch.randn((CACHE_WRITE_ROWS, 512), generator=gen, device="cuda")
    xk = torch.randn((CACHE_WRITE_ROWS, 128), generator=gen, device="cuda")
    qm = torch.empty((CACHE_WRITE_ROWS, 288), dtype=torch.uint8, device="cuda")
    qc = torch.empty((CACHE_WRITE_ROWS, 64), dtype=torch.uint8, device="cuda")
    qs = torch.empty((CACHE_WRITE_ROWS, 4), dtype=torch.uint8, device="cuda")
    for j, (kname, kind, xin, co, so, per_row) in enumerate(
            (("quantize_main", 0, xm, qm, None, 512 * 4 + ENTRY_BYTES_MAIN),
             ("quantize_index", 1, xk, qc, qs, 128 * 4 + ENTRY_BYTES_INDEX))):
        ms = _timed(ev, e0 + 8 + 2 * j, stream, K, lambda i: csa.csa2_quantize(
            kind, xin, csa.CSA2_IN_F32, CACHE_WRITE_ROWS, None, CACHE_WRITE_ROWS, co, so, stream))
        qb = CACHE_WRITE_ROWS * per_row
        res[kname] = {"kernels": [f"k_quantize<f32, {'main' if kind == 0 else 'index'}>"], "rows": CACHE_WRITE_ROWS,
                      "us_per_launch": round(1e3 * ms, 3), "algorithmic_bytes": qb,
                      "GB_s": round(qb / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(qb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del xm, xk, qm, qc, qs
    npool = CACHE_WRITE_ROWS // 2
    xp = torch.randn((2 * npool, 512), generator=gen, device="cuda")
    gp = torch.randn((2 * npool, 512), generator=gen, device="cuda")
    cp = torch.empty((npool, 288), dtype=torch.uint8, device="cuda")
    pp = torch.empty((npool, 512), dtype=torch.float32, device="cuda")
    ms = _timed(ev, e0 + 12, stream, K, lambda i: csa.csa2_pool_quantize(xp, gp, npool, None, npool, cp, pp, stream))
    pqb = npool * (2 * 2048 * 2 + ENTRY_BYTES_MAIN + 2048)  # two rows + two gate rows in, entry + pooled out
    res["pool_quantize_m2"] = {"kernels": ["k_quantize<f32, main, gate 512>"], "entries": npool,
                               "us_per_launch": round(1e3 * ms, 3), "algorithmic_bytes": pqb,
                               "GB_s": round(pqb / (ms * 1e-3) / 1e9, 1),
                               "hbm_frac": round(pqb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del xp, gp, cp, pp
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", "--config", dest="workload", type=int, default=None,
                    help="run one workload only: 0 decode 1 x 4,096; 1 decode 16 x 65,536; 2 reindex decode "
                         "64 x 16,384-entry pools of 1,048,576-entry caches; 3 prefill 4,096 x 131,072; 4 decode "
                         "4 x 1,048,576 (the headline). Default: all five, headline 4")
    ap.add_argument("--replicas", type=int, default=0, help="device copies rotated per step (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum wall time of the headline's oracle sample (a third of it for the other workloads)")
    ap.add_argument("--no-extras", action="store_true", help="skip the kernels of the rows beside the hot path")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"also run an elementwise {COPY_MIB} MiB negation (counter calibration)")
    ap.add_argument("--pmc-summary", metavar="DIR", help="summarise rocprofv3 counter CSVs under DIR and exit")
    ap.add_argument("--trace-summary", metavar="DIR", help="summarise rocprofv3 kernel-trace CSVs under DIR and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        print_pmc_summary(args.pmc_summary)
        return
    if args.trace_summary:
        print_trace_summary(args.trace_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported. Decode batches and prefill "
              "chunks shard across GPUs by sequence / query rows with no exchange, so the one-GPU figure is the "
              "per-GPU share.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    torch.cuda.set_device(0)
    order = [args.workload] if args.workload is not None else [0, 1, 2, 3, HEADLINE]
    head = order[-1]
    per = {}
    for wi in order:
        cpu_s = 0.0 if args.no_cpu_baseline else (args.cpu_seconds if wi == head else args.cpu_seconds / 3)
        per[str(wi)] = run_workload(wi, args, extras=(wi == head and not args.no_extras), cpu_seconds=cpu_s)
    read_gbs, copy_gbs = stream_bandwidth()
    if args.copy_calibration:
        src = torch.ones(COPY_MIB << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    h = per[str(head)]
    for r in per.values():
        if r["roofline"]["unit"] == "GB/s":
            r["roofline"]["frac_of_measured_read"] = round(r["roofline"]["achieved"] / read_gbs, 4)
    res = {
        "metric": METRIC,
        "value": h["queries_per_s"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4(mx)+bf16",
        "data": "synthetic (seeded N(0,1) latents/keys/queries quantised to FP4 per the pages' formats)",
        "config": {"workload": h["workload"], "workload_index": h["workload_index"], "queries": h["queries"],
                   "candidates_per_query": h["candidates_per_query"], "top_k": h["top_k"],
                   "swa_rows": h["swa_rows"], "replicas": h["replicas"]},
        "entries_scored_per_s": h["entries_scored_per_s"],
        "gpu_ms_per_step": h["gpu_ms_per_step"],
        "path_hbm_frac": h["path_hbm_frac"],
        "stage_us": h["stage_us"],
        "roofline": h["roofline"],
    }
    if "cpu_baseline" in h:
        res["cpu_baseline"] = h["cpu_baseline"]
    res["measured_stream"] = {"read_GB_s": round(read_gbs, 1), "copy_GB_s": round(copy_gbs, 1),
                              "what": "torch row sums over 16 KB rows (read) and copy (read + write), 1 GiB fp32, "
                                      "on this box"}
    res["workloads"] = per
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
