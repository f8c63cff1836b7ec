"""CPU oracle for the CSA2 path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never does.

Thin ctypes wrapper over ``csa2_oracle.c`` (plain fp64 C, one function per step
of the path); numpy arrays in, numpy arrays out.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB = os.path.join(_HERE, "libcsa2oracle.so")


def build(force: bool = True, extra_flags=(), out: str | None = None) -> str:
    out = out or _LIB
    if force or not os.path.exists(out):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden", *extra_flags, _SRC, "-o",
               out + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return out


def _bind(L):
    i32, i64, vp, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
    for n in ("orc_e2m1", "orc_e4m3", "orc_e8m0"):
        getattr(L, n).restype = dbl
        getattr(L, n).argtypes = [ctypes.c_uint]
    L.orc_main_entry_bytes.restype = i32
    L.orc_f64_to_bf16.restype = ctypes.c_uint16
    L.orc_f64_to_bf16.argtypes = [dbl]
    L.orc_index_entry_bytes.restype = i32
    L.orc_dequant_main.argtypes = [vp, i64, vp, vp]
    L.orc_dequant_index.argtypes = [vp, vp, i64, vp, vp]
    L.orc_index_score.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
    L.orc_topk.argtypes = [vp, i32, i64, vp, i64, vp, i32, i32, vp, vp]
    L.orc_sparse_attn.argtypes = [i32, i64, i64, vp, vp, i32, vp, vp, i64, i32, dbl, vp, vp, vp, vp, i32, vp]
    L.orc_decode.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, i64, i32, dbl, vp, vp,
                             vp, vp, vp, i32, vp]
    L.orc_dequant_swa_fp8.argtypes = [vp, i64, vp]
    L.orc_pool_blocks.argtypes = [vp, i32, i64, vp, i32, vp]
    L.orc_pool_latents.argtypes = [vp, vp, i32, i64, vp]
    L.orc_gather_selected.argtypes = [vp, i64, i64, vp, i32, i32, vp, vp]
    L.orc_quantize_main.argtypes = [vp, i64, vp]
    L.orc_quantize_index.argtypes = [vp, i64, vp, vp]
    L.orc_set_threads.argtypes = [i32]
    L.orc_get_threads.restype = i32
    return L


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def load_variant(path: str):
    """Load another build of the oracle (e.g. one compiled with a planted mistake)."""
    return _bind(ctypes.CDLL(path))


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous numpy arrays"
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    lib().orc_set_threads(n)


def get_threads() -> int:
    return lib().orc_get_threads()


def e2m1(code: int, L=None) -> float:
    return (L or lib()).orc_e2m1(code)


def e4m3(b: int, L=None) -> float:
    return (L or lib()).orc_e4m3(b)


def e8m0(b: int, L=None) -> float:
    return (L or lib()).orc_e8m0(b)


def f64_to_bf16(v: float, L=None) -> int:
    """bf16 bit pattern of the fp64 value v, one round-to-nearest-even step."""
    return int((L or lib()).orc_f64_to_bf16(float(v)))


def dequant_main(entries: np.ndarray, L=None):
    entries = np.ascontiguousarray(entries, np.uint8).reshape(-1, 288)
    n = entries.shape[0]
    f = np.empty((n, 512), np.float32)
    b = np.empty((n, 512), np.uint16)
    (L or lib()).orc_dequant_main(_p(entries), n, _p(f), _p(b))
    return f, b


def dequant_index(codes: np.ndarray, scales: np.ndarray, L=None):
    codes = np.ascontiguousarray(codes, np.uint8).reshape(-1, 64)
    scales = np.ascontiguousarray(scales, np.uint8).reshape(-1, 4)
    n = codes.shape[0]
    f = np.empty((n, 128), np.float32)
    b = np.empty((n, 128), np.uint16)
    (L or lib()).orc_dequant_index(_p(codes), _p(scales), n, _p(f), _p(b))
    return f, b


def quantize_main(x: np.ndarray, L=None) -> np.ndarray:
    """fp32 latents [n][512] -> main entries [n][288] (uint8)."""
    x = np.ascontiguousarray(x, np.float32).reshape(-1, 512)
    out = np.empty((x.shape[0], 288), np.uint8)
    (L or lib()).orc_quantize_main(_p(x), x.shape[0], _p(out))
    return out


def quantize_index(x: np.ndarray, L=None):
    """fp32 indexer keys [n][128] -> (codes [n][64], E8M0 scales [n][4])."""
    x = np.ascontiguousarray(x, np.float32).reshape(-1, 128)
    codes = np.empty((x.shape[0], 64), np.uint8)
    scales = np.empty((x.shape[0], 4), np.uint8)
    (L or lib()).orc_quantize_index(_p(x), x.shape[0], _p(codes), _p(scales))
    return codes, scales


def dequant_swa_fp8(rows: np.ndarray, L=None) -> np.ndarray:
    """FP8 window rows [n][528] -> exact values [n][512] (fp64)."""
    rows = np.ascontiguousarray(rows, np.uint8).reshape(-1, 528)
    out = np.empty((rows.shape[0], 512), np.float64)
    (L or lib()).orc_dequant_swa_fp8(_p(rows), rows.shape[0], _p(out))
    return out


def pool_latents(x: np.ndarray, gate: np.ndarray, L=None) -> np.ndarray:
    """m=2 softmax-gated pooling: x [2n][512], gate [2n][512] or [2n][1] -> [n][512] fp64."""
    x = np.ascontiguousarray(x, np.float32).reshape(-1, 512)
    gate = np.ascontiguousarray(gate, np.float32).reshape(x.shape[0], -1)
    n = x.shape[0] // 2
    out = np.empty((n, 512), np.float64)
    (L or lib()).orc_pool_latents(_p(x), _p(gate), gate.shape[1], n, _p(out))
    return out


def gather_selected(main_cache: np.ndarray, n_entries: int, cache_q_stride: int, idx: np.ndarray, L=None):
    """Dense copies [Q][k][288] of each query's selected entries and the dense ids [Q][k]."""
    idx = np.ascontiguousarray(idx, np.int32)
    Q, k = idx.shape
    out = np.empty((Q, k, 288), np.uint8)
    dense = np.empty((Q, k), np.int32)
    (L or lib()).orc_gather_selected(_p(np.ascontiguousarray(main_cache, np.uint8)), n_entries, cache_q_stride,
                                     _p(idx), Q, k, _p(out), _p(dense))
    return out, dense


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, np.float32)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, np.int32)


def index_score(wl, want_dots: bool = False, L=None, queries=None):
    """Scores [Q][n_cand] (fp32) of workload ``wl``; optional exact dots [Q][32][n_cand].

    ``queries`` (optional list of query ids) restricts the computation to those
    queries (rows of the result follow that list)."""
    wl_q = _subset(wl, queries)
    Q, n_cand = wl_q["Q"], wl.n_cand
    scores = np.empty((Q, n_cand), np.float32)
    dots = np.empty((Q, 32, n_cand), np.float64) if want_dots else None
    (L or lib()).orc_index_score(Q, wl.n_entries, wl_q["stride"], _p(wl_q["key_codes"]), _p(wl_q["key_scales"]),
                                 _p(wl_q["iq_codes"]), _p(wl_q["iq_scales"]), _p(wl_q["w"]),
                                 _p(wl_q["cand_blocks"]), wl.n_blocks, _p(wl_q["n_valid"]), _p(scores), _p(dots))
    return (scores, dots) if want_dots else scores


def topk(scores: np.ndarray, wl=None, k: int = 512, n_valid=None, n_entries=None, cand_blocks=None, L=None):
    scores = np.ascontiguousarray(scores, np.float32)
    Q, n_cand = scores.shape
    if wl is not None:
        n_valid = wl.n_valid if n_valid is None else n_valid
        cand_blocks = wl.cand_blocks if cand_blocks is None else cand_blocks
        n_entries = wl.n_entries if n_entries is None else n_entries
    if n_entries is None:
        n_entries = n_cand
    cb = _i32(cand_blocks)
    nb = 0 if cb is None else cb.shape[1]
    idx = np.empty((Q, k), np.int32)
    ts = np.empty((Q, k), np.float32)
    (L or lib()).orc_topk(_p(scores), Q, n_cand, _p(_i32(n_valid)), n_entries, _p(cb), nb, k, _p(idx), _p(ts))
    return idx, ts


def pool_blocks(scores: np.ndarray, n_pool: int = 2048, n_valid=None, L=None) -> np.ndarray:
    """Reindex pool [Q][n_pool] (ascending block ids, -1 padded) from Full-layer
    scores [Q][n_entries] and an optional causal limit [Q]."""
    scores = np.ascontiguousarray(scores, np.float32)
    Q, n = scores.shape
    out = np.empty((Q, n_pool), np.int32)
    (L or lib()).orc_pool_blocks(_p(scores), Q, n, _p(_i32(n_valid)), n_pool, _p(out))
    return out


def sparse_attn(wl, idx: np.ndarray, want_probs: bool = False, L=None, queries=None, n_swa=None):
    """Attention of ``wl``'s queries over ``idx`` [Q][k_sel] + the SWA window.
    Returns (out_bf16 [Q][64][512] uint16, out_f32, lse [Q][64][, probs])."""
    wl_q = _subset(wl, queries)
    idx = np.ascontiguousarray(idx, np.int32)
    Q, k_sel = idx.shape
    assert Q == wl_q["Q"]
    n_swa = wl.n_swa if n_swa is None else n_swa
    ob = np.empty((Q, 64, 512), np.uint16)
    of = np.empty((Q, 64, 512), np.float32)
    lse = np.empty((Q, 64), np.float32)
    probs = np.empty((Q, 64, k_sel + n_swa), np.float64) if want_probs else None
    (L or lib()).orc_sparse_attn(Q, wl.n_entries, wl_q["stride"], _p(wl_q["main_cache"]), _p(idx), k_sel,
                                 _p(wl_q["q"]), _p(wl_q["swa"]), wl_q["swa_q_stride"], n_swa, float(wl.scale), _p(ob),
                                 _p(of), _p(lse), _p(probs), int(wl.swa_format), _p(wl_q["rope"]))
    return (ob, of, lse, probs) if want_probs else (ob, of, lse)


def decode(wl, L=None, queries=None):
    """Fused O2 -> O4 -> O5. Returns dict(out_bf16, out_f32, lse, idx, scores)."""
    wl_q = _subset(wl, queries)
    Q, n_cand, k = wl_q["Q"], wl.n_cand, wl.k
    ob = np.empty((Q, 64, 512), np.uint16)
    of = np.empty((Q, 64, 512), np.float32)
    lse = np.empty((Q, 64), np.float32)
    idx = np.empty((Q, k), np.int32)
    sc = np.empty((Q, n_cand), np.float32)
    (L or lib()).orc_decode(Q, wl.n_entries, wl_q["stride"], _p(wl_q["key_codes"]), _p(wl_q["key_scales"]),
                            _p(wl_q["iq_codes"]), _p(wl_q["iq_scales"]), _p(wl_q["w"]), _p(wl_q["cand_blocks"]),
                            wl.n_blocks, _p(wl_q["n_valid"]), k, _p(wl_q["main_cache"]), _p(wl_q["q"]),
                            _p(wl_q["swa"]), wl_q["swa_q_stride"], wl.n_swa, float(wl.scale), _p(ob), _p(of), _p(lse),
                            _p(idx), _p(sc), int(wl.swa_format), _p(wl_q["rope"]))
    return dict(out_bf16=ob, out_f32=of, lse=lse, idx=idx, scores=sc)


def _subset(wl, queries):
    """View of a workload restricted to some queries. Independent-cache workloads
    slice the caches; shared-cache (stride 0) workloads keep the cache whole."""
    if queries is None:
        return dict(Q=wl.Q, stride=wl.cache_q_stride, key_codes=wl.key_codes, key_scales=wl.key_scales,
                    main_cache=wl.main_cache, iq_codes=wl.iq_codes, iq_scales=wl.iq_scales, w=wl.w, q=wl.q,
                    swa=wl.swa, swa_q_stride=wl.swa_q_stride, cand_blocks=_i32(wl.cand_blocks),
                    n_valid=_i32(wl.n_valid), rope=_f32(wl.rope))
    qs = list(queries)
    N, S = wl.n_entries, wl.cache_q_stride
    if S == 0:
        kc, ks, mc = wl.key_codes, wl.key_scales, wl.main_cache
    else:
        assert wl.extra.get("dense_rows", True), "query subsets need a dense host cache"
        kc = np.ascontiguousarray(np.concatenate([wl.key_codes[i * S:i * S + N] for i in qs]))
        ks = np.ascontiguousarray(np.concatenate([wl.key_scales[i * S:i * S + N] for i in qs]))
        mc = np.ascontiguousarray(np.concatenate([wl.main_cache[i * S:i * S + N] for i in qs]))
    if wl.swa_q_stride >= wl.n_swa:
        R = wl.swa_q_stride
        swa = np.ascontiguousarray(np.concatenate([wl.swa[i * R:i * R + R] for i in qs]))
        swa_stride = R
    else:  # overlapping windows of a shared chunk buffer: give each query its own copy
        swa = np.ascontiguousarray(np.concatenate([wl.swa[i * wl.swa_q_stride:i * wl.swa_q_stride + wl.n_swa]
                                                   for i in qs]))
        swa_stride = wl.n_swa
    return dict(Q=len(qs), stride=(0 if S == 0 else N), key_codes=kc, key_scales=ks, main_cache=mc,
                iq_codes=np.ascontiguousarray(wl.iq_codes[qs]), iq_scales=np.ascontiguousarray(wl.iq_scales[qs]),
                w=np.ascontiguousarray(wl.w[qs]), q=np.ascontiguousarray(wl.q[qs]), swa=swa,
                swa_q_stride=swa_stride,
                cand_blocks=None if wl.cand_blocks is None else np.ascontiguousarray(wl.cand_blocks[qs], np.int32),
                n_valid=None if wl.n_valid is None else np.ascontiguousarray(wl.n_valid[qs], np.int32),
                rope=None if wl.rope is None else np.ascontiguousarray(wl.rope[qs], np.float32))
