"""Seeded synthetic inputs for the CSA2 path (shared by the oracle and the HIP side).

The C source ``csa2_synth.c`` defines the random streams and the storage
quantisation of the inputs; this module builds it with gcc, loads it, and
assembles whole workloads as numpy arrays. Nothing here scores, selects or
attends.

Stream ids (the ``tensor_id`` of the counter): 0 main latents, 1 indexer keys,
2 indexer queries, 3 head weights, 4 attention queries, 5 SWA rows, 6 pool blocks,
7 m=2 pooling gate logits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_synth.c")
_LIB = os.path.join(_HERE, "libcsa2synth.so")

TID_MAIN, TID_IKEY, TID_IQ, TID_W, TID_Q, TID_SWA, TID_POOL, TID_GATE = range(8)

MAIN_BYTES = 288
IKEY_CODE_BYTES = 64
IKEY_SCALE_BYTES = 4
N_IHEADS = 32
N_HEADS = 64
HEAD_DIM = 512
TOPK = 512
N_SWA = 128
SWA_FP8_BYTES = 528
BLOCK = 8


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.syn_normal.restype = ctypes.c_double
        L.syn_normal.argtypes = [u64, i32, u64, u64]
        L.syn_bits.restype = u64
        L.syn_bits.argtypes = [u64, i32, u64, u64]
        L.syn_main_latents.argtypes = [u64, u64, i64, i64, vp]
        L.syn_main_latents_list.argtypes = [u64, u64, vp, i64, vp]
        L.syn_index_keys.argtypes = [u64, u64, i64, i64, vp, vp]
        L.syn_index_keys_list.argtypes = [u64, u64, vp, i64, vp, vp]
        L.syn_index_queries.argtypes = [u64, i64, i64, vp, vp]
        L.syn_head_weights.argtypes = [u64, i64, i64, vp]
        L.syn_bf16_normal.argtypes = [u64, i32, u64, i64, i64, vp]
        L.syn_pool_blocks.argtypes = [u64, u64, i64, i64, vp]
        L.syn_bf16_rows.argtypes = [u64, i32, u64, i64, i64, i32, vp]
        L.syn_f32_rows.argtypes = [u64, i32, u64, i64, i64, i32, vp]
        L.syn_fp8_rows.argtypes = [u64, i32, u64, i64, i64, vp]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def main_latents(seed: int, seq: int, first: int, n: int) -> np.ndarray:
    out = np.empty((n, MAIN_BYTES), np.uint8)
    lib().syn_main_latents(seed, seq, first, n, _p(out))
    return out


def main_latents_list(seed: int, seq: int, ids: np.ndarray) -> np.ndarray:
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    out = np.empty((len(ids), MAIN_BYTES), np.uint8)
    lib().syn_main_latents_list(seed, seq, _p(ids), len(ids), _p(out))
    return out


def index_keys(seed: int, seq: int, first: int, n: int):
    codes = np.empty((n, IKEY_CODE_BYTES), np.uint8)
    scales = np.empty((n, IKEY_SCALE_BYTES), np.uint8)
    lib().syn_index_keys(seed, seq, first, n, _p(codes), _p(scales))
    return codes, scales


def index_keys_list(seed: int, seq: int, ids: np.ndarray):
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    codes = np.empty((len(ids), IKEY_CODE_BYTES), np.uint8)
    scales = np.empty((len(ids), IKEY_SCALE_BYTES), np.uint8)
    lib().syn_index_keys_list(seed, seq, _p(ids), len(ids), _p(codes), _p(scales))
    return codes, scales


def index_queries(seed: int, first: int, n: int):
    codes = np.empty((n, N_IHEADS, IKEY_CODE_BYTES), np.uint8)
    scales = np.empty((n, N_IHEADS, IKEY_SCALE_BYTES), np.uint8)
    lib().syn_index_queries(seed, first, n, _p(codes), _p(scales))
    return codes, scales


def head_weights(seed: int, first: int, n: int) -> np.ndarray:
    w = np.empty((n, N_IHEADS), np.float32)
    lib().syn_head_weights(seed, first, n, _p(w))
    return w


def bf16_normal(seed: int, tid: int, seq: int, first: int, n: int) -> np.ndarray:
    out = np.empty((n,), np.uint16)
    lib().syn_bf16_normal(seed, tid, seq, first, n, _p(out))
    return out


def bf16_rows(seed: int, tid: int, seq: int, first_row: int, n_rows: int, width: int) -> np.ndarray:
    out = np.empty((n_rows, width), np.uint16)
    lib().syn_bf16_rows(seed, tid, seq, first_row, n_rows, width, _p(out))
    return out


def f32_rows(seed: int, tid: int, seq: int, first_row: int, n_rows: int, width: int) -> np.ndarray:
    """fp32 N(0,1) rows; on streams TID_MAIN / TID_IKEY (width 512 / 128) these
    are the unquantised sources of the stored entries ``first_row ...``."""
    assert width % 2 == 0
    out = np.empty((n_rows, width), np.float32)
    lib().syn_f32_rows(seed, tid, seq, first_row, n_rows, width, _p(out))
    return out


def fp8_rows(seed: int, tid: int, seq: int, first_row: int, n_rows: int) -> np.ndarray:
    """MXFP8 window rows [n_rows][528] of stream (tid, seq): the same N(0,1)
    elements as ``bf16_rows(..., width=512)``, quantised to E4M3 codes with an
    E8M0 scale per 32 channels."""
    out = np.empty((n_rows, SWA_FP8_BYTES), np.uint8)
    lib().syn_fp8_rows(seed, tid, seq, first_row, n_rows, _p(out))
    return out


def rope_table(positions, base: float = 10000.0) -> np.ndarray:
    """(cos, sin) [len(positions)][32][2] fp32 of standard RoPE angles
    position * base^(-2i/64) over the 32 rotary pairs (input data for the
    attention epilogue's un-rotation; the model's own table may differ)."""
    pos = np.asarray(positions, np.float64)[:, None]
    inv_freq = base ** (-np.arange(0, 64, 2, dtype=np.float64) / 64.0)
    ang = pos * inv_freq[None, :]
    return np.ascontiguousarray(np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32))


def pool_blocks(seed: int, seq: int, n_pick: int, n_total: int) -> np.ndarray:
    out = np.empty((n_pick,), np.int32)
    lib().syn_pool_blocks(seed, seq, n_pick, n_total, _p(out))
    return out


# Poison bytes for cache entries that a kernel must never read: NaN scales
# (E4M3 0x7F, E8M0 0xFF) so any stray read turns outputs into NaN.
POISON_E4M3 = 0x7F
POISON_E8M0 = 0xFF


@dataclass
class Workload:
    """One batch of the CSA2 path, all host arrays.

    Layouts (C-contiguous):
      main_cache  uint8 [rows][288]     key_codes uint8 [rows][64]   key_scales uint8 [rows][4]
      iq_codes    uint8 [Q][32][64]     iq_scales uint8 [Q][32][4]   w float32 [Q][32]
      q           uint16(bf16) [Q][64][512]
      swa         uint16(bf16) [swa_rows][512], or uint8 [swa_rows][528] FP8 rows when
                  swa_format == 1; query i's window starts at row i*swa_q_stride
      cand_blocks int32 [Q][n_blocks] or None   n_valid int32 [Q] or None
      rope        float32 [Q][32][2] (cos, sin) or None
    Query i's cache occupies rows [i*cache_q_stride, i*cache_q_stride + n_entries).
    Entries listed in ``sparse_rows`` (if not None) are the only ones holding data;
    all other rows are poison.
    """

    name: str
    Q: int
    n_entries: int
    cache_q_stride: int
    main_cache: np.ndarray
    key_codes: np.ndarray
    key_scales: np.ndarray
    iq_codes: np.ndarray
    iq_scales: np.ndarray
    w: np.ndarray
    q: np.ndarray
    swa: np.ndarray
    swa_q_stride: int
    n_swa: int
    cand_blocks: Optional[np.ndarray] = None
    n_valid: Optional[np.ndarray] = None
    k: int = TOPK
    scale: float = 1.0 / np.sqrt(512.0)
    extra: dict = field(default_factory=dict)
    swa_format: int = 0
    rope: Optional[np.ndarray] = None

    @property
    def n_blocks(self) -> int:
        return 0 if self.cand_blocks is None else int(self.cand_blocks.shape[1])

    @property
    def n_cand(self) -> int:
        return self.n_blocks * BLOCK if self.cand_blocks is not None else self.n_entries


def _swa_rows(seed, seq, n_rows, fp8):
    return fp8_rows(seed, TID_SWA, seq, 0, n_rows) if fp8 else bf16_rows(seed, TID_SWA, seq, 0, n_rows, HEAD_DIM)


def _queries(seed, Q, swa_rows_per_query, shared_swa_rows=None, swa_fp8=False):
    iq_codes, iq_scales = index_queries(seed, 0, Q)
    w = head_weights(seed, 0, Q)
    q = np.stack([bf16_rows(seed, TID_Q, i, 0, N_HEADS, HEAD_DIM) for i in range(Q)])
    if shared_swa_rows is None:
        swa = np.stack([_swa_rows(seed, i, swa_rows_per_query, swa_fp8) for i in range(Q)])
        swa = swa.reshape(Q * swa_rows_per_query, -1)
    else:
        swa = _swa_rows(seed, 0, shared_swa_rows, swa_fp8)
    return iq_codes, iq_scales, w, q, np.ascontiguousarray(swa)


def with_window_options(wl: Workload, positions=None, swa_fp8: bool = False, rope: bool = False) -> Workload:
    """Attach the optional window format and RoPE table to a built workload:
    ``swa_fp8`` regenerates its window rows as FP8 from the same streams
    (row layout unchanged), ``rope`` adds the (cos, sin) table of ``positions``
    (default: entry count + 7 i for decode queries)."""
    seed = wl.extra.get("seed", 0)
    if swa_fp8:
        if wl.extra.get("shared_swa"):
            wl.swa = _swa_rows(seed, 0, wl.swa.shape[0], True)
        else:
            per = wl.swa.shape[0] // max(wl.Q, 1)
            wl.swa = np.ascontiguousarray(np.concatenate([_swa_rows(seed, i, per, True) for i in range(wl.Q)])
                                          if wl.Q else np.zeros((0, SWA_FP8_BYTES), np.uint8))
        wl.swa_format = 1
    if rope:
        if positions is None:
            positions = (wl.extra["t0"] + np.arange(wl.Q)) if "t0" in wl.extra else wl.n_entries + 7 * np.arange(wl.Q)
        wl.rope = rope_table(positions)
    return wl


def full_decode(Q: int, N: int, seed: int = 0, n_swa: int = N_SWA, name: str = "full_decode") -> Workload:
    """Full-layer decode: Q queries, each with its own cache of N entries (m=1)."""
    main = np.concatenate([main_latents(seed, i, 0, N) for i in range(Q)]) if N else np.zeros((0, MAIN_BYTES), np.uint8)
    kc, ks = zip(*[index_keys(seed, i, 0, N) for i in range(Q)]) if N else ((np.zeros((0, 64), np.uint8),), (np.zeros((0, 4), np.uint8),))
    iq_codes, iq_scales, w, q, swa = _queries(seed, Q, n_swa)
    wl = Workload(name, Q, N, N, main, np.concatenate(kc), np.concatenate(ks), iq_codes, iq_scales, w, q,
                  swa, n_swa, n_swa)
    wl.extra["seed"] = seed
    return wl


def reindex_decode(Q: int, N: int, n_blocks: int, seed: int = 0, dense_rows: bool = True,
                   name: str = "reindex_decode") -> Workload:
    """Reindex-layer decode: each query's cache has N entries; a pool of n_blocks
    distinct aligned blocks of 8 is drawn per query. Only pool entries hold data,
    every other entry is poison.

    dense_rows=True materialises the full Q*N-row cache on the host (small N only);
    otherwise ``extra['pool_rows']`` lists the pool rows and ``main_cache`` etc.
    hold only those rows (the caller scatters them into a poisoned device cache).
    """
    blocks = np.stack([pool_blocks(seed, i, n_blocks, N // BLOCK) for i in range(Q)])
    ids = [(BLOCK * blocks[i][:, None] + np.arange(BLOCK)[None, :]).reshape(-1).astype(np.int64) for i in range(Q)]
    main_rows = [main_latents_list(seed, i, ids[i]) for i in range(Q)]
    key_rows = [index_keys_list(seed, i, ids[i]) for i in range(Q)]
    iq_codes, iq_scales, w, q, swa = _queries(seed, Q, N_SWA)
    pool_rows = np.concatenate([i * N + ids[i] for i in range(Q)])
    pm = np.concatenate(main_rows)
    pkc = np.concatenate([k[0] for k in key_rows])
    pks = np.concatenate([k[1] for k in key_rows])
    if dense_rows:
        main = np.zeros((Q * N, MAIN_BYTES), np.uint8)
        main[:, 256:] = POISON_E4M3
        kc = np.zeros((Q * N, IKEY_CODE_BYTES), np.uint8)
        ks = np.full((Q * N, IKEY_SCALE_BYTES), POISON_E8M0, np.uint8)
        main[pool_rows] = pm
        kc[pool_rows] = pkc
        ks[pool_rows] = pks
        wl = Workload(name, Q, N, N, main, kc, ks, iq_codes, iq_scales, w, q, swa, N_SWA, N_SWA,
                      cand_blocks=blocks.astype(np.int32))
    else:
        wl = Workload(name, Q, N, N, pm, pkc, pks, iq_codes, iq_scales, w, q, swa, N_SWA, N_SWA,
                      cand_blocks=blocks.astype(np.int32))
    wl.extra["pool_rows"] = pool_rows
    wl.extra["dense_rows"] = dense_rows
    wl.extra["seed"] = seed
    return wl


def prefill(T: int, n_cache: int, t0: int, seed: int = 0, m: int = 2, name: str = "prefill") -> Workload:
    """Encoder Full-layer prefill chunk: T queries at positions t0..t0+T-1 against a
    shared m-pooled cache of n_cache entries; query at position t sees entries
    with index < floor(t/m) and its own 128-token window, rows i..i+127 of a
    shared chunk buffer of T+127 bf16 rows."""
    main = main_latents(seed, 0, 0, n_cache)
    kc, ks = index_keys(seed, 0, 0, n_cache)
    iq_codes, iq_scales, w, q, swa = _queries(seed, T, 0, shared_swa_rows=T + N_SWA - 1)
    n_valid = np.array([(t0 + i) // m for i in range(T)], np.int64)
    n_valid = np.minimum(n_valid, n_cache).astype(np.int32)
    wl = Workload(name, T, n_cache, 0, main, kc, ks, iq_codes, iq_scales, w, q, swa, 1, N_SWA, n_valid=n_valid)
    wl.extra["t0"] = t0
    wl.extra["seed"] = seed
    wl.extra["shared_swa"] = True
    return wl


# The five workload shapes of the CSA2 decode/prefill hot path, by index.
WORKLOADS = {
    0: dict(kind="full_decode", Q=1, N=4096),
    1: dict(kind="full_decode", Q=16, N=65536),
    2: dict(kind="reindex_decode", Q=64, N=1 << 20, n_blocks=2048),
    3: dict(kind="prefill", T=4096, n_cache=131072, t0=258048),
    4: dict(kind="full_decode", Q=4, N=1 << 20),
}

WORKLOAD_NAMES = {
    0: "full-layer decode, 1 query x 4,096 entries",
    1: "full-layer decode, batch 16 x 65,536 entries",
    2: "reindex-layer decode, batch 64, 16,384-entry pool of a 1,048,576-entry cache",
    3: "encoder full-layer prefill, 4,096 queries x 131,072-entry m=2 cache (causal)",
    4: "long-context full-layer decode, batch 4 x 1,048,576 entries",
}


def make_workload(i: int, seed: int = 0, dense_rows: Optional[bool] = None) -> Workload:
    c = WORKLOADS[i]
    name = WORKLOAD_NAMES[i]
    if c["kind"] == "full_decode":
        return full_decode(c["Q"], c["N"], seed, name=name)
    if c["kind"] == "reindex_decode":
        return reindex_decode(c["Q"], c["N"], c["n_blocks"], seed, dense_rows=bool(dense_rows), name=name)
    return prefill(c["T"], c["n_cache"], c["t0"], seed, name=name)


def compact_pool_view(wl: Workload) -> Workload:
    """A Reindex workload built with dense_rows=False holds only the pool rows
    (query-major, blocks in ascending id). This view renumbers query i's pool
    as entries 0..8*n_blocks-1 of its own cache, so a host consumer that wants
    dense rows can run on it; entry j of the view is pool_ids(wl, i)[j]."""
    assert wl.cand_blocks is not None and not wl.extra.get("dense_rows", True)
    nb = wl.n_blocks
    return Workload(wl.name + "-compact", wl.Q, 8 * nb, 8 * nb, wl.main_cache, wl.key_codes, wl.key_scales,
                    wl.iq_codes, wl.iq_scales, wl.w, wl.q, wl.swa, wl.swa_q_stride, wl.n_swa,
                    cand_blocks=np.tile(np.arange(nb, dtype=np.int32), (wl.Q, 1)), k=wl.k, scale=wl.scale)


def pool_ids(wl: Workload, i: int) -> np.ndarray:
    """Global entry ids of query i's candidate pool, ascending."""
    return (8 * wl.cand_blocks[i][:, None].astype(np.int64) + np.arange(8)[None, :]).reshape(-1)
