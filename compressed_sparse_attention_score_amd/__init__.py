"""Python binding of the CSA2 HIP library (libcsa2.so, C ABI in include/csa2.h).

Argument marshalling only: every function here fills the C argument struct
from torch CUDA tensors (device pointers) and calls the entry point of the same
name on the current HIP stream. All computation happens in the library's
gfx950 kernels. There is no CPU fallback: importing this package fails if the
library is not built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa2.so")

CSA2_OK, CSA2_ERR_NULL, CSA2_ERR_SHAPE, CSA2_ERR_ALIGN, CSA2_ERR_WORKSPACE, CSA2_ERR_HIP, CSA2_ERR_ARG, \
    CSA2_ERR_SCRATCH = range(8)
CSA2_ATTN_SCRATCH_BYTES = 8454144
CSA2_KIND_MAIN, CSA2_KIND_INDEX = 0, 1
CSA2_OUT_F32, CSA2_OUT_BF16 = 0, 1
CSA2_IN_F32, CSA2_IN_BF16 = 0, 1
CSA2_SWA_BF16, CSA2_SWA_FP8 = 0, 1
CSA2_WS_TOPK, CSA2_WS_ATTN, CSA2_WS_DECODE, CSA2_WS_POOL = 0, 1, 2, 3
EXPORTED = ("csa2_dequant", "csa2_quantize", "csa2_pool_quantize", "csa2_build_pool", "csa2_gather_selected",
            "csa2_index_score", "csa2_topk", "csa2_sparse_attn", "csa2_sparse_attn_noalloc", "csa2_decode",
            "csa2_workspace_size",
            "csa2_status_string", "csa2_version")

_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float


class IndexArgs(ctypes.Structure):
    _fields_ = [("struct_size", _sz), ("n_queries", _i32), ("n_entries", _i64), ("cache_q_stride", _i64),
                ("key_codes", _vp), ("key_scales", _vp), ("iq_codes", _vp), ("iq_scales", _vp),
                ("head_weights", _vp), ("cand_blocks", _vp), ("n_blocks", _i32), ("n_valid", _vp)]


class TopkArgs(ctypes.Structure):
    _fields_ = [("struct_size", _sz), ("n_queries", _i32), ("n_cand", _i64), ("n_entries", _i64), ("scores", _vp),
                ("cand_blocks", _vp), ("n_blocks", _i32), ("n_valid", _vp), ("k", _i32), ("idx", _vp),
                ("top_scores", _vp)]


class PoolArgs(ctypes.Structure):
    _fields_ = [("struct_size", _sz), ("n_queries", _i32), ("n_entries", _i64), ("scores", _vp), ("n_valid", _vp),
                ("n_pool_blocks", _i32), ("pool_blocks", _vp)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("struct_size", _sz), ("n_queries", _i32), ("n_entries", _i64), ("cache_q_stride", _i64),
                ("main_cache", _vp), ("idx", _vp), ("k_sel", _i32), ("q", _vp), ("swa", _vp),
                ("swa_q_stride", _i64), ("n_swa", _i32), ("softmax_scale", _f32), ("out", _vp), ("lse", _vp),
                ("swa_format", _i32), ("rope_cos_sin", _vp)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("struct_size", _sz), ("index", IndexArgs), ("k", _i32), ("main_cache", _vp), ("q", _vp),
                ("swa", _vp), ("swa_q_stride", _i64), ("n_swa", _i32), ("softmax_scale", _f32), ("out", _vp),
                ("lse", _vp), ("idx_out", _vp), ("stage_events", _vp * 4), ("swa_format", _i32),
                ("rope_cos_sin", _vp)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"CSA2 HIP library not built: {LIB_PATH} is missing "
                          "(run __graft_entry__.build() or compressed_sparse_attention_score_amd/_build.py)")
    L = ctypes.CDLL(LIB_PATH)
    L.csa2_dequant.argtypes = [ctypes.c_int, _vp, _vp, _i64, ctypes.c_int, _vp, _vp]
    L.csa2_quantize.argtypes = [ctypes.c_int, _vp, ctypes.c_int, _i64, _vp, _i64, _vp, _vp, _vp]
    L.csa2_index_score.argtypes = [ctypes.POINTER(IndexArgs), _vp, _vp]
    L.csa2_build_pool.argtypes = [ctypes.POINTER(PoolArgs), _vp, _sz, _vp]
    L.csa2_pool_quantize.argtypes = [_vp, _vp, ctypes.c_int, _i64, _vp, _i64, _vp, _vp, _vp]
    L.csa2_gather_selected.argtypes = [_vp, _i64, _i64, _vp, _i32, _i32, _vp, _vp, _vp]
    L.csa2_topk.argtypes = [ctypes.POINTER(TopkArgs), _vp, _sz, _vp]
    L.csa2_sparse_attn.argtypes = [ctypes.POINTER(AttnArgs), _vp, _sz, _vp]
    L.csa2_sparse_attn_noalloc.argtypes = [ctypes.POINTER(AttnArgs), _vp]
    L.csa2_decode.argtypes = [ctypes.POINTER(DecodeArgs), _vp, _sz, _vp]
    L.csa2_workspace_size.argtypes = [ctypes.c_int, _vp]
    L.csa2_workspace_size.restype = _sz
    L.csa2_status_string.argtypes = [ctypes.c_int]
    L.csa2_status_string.restype = ctypes.c_char_p
    L.csa2_version.restype = ctypes.c_int
    for name in ("csa2_dequant", "csa2_quantize", "csa2_pool_quantize", "csa2_build_pool", "csa2_gather_selected", "csa2_index_score", "csa2_topk", "csa2_sparse_attn", "csa2_decode"):
        getattr(L, name).restype = ctypes.c_int
    return L


lib = _load()


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: status {status} ({csa2_status_string(status)})")
        self.status = status


def csa2_status_string(status: int) -> str:
    return lib.csa2_status_string(status).decode()


def csa2_version() -> int:
    return lib.csa2_version()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    assert t.is_cuda and t.is_contiguous(), "expected a contiguous CUDA tensor"
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, st):
    if st != CSA2_OK:
        raise Csa2Error(fn, st)


def _alloc_ws(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    # torch allocations are 512-byte aligned
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ----------------------------------------------------------------- entry points

def csa2_dequant(kind: int, codes, scales, n_entries: int, out_dtype: int, out, stream=None) -> None:
    _check("csa2_dequant", lib.csa2_dequant(kind, _ptr(codes), _ptr(scales), n_entries, out_dtype, _ptr(out),
                                            _stream(stream)))


def csa2_quantize(kind: int, x, in_dtype: int, n_entries: int, dst_rows, n_cache_rows: int, codes, scales=None,
                  stream=None) -> None:
    _check("csa2_quantize", lib.csa2_quantize(kind, _ptr(x), in_dtype, n_entries, _ptr(dst_rows), n_cache_rows,
                                              _ptr(codes), _ptr(scales), _stream(stream)))


def csa2_pool_quantize(x, gate, n_entries: int, dst_rows, n_cache_rows: int, cache, pooled=None,
                       stream=None) -> None:
    gate_width = int(gate.shape[-1])
    _check("csa2_pool_quantize", lib.csa2_pool_quantize(_ptr(x), _ptr(gate), gate_width, n_entries, _ptr(dst_rows),
                                                        n_cache_rows, _ptr(cache), _ptr(pooled), _stream(stream)))


def csa2_gather_selected(main_cache, n_entries: int, cache_q_stride: int, idx, out, dense_idx, stream=None) -> None:
    Q, k = int(idx.shape[0]), int(idx.shape[1])
    _check("csa2_gather_selected", lib.csa2_gather_selected(_ptr(main_cache), n_entries, cache_q_stride, _ptr(idx), Q,
                                                            k, _ptr(out), _ptr(dense_idx), _stream(stream)))


def pool_args(scores, n_pool_blocks, pool_blocks, n_valid=None) -> PoolArgs:
    Q, n = int(scores.shape[0]), int(scores.shape[1])
    return PoolArgs(ctypes.sizeof(PoolArgs), Q, n, _ptr(scores), _ptr(n_valid), n_pool_blocks, _ptr(pool_blocks))


def csa2_build_pool(args: PoolArgs, workspace=None, stream=None, device="cuda") -> None:
    need = csa2_workspace_size(CSA2_WS_POOL, args)
    ws = workspace if workspace is not None else _alloc_ws(need, device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_build_pool", lib.csa2_build_pool(ctypes.byref(args), _ptr(ws), nbytes, _stream(stream)))


def index_args(Q, n_entries, cache_q_stride, key_codes, key_scales, iq_codes, iq_scales, head_weights,
               cand_blocks=None, n_valid=None) -> IndexArgs:
    nb = 0 if cand_blocks is None else int(cand_blocks.shape[-1])
    return IndexArgs(ctypes.sizeof(IndexArgs), Q, n_entries, cache_q_stride, _ptr(key_codes), _ptr(key_scales),
                     _ptr(iq_codes), _ptr(iq_scales), _ptr(head_weights), _ptr(cand_blocks), nb, _ptr(n_valid))


def csa2_index_score(args: IndexArgs, scores, stream=None) -> None:
    _check("csa2_index_score", lib.csa2_index_score(ctypes.byref(args), _ptr(scores), _stream(stream)))


def topk_args(scores, n_entries, k, idx, top_scores=None, cand_blocks=None, n_valid=None) -> TopkArgs:
    Q, n_cand = int(scores.shape[0]), int(scores.shape[1])
    nb = 0 if cand_blocks is None else int(cand_blocks.shape[-1])
    return TopkArgs(ctypes.sizeof(TopkArgs), Q, n_cand, n_entries, _ptr(scores), _ptr(cand_blocks), nb, _ptr(n_valid),
                    k, _ptr(idx), _ptr(top_scores))


def csa2_workspace_size(which: int, args) -> int:
    n = lib.csa2_workspace_size(which, ctypes.cast(ctypes.byref(args), _vp))
    if n == ctypes.c_size_t(-1).value:
        raise Csa2Error("csa2_workspace_size", CSA2_ERR_ARG)
    return n


def csa2_topk(args: TopkArgs, workspace=None, stream=None, device="cuda") -> None:
    need = csa2_workspace_size(CSA2_WS_TOPK, args)
    ws = workspace if workspace is not None else _alloc_ws(need, device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_topk", lib.csa2_topk(ctypes.byref(args), _ptr(ws), nbytes, _stream(stream)))


def attn_args(Q, n_entries, cache_q_stride, main_cache, idx, q, swa, swa_q_stride, n_swa, softmax_scale, out,
              lse=None, swa_format=CSA2_SWA_BF16, rope_cos_sin=None) -> AttnArgs:
    k_sel = 0 if idx is None else int(idx.shape[-1])
    return AttnArgs(ctypes.sizeof(AttnArgs), Q, n_entries, cache_q_stride, _ptr(main_cache), _ptr(idx), k_sel, _ptr(q),
                    _ptr(swa), swa_q_stride, n_swa, softmax_scale, _ptr(out), _ptr(lse), swa_format,
                    _ptr(rope_cos_sin))


def csa2_sparse_attn(args: AttnArgs, workspace=None, stream=None, device="cuda") -> None:
    need = csa2_workspace_size(CSA2_WS_ATTN, args)
    ws = workspace if workspace is not None else _alloc_ws(need, device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_sparse_attn", lib.csa2_sparse_attn(ctypes.byref(args), _ptr(ws), nbytes, _stream(stream)))


def csa2_sparse_attn_noalloc(args: AttnArgs, stream=None) -> None:
    _check("csa2_sparse_attn_noalloc", lib.csa2_sparse_attn_noalloc(ctypes.byref(args), _stream(stream)))


def decode_args(index: IndexArgs, k, main_cache, q, swa, swa_q_stride, n_swa, softmax_scale, out, lse=None,
                idx_out=None, stage_events=None, swa_format=CSA2_SWA_BF16, rope_cos_sin=None) -> DecodeArgs:
    ev = (_vp * 4)(*(stage_events or (None, None, None, None)))
    return DecodeArgs(ctypes.sizeof(DecodeArgs), index, k, _ptr(main_cache), _ptr(q), _ptr(swa), swa_q_stride, n_swa,
                      softmax_scale, _ptr(out), _ptr(lse), _ptr(idx_out), ev, swa_format, _ptr(rope_cos_sin))


def csa2_decode(args: DecodeArgs, workspace=None, stream=None, device="cuda") -> None:
    need = csa2_workspace_size(CSA2_WS_DECODE, args)
    ws = workspace if workspace is not None else _alloc_ws(need, device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_decode", lib.csa2_decode(ctypes.byref(args), _ptr(ws), nbytes, _stream(stream)))
