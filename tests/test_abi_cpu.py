"""The C-ABI library on the host (no GPU): it loads, exports exactly what
include/csa2.h declares, the binding's structs match the header's layout, and
argument validation rejects bad calls before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

import compressed_sparse_attention_score_amd as csa  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"CSA2_API\s+[\w\s\*]+?\b(csa2_\w+)\s*\(", text)))


def test_library_exports_declared_symbols():
    names = declared_functions()
    assert names == sorted(csa.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", csa.LIB_PATH], capture_output=True, text=True, check=True)
    exported = sorted({l.split()[-1] for l in out.stdout.splitlines() if l.split()[-1].startswith("csa2_")})
    assert exported == names
    for n in names:
        assert hasattr(csa.lib, n)


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "csa2.h"\n'
                   '#define P(s, f) printf(#s "." #f " %zu\\n", offsetof(s, f));\n'
                   'int main(void){\n'
                   'printf("csa2_index_args %zu\\n", sizeof(csa2_index_args));\n'
                   'printf("csa2_topk_args %zu\\n", sizeof(csa2_topk_args));\n'
                   'printf("csa2_attn_args %zu\\n", sizeof(csa2_attn_args));\n'
                   'printf("csa2_decode_args %zu\\n", sizeof(csa2_decode_args));\n'
                   'P(csa2_index_args, n_valid) P(csa2_topk_args, top_scores) P(csa2_attn_args, lse)\n'
                   'P(csa2_decode_args, idx_out) P(csa2_decode_args, index) P(csa2_attn_args, softmax_scale)\n'
                   'P(csa2_decode_args, stage_events)\n'
                   'return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I" + os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    vals = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                          check=True).stdout.splitlines())
    assert int(vals["csa2_index_args"]) == ctypes.sizeof(csa.IndexArgs)
    assert int(vals["csa2_topk_args"]) == ctypes.sizeof(csa.TopkArgs)
    assert int(vals["csa2_attn_args"]) == ctypes.sizeof(csa.AttnArgs)
    assert int(vals["csa2_decode_args"]) == ctypes.sizeof(csa.DecodeArgs)
    assert int(vals["csa2_index_args.n_valid"]) == csa.IndexArgs.n_valid.offset
    assert int(vals["csa2_topk_args.top_scores"]) == csa.TopkArgs.top_scores.offset
    assert int(vals["csa2_attn_args.lse"]) == csa.AttnArgs.lse.offset
    assert int(vals["csa2_attn_args.softmax_scale"]) == csa.AttnArgs.softmax_scale.offset
    assert int(vals["csa2_decode_args.idx_out"]) == csa.DecodeArgs.idx_out.offset
    assert int(vals["csa2_decode_args.index"]) == csa.DecodeArgs.index.offset
    assert int(vals["csa2_decode_args.stage_events"]) == csa.DecodeArgs.stage_events.offset


def test_status_strings_and_version():
    assert csa.csa2_version() == 200
    for s in range(8):
        assert csa.csa2_status_string(s) != "unknown status"
    assert csa.csa2_status_string(99) == "unknown status"


def _fake(addr):  # host-side fake device addresses: validation never dereferences them
    return addr


def test_validation_rejects_before_launch():
    L = csa.lib
    A = 0x10000  # 16-B aligned fake pointer
    # dequant
    assert L.csa2_dequant(5, A, A, 10, 0, A, None) == csa.CSA2_ERR_ARG
    assert L.csa2_dequant(0, A, A, 10, 9, A, None) == csa.CSA2_ERR_ARG
    assert L.csa2_dequant(0, None, None, 10, 0, A, None) == csa.CSA2_ERR_NULL
    assert L.csa2_dequant(1, A, None, 10, 0, A, None) == csa.CSA2_ERR_NULL
    assert L.csa2_dequant(0, A + 8, None, 10, 0, A, None) == csa.CSA2_ERR_ALIGN
    assert L.csa2_dequant(0, A, None, -1, 0, A, None) == csa.CSA2_ERR_SHAPE
    assert L.csa2_dequant(0, None, None, 0, 0, None, None) == csa.CSA2_OK  # empty: no-op
    # quantize
    assert L.csa2_quantize(2, A, 0, 10, None, 10, A, A, None) == csa.CSA2_ERR_ARG
    assert L.csa2_quantize(0, A, 3, 10, None, 10, A, A, None) == csa.CSA2_ERR_ARG
    assert L.csa2_quantize(0, A, 0, 10, None, 9, A, None, None) == csa.CSA2_ERR_SHAPE  # cache too small
    assert L.csa2_quantize(0, A, 0, -1, None, 10, A, None, None) == csa.CSA2_ERR_SHAPE
    assert L.csa2_quantize(1, A, 0, 10, None, 10, A, None, None) == csa.CSA2_ERR_NULL
    assert L.csa2_quantize(0, None, 0, 10, None, 10, A, None, None) == csa.CSA2_ERR_NULL
    assert L.csa2_quantize(0, A + 8, 0, 10, None, 10, A, None, None) == csa.CSA2_ERR_ALIGN  # fp32 needs 16 B
    assert L.csa2_quantize(0, A + 4, 1, 10, None, 10, A, None, None) == csa.CSA2_ERR_ALIGN  # bf16 needs 8 B
    assert L.csa2_quantize(0, A, 0, 10, A + 4, 3, A, None, None) == csa.CSA2_ERR_ALIGN
    assert L.csa2_quantize(0, None, 0, 0, None, 0, None, None, None) == csa.CSA2_OK  # empty: no-op
    # m=2 pooling + quantise
    assert L.csa2_pool_quantize(A, A, 3, 10, None, 10, A, None, None) == csa.CSA2_ERR_ARG
    assert L.csa2_pool_quantize(A, A, 512, 10, None, 9, A, None, None) == csa.CSA2_ERR_SHAPE
    assert L.csa2_pool_quantize(None, A, 512, 10, None, 10, A, None, None) == csa.CSA2_ERR_NULL
    assert L.csa2_pool_quantize(A, None, 1, 10, None, 10, A, None, None) == csa.CSA2_ERR_NULL
    assert L.csa2_pool_quantize(A, A + 4, 512, 10, None, 10, A, None, None) == csa.CSA2_ERR_ALIGN
    assert L.csa2_pool_quantize(A, A + 4, 1, 10, None, 10, A, A + 8, None) == csa.CSA2_ERR_ALIGN
    assert L.csa2_pool_quantize(None, None, 1, 0, None, 0, None, None, None) == csa.CSA2_OK
    # gather of the selected entries
    assert L.csa2_gather_selected(A, 100, 100, A, 2, 1025, A, A, None) == csa.CSA2_ERR_SHAPE
    assert L.csa2_gather_selected(A, 100, 100, None, 2, 512, A, A, None) == csa.CSA2_ERR_NULL
    assert L.csa2_gather_selected(A, 100, 100, A, 2, 512, A + 8, A, None) == csa.CSA2_ERR_ALIGN
    assert L.csa2_gather_selected(None, 100, 100, None, 2, 0, None, None, None) == csa.CSA2_OK
    # pool construction
    pa = csa.PoolArgs(ctypes.sizeof(csa.PoolArgs), 2, 1000, A, None, 2048, A)
    for field, value, code in (("n_pool_blocks", 0, csa.CSA2_ERR_SHAPE), ("n_pool_blocks", 8193, csa.CSA2_ERR_SHAPE),
                               ("n_entries", 1 << 31, csa.CSA2_ERR_SHAPE), ("scores", None, csa.CSA2_ERR_NULL),
                               ("pool_blocks", None, csa.CSA2_ERR_NULL), ("scores", A + 2, csa.CSA2_ERR_ALIGN),
                               ("struct_size", 8, csa.CSA2_ERR_ARG)):
        bad = csa.PoolArgs.from_buffer_copy(pa)
        setattr(bad, field, value)
        assert L.csa2_build_pool(ctypes.byref(bad), A, 1 << 30, None) == code, field
    need = csa.csa2_workspace_size(csa.CSA2_WS_POOL, pa)
    assert need >= 2 * 125 * 4
    assert L.csa2_build_pool(ctypes.byref(pa), A, need - 1, None) == csa.CSA2_ERR_WORKSPACE
    # index score
    ia = csa.IndexArgs(ctypes.sizeof(csa.IndexArgs), 2, 100, 100, A, A, A, A, A, None, 0, None)
    bad = csa.IndexArgs.from_buffer_copy(ia)
    bad.struct_size = 8
    assert L.csa2_index_score(ctypes.byref(bad), A, None) == csa.CSA2_ERR_ARG
    bad = csa.IndexArgs.from_buffer_copy(ia)
    bad.key_codes = A + 4
    assert L.csa2_index_score(ctypes.byref(bad), A, None) == csa.CSA2_ERR_ALIGN
    bad = csa.IndexArgs.from_buffer_copy(ia)
    bad.iq_codes = None
    assert L.csa2_index_score(ctypes.byref(bad), A, None) == csa.CSA2_ERR_NULL
    bad = csa.IndexArgs.from_buffer_copy(ia)
    bad.n_entries = 1 << 31
    assert L.csa2_index_score(ctypes.byref(bad), A, None) == csa.CSA2_ERR_SHAPE
    bad = csa.IndexArgs.from_buffer_copy(ia)
    bad.n_blocks = 3  # blocks without a block list
    assert L.csa2_index_score(ctypes.byref(bad), A, None) == csa.CSA2_ERR_SHAPE
    assert L.csa2_index_score(ctypes.byref(ia), None, None) == csa.CSA2_ERR_NULL
    empty = csa.IndexArgs.from_buffer_copy(ia)
    empty.n_queries = 0
    assert L.csa2_index_score(ctypes.byref(empty), None, None) == csa.CSA2_OK
    # top-k
    ta = csa.TopkArgs(ctypes.sizeof(csa.TopkArgs), 2, 1000, 1000, A, None, 0, None, 512, A, None)
    for field, value, code in (("k", 0, csa.CSA2_ERR_SHAPE), ("k", 1025, csa.CSA2_ERR_SHAPE),
                               ("n_blocks", 5, csa.CSA2_ERR_SHAPE), ("idx", None, csa.CSA2_ERR_NULL),
                               ("scores", A + 2, csa.CSA2_ERR_ALIGN), ("struct_size", 4, csa.CSA2_ERR_ARG)):
        bad = csa.TopkArgs.from_buffer_copy(ta)
        setattr(bad, field, value)
        assert L.csa2_topk(ctypes.byref(bad), A, 1 << 30, None) == code, field
    need = csa.csa2_workspace_size(csa.CSA2_WS_TOPK, ta)
    assert need > 0
    assert L.csa2_topk(ctypes.byref(ta), None, 0, None) == csa.CSA2_ERR_WORKSPACE
    assert L.csa2_topk(ctypes.byref(ta), A, need - 1, None) == csa.CSA2_ERR_WORKSPACE
    assert L.csa2_topk(ctypes.byref(ta), A + 16, need, None) == csa.CSA2_ERR_ALIGN
    # attention
    aa = csa.AttnArgs(ctypes.sizeof(csa.AttnArgs), 4, 100, 100, A, A, 512, A, A, 128, 128, 0.04, A, None)
    for field, value, code in (("k_sel", 1025, csa.CSA2_ERR_SHAPE), ("n_swa", 129, csa.CSA2_ERR_SHAPE),
                               ("swa", None, csa.CSA2_ERR_NULL), ("q", A + 4, csa.CSA2_ERR_ALIGN),
                               ("out", None, csa.CSA2_ERR_NULL), ("idx", None, csa.CSA2_ERR_NULL),
                               ("swa_format", 2, csa.CSA2_ERR_ARG), ("rope_cos_sin", A + 4, csa.CSA2_ERR_ALIGN)):
        bad = csa.AttnArgs.from_buffer_copy(aa)
        setattr(bad, field, value)
        assert L.csa2_sparse_attn(ctypes.byref(bad), A, 1 << 30, None) == code, field
        assert L.csa2_sparse_attn_noalloc(ctypes.byref(bad), None) == code, field
    need = csa.csa2_workspace_size(csa.CSA2_WS_ATTN, aa)
    assert need > 0  # 4 queries split their slot list
    assert L.csa2_sparse_attn(ctypes.byref(aa), A, need - 1, None) == csa.CSA2_ERR_WORKSPACE
    big = csa.AttnArgs.from_buffer_copy(aa)
    big.n_queries = 2000  # enough workgroups without splitting: no workspace
    assert csa.csa2_workspace_size(csa.CSA2_WS_ATTN, big) == 0
    # decode
    da = csa.DecodeArgs(ctypes.sizeof(csa.DecodeArgs), ia, 512, A, A, A, 128, 128, 0.04, A, None, None,
                        (ctypes.c_void_p * 4)())
    bad = csa.DecodeArgs.from_buffer_copy(da)
    bad.k = 0
    assert L.csa2_decode(ctypes.byref(bad), A, 1 << 30, None) == csa.CSA2_ERR_SHAPE
    bad = csa.DecodeArgs.from_buffer_copy(da)
    bad.swa_format = -1
    assert L.csa2_decode(ctypes.byref(bad), A, 1 << 30, None) == csa.CSA2_ERR_ARG
    need = csa.csa2_workspace_size(csa.CSA2_WS_DECODE, da)
    assert need >= 2 * 100 * 4
    assert L.csa2_decode(ctypes.byref(da), A, need - 1, None) == csa.CSA2_ERR_WORKSPACE
    # invalid workspace queries
    assert L.csa2_workspace_size(7, ctypes.cast(ctypes.byref(da), ctypes.c_void_p)) == ctypes.c_size_t(-1).value
    assert L.csa2_workspace_size(0, None) == ctypes.c_size_t(-1).value
