"""GPU parity: every C-ABI entry point against the CPU oracle on the same
seeded inputs (small ragged cases spanning several tiles, edge cases, and the
five workload shapes at full size)."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_util import (QueryView, announce, bf16_np_to_f64, block_abs_dots, check_attn, check_lse, check_scores,
                      check_topk_band, gpu_attn, gpu_decode, gpu_scores, gpu_topk, oracle, to_device)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_sparse_attention_score_amd as csa


@pytest.fixture(autouse=True)
def _name(request):
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ dequant

def _dq(kind, codes, scales, n, bf16):
    width = 512 if kind == 0 else 128
    out = torch.empty((n, width), dtype=torch.int16 if bf16 else torch.float32, device="cuda")
    c = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
    s = None if scales is None else torch.from_numpy(np.ascontiguousarray(scales)).cuda()
    csa.csa2_dequant(kind, c, s, n, 1 if bf16 else 0, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _bits_equal_nan(a32, b32):
    an, bn = np.isnan(a32), np.isnan(b32)
    assert np.array_equal(an, bn)
    assert np.array_equal(a32[~an].view(np.uint32), b32[~bn].view(np.uint32))


def test_dequant_main_bitexact():
    main = synth.main_latents(7, 0, 0, 1001)
    sweep = np.zeros((256, 288), np.uint8)
    sweep[:, :256] = np.arange(256, dtype=np.uint8)[None, :]
    sweep[:, 256:] = np.arange(256, dtype=np.uint8)[:, None]
    ent = np.concatenate([main, sweep])
    f_ref, b_ref = oracle.dequant_main(ent)
    f = _dq(0, ent, None, len(ent), False)
    _bits_equal_nan(f, f_ref)
    b = _dq(0, ent, None, len(ent), True).view(np.uint16)
    bn = np.isnan(bf16_np_to_f64(b))
    assert np.array_equal(bn, np.isnan(f_ref))
    assert np.array_equal(b[~bn], b_ref[~bn])


def test_dequant_index_bitexact():
    kc, ks = synth.index_keys(7, 0, 0, 999)
    sc = np.tile(np.arange(64, dtype=np.uint8) * 4 + 1, (256, 1)).astype(np.uint8)
    ss = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 4, axis=1)
    codes, scales = np.concatenate([kc, sc]), np.concatenate([ks, ss])
    with np.errstate(over="ignore"):
        f_ref, b_ref = oracle.dequant_index(codes, scales)
    f = _dq(1, codes, scales, len(codes), False)
    _bits_equal_nan(f, f_ref)
    b = _dq(1, codes, scales, len(codes), True).view(np.uint16)
    bn = np.isnan(bf16_np_to_f64(b))
    assert np.array_equal(b[~bn], b_ref[~bn])


# ---------------------------------------------------------------- quantize

_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)


def _quant_inputs(width, n, seed):
    """Seeded fp32 rows of the cache-entry streams plus rows of edge values:
    scales from subnormal to overflow, NaN, +-inf, -0, all-zero blocks, exact
    E2M1 ties at every E4M3 scale and their neighbouring floats."""
    tid = synth.TID_MAIN if width == 512 else synth.TID_IKEY
    base = synth.f32_rows(seed, tid, 0, 0, n, width)
    rng = np.random.default_rng(seed)
    extra = []
    for sc in (1e-44, 1e-40, 1e-30, 1e-6, 1e4, 1e20, 1e37):
        with np.errstate(over="ignore"):
            extra.append((base[:8].astype(np.float64) * sc).astype(np.float32))
    sp = base[:16].copy()
    flat = sp.reshape(-1)
    flat[rng.integers(0, flat.size, 40)] = np.nan
    flat[rng.integers(0, flat.size, 10)] = np.inf
    flat[rng.integers(0, flat.size, 10)] = -np.inf
    flat[rng.integers(0, flat.size, 60)] = -0.0
    sp[3] = 0.0
    sp[4] = -0.0
    extra.append(sp)
    ties = []
    scales = [oracle.e4m3(c) for c in range(1, 0x7F)] if width == 512 else [2.0 ** e for e in range(-127, 120, 2)]
    g = 16 if width == 512 else 32
    for s in scales:
        r = np.zeros(width, np.float32)
        for b in range(width // g):
            r[g * b] = 6 * s
            r[g * b + 1:g * b + 8] = s * _MIDS
            r[g * b + 8:g * b + 15] = -s * _MIDS
        ties.append(r)
    t = np.array(ties, np.float32)
    extra += [t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(-np.inf))]
    return np.ascontiguousarray(np.concatenate([base, *extra]))


def _quantize_gpu(kind, x, bf16=False, dst_rows=None, n_cache_rows=None, fill=0xA5):
    n = x.shape[0]
    rows = n if n_cache_rows is None else n_cache_rows
    # bf16 inputs are rounded on the host so that the oracle sees the very bits
    # the kernel reads (device and host conversions may differ in NaN signs)
    xt = (torch.from_numpy(x).to(torch.bfloat16) if bf16 else torch.from_numpy(x)).cuda()
    codes = torch.full((rows, 288 if kind == 0 else 64), fill, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, 4), fill, dtype=torch.uint8, device="cuda") if kind == 1 else None
    dr = None if dst_rows is None else torch.from_numpy(np.ascontiguousarray(dst_rows, np.int64)).cuda()
    csa.csa2_quantize(kind, xt, 1 if bf16 else 0, n, dr, rows, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), (None if scales is None else scales.cpu().numpy())


def _bf16_round(x):
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_quantize_main_bitexact(bf16):
    x = _quant_inputs(512, 1001, seed=31)
    got, _ = _quantize_gpu(0, x, bf16)
    ref = oracle.quantize_main(_bf16_round(x) if bf16 else x)
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert bad.size == 0, f"rows {bad[:10]} differ, e.g. got {got[bad[0]][:8]} want {ref[bad[0]][:8]}"


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_quantize_index_bitexact(bf16):
    x = _quant_inputs(128, 999, seed=33)
    got_c, got_s = _quantize_gpu(1, x, bf16)
    ref_c, ref_s = oracle.quantize_index(_bf16_round(x) if bf16 else x)
    assert np.array_equal(got_s, ref_s), np.nonzero((got_s != ref_s).any(axis=1))[0][:10]
    assert np.array_equal(got_c, ref_c), np.nonzero((got_c != ref_c).any(axis=1))[0][:10]


def test_quantize_reproduces_generated_cache():
    """fp32 sources of seeded cache entries give back the stored entries."""
    x = synth.f32_rows(5, synth.TID_MAIN, 0, 0, 3000, 512)
    got, _ = _quantize_gpu(0, x)
    assert np.array_equal(got, synth.main_latents(5, 0, 0, 3000))
    x = synth.f32_rows(5, synth.TID_IKEY, 0, 0, 3000, 128)
    c, s = _quantize_gpu(1, x)
    kc, ks = synth.index_keys(5, 0, 0, 3000)
    assert np.array_equal(c, kc) and np.array_equal(s, ks)


@pytest.mark.parametrize("kind", [0, 1], ids=["main", "index"])
def test_quantize_scatter_rows(kind):
    """Rows go to dst_rows; -1 and out-of-range rows are skipped and the rest
    of the cache is untouched."""
    width = 512 if kind == 0 else 128
    n, cap = 700, 2000
    x = synth.f32_rows(9, synth.TID_MAIN if kind == 0 else synth.TID_IKEY, 1, 0, n, width)
    rng = np.random.default_rng(9)
    dst = rng.permutation(cap)[:n].astype(np.int64)
    dst[::50] = -1
    dst[7::50] = cap + 5
    got_c, got_s = _quantize_gpu(kind, x, dst_rows=dst, n_cache_rows=cap)
    if kind == 0:
        ref_c, ref_s = oracle.quantize_main(x), None
    else:
        ref_c, ref_s = oracle.quantize_index(x)
    ok = (dst >= 0) & (dst < cap)
    assert np.array_equal(got_c[dst[ok]], ref_c[ok])
    if kind == 1:
        assert np.array_equal(got_s[dst[ok]], ref_s[ok])
    untouched = np.setdiff1d(np.arange(cap), dst[ok])
    assert (got_c[untouched] == 0xA5).all()
    if kind == 1:
        assert (got_s[untouched] == 0xA5).all()


def test_quantize_full_size_sampled():
    """131072 new main entries and indexer keys in one launch each (the size of
    a long prefill chunk's cache write); sampled rows against the oracle."""
    n = 131072
    xm = synth.f32_rows(41, synth.TID_MAIN, 0, 0, n, 512)
    got, _ = _quantize_gpu(0, xm)
    rows = np.random.default_rng(41).choice(n, 1500, replace=False)
    rows[-1] = n - 1
    assert np.array_equal(got[rows], oracle.quantize_main(xm[rows]))
    xk = synth.f32_rows(41, synth.TID_IKEY, 0, 0, n, 128)
    c, s = _quantize_gpu(1, xk)
    rc, rs = oracle.quantize_index(xk[rows])
    assert np.array_equal(c[rows], rc) and np.array_equal(s[rows], rs)


def _pool_inputs(n, gw, seed):
    x = synth.f32_rows(seed, synth.TID_MAIN, 7, 0, 2 * n, 512)
    g = synth.f32_rows(seed, synth.TID_GATE, 0, 0, 2 * n, 512 if gw == 512 else 2)[:, :gw] * 2.0
    g = np.ascontiguousarray(g, np.float32)
    g[0:2] = 0.0                      # equal gates: the mean
    g[2], g[3] = 80.0, -80.0          # one token only
    g[4], g[5] = -80.0, 80.0
    x[6:8] *= 1e-30                   # tiny pair
    return x, g


@pytest.mark.parametrize("gw", [512, 1], ids=["per-channel", "per-token"])
def test_pool_quantize(gw):
    """m=2 pooling + encoding: the fp32 pooled rows within a few ulp of the
    fp64 pooling; the codes equal the oracle's encoding of those very fp32
    rows (the rounding decisions are taken on the same values)."""
    n = 1001
    x, g = _pool_inputs(n, gw, seed=61)
    xt, gt = torch.from_numpy(x).cuda(), torch.from_numpy(g).cuda()
    cache = torch.full((n, 288), 0xA5, dtype=torch.uint8, device="cuda")
    pooled = torch.empty((n, 512), dtype=torch.float32, device="cuda")
    csa.csa2_pool_quantize(xt, gt, n, None, n, cache, pooled)
    torch.cuda.synchronize()
    pg, cg = pooled.cpu().numpy(), cache.cpu().numpy()
    ref = oracle.pool_latents(x, g)
    mag = np.maximum(np.abs(x[0::2]), np.abs(x[1::2])).astype(np.float64)
    err = np.abs(pg.astype(np.float64) - ref)
    assert np.all(err <= 4e-6 * mag + 1e-37), f"pooled off by {np.max(err / (mag + 1e-37)):.3g} relative"
    assert np.array_equal(cg, oracle.quantize_main(pg))
    # without the pooled output, and scattered through a row list
    rng = np.random.default_rng(61)
    dst = rng.permutation(2 * n)[:n].astype(np.int64)
    dst[::97] = -1
    cache2 = torch.full((2 * n, 288), 0xA5, dtype=torch.uint8, device="cuda")
    csa.csa2_pool_quantize(xt, gt, n, torch.from_numpy(dst).cuda(), 2 * n, cache2, None)
    torch.cuda.synchronize()
    c2 = cache2.cpu().numpy()
    ok = dst >= 0
    assert np.array_equal(c2[dst[ok]], cg[ok])
    assert (c2[np.setdiff1d(np.arange(2 * n), dst[ok])] == 0xA5).all()


def test_quantize_empty_and_errors():
    x = torch.zeros((4, 512), dtype=torch.float32, device="cuda")
    c = torch.zeros((4, 288), dtype=torch.uint8, device="cuda")
    csa.csa2_quantize(0, x, 0, 0, None, 0, c)  # n = 0: no-op
    with pytest.raises(csa.Csa2Error):
        csa.csa2_quantize(2, x, 0, 4, None, 4, c)  # bad kind
    with pytest.raises(csa.Csa2Error):
        csa.csa2_quantize(0, x, 0, 4, None, 3, c)  # cache smaller than n without dst_rows
    with pytest.raises(csa.Csa2Error):
        csa.csa2_quantize(1, x, 0, 4, None, 4, c, None)  # index keys need scales
    assert (c.cpu() == 0).all()


# ------------------------------------------------------------ index scores

@pytest.mark.parametrize("Q,N", [(3, 5000), (1, 17), (2, 16), (1, 4096 + 37), (4, 131072 + 37), (16, 65536 + 37),
                                 (16, 131072 + 37)])
def test_index_score_full(Q, N):
    """Per-query scans. The last three sizes take 2, 4 and 8 batches of 64
    entries per wave (128-, 256- and 512-entry wave spans, the four waves of
    a workgroup interleaving their batches), each with a last workgroup
    range holding 37 entries."""
    wl = synth.full_decode(Q, N, seed=N)
    announce(f"full scores Q={Q} N={N}")
    ref, dots = oracle.index_score(wl, want_dots=True)
    got = gpu_scores(to_device(wl))
    check_scores(got, ref, dots, wl.w, f"full Q{Q} N{N}")


def test_index_score_reindex_pool_and_bad_blocks():
    wl = synth.reindex_decode(4, 65536, 300, seed=3, dense_rows=True)
    wl.cand_blocks = wl.cand_blocks.copy()
    wl.cand_blocks[1, 5] = -1          # absent block
    wl.cand_blocks[2, 7] = 65536 // 8  # beyond the cache
    ref, dots = oracle.index_score(wl, want_dots=True)
    got = gpu_scores(to_device(wl))
    check_scores(got, ref, dots, wl.w, "reindex")
    assert np.all(np.isneginf(got[1, 40:48])) and np.all(np.isneginf(got[2, 56:64]))


def test_index_score_causal_prefill():
    wl = synth.prefill(40, 3000, 5000, seed=4)
    ref, dots = oracle.index_score(wl, want_dots=True)
    got = gpu_scores(to_device(wl))
    check_scores(got, ref, dots, wl.w, "causal")


@pytest.mark.parametrize("T,n,t0", [(32, 2048, 4096), (70, 5003, 9900), (33, 777, 0), (97, 20000, 39000)])
def test_index_score_prefill_query_tiles(T, n, t0):
    """Many queries over one shared cache: the query-tiled kernel. Ragged query
    counts (partial waves), ragged entry counts, causal limits from 0 up to
    past the cache end."""
    wl = synth.prefill(T, n, t0, seed=40 + T)
    announce(f"prefill scores T={T} n={n} t0={t0}")
    ref, dots = oracle.index_score(wl, want_dots=True)
    got = gpu_scores(to_device(wl))
    check_scores(got, ref, dots, wl.w, f"prefill tiles T={T}")


def test_index_score_wide_block_scales():
    """E8M0 block scales far apart: key blocks at exponents -60..60, query
    blocks at -40..40 (any E8M0 byte is a valid scale per 32 channels), codes
    of both signs. The matrix core applies each block's two scales and sums
    the four block dots in fp32, where the oracle's dot is exact up to fp64
    rounding, so the score bound adds that sum's fp32 error bound; top-k over
    the GPU's scores must then match the oracle's exactly."""
    wl = synth.full_decode(3, 3000, seed=77)
    rng = np.random.default_rng(77)
    wl.key_scales = (127 + rng.integers(-60, 61, wl.key_scales.shape)).astype(np.uint8)
    wl.iq_scales = (127 + rng.integers(-40, 41, wl.iq_scales.shape)).astype(np.uint8)
    ref, dots = oracle.index_score(wl, want_dots=True)
    got = gpu_scores(to_device(wl))
    assert np.all(np.isfinite(got))
    check_scores(got, ref, dots, wl.w, "wide block scales", block_abs=block_abs_dots(wl))
    _assert_topk_exact(got, 512, wl.n_entries, what="wide block scales")


# ------------------------------------------------------------------- top-k

def _assert_topk_exact(scores, k, n_entries, cand_blocks=None, n_valid=None, what=""):
    ref_i, ref_s = oracle.topk(scores, k=k, n_valid=n_valid, n_entries=n_entries, cand_blocks=cand_blocks)
    gi, gs = gpu_topk(scores, k, n_entries, cand_blocks, n_valid)
    assert np.array_equal(gi, ref_i), f"{what}: ids differ at {np.argwhere(gi != ref_i)[:5].tolist()}"
    assert np.array_equal(np.isnan(gs), np.isnan(ref_s))
    m = ~np.isnan(ref_s)
    # bit-exact, except that a selected -0 is reported as +0 (the ranking
    # treats them as one value, and the kernels report the ranked value)
    ref_b = np.where(ref_s[m] == 0, np.float32(0.0), ref_s[m]).view(np.uint32)
    assert np.array_equal(gs[m].view(np.uint32), ref_b), what


@pytest.mark.parametrize("n", [1, 100, 511, 512, 513, 4096, 4097, 70001])
@pytest.mark.parametrize("k", [1, 7, 512, 1024])
def test_topk_exact_random(n, k):
    rng = np.random.default_rng(n * 31 + k)
    s = rng.standard_normal((3, n)).astype(np.float32)
    _assert_topk_exact(s, k, n, what=f"n{n} k{k}")


def test_topk_chunked_query_major_layout():
    """16 queries x 70,001 scores take the chunk-parallel selection with its
    compaction laid out query-major (the batch is a multiple of 8), then the
    per-query final selection; rows under causal limits from 0 to the whole
    list."""
    rng = np.random.default_rng(1616)
    s = rng.standard_normal((16, 70001)).astype(np.float32)
    nv = np.array([70001, 65536, 4099, 512, 511, 40, 1, 0, 70000, 30000, 20000, 16384, 16383, 1000, 513, 2],
                  np.int32)
    _assert_topk_exact(s, 512, 70001, n_valid=nv, what="chunked 16 x 70,001")


@pytest.mark.parametrize("n", [20000, 16000])
def test_topk_ties_nan_negzero(n):
    """n=20000 with 4 queries takes the chunk-parallel selection, n=16000 the
    one-workgroup-per-query kernel; the all-equal row keeps every candidate,
    more than that kernel holds in LDS."""
    rng = np.random.default_rng(1)
    s = np.round(rng.standard_normal((4, n)) * 3).astype(np.float32)  # heavy ties
    s[1, ::7] = -0.0
    s[1, 1::7] = 0.0
    s[2, :300] = np.nan
    s[3, :] = 2.5  # all equal: the whole list is one tie set
    _assert_topk_exact(s, 512, n, what=f"ties n{n}")


@pytest.mark.parametrize("n", [20000, 16000])
def test_topk_threshold_at_or_below_zero(n):
    """Thresholds at or below the key of +0 take the general compaction test
    (above it a single compare of the score bits decides). Row 0: every score
    negative. Row 1: 600 zeros of both signs, the rest negative, so the
    threshold is the key of +0 and -0 must tie with +0 (lower id first).
    Row 2: 300 positive scores, 600 zeros, the rest negative: the 512th score
    is a zero. Row 3: 1,000 values of +inf and NaN among negatives. Same
    kernels as the tie test: 4 x 20,000 chunk-parallel, 4 x 16,000 per query."""
    rng = np.random.default_rng(7)
    s = -np.abs(rng.standard_normal((4, n))).astype(np.float32) - np.float32(0.01)
    z = rng.choice(n, 600, replace=False)
    s[1, z] = np.where(np.arange(600) % 2 == 0, np.float32(0.0), np.float32(-0.0))
    s[2, z] = np.where(np.arange(600) % 3 == 0, np.float32(-0.0), np.float32(0.0))
    s[2, rng.choice(np.setdiff1d(np.arange(n), z), 300, replace=False)] = np.abs(rng.standard_normal(300)) + 0.5
    s[3, rng.choice(n, 1000, replace=False)] = np.where(np.arange(1000) % 2 == 0, np.float32(np.inf), np.float32(np.nan))
    _assert_topk_exact(s, 512, n, what=f"threshold <= 0 n{n}")


def test_topk_survivors_concentrated_in_one_chunk():
    """Chunk-parallel selection (3 queries x 70,001 candidates, 18 chunks of
    4,096). The final pass loads a fixed number of slots per chunk before it
    knows the counts; row 0 puts 600 top scores inside one chunk, more than
    those slots, so it takes the offset-table gather instead; row 1 is plain
    random (fixed slots); row 2 has 3,000 top scores over the first chunk."""
    rng = np.random.default_rng(9)
    n = 70001
    s = rng.standard_normal((3, n)).astype(np.float32)
    s[0, 5 * 4096:5 * 4096 + 600] = 10 + rng.standard_normal(600).astype(np.float32)
    s[2, :3000] = 10 + rng.standard_normal(3000).astype(np.float32)
    _assert_topk_exact(s, 512, n, what="concentrated")
    _assert_topk_exact(s, 1024, n, what="concentrated k1024")


def test_topk_many_queries_long_lists():
    """64 queries of 30,000 candidates: one workgroup per query with several
    compaction passes; some rows tie heavily."""
    rng = np.random.default_rng(5)
    s = rng.standard_normal((64, 30000)).astype(np.float32)
    s[3] = np.round(s[3] * 2)
    s[7, :] = -1.0
    nv = np.full(64, 30000, np.int32)
    nv[5] = 100
    nv[9] = 0
    _assert_topk_exact(s, 512, 30000, n_valid=nv, what="many queries")


@pytest.mark.parametrize("n", [20000, 5003])
def test_topk_large_batch(n):
    """1,100 queries take the 256-thread per-query workgroup (smaller batches
    the 1,024-thread one). n=20,000: four full passes of 4,096 positions and a
    ragged one; n=5,003 (not a multiple of 4): every pass guarded. Rows mix
    plain random scores, heavy ties, an all-equal row (every candidate
    survives, more than the workgroup holds in LDS), -0/NaN rows, all-negative
    rows (the general compaction test) and causal limits down to 0."""
    rng = np.random.default_rng(n)
    Q = 1100
    s = rng.standard_normal((Q, n)).astype(np.float32)
    s[1::50] = np.round(s[1::50] * 2)
    s[2] = 2.5
    s[3::50, ::7] = -0.0
    s[4::50, :200] = np.nan
    s[5::50] = -np.abs(s[5::50]) - np.float32(0.01)
    nv = np.full(Q, n, np.int32)
    nv[6::50] = rng.integers(0, n, len(nv[6::50]))
    nv[7] = 0
    nv[8] = 511
    announce(f"topk large batch Q={Q} n={n}")
    _assert_topk_exact(s, 512, n, n_valid=nv, what=f"large batch n{n}")


@pytest.mark.parametrize("Q,n", [(1024, 16380), (1024, 16381), (64, 30001)])
def test_topk_subchunk_skipping(Q, n):
    """With the threshold above zero, the per-query kernel reads only the
    sub-chunks (16 scores here) whose maximum reaches it. 1,024 queries take
    the 256-thread workgroup, 64 the 1,024-thread one; n = 16,380 leaves a
    partial last sub-chunk on aligned rows, 16,381 and 30,001 unaligned rows.
    Rows mix random scores, the top scores packed into the last sub-chunk,
    heavy ties, negative rows (no skipping), NaN and +inf, and causal limits."""
    rng = np.random.default_rng(Q + n)
    s = rng.standard_normal((Q, n)).astype(np.float32)
    s[0, -10:] = 50 + rng.standard_normal(10).astype(np.float32)
    s[1::40] = np.round(s[1::40] * 2)
    s[2::40] = -np.abs(s[2::40]) - np.float32(0.01)
    s[3::40, rng.choice(n, 40, replace=False)] = np.inf
    s[4::40, ::5] = np.nan
    nv = np.full(Q, n, np.int32)
    nv[5::40] = rng.integers(0, n, len(nv[5::40]))
    nv[6] = n - 5
    announce(f"topk sub-chunk skipping Q={Q} n={n}")
    _assert_topk_exact(s, 512, n, n_valid=nv, what=f"skipping Q{Q} n{n}")


def test_topk_large_batch_pool():
    """The 256-thread workgroup on Reindex-style lists: 1,024 queries, pools of
    2,048 blocks of 8 (16,384 candidates, four full passes) with absent
    blocks and blocks past the cache end."""
    rng = np.random.default_rng(12)
    Q, nb, n_entries = 1024, 2048, 1 << 20
    blocks = np.stack([np.sort(rng.choice(n_entries // 8 + 64, nb, replace=False)) for _ in range(Q)]).astype(np.int32)
    blocks[::37, 100:110] = -1
    s = rng.standard_normal((Q, 8 * nb)).astype(np.float32)
    announce(f"topk large batch pool Q={Q} blocks={nb}")
    _assert_topk_exact(s, 512, n_entries, cand_blocks=blocks, what="large batch pool")


def test_topk_pool_and_causal():
    rng = np.random.default_rng(2)
    blocks = np.stack([np.sort(rng.choice(50000, 700, replace=False)) for _ in range(3)]).astype(np.int32)
    s = rng.standard_normal((3, 5600)).astype(np.float32)
    _assert_topk_exact(s, 512, 400000, cand_blocks=blocks, what="pool")
    s2 = rng.standard_normal((5, 9000)).astype(np.float32)
    nv = np.array([0, 1, 511, 512, 8999], np.int32)
    _assert_topk_exact(s2, 512, 9000, n_valid=nv, what="causal")


@pytest.mark.parametrize("Q,n", [(14, 65536), (64, 65536), (6, 1 << 20)])
def test_topk_valid_entries_inside_first_subchunk(Q, n):
    """Causal limits small enough that every valid candidate lies in the first
    one or two sub-chunks of a list with more than k sub-chunks: the other
    sub-chunk maxima are empty, fewer than k are non-zero, and they may all be
    one value. Every valid candidate must then be selected. 14 x 65,536 and
    6 x 2^20 take the chunk-parallel selection, 64 x 65,536 the per-query
    kernel. Limits: 0, 1, 2, 17, 40, around a sub-chunk (64 or 512 entries
    here), 511..513; some rows hold one score repeated, so that two sub-chunk
    maxima are equal."""
    rng = np.random.default_rng(Q + n)
    s = rng.standard_normal((Q, n)).astype(np.float32)
    lims = [2, 17, 40, 63, 64, 65, 100, 511, 512, 513, 0, 1, 511, 1023]
    nv = np.array([lims[i % len(lims)] for i in range(Q)], np.int32)
    s[1, :] = 1.5
    if Q > 4:
        s[4::7, :] = -2.0
    announce(f"topk first sub-chunk Q={Q} n={n}")
    _assert_topk_exact(s, 512, n, n_valid=nv, what=f"first sub-chunk Q{Q} n{n}")


@pytest.mark.parametrize("Q,n", [(2, 1 << 20), (64, 1 << 19)])
def test_build_pool_few_valid_blocks(Q, n):
    """Pools asked for 2,048 blocks where the causal limit leaves only a few
    blocks inside the first sub-chunk of block maxima: every valid block must
    be kept and the rest padded (2 x 2^20: chunk-parallel selection over
    131,072 blocks; 64 x 2^19: the per-query kernel over 65,536 blocks)."""
    rng = np.random.default_rng(n + Q)
    sc = rng.standard_normal((Q, n)).astype(np.float32)
    lims = [40, 130, 8, 1, 257, 0, 4000]
    nv = np.array([lims[i % len(lims)] for i in range(Q)], np.int32)
    sc[min(1, Q - 1), :] = 0.75
    ref = oracle.pool_blocks(sc, 2048, nv)
    got = _gpu_pool(sc, 2048, nv)
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert bad.size == 0, f"queries {bad[:5]} differ"


def test_topk_empty_candidates():
    s = np.zeros((2, 0), np.float32)
    gi, _ = gpu_topk(s, 512, 0)
    assert np.all(gi == -1)


# --------------------------------------------------------------- attention

def test_sparse_attn_with_oracle_ids():
    wl = synth.full_decode(3, 2000, seed=11)
    sc = oracle.index_score(wl)
    idx, _ = oracle.topk(sc, wl)
    _, of, lse = oracle.sparse_attn(wl, idx)
    ob, glse = gpu_attn(to_device(wl), idx)
    check_attn(ob, of, "attn")
    check_lse(glse, lse, "attn lse")


@pytest.mark.parametrize("Q", [1, 12, 40, 700])
def test_sparse_attn_split_layouts(Q):
    """Q=1 splits the slot list into 10 ranges, Q=12 too (120 (query, range)
    pairs, the queries in two groups of 8 with 4 idle places), Q=40 into 3,
    Q=700 not at all."""
    wl = synth.full_decode(Q, 600, seed=Q)
    rng = np.random.default_rng(Q)
    idx = np.stack([rng.choice(600, 512, replace=False) for _ in range(Q)]).astype(np.int32)
    _, of, lse = oracle.sparse_attn(wl, idx)
    ob, glse = gpu_attn(to_device(wl), idx)
    check_attn(ob, of, f"attn Q{Q}")
    check_lse(glse, lse, f"attn Q{Q} lse")


def test_sparse_attn_edge_cases():
    wl = synth.full_decode(2, 300, seed=5, n_swa=37)
    db = to_device(wl)
    rng = np.random.default_rng(5)
    # -1 padding and out-of-range ids are skipped; ragged k_sel and window
    idx = np.full((2, 77), -1, np.int32)
    idx[:, :50] = rng.choice(300, 50, replace=False)
    idx[0, 60] = 300
    idx[1, 61] = 10 ** 6
    _, of, lse = oracle.sparse_attn(wl, idx)
    ob, glse = gpu_attn(db, idx)
    check_attn(ob, of, "padded")
    check_lse(glse, lse, "padded lse")
    # SWA only (k_sel = 0)
    _, of, lse = oracle.sparse_attn(wl, np.zeros((2, 0), np.int32))
    ob, glse = gpu_attn(db, None)
    check_attn(ob, of, "swa only")
    # selection only (no window)
    _, of, lse = oracle.sparse_attn(wl, idx, n_swa=0)
    ob, glse = gpu_attn(db, idx, n_swa=0)
    check_attn(ob, of, "no window")
    # empty joint set: zeros, lse = -inf
    ob, glse = gpu_attn(db, np.full((2, 8), -1, np.int32), n_swa=0)
    assert np.all(ob == 0) and np.all(np.isneginf(glse))


@pytest.mark.parametrize("Q,fp8,rope", [(1, True, True), (3, True, False), (2, False, True), (40, True, True),
                                         (700, True, True)])
def test_sparse_attn_fp8_window_and_rope(Q, fp8, rope):
    """FP8 (MXFP8, 528-B) window rows and the RoPE un-rotation epilogue, in
    the split (small Q, merged by the combine kernel) and unsplit layouts."""
    wl = synth.with_window_options(synth.full_decode(Q, 600, seed=50 + Q), swa_fp8=fp8, rope=rope)
    rng = np.random.default_rng(Q)
    idx = np.stack([rng.choice(600, 512, replace=False) for _ in range(Q)]).astype(np.int32)
    _, of, lse = oracle.sparse_attn(wl, idx)
    ob, glse = gpu_attn(to_device(wl), idx)
    check_attn(ob, of, f"attn fp8={fp8} rope={rope} Q{Q}")
    check_lse(glse, lse, "lse")


def test_sparse_attn_fp8_window_edge_cases():
    wl = synth.with_window_options(synth.full_decode(2, 300, seed=6, n_swa=37), swa_fp8=True, rope=True)
    db = to_device(wl)
    _, of, lse = oracle.sparse_attn(wl, np.zeros((2, 0), np.int32))  # window only, ragged
    ob, glse = gpu_attn(db, None)
    check_attn(ob, of, "fp8 window only")
    check_lse(glse, lse, "fp8 window only lse")
    rng = np.random.default_rng(6)
    idx = np.full((2, 45), -1, np.int32)  # mixed tile: selection ends inside a tile
    idx[:, :40] = rng.choice(300, 40, replace=False)
    _, of, lse = oracle.sparse_attn(wl, idx)
    ob, glse = gpu_attn(db, idx)
    check_attn(ob, of, "fp8 mixed tile")


# -------------------------------------------------------- pool construction

def _gpu_pool(scores_np, n_pool, n_valid=None):
    s = torch.from_numpy(np.ascontiguousarray(scores_np, np.float32)).cuda()
    out = torch.empty((s.shape[0], n_pool), dtype=torch.int32, device="cuda")
    nv = None if n_valid is None else torch.from_numpy(np.ascontiguousarray(n_valid, np.int32)).cuda()
    csa.csa2_build_pool(csa.pool_args(s, n_pool, out, nv))
    torch.cuda.synchronize()
    return to_np_i32(out)


def to_np_i32(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("Q,n,n_pool,limit", [(2, 1 << 20, 2048, False), (3, 8 * 3000 + 5, 1000, True),
                                               (64, 65536, 2048, True), (1, 100, 2048, False),
                                               (5, 4096, 8192, True), (4, 4097, 1, False)])
def test_build_pool_exact(Q, n, n_pool, limit):
    """Same scores on both sides: the pool ids are compared exactly (ties on a
    coarse grid, NaN, -0 / +0, -inf, ragged last block, causal limits, more
    blocks asked for than hold a valid entry)."""
    rng = np.random.default_rng(n + Q)
    sc = (np.round(rng.standard_normal((Q, n)) * 8) / 8).astype(np.float32)
    sc[0, rng.integers(0, n, 50)] = np.nan
    if Q > 1:
        sc[1, ::5] = -0.0
    if Q > 2:
        sc[2, rng.integers(0, n, 50)] = -np.inf
    n_valid = rng.integers(n // 3, n + 1, Q).astype(np.int32) if limit else None
    ref = oracle.pool_blocks(sc, n_pool, n_valid)
    got = _gpu_pool(sc, n_pool, n_valid)
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert bad.size == 0, f"queries {bad[:5]} differ"


def test_pool_feeds_reindex_layer():
    """A Full layer's GPU scores -> pool -> the Reindex layer's scores over
    that pool on the same cache, against the oracle."""
    wl = synth.full_decode(2, 1 << 16, seed=31)
    sc = gpu_scores(to_device(wl))
    pool = _gpu_pool(sc, 2048)
    assert np.array_equal(pool, oracle.pool_blocks(sc, 2048))
    wl.cand_blocks = pool
    ref, dots = oracle.index_score(wl, want_dots=True)
    got = gpu_scores(to_device(wl))
    check_scores(got, ref, dots, wl.w, "reindex over the built pool")
    ents = (8 * pool[:, :, None] + np.arange(8)[None, None, :]).reshape(2, -1)
    np.testing.assert_array_equal(got, np.take_along_axis(sc, ents, axis=1))


# -------------------------------------------------------- Reuse layers

def test_gather_selected_and_reuse_attention():
    """The dense copy of the selection matches the oracle byte for byte, and a
    later layer's attention over it (dense ids) equals attention over the
    original cache with the original ids, bit for bit."""
    wl = synth.full_decode(5, 3000, seed=71)
    rng = np.random.default_rng(71)
    idx = np.stack([rng.choice(3000, 512, replace=False) for _ in range(5)]).astype(np.int32)
    idx[0, 3] = -1
    idx[1, 100] = 3000
    idx[4, -5:] = -1
    db = to_device(wl)
    it = torch.from_numpy(idx).cuda()
    out = torch.empty((5, 512, 288), dtype=torch.uint8, device="cuda")
    dense = torch.empty((5, 512), dtype=torch.int32, device="cuda")
    csa.csa2_gather_selected(db.main_cache, wl.n_entries, wl.cache_q_stride, it, out, dense)
    torch.cuda.synchronize()
    ref_g, ref_d = oracle.gather_selected(wl.main_cache, wl.n_entries, wl.cache_q_stride, idx)
    assert np.array_equal(out.cpu().numpy(), ref_g) and np.array_equal(dense.cpu().numpy(), ref_d)
    ob, glse = gpu_attn(db, idx)
    import dataclasses
    dd = dataclasses.replace(db, main_cache=out.view(-1, 288), n_entries=512, cache_q_stride=512)
    ob2, glse2 = gpu_attn(dd, dense.cpu().numpy())
    assert np.array_equal(ob, ob2) and np.array_equal(glse.view(np.uint32), glse2.view(np.uint32))
    _, of, _ = oracle.sparse_attn(wl, idx)
    check_attn(ob2, of, "reuse layer over the gathered list")


# ------------------------------------------------------------ fused decode

def _check_decode(wl, queries=None, what=""):
    db = to_device(wl)
    ob, glse, gidx = gpu_decode(db)
    ref = oracle.decode(wl, queries=queries)
    qs = list(range(wl.Q)) if queries is None else list(queries)
    check_topk_band(gidx[qs], ref["scores"], ref["idx"], QueryView(wl, qs), wl.k, what)
    # attention with the GPU's own selection isolates the attention step
    _, of_own, lse_own = oracle.sparse_attn(wl, gidx[qs], queries=qs)
    check_attn(ob[qs], of_own, what + " (own ids)")
    check_lse(glse[qs], lse_own, what + " lse")
    # end to end against the oracle's selection (differences only from band swaps)
    check_attn(ob[qs], ref["out_f32"], what + " (oracle ids)")
    return gidx


def test_decode_full_small():
    _check_decode(synth.full_decode(2, 4096 + 300, seed=21), what="full small")


def test_decode_fp8_window_and_rope():
    wl = synth.with_window_options(synth.full_decode(3, 3000, seed=24), swa_fp8=True, rope=True)
    _check_decode(wl, what="decode fp8 rope")


def test_decode_prefill_fp8_window_and_rope():
    wl = synth.with_window_options(synth.prefill(40, 2048, 3000, seed=25), swa_fp8=True, rope=True)
    _check_decode(wl, what="prefill fp8 rope")


def test_decode_reindex_small_poisoned():
    wl = synth.reindex_decode(3, 1 << 16, 2048, seed=22, dense_rows=True)
    gidx = _check_decode(wl, what="reindex small")
    for qi in range(wl.Q):
        pool = set((8 * wl.cand_blocks[qi][:, None] + np.arange(8)[None, :]).reshape(-1).tolist())
        assert set(gidx[qi].tolist()) <= pool


def test_decode_prefill_small():
    _check_decode(synth.prefill(50, 2048, 3000, seed=23), what="prefill small")


@pytest.mark.parametrize("T,n,t0", [(70, 5003, 9900), (64, 40000, 79000)])
def test_decode_prefill_query_tiles(T, n, t0):
    """Decode over a query-tiled prefill: the selection uses the sub-chunk
    maxima recorded by the tiled scoring kernel."""
    _check_decode(synth.prefill(T, n, t0, seed=50 + T), what=f"prefill tiles T={T}")


def test_decode_chunked_selection_paths():
    """Lists long enough for the chunk-parallel selection (3 queries x 20,000
    entries, 5 compaction chunks of 4,096), whose final step runs inside the
    attention kernel. Query 0: every key equal, so every score ties, every
    candidate survives the compaction and the lowest 512 ids win (streaming
    path). Query 1: 1,000 entries of chunk 1 carry the query's best key, a tie
    set larger than that chunk's register slots (offset-table path). Query 2:
    random (fixed slots). The tied queries' id sets are compared exactly."""
    wl = synth.full_decode(3, 20000, seed=31)
    n = wl.n_entries
    wl.key_codes[0:n] = wl.key_codes[0]
    wl.key_scales[0:n] = wl.key_scales[0]
    s1 = oracle.index_score(wl, queries=[1])[0]
    best = n + int(np.argmax(s1))
    wl.key_codes[n + 4196:n + 5196] = wl.key_codes[best]
    wl.key_scales[n + 4196:n + 5196] = wl.key_scales[best]
    gidx = _check_decode(wl, what="chunked selection")
    ref = oracle.decode(wl, queries=[0, 1])
    assert np.array_equal(gidx[0], np.arange(512, dtype=np.int32))
    assert np.array_equal(np.sort(gidx[1]), np.sort(ref["idx"][1][:512]))


def test_decode_chunked_long_tie_list():
    """2 queries x 65,536 entries (16 compaction chunks). In query 0 every
    32nd entry carries the query's best key: 2,048 tied candidates survive
    the compaction, 128 per chunk, which the attention kernel's final
    selection holds in registers but cannot spread over its threads (more
    than 1,024); the lowest 512 ids of the tie set win. Query 1 is random
    (its few hundred survivors take the spread path)."""
    wl = synth.full_decode(2, 65536, seed=35)
    s0 = oracle.index_score(wl, queries=[0])[0]
    best = int(np.argmax(s0))
    ties = np.arange(0, 65536, 32)
    wl.key_codes[ties] = wl.key_codes[best]
    wl.key_scales[ties] = wl.key_scales[best]
    announce("chunked long tie list")
    gidx = _check_decode(wl, what="chunked tie list")
    assert np.array_equal(gidx[0], np.sort(np.union1d(ties, [best]))[:512].astype(np.int32))


@pytest.mark.parametrize("k", [7, 1024])
def test_decode_chunked_other_k(k):
    """k other than 512 through the chunk-parallel selection finished in the
    attention kernel (3 queries x 20,000 entries): 7 selected slots leave
    most of the first tile to the window; 1,024 fill 32 tiles before it."""
    wl = dataclasses.replace(synth.full_decode(3, 20000, seed=34 + k), k=k)
    _check_decode(wl, what=f"chunked k={k}")


def test_decode_chunked_causal_limits_and_no_ids():
    """A 40-query prefill over 20,000 entries at positions 990..1029: the
    causal limits (495..514 entries) straddle k = 512, so some queries select
    every valid entry and pad with -1, inside the attention kernel's final
    selection (chunk-parallel lists: fewer than 64 queries, more than 16,384
    candidates). The same call without an id output gives the same
    attention, bit for bit."""
    wl = synth.prefill(40, 20000, 990, seed=33)
    assert wl.n_valid.min() < 512 < wl.n_valid.max()
    gidx = _check_decode(wl, what="chunked causal")
    db = to_device(wl)
    out, lse, idx = db.new_outputs()
    csa.csa2_decode(db.decode_args(out, lse, idx))
    out2, lse2, _ = db.new_outputs()
    csa.csa2_decode(db.decode_args(out2, lse2, None))
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), gidx)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("T,t0", [(40, 0), (70, 0), (40, 120), (70, 960)])
def test_decode_prefill_from_position_zero(T, t0):
    """A prefill chunk over a long (65,536-entry) m=2 cache starting at
    position t0: limits floor(t/2) from 0 up, all inside the first sub-chunks
    of the list (t0 = 0), around one sub-chunk (t0 = 120) or around k
    (t0 = 960). 40 queries take the chunk-parallel selection finished in the
    attention kernel, 70 the per-query kernel."""
    _check_decode(synth.prefill(T, 65536, t0, seed=60 + T + t0), what=f"prefill from t0={t0} T={T}")


@pytest.mark.parametrize("T,n,t0", [(40, 3001, 0), (9, 4096, 9000)])
def test_decode_raw_selection(T, n, t0):
    """Fewer than 64 queries over a plain list of at most 4,096 entries: the
    attention kernel selects straight from the scores. t0 = 0: causal limits
    from 0 up (queries with fewer than k valid entries pad with -1, one with
    none attends over its window only), a list that is not a multiple of 16;
    t0 past the cache end: every entry valid, the longest such list."""
    announce(f"raw selection T={T} n={n} t0={t0}")
    _check_decode(synth.prefill(T, n, t0, seed=70 + T), what=f"raw selection T={T}")


def test_decode_raw_selection_ties():
    """Raw-score selection with query 0's 4,096 keys all equal: every score
    ties and the lowest 512 ids win. Query 1 is random."""
    wl = synth.full_decode(2, 4096, seed=36)
    wl.key_codes[0:4096] = wl.key_codes[0]
    wl.key_scales[0:4096] = wl.key_scales[0]
    announce("raw selection ties")
    gidx = _check_decode(wl, what="raw ties")
    assert np.array_equal(gidx[0], np.arange(512, dtype=np.int32))


def test_decode_fewer_than_k_entries():
    _check_decode(synth.full_decode(2, 300, seed=24), what="n<k")


def test_decode_deterministic():
    wl = synth.full_decode(4, 9000, seed=25)
    db = to_device(wl)
    a = gpu_decode(db)
    b = gpu_decode(db)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))



@pytest.mark.parametrize("Q,n", [(1, 4096), (3, 20000), (16, 3000)])
def test_decode_graph_capture_replays(Q, n):
    """csa2_decode captured in a HIP graph on the caller's stream: three
    replays, each after eager work and a synchronisation, must reproduce the
    eager outputs bit for bit (1 x 4,096: the selection from raw scores
    inside attention; 3 x 20,000: compaction and the fused final selection;
    16 x 3,000: raw selection with the query-major scan)."""
    announce(f"graph capture Q={Q} n={n}")
    wl = synth.full_decode(Q, n, seed=Q + n)
    db = to_device(wl)
    out, lse, idx = db.new_outputs()
    da = db.decode_args(out, lse, idx)
    ws = torch.empty(max(1, csa.csa2_workspace_size(csa.CSA2_WS_DECODE, da)), dtype=torch.uint8, device="cuda")
    csa.csa2_decode(da, ws)
    torch.cuda.synchronize()
    ref = [out.clone(), lse.clone(), idx.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        csa.csa2_decode(da, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        csa.csa2_decode(da, ws)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(0)
        lse.fill_(0)
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((out, lse, idx), ref):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {r}"
        csa.csa2_decode(da, ws)  # eager work between the replays
        torch.cuda.synchronize()
    del g


# ------------------------------------------------- full-size workload shapes

def test_decode_1x4096_full():
    _check_decode(synth.make_workload(0), what="decode 1 x 4,096")


def test_decode_16x65536_full():
    _check_decode(synth.make_workload(1), what="decode 16 x 65,536")


def test_decode_4x1048576_full():
    _check_decode(synth.make_workload(4), what="decode 4 x 1,048,576")


def test_reindex_decode_64x16384_pool_full():
    """1,048,576-entry caches, 2,048 random blocks of 8 per query; the oracle
    runs on the pool rows re-indexed into a compact cache."""
    wl = synth.make_workload(2, dense_rows=False)
    db = to_device(wl)
    ob, glse, gidx = gpu_decode(db)
    # compact view: query i's pool becomes entries 0..16383 of its own cache
    comp = synth.compact_pool_view(wl)
    ref = oracle.decode(comp)
    pools = [synth.pool_ids(wl, i) for i in range(wl.Q)]
    # map the GPU's global ids back to compact ids
    comp_gidx = np.stack([np.searchsorted(pools[i], gidx[i]) for i in range(wl.Q)]).astype(np.int32)
    for i in range(wl.Q):
        assert np.array_equal(pools[i][comp_gidx[i]], gidx[i]), "GPU selected an entry outside the pool"
    check_topk_band(comp_gidx, ref["scores"], ref["idx"], comp, wl.k, "reindex 64 x 16,384")
    _, of_own, _ = oracle.sparse_attn(comp, comp_gidx)
    check_attn(ob, of_own, "reindex 64 x 16,384 (own ids)")
    check_attn(ob, ref["out_f32"], "reindex 64 x 16,384 (oracle ids)")


def test_prefill_4096x131072_sampled_queries():
    """64 of the 4,096 queries: every position a query takes inside a
    32-query scorer workgroup (4 waves x 2 sets x 4 queries) twice, spread
    over the chunk, plus the first and last query."""
    wl = synth.make_workload(3)
    qs = sorted({r + 32 * ((37 * r + 61 * s) % 128) for r in range(32) for s in range(2)} | {0, 4095})
    assert len(qs) >= 64 and {q % 32 for q in qs} == set(range(32))
    _check_decode(wl, queries=qs, what="prefill 4,096 x 131,072")
