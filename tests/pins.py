"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``check_*`` takes an oracle library handle ``L`` (the real build, or a
build with a planted mistake) and raises AssertionError when the oracle
disagrees with:
  * the element-format definitions (golden E2M1 table; torch's own
    float8_e4m3fn / float8_e8m0fnu conversions),
  * the byte figures the pages print (tests/golden/kv_layout.txt),
  * independent numpy / torch computations of the same closed forms
    (matmul-based indexer scores, library sort for top-k, library SDPA for
    select-all attention),
  * invariants (ReLU before weighting, exact dots, tie order, permutation
    invariance, softmax weights summing to 1, single-entry and zero-query cases).
"""
from __future__ import annotations

import copy
import math
import os

import numpy as np
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_e2m1() -> np.ndarray:
    vals = np.zeros(16, np.float64)
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def golden_layout() -> dict:
    out = {}
    with open(os.path.join(GOLDEN, "kv_layout.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            out[k] = float(v)
    return out


def lib_e4m3(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def lib_e8m0(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., B] bytes -> [..., 2B] 4-bit codes, channel 2j = low nibble of byte j."""
    lo = codes & 0x0F
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)


def ref_dequant_main(entries: np.ndarray) -> np.ndarray:
    e = np.asarray(entries, np.uint8).reshape(-1, 288)
    vals = golden_e2m1()[nibbles(e[:, :256])]
    sc = lib_e4m3(e[:, 256:])
    return vals * np.repeat(sc, 16, axis=1)


def ref_dequant_index(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, np.uint8).reshape(-1, 64)
    s = np.asarray(scales, np.uint8).reshape(-1, 4)
    return golden_e2m1()[nibbles(c)] * np.repeat(lib_e8m0(s), 32, axis=1)


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- formats ---

def check_format_tables(L):
    g = golden_e2m1()
    for c in range(16):
        v = oracle.e2m1(c, L)
        assert v == g[c] and math.copysign(1, v) == math.copysign(1, g[c]), (c, v, g[c])
    ref4 = lib_e4m3(np.arange(256, dtype=np.uint8))
    ref8 = lib_e8m0(np.arange(256, dtype=np.uint8))
    for b in range(256):
        v4, v8 = oracle.e4m3(b, L), oracle.e8m0(b, L)
        if math.isnan(ref4[b]):
            assert math.isnan(v4), b
        else:
            assert v4 == ref4[b] and math.copysign(1, v4) == math.copysign(1, ref4[b]), (b, v4, ref4[b])
        if math.isnan(ref8[b]):
            assert math.isnan(v8), b
        else:
            assert v8 == ref8[b], (b, v8, ref8[b])


def check_layout(L):
    g = golden_layout()
    assert L.orc_main_entry_bytes() == g["main_entry_bytes"]
    assert L.orc_index_entry_bytes() == g["index_entry_bytes"]
    per_entry = L.orc_main_entry_bytes() + L.orc_index_entry_bytes()
    # three m=2 encoder caches and one m=1 decoder cache
    entries_per_token = 3 * 0.5 + 1 * 1.0
    assert entries_per_token == g["entries_per_token"]
    assert entries_per_token * per_entry == g["kv_bytes_per_token"]
    gib = g["kv_bytes_per_token"] * g["context_limit_tokens"] / 2**30
    assert round(gib, 2) == g["kv_gib_at_limit"]


def check_dequant(L, seed=3):
    main = synth.main_latents(seed, 0, 0, 300)
    kc, ks = synth.index_keys(seed, 0, 0, 300)
    # hand-built entry: byte 0x71 -> channel 0 code 1 (0.5), channel 1 code 7 (6.0)
    hand = np.zeros((1, 288), np.uint8)
    hand[0, 0] = 0x71
    hand[0, 1] = 0x9A  # channel 2 code 0xA (-1.0), channel 3 code 9 (-0.5)
    hand[0, 256] = 0x38  # E4M3 1.0 for channels 0..15
    hand[0, 257] = 0x40  # E4M3 2.0 for channels 16..31
    hand[0, 8] = 0x0F  # channel 16 code 0xF (-6.0) -> -12.0
    # all E4M3 scale codes incl. subnormals and NaN, all nibbles
    sweep = np.zeros((256, 288), np.uint8)
    sweep[:, :256] = np.arange(256, dtype=np.uint8)[None, :]
    sweep[:, 256:] = np.arange(256, dtype=np.uint8)[:, None]
    for ent in (main, hand, sweep):
        f, b = oracle.dequant_main(ent, L)
        ref = ref_dequant_main(ent)
        ref32 = ref.astype(np.float32)
        nan = np.isnan(ref32)
        assert np.array_equal(np.isnan(f), nan)
        assert np.array_equal(f[~nan].view(np.uint32), ref32[~nan].view(np.uint32))
        # bf16 output equals the exact value (products have <= 6 significant bits)
        bb = bf16_to_f64(b)
        assert np.array_equal(np.isnan(bb), nan)
        assert np.array_equal(bb[~nan], ref[~nan])
    f, _ = oracle.dequant_main(hand, L)
    assert f[0, 0] == 0.5 and f[0, 1] == 6.0 and f[0, 2] == -1.0 and f[0, 3] == -0.5 and f[0, 16] == -12.0
    # indexer keys, plus all E8M0 scales
    sweep_c = np.tile(np.arange(64, dtype=np.uint8) * 4 + 1, (256, 1)).astype(np.uint8)
    sweep_s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 4, axis=1)
    for c, s in ((kc, ks), (sweep_c, sweep_s)):
        f, _ = oracle.dequant_index(c, s, L)
        ref = ref_dequant_index(c, s)
        with np.errstate(over="ignore"):
            ref32 = ref.astype(np.float32)
        nan = np.isnan(ref32)
        assert np.array_equal(np.isnan(f), nan)
        assert np.array_equal(f[~nan].view(np.uint32), ref32[~nan].view(np.uint32))


def ref_bf16_rne(v: float) -> int:
    """bf16 bit pattern nearest to the fp64 value v, ties to the even
    mantissa, by exact rational arithmetic (fractions.Fraction): the value is
    divided by the bf16 unit of its binade (2^(E-7), or 2^-133 below 2^-126),
    the quotient rounded to an integer, and the result encoded. Magnitudes
    from the largest finite bf16 plus half a unit up become infinity."""
    from fractions import Fraction
    if math.isnan(v):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    if math.isinf(v):
        return sign | 0x7F80
    a = abs(Fraction(v))
    if a == 0:
        return sign
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    assert Fraction(2) ** E <= a < Fraction(2) ** (E + 1)
    sub = E < -126
    unit = Fraction(2) ** (-133 if sub else E - 7)
    n = a / unit
    r = n.numerator // n.denominator
    rem = n - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    if sub:
        return sign | r  # r = 128 is the least normal, 0x0080
    if r == 256:
        E, r = E + 1, 128
    if E > 127:
        return sign | 0x7F80
    return sign | ((E + 127) << 7) | (r - 128)


def check_bf16_rounding(L, seed=2):
    """The oracle's fp64 -> bf16 conversion is one round-to-nearest-even step.
    1 + 2^-8 + 2^-30 lies just above the midpoint of 1 and 1 + 2^-7 and must
    give 1 + 2^-7 (rounding through fp32 first lands on the midpoint and then
    on 1.0). Random values just off bf16 midpoints (by 2^-30 to 2^-50 of
    their size), exact midpoints of both mantissa parities, the subnormal
    range, the overflow boundary, zeros of both signs, infinities and NaN are
    checked against the rational reference above."""
    assert oracle.f64_to_bf16(1 + 2.0 ** -8 + 2.0 ** -30, L) == 0x3F81
    assert oracle.f64_to_bf16(1 + 2.0 ** -8, L) == 0x3F80          # tie, even mantissa 0
    assert oracle.f64_to_bf16(1 + 3 * 2.0 ** -8, L) == 0x3F82      # tie, odd mantissa 1 rounds up
    assert oracle.f64_to_bf16(-(1 + 2.0 ** -8 + 2.0 ** -30), L) == 0xBF81
    rng = np.random.default_rng(seed)
    vals = [0.0, -0.0, math.inf, -math.inf, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -135,
            2.0 ** -126 - 2.0 ** -134, 2.0 ** -126 - 2.0 ** -135, 5e-324, -5e-324,
            (2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -8) * 2.0 ** 127, (2 - 2.0 ** -8 - 2.0 ** -40) * 2.0 ** 127,
            2.0 ** 128, 1e300, -1e300]
    for _ in range(3000):
        e = int(rng.integers(-140, 128))
        m = int(rng.integers(0, 256))
        mid = (1 + (2 * m + 1) / 256.0) * 2.0 ** e  # a bf16 midpoint (exact in fp64)
        off = 2.0 ** -float(rng.integers(30, 51))
        vals += [mid, mid * (1 + off), mid * (1 - off), -mid * (1 + off)]
        vals.append(float(rng.standard_normal()) * 2.0 ** float(rng.integers(-135, 128)))
    for v in vals:
        got, want = oracle.f64_to_bf16(v, L), ref_bf16_rne(v)
        assert got == want, (v.hex(), hex(got), hex(want))
    got_nan = oracle.f64_to_bf16(math.nan, L)
    assert (got_nan & 0x7F80) == 0x7F80 and (got_nan & 0x7F) != 0


# ---------------------------------------------------------------- indexer ---

def _ref_scores(wl, queries=None):
    """Independent indexer scores: numpy dequant + matmul + ReLU + weighted sum."""
    qs = range(wl.Q) if queries is None else queries
    out = []
    for i in qs:
        qd = ref_dequant_index(wl.iq_codes[i], wl.iq_scales[i])  # [32][128]
        if wl.cand_blocks is None:
            ents = np.arange(wl.n_entries)
        else:
            ents = (8 * wl.cand_blocks[i][:, None] + np.arange(8)[None, :]).reshape(-1)
        rows = i * wl.cache_q_stride + ents
        kd = ref_dequant_index(wl.key_codes[rows], wl.key_scales[rows])  # [n][128]
        d = qd @ kd.T  # [32][n]
        s = (wl.w[i].astype(np.float64)[:, None] * np.maximum(d, 0.0)).sum(axis=0)
        lim = wl.n_entries if wl.n_valid is None else min(int(wl.n_valid[i]), wl.n_entries)
        s = np.where(ents < lim, s, -np.inf)
        out.append(s)
    return np.stack(out)


def check_index_scores(L, seed=5):
    wl = synth.full_decode(3, 700, seed)
    sc, dots = oracle.index_score(wl, want_dots=True, L=L)
    ref = _ref_scores(wl)
    assert np.allclose(sc, ref, rtol=2e-7, atol=1e-30), np.abs(sc - ref).max()
    # exact dots: an exactly-rounded sum in a different (reversed) order agrees bit for bit
    for i in range(wl.Q):
        qd = ref_dequant_index(wl.iq_codes[i], wl.iq_scales[i])
        for e in (0, 17, 699):
            kd = ref_dequant_index(wl.key_codes[i * 700 + e], wl.key_scales[i * 700 + e])[0]
            for h in (0, 13, 31):
                exact = math.fsum(list((qd[h] * kd)[::-1]))
                assert dots[i, h, e] == exact, (i, h, e)
    # one-hot weights -> score = ReLU(d_h)
    for h in (0, 7, 31):
        wl1 = synth.full_decode(1, 200, seed)
        wl1.w[:] = 0
        wl1.w[0, h] = 1.0
        s1, d1 = oracle.index_score(wl1, want_dots=True, L=L)
        assert np.array_equal(s1[0], np.maximum(d1[0, h], 0).astype(np.float32)), h
    # zero keys -> score 0
    wl0 = synth.full_decode(1, 64, seed)
    wl0.key_codes[:] = 0
    s0 = oracle.index_score(wl0, L=L)
    assert np.all(s0 == 0)
    # ReLU comes before weighting: negative weight on a negative dot contributes 0
    wln = synth.full_decode(1, 256, seed)
    wln.w[:] = -1.0
    sn, dn = oracle.index_score(wln, want_dots=True, L=L)
    expect = -np.maximum(dn[0], 0).sum(axis=0)
    assert np.allclose(sn[0], expect, rtol=1e-6)
    assert np.all(sn[0] <= 0)


def check_candidate_sets(L, seed=9):
    # Reindex pool scores equal the Full-layer scores at entries 8b+r
    wlr = synth.reindex_decode(2, 4096, 64, seed, dense_rows=True)
    sr = oracle.index_score(wlr, L=L)
    assert np.allclose(sr, _ref_scores(wlr), rtol=2e-7)
    full = synth.Workload("f", wlr.Q, wlr.n_entries, wlr.cache_q_stride, wlr.main_cache, wlr.key_codes,
                          wlr.key_scales, wlr.iq_codes, wlr.iq_scales, wlr.w, wlr.q, wlr.swa, wlr.swa_q_stride,
                          wlr.n_swa)
    with np.errstate(invalid="ignore"):
        sf = oracle.index_score(full, L=L)
    for i in range(wlr.Q):
        ents = (8 * wlr.cand_blocks[i][:, None] + np.arange(8)[None, :]).reshape(-1)
        assert np.array_equal(sr[i], sf[i][ents])
    # causal limit: entries >= n_valid are -inf, the rest unchanged
    wlc = synth.prefill(5, 300, 40, seed, m=2)  # n_valid = 20..22
    sc = oracle.index_score(wlc, L=L)
    assert np.allclose(sc, _ref_scores(wlc), rtol=2e-7)
    for i in range(5):
        nv = wlc.n_valid[i]
        assert np.all(np.isneginf(sc[i, nv:])) and np.all(np.isfinite(sc[i, :nv]))


# ---------------------------------------------------------------- top-k ----

def _ref_topk(scores_row, ents, k):
    """Brute force: rank by (score desc, id asc; NaN last), keep k, list by id."""
    pairs = [(float(s), int(e)) for s, e in zip(scores_row, ents)]
    pairs.sort(key=lambda t: (0 if not math.isnan(t[0]) else 1, -t[0] if not math.isnan(t[0]) else 0, t[1]))
    top = sorted(e for _, e in pairs[:k])
    return top + [-1] * (k - len(top))


def check_topk(L, seed=11):
    rng = np.random.default_rng(seed)
    for n in (1, 511, 512, 513, 2048):
        s = rng.standard_normal((2, n)).astype(np.float32)
        idx, ts = oracle.topk(s, k=512, L=L)
        for i in range(2):
            assert list(idx[i]) == _ref_topk(s[i], range(n), 512), n
            m = min(n, 512)
            assert np.array_equal(ts[i, :m], s[i][idx[i, :m]])
            assert np.all(np.isneginf(ts[i, m:]))
            # every kept score >= every dropped score
            if n > 512:
                dropped = np.setdiff1d(np.arange(n), idx[i, :m])
                assert ts[i, :m].min() >= s[i][dropped].max()
    # ties: equal keys go to the lower index; -0 == +0
    s = np.zeros((1, 3000), np.float32)
    s[0, ::3] = 1.0
    s[0, 1::3] = -0.0
    idx, _ = oracle.topk(s, k=512, L=L)
    assert list(idx[0]) == list(range(0, 1536, 3))
    s2 = np.zeros((1, 1200), np.float32)
    s2[0, 600:] = 1.0
    s2[0, :600:2] = -0.0
    idx2, _ = oracle.topk(s2, k=700, L=L)
    assert list(idx2[0]) == list(range(100)) + list(range(600, 1200))
    # quantised scores with many duplicates, brute force
    s3 = np.round(rng.standard_normal((3, 4000)) * 4).astype(np.float32)
    idx3, _ = oracle.topk(s3, k=512, L=L)
    for i in range(3):
        assert list(idx3[i]) == _ref_topk(s3[i], range(4000), 512)
    # NaN ranks below every number
    s4 = rng.standard_normal((1, 600)).astype(np.float32)
    s4[0, :200] = np.nan
    idx4, _ = oracle.topk(s4, k=512, L=L)
    assert list(idx4[0]) == list(range(112)) + list(range(200, 600))
    # n_valid and pool translation
    s5 = rng.standard_normal((2, 64)).astype(np.float32)
    blocks = np.array([[3, 9, 10, 40, 41, 50, 60, 70], [0, 1, 2, 3, 4, 5, 6, 7]], np.int32)
    idx5, _ = oracle.topk(s5, k=16, n_valid=np.array([400, 30], np.int32), n_entries=1000, cand_blocks=blocks, L=L)
    for i in range(2):
        ents = (8 * blocks[i][:, None] + np.arange(8)[None, :]).reshape(-1)
        lim = [400, 30][i]
        keep = ents < lim
        assert list(idx5[i]) == _ref_topk(s5[i][keep], ents[keep], 16)


# ------------------------------------------------------------ attention ----

def _dense_ref(q_bf16, kv_f64, scale):
    """Library SDPA in fp64 (torch CPU math path)."""
    qq = torch.from_numpy(bf16_to_f64(q_bf16))[:, None, :]  # [64 heads][1][512]
    kk = torch.from_numpy(kv_f64)[None].expand(64, *kv_f64.shape).contiguous()  # [64][J][512]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, kk, scale=scale)
    logits = (qq @ kk.transpose(1, 2)) * scale
    lse = torch.logsumexp(logits[:, 0, :], dim=-1)
    return o[:, 0, :].numpy(), lse.numpy()


def assert_nearest_bf16(bits: np.ndarray, x: np.ndarray, rel_slack: float = 1e-12) -> None:
    """Each bf16 value is a nearest bf16 to the fp64 reference x: no farther
    from x than the bf16 values one unit below and above it (same sign), up to
    rel_slack of |x| for the reference's own fp64 rounding."""
    b = np.asarray(bits, np.uint16).reshape(-1).astype(np.int64)
    xv = np.asarray(x, np.float64).reshape(-1)
    mag = b & 0x7FFF
    neg = (b & 0x8000) != 0
    nonzero = mag != 0
    assert np.all(~nonzero | (neg == (xv < 0))), "bf16 sign differs from the reference"

    def val(m):
        return bf16_to_f64(m.astype(np.uint16))

    ax = np.abs(xv)
    d0 = np.abs(ax - val(mag))
    dn = np.abs(ax - val(np.maximum(mag - 1, 0)))
    dp = np.abs(ax - val(np.minimum(mag + 1, 0x7F7F)))
    slack = rel_slack * ax + 1e-300
    assert np.all(d0 <= np.minimum(dn, dp) + slack), "a bf16 output is not a nearest bf16 of the reference"


def check_attention(L, seed=13):
    n = 200
    wl = synth.full_decode(2, n, seed)
    idx = np.tile(np.arange(n, dtype=np.int32), (2, 1))
    ob, of, lse, probs = oracle.sparse_attn(wl, idx, want_probs=True, L=L)
    for i in range(2):
        kv = np.concatenate([ref_dequant_main(wl.main_cache[i * n:(i + 1) * n]),
                             bf16_to_f64(wl.swa[i * 128:(i + 1) * 128])])
        o_ref, lse_ref = _dense_ref(wl.q[i], kv, wl.scale)
        assert np.allclose(of[i], o_ref, rtol=1e-6, atol=1e-7), np.abs(of[i] - o_ref).max()
        assert np.allclose(lse[i], lse_ref, rtol=1e-6)
        assert np.allclose(bf16_to_f64(ob[i]), o_ref, rtol=8e-3, atol=1e-6)
        assert_nearest_bf16(ob[i], o_ref)
    assert np.allclose(probs.sum(axis=-1), 1.0, atol=1e-12)
    # permutation invariance of the selected list
    perm = np.random.default_rng(seed).permutation(n)
    _, of2, lse2 = oracle.sparse_attn(wl, idx[:, perm].copy(), L=L)
    assert np.allclose(of2, of, rtol=1e-6, atol=1e-7) and np.allclose(lse2, lse, rtol=1e-6)
    # padding (-1) and out-of-range ids are skipped
    idx_pad = np.full((2, 300), -1, np.int32)
    idx_pad[:, :n] = idx
    idx_pad[:, n] = n + 5
    _, of3, _ = oracle.sparse_attn(wl, idx_pad, L=L)
    assert np.allclose(of3, of, rtol=1e-6, atol=1e-7)
    # a single entry: o = v exactly
    one = np.full((2, 4), -1, np.int32)
    one[:, 2] = 7
    _, of4, _ = oracle.sparse_attn(wl, one, n_swa=0, L=L)
    for i in range(2):
        v = ref_dequant_main(wl.main_cache[i * n + 7])[0]
        assert np.array_equal(of4[i], np.broadcast_to(v.astype(np.float32), (64, 512)))
    # zero query: o = mean of the values
    wlz = synth.full_decode(1, n, seed)
    wlz.q[:] = 0
    _, of5, _ = oracle.sparse_attn(wlz, idx[:1], L=L)
    kv = np.concatenate([ref_dequant_main(wlz.main_cache[:n]), bf16_to_f64(wlz.swa[:128])])
    assert np.allclose(of5[0], np.broadcast_to(kv.mean(axis=0), (64, 512)), rtol=1e-6, atol=1e-7)
    # empty joint set: zeros and lse = -inf
    _, of6, lse6 = oracle.sparse_attn(wl, np.full((2, 8), -1, np.int32), n_swa=0, L=L)
    assert np.all(of6 == 0) and np.all(np.isneginf(lse6))


def check_decode_composition(L, seed=17):
    wl = synth.full_decode(2, 1500, seed)
    r = oracle.decode(wl, L=L)
    sc = oracle.index_score(wl, L=L)
    idx, _ = oracle.topk(sc, wl, L=L)
    ob, of, lse = oracle.sparse_attn(wl, idx, L=L)
    assert np.array_equal(r["scores"], sc) and np.array_equal(r["idx"], idx)
    assert np.array_equal(r["out_bf16"], ob) and np.array_equal(r["lse"], lse)
    # the selection is the true top-512 of the independent scores
    ref = _ref_scores(wl)
    for i in range(wl.Q):
        assert list(idx[i]) == _ref_topk(ref[i].astype(np.float32), range(wl.n_entries), 512)


# ------------------------------------------------------------- cache write ---

_E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
# Nearest E2M1 codes (OCP MX: round to nearest, ties to even) at the midpoints
# of the value table, and just below / just above them.
_AT_MID = [0, 2, 2, 4, 4, 6, 6]
_BELOW_MID = [0, 1, 2, 3, 4, 5, 6]
_ABOVE_MID = [1, 2, 3, 4, 5, 6, 7]


def _lib_e4m3_encode(v: np.ndarray) -> np.ndarray:
    """torch's float32 -> float8_e4m3fn conversion (RNE), as code bytes."""
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def check_quantize(L, seed=21):
    # (1) quantising the fp32-rounded sources reproduces the generator's stored
    # entries (an independent implementation of the same rule, from fp64)
    xm = synth.f32_rows(seed, synth.TID_MAIN, 0, 0, 600, 512)
    ent = synth.main_latents(seed, 0, 0, 600)
    assert np.array_equal(oracle.quantize_main(xm, L), ent)
    xk = synth.f32_rows(seed, synth.TID_IKEY, 0, 0, 600, 128)
    kc, ks = synth.index_keys(seed, 0, 0, 600)
    c, sc = oracle.quantize_index(xk, L)
    assert np.array_equal(c, kc) and np.array_equal(sc, ks)
    # (2) re-quantising dequantised entries gives them back: byte for byte for
    # main entries (their largest code is always 6); by value for indexer keys,
    # whose ceil-log2 scale drops by one where a block's largest code is <= 3
    assert np.array_equal(oracle.quantize_main(ref_dequant_main(ent).astype(np.float32), L), ent)
    d = ref_dequant_index(kc, ks)
    c, sc = oracle.quantize_index(d.astype(np.float32), L)
    assert np.array_equal(ref_dequant_index(c, sc), d)
    top = np.abs(d).reshape(-1, 4, 32).max(axis=2) > 3 * lib_e8m0(ks)
    assert top.any() and (~top).any() and np.array_equal(sc[top], ks[top])
    assert np.array_equal(sc[~top].astype(int), ks[~top].astype(int) - 1)
    # (3) the element error is at most half the local E2M1 spacing of x / s
    q = oracle.quantize_main(xm, L)
    s = np.repeat(lib_e4m3(q[:, 256:]), 16, axis=1)
    y = np.abs(xm.astype(np.float64)) / s
    err = np.abs(np.abs(ref_dequant_main(q)) / s - y)
    half = np.where(y <= 2, 0.25, np.where(y <= 4, 0.5, 1.0))
    assert np.all((err <= half) | (y >= 6))

    # (4) main scales: every finite E4M3 code, its midpoints, saturation, and
    # torch's own conversion of amax / 6 on random magnitudes
    vals = lib_e4m3(np.arange(0x7F, dtype=np.uint8))
    amax = [6 * vals, 6 * (vals[:-1] + vals[1:]) / 2, np.array([6 * 448 * 1.01, 6 * 480.0, 1e30, np.inf])]
    want = [np.arange(0x7F), [c if c % 2 == 0 else c + 1 for c in range(0x7E)], [0x7E] * 4]
    rng = np.random.default_rng(seed)
    r = np.exp2(rng.uniform(-12, 11, 4000)).astype(np.float32)
    amax.append(r)
    want.append(_lib_e4m3_encode((r.astype(np.float64) / 6).astype(np.float32)))
    a = np.concatenate(amax).astype(np.float32)
    w = np.concatenate([np.asarray(v, np.int64) for v in want])
    pad = (-len(a)) % 32
    a = np.concatenate([a, np.zeros(pad, np.float32)])
    w = np.concatenate([w, np.zeros(pad, np.int64)])
    x = np.zeros((len(a) // 32, 512), np.float32)
    x.reshape(-1, 32, 16)[:, :, 5] = -a.reshape(-1, 32)  # amax is a magnitude
    got = oracle.quantize_main(x, L)[:, 256:].reshape(-1)
    assert np.array_equal(got.astype(np.int64), w), np.nonzero(got.astype(np.int64) != w)

    # (5) element codes at a scale of exactly 1 (amax 6): ties, neighbours, signs
    row = np.zeros((3, 512), np.float32)
    tie = [6.0, *_E2M1_MIDS, *(-_E2M1_MIDS), -0.0]
    row[0, :16] = tie
    row[1, :16] = [6.0, *np.nextafter(_E2M1_MIDS.astype(np.float32), np.float32(0)), 0, 0, 0, 0, 0, 0, 0, np.nan]
    row[2, :16] = [6.0, *np.nextafter(_E2M1_MIDS.astype(np.float32), np.float32(np.inf)), *([0.0] * 7), 6.3]
    # a block whose scale rounds to zero, and one saturated at 448
    row[0, 16:32] = [-1e-4, 2e-4, -3e-4, *([0.0] * 13)]
    row[0, 32:48] = [6000.0, 2700.0, 2000.0, -6000.0, *([0.0] * 12)]
    row[0, 48:64] = [np.inf, 448.0, 224.0, *([0.0] * 13)]
    q = oracle.quantize_main(row, L)
    codes = nibbles(q[:, :256])
    assert list(q[:, 256]) == [0x38, 0x38, 0x38]
    assert list(codes[0, :16]) == [7, *_AT_MID, *(8 | np.array(_AT_MID)), 8]
    assert list(codes[1, :16]) == [7, *_BELOW_MID, *([0] * 7), 0]
    assert list(codes[2, :16]) == [7, *_ABOVE_MID, *([0] * 7), 7]
    assert q[0, 257] == 0 and not codes[0, 16:32].any()
    assert q[0, 258] == 0x7E and list(codes[0, 32:36]) == [7, 7, 6, 15]
    assert q[0, 259] == 0x7E and list(codes[0, 48:51]) == [7, 2, 1]

    # (6) indexer scales: exact powers of two, the next float up, clamps, zero
    es = np.arange(-127, 126)  # 6 * 2^126 is beyond the fp32 range
    a = np.concatenate([6 * np.exp2(es), np.nextafter((6 * np.exp2(es[:-1])).astype(np.float32), np.float32(np.inf)),
                        [1e-45, 0.0, 3e38]]).astype(np.float32)
    w = np.concatenate([es + 127, es[:-1] + 128, [0, 127, 253]])
    r = np.exp2(rng.uniform(-60, 60, 3000)).astype(np.float32)
    a = np.concatenate([a, r])
    # smallest e with 6 * 2^e >= amax, from Python's exact frexp
    w = np.concatenate([w, [(lambda m, e: e + 127 - (m == 0.5))(*math.frexp(float(v) / 6.0)) for v in r]])
    pad = (-len(a)) % 4
    a = np.concatenate([a, np.zeros(pad, np.float32)])
    w = np.concatenate([w, np.full(pad, 127)])
    x = np.zeros((len(a) // 4, 128), np.float32)
    x.reshape(-1, 4, 32)[:, :, 31] = a.reshape(-1, 4)
    _, sc = oracle.quantize_index(x, L)
    assert np.array_equal(sc.reshape(-1).astype(np.int64), w)
    # element codes at scale 2^0 (amax 6), and at 2^-3 (amax 0.75)
    x = np.zeros((2, 128), np.float32)
    x[0, :16] = tie
    x[1, :8] = [0.75, *(_E2M1_MIDS / 8)]
    x[1, 64:80] = [-0.0] * 16  # all-zero block: scale 2^0, codes 0
    c, sc = oracle.quantize_index(x, L)
    cc = nibbles(c)
    assert list(sc[0]) == [127, 127, 127, 127] and list(sc[1]) == [124, 127, 127, 127]
    assert list(cc[0, :16]) == [7, *_AT_MID, *(8 | np.array(_AT_MID)), 8]
    assert list(cc[1, :8]) == [7, *_AT_MID] and not cc[1, 64:80].any()


# ------------------------------------------------- window format and RoPE ---

def _with(wl, **kw):
    w2 = copy.copy(wl)
    w2.extra = dict(wl.extra)
    for k, v in kw.items():
        setattr(w2, k, v)
    return w2


def check_window_options(L, seed=23):
    # (1) FP8 window rows (R14): codes through torch's float8_e4m3fn, scales
    # through float8_e8m0fnu, scale b for channels 32b..32b+31
    rows = synth.fp8_rows(seed, synth.TID_SWA, 0, 0, 40)
    sweep = np.zeros((2, 528), np.uint8)
    sweep[0, :512] = np.arange(512) % 256
    sweep[0, 512:] = np.arange(112, 128)
    sweep[1, :512] = (np.arange(512) * 7) % 256
    sweep[1, 512:] = np.arange(120, 136)
    for r in (rows, sweep):
        ref = lib_e4m3(r[:, :512]) * np.repeat(lib_e8m0(r[:, 512:]), 32, axis=1)
        got = oracle.dequant_swa_fp8(r, L)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], ref[~nan])

    # (2) attention over FP8 rows equals attention over the same values as bf16 rows
    wl = synth.full_decode(3, 600, seed=seed)
    idx = np.stack([np.random.default_rng(seed + i).choice(600, 512, replace=False) for i in range(3)]).astype(np.int32)
    wl8 = synth.with_window_options(_with(wl), swa_fp8=True)
    vals = lib_e4m3(wl8.swa[:, :512]) * np.repeat(lib_e8m0(wl8.swa[:, 512:]), 32, axis=1)
    vb = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(vb.to(torch.float64).numpy(), vals)  # exact in bf16
    wlb = _with(wl, swa=np.ascontiguousarray(vb.view(torch.int16).numpy().view(np.uint16)), swa_format=0)
    a8, b8 = oracle.sparse_attn(wl8, idx, L=L), oracle.sparse_attn(wlb, idx, L=L)
    for x, y in zip(a8, b8):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)

    # (3) RoPE un-rotation (R15) of the rotary pairs (448 + 2i, 449 + 2i)
    plain = oracle.sparse_attn(wl, idx, L=L)
    ident = np.zeros((3, 32, 2), np.float32)
    ident[:, :, 0] = 1.0
    got = oracle.sparse_attn(_with(wl, rope=ident), idx, L=L)
    assert np.array_equal(got[0], plain[0]) and np.array_equal(got[1], plain[1])
    quarter = np.zeros((3, 32, 2), np.float32)
    quarter[:, :, 1] = 1.0  # cos 0, sin 1: (a, b) -> (b, -a)
    got = oracle.sparse_attn(_with(wl, rope=quarter), idx, L=L)[1]
    pf = plain[1]
    assert np.array_equal(got[:, :, :448], pf[:, :, :448])
    assert np.array_equal(got[:, :, 448::2], pf[:, :, 449::2])
    assert np.array_equal(got[:, :, 449::2], -pf[:, :, 448::2])
    tab = synth.rope_table(600 + 7 * np.arange(3))
    un = oracle.sparse_attn(_with(wl, rope=tab), idx, L=L)
    assert np.array_equal(un[2], plain[2])  # lse unchanged
    a, b = un[1][:, :, 448::2].astype(np.float64), un[1][:, :, 449::2].astype(np.float64)
    c, sn = tab[:, None, :, 0].astype(np.float64), tab[:, None, :, 1].astype(np.float64)
    fa, fb = a * c - b * sn, a * sn + b * c  # forward rotation by the same angles
    tol = 1e-6 * np.abs(pf).max()
    assert np.abs(fa - pf[:, :, 448::2]).max() <= tol and np.abs(fb - pf[:, :, 449::2]).max() <= tol
    assert np.array_equal(un[1][:, :, :448], pf[:, :, :448])


# ------------------------------------------------------- pool construction ---

def _ref_pool(scores_row: np.ndarray, lim: int, n_pool: int) -> list:
    """Brute force of R16: block max over valid entries (NaN lowest), then a
    plain sort by (score desc, block asc) with NaN last."""
    n = len(scores_row)
    nb_valid = (min(lim, n) + 7) // 8
    blocks = []
    for b in range(nb_valid):
        seg = scores_row[8 * b:min(8 * b + 8, lim)].astype(np.float64)
        num = seg[~np.isnan(seg)]
        best = float(num.max()) if num.size else float("nan")
        blocks.append((b, best))
    blocks.sort(key=lambda t: (1, 0.0, t[0]) if math.isnan(t[1]) else (0, -t[1], t[0]))
    keep = sorted(b for b, _ in blocks[:n_pool])
    return keep + [-1] * (n_pool - len(keep))


def check_pool(L, seed=29):
    rng = np.random.default_rng(seed)
    # random scores with ties (coarse grid), NaNs, -0 / +0 and -inf
    n = 8 * 300 + 5  # ragged last block
    sc = np.round(rng.standard_normal((4, n)) * 4) / 4
    sc = sc.astype(np.float32)
    sc[0, rng.integers(0, n, 200)] = np.nan
    sc[1, ::7] = -0.0
    sc[1, 3::7] = 0.0
    sc[2, rng.integers(0, n, 100)] = -np.inf
    sc[3, :] = 1.0  # every block ties: the lowest ids win
    n_valid = np.array([n, 1001, 8 * 17 + 3, 777], np.int32)
    for n_pool in (1, 16, 100, 303):
        got = oracle.pool_blocks(sc, n_pool, n_valid, L=L)
        for q in range(4):
            assert list(got[q]) == _ref_pool(sc[q], int(n_valid[q]), n_pool), (n_pool, q)
    # a straddling block ignores its entries past the limit
    s1 = np.zeros((1, 64), np.float32)
    s1[0, 13] = 100.0  # entry 13 lies in block 1, past a limit of 12
    s1[0, 2] = 1.0
    assert list(oracle.pool_blocks(s1, 1, np.array([12], np.int32), L=L)[0]) == [0]
    assert list(oracle.pool_blocks(s1, 1, np.array([14], np.int32), L=L)[0]) == [1]
    # more blocks requested than valid: all valid blocks in order, then -1
    got = oracle.pool_blocks(s1, 5, np.array([20], np.int32), L=L)[0]
    assert list(got) == [0, 1, 2, -1, -1]
    # no limit given: the whole row, and the last block is the ragged one
    s2 = np.full((1, 21), -1.0, np.float32)
    s2[0, 20] = 5.0
    assert list(oracle.pool_blocks(s2, 1, L=L)[0]) == [2]


# ------------------------------------------------------------ m=2 pooling ---

def check_pooling(L, seed=31):
    from scipy.special import softmax
    rng = np.random.default_rng(seed)
    n = 40
    x = rng.standard_normal((2 * n, 512)).astype(np.float32)
    g = (rng.standard_normal((2 * n, 512)) * 2).astype(np.float32)
    got = oracle.pool_latents(x, g, L=L)
    # the two-way softmax of the gates, from a library routine, weights the pair
    w = softmax(np.stack([g[0::2], g[1::2]]).astype(np.float64), axis=0)
    ref = w[0] * x[0::2] + w[1] * x[1::2]
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)
    lo, hi = np.minimum(x[0::2], x[1::2]), np.maximum(x[0::2], x[1::2])
    assert np.all(got >= lo - 1e-12) and np.all(got <= hi + 1e-12)  # a convex mix
    # equal gates: the plain mean; a gate 60 higher: that token alone
    eq = oracle.pool_latents(x, np.zeros_like(g), L=L)
    assert np.array_equal(eq, (x[0::2].astype(np.float64) + x[1::2]) / 2)
    far = np.zeros_like(g)
    far[0::2] = 60.0
    assert np.allclose(oracle.pool_latents(x, far, L=L), x[0::2], rtol=1e-15, atol=0)
    # swapping the two tokens (and their gates) changes nothing
    xs, gs = x.reshape(n, 2, 512)[:, ::-1].reshape(2 * n, 512), g.reshape(n, 2, 512)[:, ::-1].reshape(2 * n, 512)
    assert np.array_equal(oracle.pool_latents(xs, gs, L=L), got)
    # one logit per token equals that logit in every channel
    gt = g[:, :1]
    assert np.array_equal(oracle.pool_latents(x, gt, L=L), oracle.pool_latents(x, np.repeat(gt, 512, axis=1), L=L))


# ---------------------------------------------------- Reuse-layer gather ---

def check_gather(L, seed=37):
    wl = synth.full_decode(3, 700, seed=seed)
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(700, 300, replace=False) for _ in range(3)]).astype(np.int32)
    idx[0, 5] = -1
    idx[1, 7] = 700
    idx[2, -1] = 10 ** 6
    g, dense = oracle.gather_selected(wl.main_cache, 700, 700, idx, L=L)
    for q in range(3):
        for j in range(300):
            e = idx[q, j]
            if 0 <= e < 700:
                assert dense[q, j] == j and np.array_equal(g[q, j], wl.main_cache[q * 700 + e])
            else:
                assert dense[q, j] == -1 and not g[q, j].any()
    # attention over the dense list with dense ids = attention over the cache
    dl = copy.copy(wl)
    dl.main_cache, dl.n_entries, dl.cache_q_stride = g.reshape(-1, 288), 300, 300
    a, b = oracle.sparse_attn(wl, idx, L=L), oracle.sparse_attn(dl, dense, L=L)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)


ALL_CHECKS = [check_format_tables, check_layout, check_bf16_rounding, check_dequant, check_index_scores, check_candidate_sets,
              check_topk, check_attention, check_decode_composition, check_quantize, check_window_options,
              check_pool, check_pooling, check_gather]
