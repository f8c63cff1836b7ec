"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the CPU oracle under the acceptance rules:

  * dequantisation: bit-exact (NaN positions equal);
  * indexer scores: |gpu - oracle| <= 1e-5 * sum_h |w_h| max(d_h, 0) (the fp32
    accumulation of 32 exact head terms; the oracle rounds once);
  * top-k on identical scores: identical ids and scores;
  * top-k end to end: the band rule — entries whose oracle score lies within
    1e-5 relative of the oracle's k-th largest score are don't-care, every other entry
    has the same membership, and the GPU returns min(k, n_valid) distinct valid
    ids followed by -1;
  * attention: max |gpu - oracle| <= 1e-2 * max |oracle| (bf16 out, fp32
    accumulation).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import compressed_sparse_attention_score_amd as csa
import oracle
from synth.device import to_device

SCORE_RTOL = 1e-5
BAND_RTOL = 1e-5
ATTN_TOL = 1e-2


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_np_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gpu_scores(db) -> np.ndarray:
    scores = torch.empty((db.Q, max(db.n_cand, 1)), dtype=torch.float32, device="cuda")
    csa.csa2_index_score(db.index_args(), scores)
    torch.cuda.synchronize()
    return to_np(scores)[:, :db.n_cand]


def gpu_topk(scores_np: np.ndarray, k: int, n_entries: int, cand_blocks=None, n_valid=None):
    s = torch.from_numpy(np.ascontiguousarray(scores_np, np.float32)).cuda()
    Q = s.shape[0]
    idx = torch.empty((Q, k), dtype=torch.int32, device="cuda")
    ts = torch.empty((Q, k), dtype=torch.float32, device="cuda")
    cb = None if cand_blocks is None else torch.from_numpy(np.ascontiguousarray(cand_blocks, np.int32)).cuda()
    nv = None if n_valid is None else torch.from_numpy(np.ascontiguousarray(n_valid, np.int32)).cuda()
    csa.csa2_topk(csa.topk_args(s, n_entries, k, idx, ts, cb, nv))
    torch.cuda.synchronize()
    return to_np(idx), to_np(ts)


def gpu_attn(db, idx_np: np.ndarray | None, n_swa=None):
    out = torch.empty((db.Q, 64, 512), dtype=torch.int16, device="cuda")
    lse = torch.empty((db.Q, 64), dtype=torch.float32, device="cuda")
    idx = None if idx_np is None else torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).cuda()
    csa.csa2_sparse_attn(db.attn_args(idx, out, lse, n_swa=n_swa))
    torch.cuda.synchronize()
    return to_np(out).view(np.uint16), to_np(lse)


def gpu_decode(db):
    out, lse, idx = db.new_outputs()
    csa.csa2_decode(db.decode_args(out, lse, idx))
    torch.cuda.synchronize()
    return to_np(out).view(np.uint16), to_np(lse), to_np(idx)


FP32_U = 2.0 ** -24   # unit roundoff of fp32


def check_scores(gpu: np.ndarray, ref: np.ndarray, dots: np.ndarray, w: np.ndarray, what="", block_abs=None):
    """dots [Q][32][n] from the oracle; w [Q][32]. block_abs [Q][32][n]
    (optional) = sum over the four 32-channel blocks of |block dot|: when block
    scales lie far apart the four block dots no longer sum exactly in fp32,
    and each head may be off by the fp32 summation bound gamma_4 = 4u of that
    sum (ReLU is 1-Lipschitz, so the score by sum_h |w_h| times it)."""
    inv_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu), inv_ref), f"{what}: invalid-candidate pattern differs"
    wa = np.abs(w.astype(np.float64))
    s_abs = np.einsum("qh,qhn->qn", wa, np.maximum(dots, 0.0))
    with np.errstate(invalid="ignore"):
        err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    bound = SCORE_RTOL * s_abs + 1e-30
    if block_abs is not None:
        bound = bound + 4 * FP32_U * np.einsum("qh,qhn->qn", wa, block_abs)
    bad = (err > bound) & ~inv_ref
    assert not bad.any(), f"{what}: {bad.sum()} scores off, worst {np.max(err[~inv_ref] / bound[~inv_ref]):.3g}x bound"


E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mxfp4_values(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[..., 64] E2M1 code bytes (channel 2j low nibble) and [..., 4] E8M0
    scales -> [..., 128] fp64 values (tolerance helper, not a reference)."""
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], 128)
    v = E2M1_MAG[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    return v * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)


def block_abs_dots(wl) -> np.ndarray:
    """[Q][32][n_cand] sum over the 32-channel blocks of |q_h . k| of each
    block (independent caches, plain ranges)."""
    assert wl.cand_blocks is None and wl.cache_q_stride == wl.n_entries
    out = np.empty((wl.Q, 32, wl.n_entries))
    for i in range(wl.Q):
        qv = mxfp4_values(wl.iq_codes[i], wl.iq_scales[i]).reshape(32, 4, 32)
        rows = slice(i * wl.n_entries, (i + 1) * wl.n_entries)
        kv = mxfp4_values(wl.key_codes[rows], wl.key_scales[rows]).reshape(-1, 4, 32)
        out[i] = np.abs(np.einsum("hbc,nbc->hnb", qv, kv)).sum(axis=-1)
    return out


def valid_entries(wl, qi):
    if wl.cand_blocks is None:
        ents = np.arange(wl.n_entries)
    else:
        ents = (8 * wl.cand_blocks[qi][:, None].astype(np.int64) + np.arange(8)[None, :]).reshape(-1)
    lim = wl.n_entries if wl.n_valid is None else min(int(wl.n_valid[qi]), wl.n_entries)
    return ents[(ents >= 0) & (ents < lim)]


def check_topk_band(gpu_idx: np.ndarray, ref_scores: np.ndarray, ref_idx: np.ndarray, wl, k: int, what=""):
    """Band rule. ref_scores [Q][n_cand] by candidate position."""
    for qi in range(gpu_idx.shape[0]):
        ents = valid_entries(wl, qi)
        nvalid = len(ents)
        m = min(k, nvalid)
        g = gpu_idx[qi]
        assert np.all(g[m:] == -1), f"{what} q{qi}: padding"
        gs = g[:m]
        assert len(set(gs.tolist())) == m, f"{what} q{qi}: duplicate ids"
        assert set(gs.tolist()) <= set(ents.tolist()), f"{what} q{qi}: invalid ids"
        if nvalid <= k:
            continue
        # oracle score of an entry id
        if wl.cand_blocks is None:
            def score_of(e, _r=ref_scores[qi]):
                return float(_r[e])
        else:
            allents = (8 * wl.cand_blocks[qi][:, None].astype(np.int64) + np.arange(8)[None, :]).reshape(-1)
            order = np.argsort(allents, kind="stable")

            def score_of(e, _r=ref_scores[qi], _a=allents, _o=order):
                pos = _o[np.searchsorted(_a[_o], e)]
                return float(_r[pos])
        # the oracle lists its selection by entry id: tau is its lowest score
        tau = min(score_of(int(e)) for e in ref_idx[qi][:k])
        band = BAND_RTOL * abs(tau)
        rset, gset = set(ref_idx[qi].tolist()), set(gs.tolist())
        for e in rset ^ gset:
            se = score_of(e)
            assert abs(se - tau) <= band, f"{what} q{qi}: entry {e} score {se} outside band of tau {tau}"


class QueryView:
    """The workload fields the band check reads, restricted to queries qs."""

    def __init__(self, wl, qs):
        self.n_entries = wl.n_entries
        self.cand_blocks = None if wl.cand_blocks is None else wl.cand_blocks[qs]
        self.n_valid = None if wl.n_valid is None else wl.n_valid[qs]


def check_attn(gpu_bf16: np.ndarray, ref_f32: np.ndarray, what=""):
    g = bf16_np_to_f64(gpu_bf16)
    r = ref_f32.astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    scale = max(np.max(np.abs(r)), 1e-30)
    err = np.max(np.abs(g - r)) if r.size else 0.0
    assert err <= ATTN_TOL * scale, f"{what}: max abs err {err:.3g} > {ATTN_TOL} * {scale:.3g}"
    return err / scale


def check_lse(gpu: np.ndarray, ref: np.ndarray, what=""):
    inf_r = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu), inf_r), f"{what}: lse -inf pattern"
    assert np.allclose(gpu[~inf_r], ref[~inf_r], rtol=1e-4, atol=1e-3), f"{what}: lse"


__all__ = ["block_abs_dots", "mxfp4_values", "announce", "to_device", "gpu_scores", "gpu_topk", "gpu_attn", "gpu_decode", "check_scores",
           "check_topk_band", "QueryView", "check_attn", "check_lse", "oracle", "bf16_np_to_f64", "valid_entries"]
