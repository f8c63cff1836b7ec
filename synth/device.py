"""Copy a host ``synth.Workload`` into device memory as a DeviceBatch."""
from __future__ import annotations

import numpy as np
import torch

from compressed_sparse_attention_score_amd.batch import DeviceBatch

from . import IKEY_CODE_BYTES, IKEY_SCALE_BYTES, MAIN_BYTES, POISON_E4M3, POISON_E8M0


def _t(a, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def to_device(wl, device="cuda") -> DeviceBatch:
    if wl.extra.get("pool_rows") is not None and not wl.extra.get("dense_rows", True):
        # sparse host cache: poison every row on the device, then scatter the pool rows
        rows = wl.Q * wl.cache_q_stride
        main = torch.zeros((rows, MAIN_BYTES), dtype=torch.uint8, device=device)
        main[:, 256:] = POISON_E4M3
        kc = torch.zeros((rows, IKEY_CODE_BYTES), dtype=torch.uint8, device=device)
        ks = torch.full((rows, IKEY_SCALE_BYTES), POISON_E8M0, dtype=torch.uint8, device=device)
        pr = torch.from_numpy(wl.extra["pool_rows"]).to(device)
        main[pr] = _t(wl.main_cache, device)
        kc[pr] = _t(wl.key_codes, device)
        ks[pr] = _t(wl.key_scales, device)
    else:
        main, kc, ks = _t(wl.main_cache, device), _t(wl.key_codes, device), _t(wl.key_scales, device)
    return DeviceBatch(
        Q=wl.Q, n_entries=wl.n_entries, cache_q_stride=wl.cache_q_stride, main_cache=main, key_codes=kc,
        key_scales=ks, iq_codes=_t(wl.iq_codes, device), iq_scales=_t(wl.iq_scales, device), w=_t(wl.w, device),
        q=_t(wl.q, device, torch.int16), swa=_t(wl.swa, device, None if wl.swa_format else torch.int16),
        swa_q_stride=wl.swa_q_stride, n_swa=wl.n_swa, k=wl.k, scale=float(wl.scale),
        cand_blocks=None if wl.cand_blocks is None else _t(wl.cand_blocks.astype(np.int32), device),
        n_valid=None if wl.n_valid is None else _t(wl.n_valid.astype(np.int32), device),
        swa_format=int(wl.swa_format), rope=None if wl.rope is None else _t(wl.rope.astype(np.float32), device))
