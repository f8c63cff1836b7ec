"""A batch of CSA2 inputs resident in device memory, and the C argument structs
that describe it. Plumbing only: holds torch CUDA tensors and their sizes."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import attn_args, decode_args, index_args


@dataclass
class DeviceBatch:
    Q: int
    n_entries: int
    cache_q_stride: int
    main_cache: torch.Tensor    # uint8 [rows][288]
    key_codes: torch.Tensor     # uint8 [rows][64]
    key_scales: torch.Tensor    # uint8 [rows][4]
    iq_codes: torch.Tensor      # uint8 [Q][32][64]
    iq_scales: torch.Tensor     # uint8 [Q][32][4]
    w: torch.Tensor             # float32 [Q][32]
    q: torch.Tensor             # int16 (bf16 bits) [Q][64][512]
    swa: torch.Tensor           # int16 (bf16 bits) [rows][512], or uint8 [rows][528] FP8 rows
    swa_q_stride: int
    n_swa: int
    k: int = 512
    scale: float = 512 ** -0.5
    cand_blocks: Optional[torch.Tensor] = None  # int32 [Q][n_blocks]
    n_valid: Optional[torch.Tensor] = None      # int32 [Q]
    swa_format: int = 0                         # CSA2_SWA_BF16 / CSA2_SWA_FP8
    rope: Optional[torch.Tensor] = None         # float32 [Q][32][2] (cos, sin)

    @property
    def n_cand(self) -> int:
        return 8 * int(self.cand_blocks.shape[1]) if self.cand_blocks is not None else self.n_entries

    def index_args(self):
        return index_args(self.Q, self.n_entries, self.cache_q_stride, self.key_codes, self.key_scales, self.iq_codes,
                          self.iq_scales, self.w, self.cand_blocks, self.n_valid)

    def attn_args(self, idx, out, lse=None, n_swa=None):
        return attn_args(self.Q, self.n_entries, self.cache_q_stride, self.main_cache, idx, self.q, self.swa,
                         self.swa_q_stride, self.n_swa if n_swa is None else n_swa, self.scale, out, lse,
                         self.swa_format, self.rope)

    def decode_args(self, out, lse=None, idx_out=None, stage_events=None):
        return decode_args(self.index_args(), self.k, self.main_cache, self.q, self.swa, self.swa_q_stride, self.n_swa,
                           self.scale, out, lse, idx_out, stage_events, self.swa_format, self.rope)

    def new_outputs(self):
        dev = self.q.device
        out = torch.empty((self.Q, 64, 512), dtype=torch.int16, device=dev)
        lse = torch.empty((self.Q, 64), dtype=torch.float32, device=dev)
        idx = torch.empty((self.Q, self.k), dtype=torch.int32, device=dev)
        return out, lse, idx
