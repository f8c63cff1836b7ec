"""The allocation-free attention entry point (csa2_sparse_attn_noalloc)
against csa2_sparse_attn with a caller workspace: same kernels, so the
outputs and lse must be identical, on two calls in a row (the second smaller,
so it runs over the static scratch the first one left behind), for a batch
that splits its slot list (scratch in use) and one that does not."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import announce, check_attn, oracle, to_device

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_sparse_attention_score_amd as csa


def _run(db, idx_np, noalloc):
    out = torch.empty((db.Q, 64, 512), dtype=torch.int16, device="cuda")
    lse = torch.empty((db.Q, 64), dtype=torch.float32, device="cuda")
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).cuda()
    args = db.attn_args(idx, out, lse)
    if noalloc:
        csa.csa2_sparse_attn_noalloc(args)
    else:
        csa.csa2_sparse_attn(args)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), lse.cpu().numpy()


@pytest.mark.parametrize("sizes", [((5, 3000, 512), (2, 900, 300)), ((300, 700, 512), (3, 600, 77))])
def test_noalloc_matches_workspace_call(sizes):
    for Q, N, k in sizes:  # second call smaller than the first
        announce(f"noalloc attention Q={Q} N={N} k={k}")
        wl = synth.with_window_options(synth.full_decode(Q, N, seed=Q + N), swa_fp8=(Q == 2), rope=(Q == 2))
        rng = np.random.default_rng(Q * 7 + N)
        idx = np.stack([rng.choice(N, k, replace=False) for _ in range(Q)]).astype(np.int32)
        idx[0, :3] = -1
        db = to_device(wl)
        need = csa.csa2_workspace_size(csa.CSA2_WS_ATTN, db.attn_args(None, db.q, None))
        assert need <= csa.CSA2_ATTN_SCRATCH_BYTES
        ob, lb = _run(db, idx, False)
        oa, la = _run(db, idx, True)
        assert np.array_equal(oa, ob), "outputs differ from the workspace call"
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), "lse differs"
        qs = [0, Q - 1]
        _, of, _ = oracle.sparse_attn(wl, idx[qs], queries=qs)
        check_attn(oa[qs], of, f"noalloc Q={Q}")
