"""The allocation-free head entry point (dflash_head_topk_noalloc, scratch in
the library's static per-GPU array) against dflash_head_topk with a caller
workspace: identical values and ids on two calls in a row, the second smaller
than the first, so that it runs over the first call's leftover scratch."""

import numpy as np
import pytest
import torch

from oracle.head import head_topk as oracle_topk

pytestmark = pytest.mark.gpu


def _inputs(M, D, V, seed):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(M, D, generator=g).to(torch.bfloat16)
    W = (0.02 * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    return h, W


def test_noalloc_matches_workspace_entry(dfl, dev):
    for M, D, V, seed in ((224, 512, 20000, 11), (7, 256, 4096, 12), (56, 264, 3001, 13)):
        h, W = _inputs(M, D, V, seed)
        hd, Wd = h.to(dev), W.to(dev)
        print(f"noalloc case M={M} D={D} V={V}", flush=True)
        tv, ti = dfl.head_topk_noalloc(hd, Wd)
        rv, ri = dfl.head_topk(hd, Wd)
        torch.cuda.synchronize()
        assert torch.equal(ti, ri), M
        assert torch.equal(tv.view(torch.int32), rv.view(torch.int32)), M
        ov, oi, _ = oracle_topk(h, W)
        assert np.array_equal(ti.cpu().numpy(), oi)
        assert np.array_equal(tv.cpu().numpy(), ov)


def test_noalloc_rejects_oversized_scratch(dfl, dev):
    # 2^18 rows need 32 MiB of partial lists; rejected before any launch
    h = torch.zeros((1 << 18, 8), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((16, 8), dtype=torch.bfloat16, device=dev)
    with pytest.raises(dfl.DFlashError, match="workspace too small"):
        dfl.head_topk_noalloc(h, W)
