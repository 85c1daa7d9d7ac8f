"""GPU parity of dflash_verify_greedy_fused (greedy verification with the
target's argmax taken in the LM-head GEMM epilogue) against the oracle's
verify_greedy on exact target logits."""

import numpy as np
import pytest
import torch

from oracle.verify import verify_greedy_hidden

pytestmark = pytest.mark.gpu


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def block(seed, B, T, D, V, agree=0.8, grid=False):
    """Target hidden states planted toward random tokens; drafts equal to
    the target argmax with probability `agree` per slot."""
    rng = np.random.default_rng(seed)
    if grid:
        W = rng.integers(-1, 2, (V, D)).astype(np.float32)
        h = rng.integers(-1, 2, (B * T, D)).astype(np.float32)
    else:
        W = (0.02 * rng.standard_normal((V, D))).astype(np.float32)
        h = rng.standard_normal((B * T, D)).astype(np.float32)
        c = rng.integers(0, V, B * T)
        h += (6.0 * W[c] / np.maximum((W[c] ** 2).sum(1, keepdims=True), 1e-6)).astype(np.float32)
    return bf16(h), bf16(W), rng


@pytest.mark.parametrize("B,T,D,V,grid", [(3, 8, 256, 4096, False), (2, 16, 512, 5000, False),
                                          (4, 8, 64, 3001, True), (1, 8, 5120, 151936, False),
                                          (4, 16, 5120, 20000, False)])
def test_matches_oracle(dfl, dev, B, T, D, V, grid):
    h, W, rng = block(B * 7 + T + V, B, T, D, V, grid=grid)
    from oracle.head import head_logits
    g = head_logits(h, W).reshape(B, T, V).argmax(-1)
    d = g[:, :T - 1].copy()
    flip = rng.random(d.shape) > 0.8
    d[flip] = (d[flip] + 1) % V
    draft = torch.from_numpy(d.astype(np.int32))
    out, n = dfl.verify_greedy_fused(h.to(dev), W.to(dev), draft.to(dev))
    torch.cuda.synchronize()
    o0, n0 = verify_greedy_hidden(h, W, d)
    assert np.array_equal(n.cpu().numpy(), n0)
    assert np.array_equal(out.cpu().numpy(), o0)


@pytest.mark.parametrize("B,T,D,V,tau,boost", [(8, 8, 256, 4096, 1.0, 6.0), (8, 8, 5120, 151936, 1.0, 8.0),
                                               (3, 16, 512, 3001, 0.7, 5.0), (8, 8, 5120, 151936, 1.0, 0.0),
                                               (16, 8, 1024, 20000, 1.3, 7.0),
                                               # the MFMA statistics GEMM: one 128-row block at the full
                                               # vocabulary, and two 240-row blocks (M = 480)
                                               (16, 8, 5120, 151936, 1.0, 8.0), (30, 16, 512, 9000, 1.0, 6.0)])
def test_sample_fused_matches_oracle(dfl, dev, B, T, D, V, tau, boost):
    """Exact agreement with the sampler on exact logits, except for requests
    whose decisions lie within the float32 error of a boundary (margin 1e-5),
    and at most two of those."""
    from oracle.verify import verify_sample_hidden
    rng = np.random.default_rng(B + T + D + V)
    W = (0.02 * rng.standard_normal((V, D))).astype(np.float32)
    h = rng.standard_normal((B * T, D)).astype(np.float32)
    d = rng.integers(0, V, (B, T - 1))
    if boost > 0:  # target rows lean toward the drafts: acceptances
        rows = (np.arange(B)[:, None] * T + np.arange(T - 1)[None]).ravel()
        wd = W[d.ravel()]
        h[rows] += (boost * wd / (wd ** 2).sum(1, keepdims=True)).astype(np.float32)
    hb, Wb = bf16(h), bf16(W)
    rid = np.arange(B, dtype=np.int64) * 11 + 3
    pos0 = np.full(B, 512, np.int64)
    out, n = dfl.verify_sample_fused(hb.to(dev), Wb.to(dev), torch.from_numpy(d.astype(np.int32)).to(dev), tau, 6,
                                     torch.from_numpy(rid).to(dev), torch.from_numpy(pos0).to(dev))
    torch.cuda.synchronize()
    o0, n0, margin = verify_sample_hidden(hb, Wb, d, tau, 6, rid, pos0, return_margins=True)
    out, n = out.cpu().numpy(), n.cpu().numpy()
    same = (n == n0) & np.all(out == o0, axis=1)
    assert np.all(same | (margin < 1e-5)), (np.nonzero(~same), margin[~same])
    # a request lies within 1e-5 of a boundary with probability about 1e-4
    # (a few decisions per request, each within 1e-5 on either side), so more
    # than two mismatches in a call would not be rounding
    assert (~same).sum() <= 2, np.nonzero(~same)
