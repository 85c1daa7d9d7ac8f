"""GPU parity of the sampled-path selector (dflash_select_path_sampled) and
of verification with a general proposal (dflash_verify_sample_q) against the
oracle, the one-hot reduction to dflash_verify_sample, and a chi-square test
that the GPU's draft-then-verify pipeline emits the target's law."""

import numpy as np
import pytest
import torch
from scipy import stats

from oracle.selector import select_path_sampled as oracle_sampled
from oracle.verify import verify_sample_q as oracle_verify_q

pytestmark = pytest.mark.gpu
K = 16


def lattice(seed, B, P, V, r, scale=0.3):
    rng = np.random.default_rng(seed)
    val = np.sort(rng.standard_normal((B, P, K)).astype(np.float32), -1)[..., ::-1].copy()
    idx = np.stack([np.stack([rng.choice(V, K, replace=False) for _ in range(P)]) for _ in range(B)])
    F_l = (scale * rng.standard_normal((V, r))).astype(np.float32)
    F_r = (scale * rng.standard_normal((V, r))).astype(np.float32)
    return val, idx.astype(np.int32), F_l, F_r


def t(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("B,P,V,r,anchored", [(4, 1, 100, 4, False), (4, 2, 300, 8, True), (5, 7, 4096, 32, False),
                                              (8, 7, 151936, 192, False), (8, 7, 151936, 192, True),
                                              (2, 15, 5000, 192, True), (3, 6, 1000, 256, False)])
def test_selector_matches_oracle(dfl, dev, B, P, V, r, anchored):
    val, idx, F_l, F_r = lattice(B * 13 + P * 5 + r, B, P, V, r)
    rid = np.arange(B, dtype=np.int64) * 977 + 5
    pos0 = np.arange(B, dtype=np.int64) * 64 + 4096
    anchor = np.random.default_rng(1).integers(0, V, B).astype(np.int32) if anchored else None
    if anchored and B >= 2:
        anchor[1] = V + 3  # outside the vocabulary: no anchor term
    rank, tok, q = dfl.select_path_sampled(t(val, dev), t(idx, dev), t(F_l, dev), t(F_r, dev), 123, t(rid, dev),
                                           t(pos0, dev), anchor=None if anchor is None else t(anchor, dev))
    torch.cuda.synchronize()
    r0, t0, q0 = oracle_sampled(val, idx, F_l, F_r, 123, rid, pos0, anchor=anchor)
    assert np.array_equal(rank.cpu().numpy(), r0)
    assert np.array_equal(tok.cpu().numpy(), t0)
    np.testing.assert_allclose(q.cpu().numpy(), q0, rtol=1e-12, atol=1e-15)


def test_selector_zero_tables_give_softmax_of_values(dfl, dev):
    val, idx, F_l, F_r = lattice(2, 6, 7, 900, 16)
    z = np.zeros_like(F_l)
    rank, tok, q = dfl.select_path_sampled(t(val, dev), t(idx, dev), t(z, dev), t(z, dev), 9,
                                           t(np.arange(6, dtype=np.int64), dev), t(np.zeros(6, np.int64), dev))
    v = val.astype(np.float64)
    ref = np.exp(v - v.max(-1, keepdims=True))
    np.testing.assert_allclose(q.cpu().numpy(), ref / ref.sum(-1, keepdims=True), rtol=1e-13, atol=1e-16)


def planted_block(seed, B, T, V, idx, boost):
    """Target logits whose row t favours position t's candidates by `boost`."""
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((B, T, V)).astype(np.float32)
    for b in range(B):
        for p in range(T - 1):
            L[b, p, idx[b, p]] += np.float32(boost)
    return L


@pytest.mark.parametrize("B,T,V,boost", [(8, 8, 4096, 6.0), (8, 8, 151936, 9.0), (4, 16, 5000, 7.0),
                                         (6, 2, 333, 3.0), (8, 8, 151936, 0.0)])
def test_verify_q_matches_oracle(dfl, dev, B, T, V, boost):
    P = T - 1
    val, idx, F_l, F_r = lattice(B + T + V, B, P, V, 16)
    rid = np.arange(B, dtype=np.int64) + 40
    pos0 = np.full(B, 128, np.int64)
    _, d, q = oracle_sampled(val, idx, F_l, F_r, 77, rid, pos0)
    L = planted_block(V + B, B, T, V, idx, boost)
    out, n = dfl.verify_sample_q(t(L, dev), t(d, dev), t(idx, dev), t(q, dev), 1.0, 77, t(rid, dev), t(pos0, dev))
    torch.cuda.synchronize()
    o0, n0 = oracle_verify_q(L, d, idx, q, 1.0, 77, rid, pos0)
    assert np.array_equal(n.cpu().numpy(), n0)
    assert np.array_equal(out.cpu().numpy(), o0)


def test_verify_q_one_hot_is_verify_sample(dfl, dev):
    B, T, V = 16, 8, 20000
    rng = np.random.default_rng(5)
    L = rng.standard_normal((B, T, V)).astype(np.float32) * 3
    d = rng.integers(0, V, (B, T - 1)).astype(np.int32)
    L[np.arange(B)[:, None], np.arange(T - 1)[None], d] += 8.0
    qi = rng.integers(0, V, (B, T - 1, K)).astype(np.int32)
    qi[..., 3] = d
    qp = np.zeros((B, T - 1, K))
    qp[..., 3] = 1.0
    rid, pos0 = t(np.arange(B, dtype=np.int64) * 3, dev), t(np.full(B, 9, np.int64), dev)
    a = dfl.verify_sample(t(L, dev), t(d, dev), 1.0, 4, rid, pos0)
    b = dfl.verify_sample_q(t(L, dev), t(d, dev), t(qi, dev), t(qp, dev), 1.0, 4, rid, pos0)
    torch.cuda.synchronize()
    assert np.array_equal(a[0].cpu().numpy(), b[0].cpu().numpy())
    assert np.array_equal(a[1].cpu().numpy(), b[1].cpu().numpy())


def test_pipeline_emits_the_target_law(dfl, dev):
    """Sampled selector then verify_sample_q, all on the GPU, 2^16 requests of
    one position: the emitted token follows p, and the acceptance rate is
    sum_v min(p(v), q(v))."""
    N, V = 1 << 16, 64
    rng = np.random.default_rng(11)
    val1 = np.sort(rng.standard_normal(K).astype(np.float32))[::-1].copy()
    idx1 = rng.choice(V, K, replace=False).astype(np.int32)
    row0 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    row0[idx1[:4]] += 1.5
    F = np.zeros((V, 4), np.float32)
    val = t(np.broadcast_to(val1, (N, 1, K)), dev)
    idx = t(np.broadcast_to(idx1, (N, 1, K)), dev)
    rid = torch.arange(N, dtype=torch.int64, device=dev)
    pos0 = torch.full((N,), 700, dtype=torch.int64, device=dev)
    rank, tok, q = dfl.select_path_sampled(val, idx, t(F, dev), t(F, dev), 31, rid, pos0)
    L = t(np.broadcast_to(np.stack([row0, rng.standard_normal(V).astype(np.float32)]), (N, 2, V)), dev)
    out, n = dfl.verify_sample_q(L, tok, idx, q, 1.0, 31, rid, pos0)
    torch.cuda.synchronize()
    first = out[:, 0].cpu().numpy()
    p = np.exp(row0.astype(np.float64) - row0.max())
    p /= p.sum()
    obs = np.bincount(first, minlength=V).astype(np.float64)
    keep = N * p >= 5
    o, e = obs[keep], N * p[keep]
    if (~keep).any():  # the rare tokens as one bin
        o, e = np.append(o, obs[~keep].sum()), np.append(e, N * p[~keep].sum())
    assert stats.chisquare(o, e).pvalue > 1e-3
    q1 = q[0, 0].cpu().numpy()
    acc = sum(min(p[idx1[j]], q1[j]) for j in range(K))
    rate = (n.cpu().numpy() == 2).mean()
    assert abs(rate - acc) < 4 * np.sqrt(acc * (1 - acc) / N)
