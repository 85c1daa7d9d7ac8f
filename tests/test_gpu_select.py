"""GPU parity of dflash_select_path against the oracle (exact paths, exact
float32 scores) and against brute force on small lattices."""

import numpy as np
import pytest
import torch

from oracle.selector import select_path as oracle_select

pytestmark = pytest.mark.gpu
K = 16


def lattice(seed, B, P, V, r, scale=1.0):
    rng = np.random.default_rng(seed)
    val = np.sort(rng.standard_normal((B, P, K)).astype(np.float32), -1)[..., ::-1].copy()
    idx = np.stack([np.stack([rng.choice(V, K, replace=False) for _ in range(P)]) for _ in range(B)])
    F_l = (scale * rng.standard_normal((V, r))).astype(np.float32)
    F_r = (scale * rng.standard_normal((V, r))).astype(np.float32)
    return val, idx.astype(np.int32), F_l, F_r


def run(dfl, dev, val, idx, F_l, F_r):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    rank, tok, score = dfl.select_path(t(val), t(idx), t(F_l), t(F_r))
    torch.cuda.synchronize()
    return rank.cpu().numpy(), tok.cpu().numpy(), score.cpu().numpy()


@pytest.mark.parametrize("B,P,V,r", [(4, 1, 100, 4), (4, 2, 100, 8), (3, 3, 500, 32), (5, 7, 4096, 32),
                                     (2, 7, 4096, 192), (2, 15, 4096, 192), (3, 6, 1000, 256),
                                     (2, 15, 300, 4), (1, 11, 2000, 64)])
def test_matches_oracle(dfl, dev, B, P, V, r):
    val, idx, F_l, F_r = lattice(B * 31 + P * 7 + r, B, P, V, r)
    rank, tok, score = run(dfl, dev, val, idx, F_l, F_r)
    r0, t0, s0, _ = oracle_select(val, idx, F_l, F_r)
    assert np.array_equal(rank, r0)
    assert np.array_equal(tok, t0)
    assert np.array_equal(score, s0)


def test_zero_tables_pick_top1(dfl, dev):
    val, idx, F_l, F_r = lattice(3, 6, 7, 900, 16)
    rank, tok, _ = run(dfl, dev, val, idx, np.zeros_like(F_l), np.zeros_like(F_r))
    assert np.all(rank == 0)
    assert np.array_equal(tok, idx[:, :, 0])


def test_brute_force_small(dfl, dev):
    val, idx, F_l, F_r = lattice(9, 2, 4, 700, 24)
    rank, _, _ = run(dfl, dev, val, idx, F_l, F_r)
    for b in range(2):
        pairs = [F_l[idx[b, p]].astype(np.float64) @ F_r[idx[b, p + 1]].astype(np.float64).T
                 for p in range(3)]
        best, arg = -np.inf, None
        for path in np.ndindex(*([K] * 4)):
            s = sum(float(val[b, p, path[p]]) for p in range(4)) + \
                sum(pairs[p][path[p], path[p + 1]] for p in range(3))
            if s > best + 1e-12:
                best, arg = s, path
        assert tuple(rank[b]) == arg


def test_batch32_block8_shapes(dfl, dev):
    """Batch 32, block 8, rank 192 over a 151936-row table."""
    rng = np.random.default_rng(12)
    V, r, B, P = 151936, 192, 32, 7
    F_l = (0.04 * rng.standard_normal((V, r))).astype(np.float32)
    F_r = (0.04 * rng.standard_normal((V, r))).astype(np.float32)
    val = np.sort(rng.standard_normal((B, P, K)).astype(np.float32) * 0.05, -1)[..., ::-1].copy()
    idx = rng.integers(0, V, (B, P, K)).astype(np.int32)
    rank, tok, score = run(dfl, dev, val, idx, F_l, F_r)
    r0, t0, s0, _ = oracle_select(val, idx, F_l, F_r)
    assert np.array_equal(rank, r0) and np.array_equal(tok, t0) and np.array_equal(score, s0)


# ------------------------------------------------------------ anchored selector
def run_anchored(dfl, dev, val, idx, F_l, F_r, anchor):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    rank, tok, score = dfl.select_path(t(val), t(idx), t(F_l), t(F_r), anchor=t(anchor.astype(np.int32)))
    torch.cuda.synchronize()
    return rank.cpu().numpy(), tok.cpu().numpy(), score.cpu().numpy()


@pytest.mark.parametrize("B,P,V,r", [(4, 1, 100, 4), (4, 2, 100, 8), (5, 7, 4096, 32), (2, 7, 4096, 192),
                                     (2, 15, 4096, 192), (32, 7, 151936, 192)])
def test_anchored_matches_oracle(dfl, dev, B, P, V, r):
    val, idx, F_l, F_r = lattice(B * 13 + P + r, B, P, V, r)
    anchor = np.random.default_rng(P + r).integers(0, V, B)
    if B >= 3:
        anchor[:3] = [-1, V, 5 * V]              # outside the vocabulary: pair 0
    rank, tok, score = run_anchored(dfl, dev, val, idx, F_l, F_r, anchor)
    r0, t0, s0, _ = oracle_select(val, idx, F_l, F_r, anchor=anchor)
    assert np.array_equal(rank, r0) and np.array_equal(tok, t0) and np.array_equal(score, s0)


def test_anchor_changes_the_path_only_through_position_0(dfl, dev):
    """A dominant anchor edge fixes position 0 to the candidate pairing best
    with the anchor; an anchor whose feature row is zero reproduces the
    unanchored selector."""
    val, idx, F_l, F_r = lattice(77, 6, 7, 2000, 16)
    F_l = F_l.copy()
    F_l[11] = 0.0
    plain = run(dfl, dev, val, idx, F_l, F_r)
    zero = run_anchored(dfl, dev, val, idx, F_l, F_r, np.full(6, 11))
    assert all(np.array_equal(a, b) for a, b in zip(plain, zero))
    F_l[11, 0] = 1e4
    rank, _, _ = run_anchored(dfl, dev, val, idx, F_l, F_r, np.full(6, 11))
    assert np.array_equal(rank[:, 0], np.argmax(F_r[idx[:, 0], 0], axis=1))
