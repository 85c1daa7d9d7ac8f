"""Pins for the oracle's pair selector: brute-force enumeration of every path,
a library matmul for the pair scores, and closed-form special cases."""

import itertools

import numpy as np
import pytest

from oracle.selector import pair_scores, select_path

K = 16


def make_case(seed, B, P, V=300, r=8, scale=1.0):
    rng = np.random.default_rng(seed)
    val = np.sort(rng.standard_normal((B, P, K)).astype(np.float32), axis=-1)[..., ::-1].copy()
    idx = np.stack([np.stack([rng.choice(V, K, replace=False) for _ in range(P)]) for _ in range(B)])
    F_l = (scale * rng.standard_normal((V, r))).astype(np.float32)
    F_r = (scale * rng.standard_normal((V, r))).astype(np.float32)
    return val, idx.astype(np.int32), F_l, F_r


def brute_force(val, idx, F_l, F_r):
    """Score every one of the 16^P paths; pair scores from a library matmul."""
    P = val.shape[0]
    pairs = [F_l[idx[p]].astype(np.float64) @ F_r[idx[p + 1]].astype(np.float64).T
             for p in range(P - 1)]
    grids = np.meshgrid(*[np.arange(K)] * P, indexing="ij")
    score = np.zeros([K] * P)
    for p in range(P):
        score = score + val[p].astype(np.float64)[grids[p]]
    for p in range(P - 1):
        score = score + pairs[p][grids[p], grids[p + 1]]
    flat = score.ravel()
    order = np.argsort(-flat, kind="stable")
    best, second = flat[order[0]], flat[order[1]]
    return np.array(np.unravel_index(order[0], score.shape)), best, best - second


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5])
def test_against_brute_force(P):
    val, idx, F_l, F_r = make_case(10 + P, B=3, P=P)
    rank, tok, s32, s64 = select_path(val, idx, F_l, F_r)
    for b in range(3):
        path, best, gap = brute_force(val[b], idx[b], F_l, F_r)
        assert gap > 1e-9  # unique optimum for these seeds
        assert list(rank[b]) == list(path)
        assert list(tok[b]) == [idx[b, p, path[p]] for p in range(P)]
        assert abs(s64[b] - best) <= 1e-12 * (1 + abs(best))
        assert s32[b] == np.float32(s64[b])


@pytest.mark.slow
def test_brute_force_block8():
    """One full block-8 lattice (P = 7): all 16^7 = 268M paths, chunked."""
    val, idx, F_l, F_r = make_case(99, B=1, P=7, V=4096, r=32, scale=0.5)
    val, idx = val[0], idx[0]
    pairs = [F_l[idx[p]].astype(np.float64) @ F_r[idx[p + 1]].astype(np.float64).T for p in range(6)]
    v64 = val.astype(np.float64)
    # tail[i1..i6] = every term of positions 1..6, built by broadcasting
    shape = [K] * 6
    g = np.meshgrid(*[np.arange(K)] * 6, indexing="ij")
    tail = np.zeros(shape)
    for q in range(6):
        tail = tail + v64[q + 1][g[q]]
    for q in range(5):
        tail = tail + pairs[q + 1][g[q], g[q + 1]]
    best, arg = -np.inf, None
    for i0 in range(K):
        s = v64[0][i0] + pairs[0][i0][g[0]] + tail
        j = int(np.argmax(s))
        if s.flat[j] > best:
            best, arg = s.flat[j], (i0,) + np.unravel_index(j, s.shape)
    rank, tok, s32, s64 = select_path(val[None], idx[None], F_l, F_r)
    assert list(rank[0]) == [int(a) for a in arg]
    assert abs(s64[0] - best) <= 1e-12 * (1 + abs(best))


def test_pair_scores_equal_library_matmul():
    _, idx, F_l, F_r = make_case(5, B=1, P=2, r=192)
    seq = pair_scores(idx[0, 0], idx[0, 1], F_l, F_r)
    lib = F_l[idx[0, 0]].astype(np.float64) @ F_r[idx[0, 1]].astype(np.float64).T
    assert np.allclose(seq, lib, rtol=1e-13, atol=1e-13)


def test_zero_tables_give_top1_path():
    val, idx, F_l, F_r = make_case(6, B=4, P=7)
    rank, tok, _, s64 = select_path(val, idx, np.zeros_like(F_l), np.zeros_like(F_r))
    assert np.all(rank == 0)
    assert np.allclose(s64, val[:, :, 0].astype(np.float64).sum(-1))


def test_single_position_is_argmax():
    rng = np.random.default_rng(7)
    val = rng.standard_normal((5, 1, K)).astype(np.float32)
    idx = np.tile(np.arange(K, dtype=np.int32), (5, 1, 1))
    F = rng.standard_normal((K, 4)).astype(np.float32)
    rank, _, _, _ = select_path(val, idx, F, F)
    assert list(rank[:, 0]) == list(np.argmax(val[:, 0], -1))


def test_ties_take_lowest_rank():
    val = np.zeros((1, 4, K), dtype=np.float32)
    idx = np.tile(np.arange(K, dtype=np.int32), (1, 4, 1))
    F = np.ones((K, 4), dtype=np.float32)
    rank, _, _, _ = select_path(val, idx, F, F)
    assert np.all(rank == 0)


def test_reported_score_is_path_score_and_shift_invariant():
    val, idx, F_l, F_r = make_case(8, B=2, P=6)
    rank, _, _, s64 = select_path(val, idx, F_l, F_r)
    for b in range(2):
        path = rank[b]
        resum = sum(float(val[b, p, path[p]]) for p in range(6))
        resum += sum(float(pair_scores(idx[b, p], idx[b, p + 1], F_l, F_r)[path[p], path[p + 1]])
                     for p in range(5))
        assert abs(resum - s64[b]) <= 1e-12 * (1 + abs(resum))
    shifted = val.copy()
    shifted[:, 3] += np.float32(4.0)
    rank2, _, _, _ = select_path(shifted, idx, F_l, F_r)
    assert np.array_equal(rank, rank2)


# ------------------------------------------------------------ anchored variant
def brute_force_anchored(val, idx, F_l, F_r, a):
    """Every path with the anchor's pair term on position 0 (library matmul)."""
    extra = (F_l[[a]].astype(np.float64) @ F_r[idx[0]].astype(np.float64).T)[0]
    v = val.astype(np.float64).copy()
    v[0] = v[0] + extra
    return brute_force(v, idx, F_l, F_r)


@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_anchored_against_brute_force(P):
    val, idx, F_l, F_r = make_case(40 + P, 6, P)
    anchor = np.random.default_rng(P).integers(0, F_l.shape[0], 6)
    rank, tok, score, score64 = select_path(val, idx, F_l, F_r, anchor=anchor)
    for b in range(6):
        path, best, gap = brute_force_anchored(val[b], idx[b], F_l, F_r, int(anchor[b]))
        if gap > 1e-9:
            assert list(rank[b]) == list(path)
        assert abs(score64[b] - best) <= 1e-9 * max(1.0, abs(best))


def test_anchor_with_zero_features_or_outside_vocab_is_unanchored():
    val, idx, F_l, F_r = make_case(7, 5, 4)
    F_l0 = F_l.copy()
    F_l0[3] = 0.0
    plain = select_path(val, idx, F_l0, F_r)
    zero = select_path(val, idx, F_l0, F_r, anchor=np.full(5, 3))
    outside = select_path(val, idx, F_l0, F_r, anchor=np.array([-1, 300, 10**6, -7, 301]))
    for r in (zero, outside):
        assert np.array_equal(r[0], plain[0]) and np.array_equal(r[3], plain[3])


def test_dominant_anchor_edge_fixes_the_first_choice():
    """An anchor pair term far larger than everything else picks position 0's
    candidate with the largest pair score with the anchor, then the
    unanchored DP of the remaining positions given that start."""
    val, idx, F_l, F_r = make_case(9, 4, 3, r=4)
    F_l = F_l.copy()
    F_l[5] = 0.0
    F_l[5, 0] = 1000.0
    rank, _, _, _ = select_path(val, idx, F_l, F_r, anchor=np.full(4, 5))
    for b in range(4):
        assert rank[b, 0] == int(np.argmax(F_r[idx[b, 0], 0]))
