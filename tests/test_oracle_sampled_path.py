"""Pins for the oracle's sampled-path selector and the verifier with a general
(sparse) proposal q: the path law against brute-force enumeration of the
chain distribution, the proposals against exact conditionals, closed-form
limits, the one-hot reduction to the deterministic sampler, and chi-square
tests that the whole draft-then-verify pipeline emits the target's law."""

import itertools

import numpy as np
from scipy import stats

from oracle.philox import philox4x64_10
from oracle.selector import select_path, select_path_sampled
from oracle.verify import verify_sample, verify_sample_q


def case(seed, P, K, V=40, r=6, scale=0.6, unary=1.0):
    rng = np.random.default_rng(seed)
    val = (unary * rng.standard_normal((P, K))).astype(np.float32)
    idx = np.stack([rng.choice(V, K, replace=False) for _ in range(P)]).astype(np.int32)
    F_l = (scale * rng.standard_normal((V, r))).astype(np.float32)
    F_r = (scale * rng.standard_normal((V, r))).astype(np.float32)
    return val, idx, F_l, F_r


def chain_scores(val, idx, F_l, F_r):
    """Score of every path (K^P of them), pair scores by a library matmul."""
    P, K = val.shape
    pairs = [F_l[idx[p]].astype(np.float64) @ F_r[idx[p + 1]].astype(np.float64).T for p in range(P - 1)]
    grids = np.meshgrid(*[np.arange(K)] * P, indexing="ij")
    s = np.zeros([K] * P)
    for p in range(P):
        s = s + val[p].astype(np.float64)[grids[p]]
    for p in range(P - 1):
        s = s + pairs[p][grids[p], grids[p + 1]]
    return s


def law(scores):
    e = np.exp(scores - scores.max())
    return e / e.sum()


def test_path_law_matches_enumeration():
    P, K, N = 3, 4, 12000
    val, idx, F_l, F_r = case(1, P, K)
    pi = law(chain_scores(val, idx, F_l, F_r)).ravel()
    rank, tok, q = select_path_sampled(np.broadcast_to(val, (N, P, K)), np.broadcast_to(idx, (N, P, K)),
                                       F_l, F_r, 7, np.arange(N), np.full(N, 100))
    flat = np.ravel_multi_index(tuple(rank.T.astype(np.int64)), (K,) * P)
    obs = np.bincount(flat, minlength=K ** P)
    assert stats.chisquare(obs, N * pi).pvalue > 1e-3
    assert np.array_equal(tok, idx[np.arange(P)[None, :], rank])


def test_proposals_are_the_exact_conditionals():
    """q[p] = pi(i_p | drawn prefix), by summing the enumerated law over the
    suffixes; with an anchor, position 0 gains pair(anchor, .)."""
    P, K = 4, 4
    val, idx, F_l, F_r = case(2, P, K)
    for anchor in (None, 5):
        scores = chain_scores(val, idx, F_l, F_r)
        if anchor is not None:
            a0 = F_l[anchor].astype(np.float64) @ F_r[idx[0]].astype(np.float64).T
            scores = scores + a0.reshape((K,) + (1,) * (P - 1))
        pi = law(scores)
        N = 6
        rank, tok, q = select_path_sampled(np.broadcast_to(val, (N, P, K)), np.broadcast_to(idx, (N, P, K)),
                                           F_l, F_r, 3, np.arange(N) * 7 + 1, np.full(N, 9),
                                           anchor=None if anchor is None else np.full(N, anchor))
        for b in range(N):
            for p in range(P):
                marg = pi[tuple(rank[b, :p])].reshape(K, -1).sum(axis=1)
                assert np.allclose(q[b, p], marg / marg.sum(), rtol=1e-12, atol=1e-15)


def test_zero_pair_tables_give_independent_softmax():
    P, K = 5, 16
    val, idx, F_l, F_r = case(3, P, K, scale=0.0)
    rank, tok, q = select_path_sampled(val[None], idx[None], F_l, F_r, 1, [4], [0])
    v = val.astype(np.float64)
    ref = np.exp(v - v.max(axis=1, keepdims=True))
    assert np.allclose(q[0], ref / ref.sum(axis=1, keepdims=True), rtol=1e-14, atol=0)


def test_sharp_limit_is_the_max_sum_path():
    """Scores scaled by 1000: the law concentrates on the max-sum path."""
    P, K = 6, 16
    val, idx, F_l, F_r = case(4, P, K, scale=1.0)
    big_val = (val * 1000.0).astype(np.float32)
    s = np.float32(np.sqrt(1000.0))
    rank_g, tok_g, _, _ = select_path(big_val[None], idx[None], F_l * s, F_r * s)
    rank, tok, q = select_path_sampled(big_val[None], idx[None], F_l * s, F_r * s, 5, [11], [3])
    assert np.array_equal(rank, rank_g) and np.array_equal(tok, tok_g)
    assert np.all(q[0, np.arange(P), rank[0]] > 1 - 1e-9)


def test_draw_uses_word_2_of_the_slot_block():
    """Two equally likely candidates at one position: the draw is candidate 1
    exactly when word 2 of block (1, request, pos0 + 1, 0) gives u >= 1/2."""
    val = np.zeros((1, 1, 2), np.float32)
    idx = np.array([[[3, 8]]], np.int32)
    F = np.zeros((10, 4), np.float32)
    for rid in range(40):
        rank, tok, q = select_path_sampled(val, idx, F, F, 99, [rid], [50])
        w2 = philox4x64_10((1, rid, 51, 0), (99, 0))[2]
        assert rank[0, 0] == (1 if (w2 >> 11) * 2.0 ** -53 >= 0.5 else 0)
        assert np.all(q == 0.5)


# ------------------------------------------------------ verify with proposal q
def p_of(row):
    e = np.exp(row - row.max())
    return e / e.sum()


def chi2_pvalue(tokens, p, n):
    obs = np.bincount(tokens, minlength=p.size).astype(np.float64)
    exp = n * p
    keep = exp >= 5
    o = np.append(obs[keep], obs[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        o, e = o[:-1], e[:-1]
    return stats.chisquare(o, e).pvalue


def test_one_hot_proposal_is_the_deterministic_sampler():
    rng = np.random.default_rng(5)
    B, T, V, K = 24, 6, 50, 16
    L = rng.standard_normal((B, T, V)) * 2.0
    d = rng.integers(0, V, (B, T - 1))
    L[np.arange(B)[:, None], np.arange(T - 1)[None], d] += 3.0  # some acceptances
    qi = rng.integers(0, V, (B, T - 1, K))
    qi[..., 0] = d
    qp = np.zeros((B, T - 1, K))
    qp[..., 0] = 1.0
    ref = verify_sample(L, d, 1.0, 21, np.arange(B) * 3, np.full(B, 77))
    got = verify_sample_q(L, d, qi, qp, 1.0, 21, np.arange(B) * 3, np.full(B, 77))
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def lattice(seed, P, K, V):
    rng = np.random.default_rng(seed)
    val = rng.standard_normal((P, K)).astype(np.float32)
    idx = np.stack([rng.choice(V, K, replace=False) for _ in range(P)]).astype(np.int32)
    F_l = (0.7 * rng.standard_normal((V, 4))).astype(np.float32)
    F_r = (0.7 * rng.standard_normal((V, 4))).astype(np.float32)
    return val, idx, F_l, F_r


def test_drawn_draft_then_verify_emits_the_target_law():
    """Draft drawn from q (a one-position lattice), verified against p: the
    first emitted token follows p whatever q is."""
    V, K, N = 12, 4, 1 << 14
    val, idx, F_l, F_r = lattice(6, 1, K, V)
    rng = np.random.default_rng(7)
    row0 = rng.standard_normal(V) * 1.5
    row0[idx[0, 1]] += 1.0  # overlap between p and q of several sizes
    rid, pos0 = np.arange(N), np.full(N, 300)
    rank, tok, q = select_path_sampled(np.broadcast_to(val, (N, 1, K)), np.broadcast_to(idx, (N, 1, K)),
                                       F_l, F_r, 13, rid, pos0)
    L = np.tile(np.stack([row0, rng.standard_normal(V)])[None], (N, 1, 1))
    out, n = verify_sample_q(L, tok, np.broadcast_to(idx, (N, 1, K)), q, 1.0, 13, rid, pos0)
    assert chi2_pvalue(out[:, 0], p_of(row0), N) > 1e-3
    # acceptance rate = sum_v min(p(v), q(v))
    acc = sum(min(p_of(row0)[idx[0, j]], q[0, 0, j]) for j in range(K))
    assert abs((n == 2).mean() - acc) < 4 * np.sqrt(acc * (1 - acc) / N)


def test_second_slot_follows_its_row_given_the_first_accepted():
    V, K, N = 10, 4, 1 << 14
    val, idx, F_l, F_r = lattice(8, 2, K, V)
    rng = np.random.default_rng(9)
    row0 = np.full(V, -3.0)
    row0[idx[0]] = val[0] + 2.0  # the first slot is accepted often
    row1 = rng.standard_normal(V) * 1.2
    rid, pos0 = np.arange(N) + 1000, np.zeros(N, np.int64)
    rank, tok, q = select_path_sampled(np.broadcast_to(val, (N, 2, K)), np.broadcast_to(idx, (N, 2, K)),
                                       F_l, F_r, 17, rid, pos0)
    L = np.tile(np.stack([row0, row1, rng.standard_normal(V)])[None], (N, 1, 1))
    out, n = verify_sample_q(L, tok, np.broadcast_to(idx, (N, 2, K)), q, 1.0, 17, rid, pos0)
    sel = n >= 2
    assert sel.mean() > 0.3
    assert chi2_pvalue(out[sel, 1], p_of(row1), int(sel.sum())) > 1e-3


def test_proposal_equal_to_target_always_accepts():
    """q = p on a support that holds all of p's mass: p / q = 1, every draft
    is accepted (acceptance is u * q(d) * Z < e(d), u < 1)."""
    V, K, B, T = 30, 4, 64, 4
    rng = np.random.default_rng(10)
    L = np.full((B, T, V), -1e4)
    qi = np.zeros((B, T - 1, K), np.int64)
    qp = np.zeros((B, T - 1, K))
    d = np.zeros((B, T - 1), np.int64)
    for b in range(B):
        for t in range(T - 1):
            ids = rng.choice(V, K, replace=False)
            lv = rng.standard_normal(K)
            L[b, t, ids] = lv
            qi[b, t], qp[b, t] = ids, p_of(lv)
            d[b, t] = ids[rng.integers(K)]
    out, n = verify_sample_q(L, d, qi, qp, 1.0, 3, np.arange(B), np.zeros(B, np.int64))
    assert np.all(n == T) and np.array_equal(out[:, :T - 1], d)
