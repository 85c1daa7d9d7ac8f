"""Pins for the oracle's verifiers: greedy against the target's own argmax
continuation; sampling against the target distribution (exact law on a grid
of uniforms, chi-square on Philox draws) and its closed-form special cases."""

import math
import numpy as np
import pytest
from scipy import stats

from oracle.verify import (decide_bonus, decide_slot, row_weights, uniforms,
                           verify_greedy, verify_sample)


# ---------------------------------------------------------------- greedy
def test_greedy_emits_target_argmax_continuation():
    rng = np.random.default_rng(0)
    B, T, V = 64, 8, 50
    L = rng.standard_normal((B, T, V))
    g = np.argmax(L, -1)
    d = g[:, :T - 1].copy()
    # corrupt drafts at a random slot (or none) per request
    cut = rng.integers(0, T, B)
    for b in range(B):
        if cut[b] < T - 1:
            d[b, cut[b]] = (g[b, cut[b]] + 1 + rng.integers(0, V - 1)) % V
    out, n = verify_greedy(L, d)
    for b in range(B):
        assert n[b] == min(cut[b], T - 1) + 1
        assert list(out[b, :n[b]]) == list(g[b, :n[b]])   # every token = target argmax
        assert np.all(out[b, n[b]:] == -1)
        if n[b] - 1 < T - 1:
            assert d[b, n[b] - 1] != g[b, n[b] - 1]        # stopped at a mismatch


def test_greedy_all_match_and_first_mismatch():
    L = np.zeros((2, 4, 6)); L[:, :, 3] = 1.0
    out, n = verify_greedy(L, np.array([[3, 3, 3], [2, 3, 3]]))
    assert list(n) == [4, 1]
    assert list(out[0]) == [3, 3, 3, 3] and list(out[1]) == [3, -1, -1, -1]


def test_greedy_ties_lowest_id():
    L = np.zeros((1, 2, 5)); L[0, 0, [1, 3]] = 2.0
    out, n = verify_greedy(L, np.array([[3]]))
    assert n[0] == 1 and out[0, 0] == 1


# ---------------------------------------------------------------- sampling
def p_of(row, tau=1.0):
    e = np.exp((row - row.max()) / tau)
    return e / e.sum()


def test_slot_law_on_uniform_grid():
    """The emitted token's law is p exactly: integrate decide_slot over a
    midpoint grid of (u_acc, u_res); error bounded by the grid step."""
    rng = np.random.default_rng(1)
    row = rng.standard_normal(8) * 1.5
    e = row_weights(row, 1.0)
    p = p_of(row)
    N = 4000
    grid = (np.arange(N) + 0.5) / N
    for d in range(8):
        acc = np.mean([decide_slot(e, d, u, 0.5)[0] for u in grid])
        assert abs(acc - p[d]) <= 1.0 / N
        res = np.bincount([decide_slot(e, d, 1.0 - 1e-12, u)[1] for u in grid], minlength=8) / N
        assert res[d] == 0.0
        law = (1 - acc) * res
        law[d] += acc
        assert np.max(np.abs(law - p)) <= 3.0 / N
    bonus = np.bincount([decide_bonus(e, u) for u in grid], minlength=8) / N
    assert np.max(np.abs(bonus - p)) <= 2.0 / N


def chi2_pvalue(tokens, p, n):
    obs = np.bincount(tokens, minlength=p.size).astype(np.float64)
    exp = n * p
    keep = exp >= 5
    o = np.append(obs[keep], obs[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        o, e = o[:-1], e[:-1]
    return stats.chisquare(o, e).pvalue


def test_chi_square_first_token_follows_target():
    rng = np.random.default_rng(2)
    V, N = 32, 1 << 14
    row0 = rng.standard_normal(V) * 2.0
    L = np.tile(np.stack([row0, rng.standard_normal(V)])[None], (N, 1, 1))
    d = np.full((N, 1), int(np.argsort(row0)[-3]))  # a plausible, not top, draft
    out, n = verify_sample(L, d, 1.0, 11, np.arange(N), np.full(N, 500))
    first = out[:, 0]
    assert chi2_pvalue(first, p_of(row0), N) > 1e-3


def test_chi_square_second_slot_conditional():
    rng = np.random.default_rng(3)
    V, N = 24, 1 << 13
    row0 = rng.standard_normal(V); row0[5] += 4.0   # d0 = 5 accepted often
    row1 = rng.standard_normal(V) * 1.5
    L = np.tile(np.stack([row0, row1, rng.standard_normal(V)])[None], (N, 1, 1))
    d = np.tile(np.array([[5, int(np.argmin(row1))]]), (N, 1))
    out, n = verify_sample(L, d, 1.0, 12, np.arange(N), np.zeros(N, np.int64))
    sel = n >= 2
    assert abs(sel.mean() - p_of(row0)[5]) < 4 * np.sqrt(p_of(row0)[5] * (1 - p_of(row0)[5]) / N)
    assert chi2_pvalue(out[sel, 1], p_of(row1), int(sel.sum())) > 1e-3


def test_temperature_scales_distribution():
    rng = np.random.default_rng(4)
    V, N, tau = 16, 1 << 13, 0.5
    row0 = rng.standard_normal(V)
    L = np.tile(np.stack([row0, row0])[None], (N, 1, 1))
    out, _ = verify_sample(L, np.full((N, 1), 0), tau, 13, np.arange(N), np.zeros(N, np.int64))
    assert chi2_pvalue(out[:, 0], p_of(row0, tau), N) > 1e-3


def test_large_margin_always_accepts_and_negative_never():
    V, N = 40, 2000
    L = np.zeros((N, 3, V)); L[:, 0, 7] = 50.0; L[:, 1, 9] = -50.0
    d = np.tile(np.array([[7, 9]]), (N, 1))
    out, n = verify_sample(L, d, 1.0, 3, np.arange(N), np.zeros(N, np.int64))
    assert np.all(out[:, 0] == 7)          # p(7) rounds to 1: always accepted
    assert np.all(n == 2)                  # slot 2 rejected (prob 2^-53 otherwise)
    assert np.all(out[:, 1] != 9)          # residual never emits the rejected draft


def test_equal_logits_are_uniform():
    V, N = 20, 1 << 13
    L = np.zeros((N, 2, V))
    out, _ = verify_sample(L, np.full((N, 1), 0), 1.0, 21, np.arange(N), np.zeros(N, np.int64))
    assert chi2_pvalue(out[:, 0], np.full(V, 1.0 / V), N) > 1e-3


def test_batch_composition_invariance():
    rng = np.random.default_rng(5)
    B, T, V = 12, 5, 30
    L = rng.standard_normal((B, T, V)) * 3
    d = rng.integers(0, V, (B, T - 1))
    rid = rng.integers(0, 2**62, B)
    pos = rng.integers(0, 2**40, B)
    out, n = verify_sample(L, d, 1.0, 9, rid, pos)
    perm = rng.permutation(B)
    out2, n2 = verify_sample(L[perm], d[perm], 1.0, 9, rid[perm], pos[perm])
    assert np.array_equal(out2, out[perm]) and np.array_equal(n2, n[perm])
    sub = perm[:3]
    out3, n3 = verify_sample(L[sub], d[sub], 1.0, 9, rid[sub], pos[sub])
    assert np.array_equal(out3, out[sub])


def test_philox_visible_through_residual_draw():
    """All-equal logits over V = 2^k + 1 and d = V - 1: the residual has 2^k
    equal weights, so the replacement token is exactly floor(u_res * 2^k) =
    w1 >> (64 - k) whenever slot 1 rejects."""
    k = 10
    V = (1 << k) + 1
    N = 300
    L = np.zeros((N, 2, V))
    out, n = verify_sample(L, np.full((N, 1), V - 1), 1.0, 5, np.arange(N), np.full(N, 7))
    for b in range(N):
        u_acc, u_res = uniforms(5, b, 8)
        if u_acc * V >= 1.0:                      # rejected
            assert out[b, 0] == int(u_res * (1 << k))


def test_chi_square_bonus_token_after_full_accept():
    rng = np.random.default_rng(6)
    V, N = 28, 1 << 13
    row0 = np.zeros(V); row0[4] = 60.0              # slot 1 always accepted
    row1 = rng.standard_normal(V) * 1.5
    L = np.tile(np.stack([row0, row1])[None], (N, 1, 1))
    out, n = verify_sample(L, np.full((N, 1), 4), 1.0, 17, np.arange(N), np.zeros(N, np.int64))
    assert np.all(n == 2) and np.all(out[:, 0] == 4)
    assert chi2_pvalue(out[:, 1], p_of(row1), N) > 1e-3


# ------------------------------------------------- top-k / top-p sampling
from oracle.verify import filtered_set, verify_sample_topkp  # noqa: E402


def _greedyish(seed, B=24, T=8, V=40):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((B, T, V)) * 2.0
    g = np.argmax(L, -1)
    d = g[:, :T - 1].copy()
    cut = rng.integers(0, T, B)
    for b in range(B):
        if cut[b] < T - 1:
            d[b, cut[b]] = (g[b, cut[b]] + 1) % V
    return L, d, rng


@pytest.mark.parametrize("top_k,top_p", [(1, 0.95), (1, 1.0), (40, 1e-9), (7, 1e-30)])
def test_topkp_single_token_is_greedy(top_k, top_p):
    """Keeping one token makes p' one-hot at the argmax: every draft equal to
    the argmax is accepted, any other rejected and replaced by the argmax,
    and the bonus is the argmax, for any uniforms: exactly verify_greedy."""
    L, d, rng = _greedyish(11)
    for seed in (0, 5, 77):
        rid = rng.integers(0, 2**40, L.shape[0])
        p0 = rng.integers(0, 2**30, L.shape[0])
        o, n = verify_sample_topkp(L, d, 1.0, top_k, top_p, seed, rid, p0)
        o0, n0 = verify_greedy(L, d)
        assert np.array_equal(o, o0) and np.array_equal(n, n0)
        # the margins see empty residuals (an accepted one-token set): the
        # decisions are the same, and only the acceptance tests bound them
        o1, n1, mg = verify_sample_topkp(L, d, 1.0, top_k, top_p, seed, rid, p0, return_margins=True)
        assert np.array_equal(o1, o) and np.array_equal(n1, n) and np.all(mg >= 0)


def test_topkp_worked_nucleus():
    """p = (0.5, 0.3, 0.15, 0.05) on shuffled ids: top-p 0.9 keeps the three
    largest (0.5 + 0.3 < 0.9 <= 0.95); 0.45 keeps one, 0.55 two; top-k 2
    caps at two; weights stay proportional to p."""
    ids = np.array([7, 2, 9, 4])
    row = np.full(12, -np.inf)
    row[ids] = np.log([0.5, 0.3, 0.15, 0.05])
    row[np.isinf(row)] = -50.0
    for top_k, top_p, kept in [(20, 0.9, [7, 2, 9]), (20, 0.45, [7]), (20, 0.55, [7, 2]),
                               (2, 0.99, [7, 2]), (3, 1.0, [7, 2, 9])]:
        got, w, Z = filtered_set(row, 1.0, top_k, top_p)
        assert list(got) == sorted(kept)
        p = {7: 0.5, 2: 0.3, 9: 0.15}
        ref = np.array([p[i] for i in got])
        assert np.allclose(w / Z, ref / ref.sum(), rtol=1e-12)


def test_topkp_ties_at_the_k_boundary_keep_lower_ids():
    row = np.array([1.0, 3.0, 3.0, 3.0, 0.0, 3.0])
    got, w, Z = filtered_set(row, 1.0, 2, 1.0)
    assert list(got) == [1, 2] and np.allclose(w, 1.0) and Z == 2.0


def test_topkp_kept_set_is_the_shortest_ranked_prefix():
    """Invariant on random rows: the kept tokens are the best-ranked ones, the
    mass before the last kept token is below top_p * Zk and the kept mass
    reaches it (unless top-k ran out), and the weights are exp((l - max)/tau)."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(1, 300))
        row = rng.standard_normal(V) * rng.uniform(0.1, 5.0)
        tau = rng.uniform(0.3, 2.0)
        k, tp = int(rng.integers(1, 70)), float(rng.uniform(0.05, 1.0))
        ids, w, Z = filtered_set(row, 1.0 / tau, k, tp)
        rank = np.lexsort((np.arange(V), -row))
        assert set(ids) == set(rank[:ids.size])
        e_all = np.exp((row[rank[:min(k, V)]] - row.max()) / tau)
        zk, cum = e_all.sum(), np.cumsum(e_all)
        n = ids.size
        assert n == 1 or cum[n - 2] < tp * zk * (1 + 1e-12)
        assert n == min(k, V) or cum[n - 1] >= tp * zk * (1 - 1e-12)
        assert np.allclose(w, np.exp((row[ids] - row.max()) / tau), rtol=1e-12)
        assert np.isclose(Z, w.sum(), rtol=1e-12)


def test_topkp_chi_square_first_token_follows_filtered_target():
    """Over many Philox counters, the first emitted token follows p'
    (top-20, top-p 0.8), for a draft inside the kept set and one outside."""
    rng = np.random.default_rng(21)
    V, N = 60, 40000
    row = rng.standard_normal(V) * 1.5
    ids, w, Z = filtered_set(row, 1.0, 20, 0.8)
    p = np.zeros(V)
    p[ids] = w / Z
    outside = int(np.setdiff1d(np.arange(V), ids)[0])
    for d0 in (int(ids[np.argsort(-w)[1]]), outside):
        L = np.broadcast_to(np.stack([row, rng.standard_normal(V)])[None], (N, 2, V))
        o, _ = verify_sample_topkp(L, np.full((N, 1), d0), 1.0, 20, 0.8, 4, np.arange(N), np.full(N, 9))
        obs = np.bincount(o[:, 0], minlength=V)
        assert obs[p == 0].sum() == 0
        keep = p > 0
        chi = stats.chisquare(obs[keep], N * p[keep])
        assert chi.pvalue > 1e-3, chi


def test_topkp_chi_square_bonus_follows_filtered_last_row():
    """A draft with overwhelming weight is always accepted (T = 2), so the
    bonus is drawn from the filtered last row."""
    rng = np.random.default_rng(22)
    V, N = 50, 30000
    r0 = rng.standard_normal(V)
    r0[13] = 60.0
    r1 = rng.standard_normal(V) * 2.0
    L = np.broadcast_to(np.stack([r0, r1])[None], (N, 2, V))
    o, n = verify_sample_topkp(L, np.full((N, 1), 13), 1.0, 10, 0.9, 8, np.arange(N), np.zeros(N))
    assert np.all(n == 2) and np.all(o[:, 0] == 13)
    ids, w, Z = filtered_set(r1, 1.0, 10, 0.9)
    obs = np.bincount(o[:, 1], minlength=V)
    assert obs[np.setdiff1d(np.arange(V), ids)].sum() == 0
    chi = stats.chisquare(obs[ids], N * w / Z)
    assert chi.pvalue > 1e-3, chi


def test_topkp_unfiltered_limit_keeps_every_weighted_token():
    rng = np.random.default_rng(23)
    row = rng.standard_normal(500) * 3.0
    ids, w, Z = filtered_set(row, 1.0, 10**9, 1.0)
    assert np.array_equal(ids, np.arange(500))
    assert np.allclose(w, row_weights(row, 1.0), rtol=1e-15)


# ------------------------------------------ greedy from target hidden states
def test_greedy_from_hidden_states_planted_argmax():
    """Target rows planted as s * W[c_t]: the row's logit of c_t is s |W[c_t]|^2,
    far above every other, so g[t] = c_t by construction; drafts matching the
    first k of them are accepted, then g[k] is emitted."""
    from oracle.verify import verify_greedy_hidden
    rng = np.random.default_rng(21)
    V, D, T = 500, 256, 6
    W = np.round(rng.standard_normal((V, D)) * 8) / 8            # exactly representable in bf16
    c = rng.choice(V, T, replace=False)
    h = 4.0 * W[c]                                              # one block, rows t = 0..T-1
    for k in range(T):
        d = c[:T - 1].copy()
        if k < T - 1:
            d[k] = (c[k] + 1) % V                               # first mismatch at slot k + 1
        out, n = verify_greedy_hidden(h, W, d[None])
        assert n[0] == k + 1
        assert list(out[0, :k + 1]) == list(c[:k + 1])
        assert np.all(out[0, k + 1:] == -1)


def test_greedy_from_hidden_ties_take_the_lowest_id():
    """Integer-grid rows where several vocabulary rows reach the maximum."""
    from oracle.verify import verify_greedy_hidden
    W = np.zeros((40, 8))
    W[[7, 19, 33], 0] = 1.0                                      # three equal maxima for h = e_0
    W[5, 1] = 1.0
    h = np.zeros((2, 8))
    h[:, 0] = 1.0
    out, n = verify_greedy_hidden(h, W, np.array([[7]]))
    assert n[0] == 2 and list(out[0]) == [7, 7]
    out, n = verify_greedy_hidden(h, W, np.array([[19]]))
    assert n[0] == 1 and out[0, 0] == 7


def test_sample_from_hidden_states_equals_sampling_integer_logits():
    """Integer-grid hidden states and head rows: the logits are integers,
    computed here by an int64 matrix product, and the hidden-state sampler
    must decide exactly as the sampler given those logits."""
    from oracle.verify import verify_sample_hidden
    rng = np.random.default_rng(23)
    B, T, V, D = 6, 5, 300, 32
    W = rng.integers(-2, 3, (V, D))
    h = rng.integers(-2, 3, (B * T, D))
    z = (h.astype(np.int64) @ W.astype(np.int64).T).reshape(B, T, V)
    d = np.argsort(-z[:, :T - 1], axis=-1, kind="stable")[..., 1]   # second-best tokens as drafts
    rid, pos0 = np.arange(B) * 5 + 2, np.full(B, 40)
    ref = verify_sample(z.astype(np.float64) * 0.25, d, 1.0, 8, rid, pos0)
    got = verify_sample_hidden(h * 0.5, W * 0.5, d, 1.0, 8, rid, pos0)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


# --- the admissibility helpers (distance of a decision from its boundary) ---

def test_edge_margin_hand_computed():
    """c = 1, 3, 6, 10: targets inside bins, on an edge, in the first and the
    last bin; zero-weight bins; targets at or past the total."""
    from oracle.verify import _edge_margin
    w = np.array([1.0, 2.0, 3.0, 4.0])
    assert _edge_margin(w, 4.5) == pytest.approx(0.15)     # bin 2: 1.5 to both edges
    assert _edge_margin(w, 3.0) == 0.0                      # exactly on the edge 3
    assert _edge_margin(w, 0.2) == pytest.approx(0.08)      # bin 0: 0 is no edge, 0.8 to 1
    assert _edge_margin(w, 9.9) == pytest.approx(0.39)      # last bin: 10 is no edge, 3.9 to 6
    assert _edge_margin(w, 10.0) == pytest.approx(0.4)      # past the total: falls back to bin 3
    z = np.array([0.0, 2.0, 0.0, 0.0, 3.0])                 # c = 0, 2, 2, 2, 5
    assert _edge_margin(z, 2.5) == pytest.approx(0.1)       # the only edge is 2
    assert _edge_margin(z, 1.0) == pytest.approx(0.2)
    assert _edge_margin(np.array([0.0, 0.0, 7.0]), 3.0) == math.inf   # one token can be drawn
    assert _edge_margin(np.array([5.0, 0.0, 0.0]), 0.1) == math.inf
    # no mass (the residual of a filtered set that is only the drafted
    # token): nothing is drawn, so no boundary either
    assert _edge_margin(np.zeros(3), 0.0) == math.inf
    assert _edge_margin(np.zeros(0), 0.0) == math.inf


def test_edge_margin_is_the_distance_to_a_change_of_token():
    """Moving the target by less than the margin (times the mass) keeps the
    drawn token; moving it by slightly more, one way or the other, changes it."""
    from oracle.verify import _edge_margin, inverse_cdf
    rng = np.random.default_rng(21)
    for trial in range(300):
        n = int(rng.integers(1, 12))
        w = rng.random(n) * (rng.random(n) > 0.3)
        if w.sum() == 0:
            w[int(rng.integers(n))] = 1.0
        tot = float(np.cumsum(w)[-1])
        t = float(rng.random()) * tot
        m = _edge_margin(w, t)
        tok = inverse_cdf(w, t)
        if m == math.inf:
            assert np.count_nonzero(w) == 1
            continue
        step = m * tot
        for f in (-0.99, 0.99):
            if t + f * step >= 0:
                assert inverse_cdf(w, t + f * step) == tok
        moved = [inverse_cdf(w, t + f * step) for f in (-1.01, 1.01) if t + f * step >= 0]
        assert any(v != tok for v in moved), (w, t, m)


def test_cut_margin_hand_computed():
    """e = 1, 1/2, 1/4, 1/8 (Zk = 1.875), nucleus bound top_p * Zk against the
    masses before tokens 1, 2, 3 (1, 1.5, 1.75)."""
    from oracle.verify import _cut_margin
    row = np.log(np.array([1.0, 0.5, 0.25, 0.125]))
    assert _cut_margin(row, 1.0, 4, 0.8) == 0.0                          # bound 1.5 = mass before token 2
    assert _cut_margin(row, 1.0, 4, 0.7) == pytest.approx(0.1875 / 1.875)  # bound 1.3125
    assert _cut_margin(row, 1.0, 2, 0.7) == pytest.approx(0.05 / 1.5)     # top-2: Zk 1.5, bound 1.05
    assert _cut_margin(row, 1.0, 1, 0.5) == math.inf                       # one token: nothing to cut
    # order and temperature: the same weights from a permuted row at tau = 2
    perm = np.array([2, 0, 3, 1])
    assert _cut_margin(2.0 * row[perm], 0.5, 4, 0.7) == pytest.approx(0.1)


def test_cut_margin_is_the_distance_to_a_change_of_set():
    """Moving top_p by less than the margin keeps the filtered set; by slightly
    more in one direction or the other it changes."""
    from oracle.verify import _cut_margin, filtered_set
    rng = np.random.default_rng(22)
    for trial in range(200):
        V = int(rng.integers(2, 40))
        row = rng.standard_normal(V) * 2.0
        k = int(rng.integers(2, V + 1))
        p = float(rng.uniform(0.2, 0.95))
        m = _cut_margin(row, 1.0, k, p)
        ids = filtered_set(row, 1.0, k, p)[0]
        for f in (-0.99, 0.99):
            assert np.array_equal(filtered_set(row, 1.0, k, p + f * m)[0], ids)
        moved = [filtered_set(row, 1.0, k, p + f * m)[0] for f in (-1.01, 1.01) if 0 < p + f * m <= 1]
        assert any(not np.array_equal(x, ids) for x in moved), (row, k, p, m)
