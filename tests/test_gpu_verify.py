"""GPU parity of dflash_verify_greedy / dflash_verify_sample against the oracle:
exact tokens and lengths per Philox counter, the target distribution by
chi-square, Philox bits visible through the public call, batch invariance."""

import numpy as np
import pytest
import torch
from scipy import stats

from oracle.verify import uniforms, verify_greedy as og, verify_sample as osamp

pytestmark = pytest.mark.gpu


def greedy_case(seed, B, T, V, scale=1.0):
    rng = np.random.default_rng(seed)
    L = (rng.standard_normal((B, T, V)) * scale).astype(np.float32)
    g = np.argmax(L, -1)
    d = g[:, :T - 1].copy()
    cut = rng.integers(0, T, B)
    for b in range(B):
        if cut[b] < T - 1:
            d[b, cut[b]] = (g[b, cut[b]] + 1) % V
    return L, d.astype(np.int32)


@pytest.mark.parametrize("B,T,V", [(1, 8, 4096), (8, 8, 151936), (32, 8, 4097), (3, 2, 100),
                                   (5, 16, 20000), (2, 8, 1), (4, 8, 5)])
def test_greedy_matches_oracle(dfl, dev, B, T, V):
    L, d = greedy_case(B + T + V, B, T, V)
    o, n = dfl.verify_greedy(torch.from_numpy(L).to(dev), torch.from_numpy(d).to(dev))
    o0, n0 = og(L, d)
    assert np.array_equal(o.cpu().numpy(), o0) and np.array_equal(n.cpu().numpy(), n0)


def test_greedy_ties_lowest_id(dfl, dev):
    L = np.zeros((2, 3, 9000), np.float32)
    L[:, :, [17, 4500, 8999]] = 3.0
    d = np.array([[17, 17], [4500, 17]], np.int32)
    o, n = dfl.verify_greedy(torch.from_numpy(L).to(dev), torch.from_numpy(d).to(dev))
    o0, n0 = og(L, d)
    assert np.array_equal(o.cpu().numpy(), o0) and list(n0) == [3, 1]


def sample(dfl, dev, L, d, tau, seed, rid, pos):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    o, n = dfl.verify_sample(t(L), t(d), tau, seed, t(rid.astype(np.int64)), t(pos.astype(np.int64)))
    torch.cuda.synchronize()
    return o.cpu().numpy(), n.cpu().numpy()


@pytest.mark.parametrize("B,T,V,scale,tau", [(64, 8, 1000, 3.0, 1.0), (32, 8, 4097, 4.0, 1.0),
                                             (16, 8, 151936, 8.0, 1.0), (40, 5, 300, 2.0, 0.7),
                                             (8, 16, 5000, 6.0, 1.3), (20, 2, 3, 1.0, 1.0),
                                             # tau 0.02: weights down to exp(-1e3), subnormal and zero
                                             (16, 8, 5000, 4.0, 0.02)])
def test_sample_matches_oracle_per_counter(dfl, dev, B, T, V, scale, tau):
    rng = np.random.default_rng(B * 3 + V)
    L = (rng.standard_normal((B, T, V)) * scale).astype(np.float32)
    g = np.argmax(L, -1)
    d = g[:, :T - 1].astype(np.int32)                   # drafts = target argmax: long accepts
    d[::3, T // 2 - 1] = rng.integers(0, V, len(d[::3]))  # some plausible misses
    rid = rng.integers(0, 2**62, B)
    pos = rng.integers(0, 2**40, B)
    o, n = sample(dfl, dev, L, d, tau, 1234, rid, pos)
    o0, n0, margin = osamp(L, d, tau, 1234, rid, pos, return_margins=True)
    ok = (o == o0).all(1) & (n == n0)
    # a mismatch is only admissible for a decision within 1e-12 of its boundary
    assert np.all(ok | (margin < 1e-12)), (np.nonzero(~ok), margin[~ok])
    assert ok.mean() == 1.0 or (~ok).sum() <= 1


def test_sample_distribution_chi_square(dfl, dev):
    rng = np.random.default_rng(8)
    V, N = 32, 1 << 18
    row0 = rng.standard_normal(V) * 2.0
    L = np.broadcast_to(np.stack([row0, rng.standard_normal(V)]).astype(np.float32)[None], (N, 2, V))
    d = np.full((N, 1), int(np.argsort(row0)[-3]), np.int32)
    o, n = sample(dfl, dev, L, d, 1.0, 99, np.arange(N), np.full(N, 77))
    p = np.exp(row0 - row0.max()); p /= p.sum()
    obs = np.bincount(o[:, 0], minlength=V)
    exp = N * p
    keep = exp >= 5
    f_obs, f_exp = obs[keep], exp[keep]
    if (~keep).any():
        f_obs = np.append(f_obs, obs[~keep].sum())
        f_exp = np.append(f_exp, exp[~keep].sum())
    assert stats.chisquare(f_obs, f_exp * f_obs.sum() / f_exp.sum()).pvalue > 1e-3


def _f32(x):
    return float(np.float32(x))


def _band_rows(seed, rid, pos, V, delta):
    """Two crafted requests per sign of delta, each with T = 2 (one draft
    slot, then the bonus row):
    * 'accept': row 0 puts the draft d = 5 at p(d) = u_acc (1 + delta) (its
      logit and the logit of token 7 tuned in float32; the rest 0), so the
      acceptance test u_acc Z < e(d) sits inside the float32 band;
    * 'draw': row 0 accepts surely (draft logit 40) and row 1 (the bonus)
      puts the draw target u_res Z at (1 + delta) times a cumulative edge
      (the weight of token 0 tuned; the rest 1)."""
    from oracle.verify import uniforms
    rows, drafts = [], []
    for r, kind in zip(rid, ("accept", "draw")):
        L = np.zeros((2, V), np.float32)
        u_acc, _ = uniforms(seed, int(r), int(pos) + 1)
        _, u_res = uniforms(seed, int(r), int(pos) + 2)
        if kind == "accept":
            p = u_acc * (1.0 + delta)
            ld = _f32(np.log(p * (V - 1) / (1.0 - p)))
            ex = np.exp(np.float64(ld)) / p - np.exp(np.float64(ld)) - (V - 2)
            L[0, 5], L[0, 7] = ld, _f32(np.log(ex))
        else:
            L[0, 5] = 40.0
            k = u_res * (1.0 + delta)
            J = int(np.floor(k * (V - 1) - (1.0 - k)))
            w = (k * (V - 1) - J) / (1.0 - k)
            L[1, 0] = _f32(np.log(w))
        rows.append(L)
        drafts.append([5])
    return np.stack(rows), np.array(drafts, np.int32)


def test_sample_decisions_next_to_their_boundary(dfl, dev):
    """Acceptance tests and draws placed between 1e-12 and 1e-7 (relative)
    from their boundary (float32 logits tuned in float64): decided in float64
    on the GPU, they equal the oracle's.  Float32 masses could not decide
    them; float64 ones err by ~1e-16."""
    from oracle.verify import _edge_margin, row_weights, uniforms
    seed, V = 4242, 2 * 4096 + 77
    Ls, ds, rids, poss = [], [], [], []
    for j, delta in enumerate((3e-8, -3e-8, 1e-8, -1e-8)):
        rid = np.array([1000 + 2 * j, 1001 + 2 * j])
        pos = 50 + j
        L, d = _band_rows(seed, rid, pos, V, delta)
        # the crafted decisions really are that close (float64, as the oracle sees them)
        u_acc, _ = uniforms(seed, int(rid[0]), pos + 1)
        e = row_weights(L[0, 0], 1.0)
        rel = e[5] / e.sum() / u_acc - 1.0
        assert 1e-12 < abs(rel) < 2e-7 and np.sign(rel) == np.sign(delta), rel
        _, u_res = uniforms(seed, int(rid[1]), pos + 2)
        e = row_weights(L[1, 1], 1.0)
        mg = _edge_margin(e, u_res * e.sum())
        assert 1e-12 < mg < 2e-7, mg
        Ls.append(L); ds.append(d); rids.append(rid); poss.append(np.full(2, pos))
    L, d = np.concatenate(Ls), np.concatenate(ds)
    rid, pos = np.concatenate(rids), np.concatenate(poss)
    o, n = sample(dfl, dev, L, d, 1.0, seed, rid, pos)
    o0, n0 = osamp(L, d, 1.0, seed, rid, pos)
    assert np.array_equal(o, o0) and np.array_equal(n, n0)
    # both outcomes of the acceptance test occur
    assert set(n[0::2].tolist()) == {1, 2}, n


def test_philox_bits_through_public_call(dfl, dev):
    """Equal logits, V = 2^23 + 1, draft = V - 1: a rejection emits exactly
    floor(u_res * 2^23) = w1 >> 41 of Philox4x64-10 for that request."""
    V, B = (1 << 23) + 1, 64
    L = torch.zeros((B, 2, V), dtype=torch.float32, device=dev)
    d = torch.full((B, 1), V - 1, dtype=torch.int32, device=dev)
    rid = np.arange(B) * 1000003 + 17
    o, n = dfl.verify_sample(L, d, 1.0, 2024, torch.from_numpy(rid).to(dev),
                             torch.full((B,), 31, dtype=torch.int64, device=dev))
    o, n = o.cpu().numpy(), n.cpu().numpy()
    for b in range(B):
        u_acc, u_res = uniforms(2024, int(rid[b]), 32)
        if u_acc * V >= 1.0:
            assert n[b] == 1 and o[b, 0] == int(u_res * (1 << 23))
        else:
            assert o[b, 0] == V - 1


def test_batch_composition_invariance(dfl, dev):
    rng = np.random.default_rng(10)
    B, T, V = 24, 8, 3000
    L = (rng.standard_normal((B, T, V)) * 5).astype(np.float32)
    d = np.argmax(L, -1)[:, :T - 1].astype(np.int32)
    rid = rng.integers(0, 2**62, B)
    pos = rng.integers(0, 2**30, B)
    o, n = sample(dfl, dev, L, d, 1.0, 5, rid, pos)
    perm = rng.permutation(B)
    o2, n2 = sample(dfl, dev, L[perm], d[perm], 1.0, 5, rid[perm], pos[perm])
    assert np.array_equal(o2, o[perm]) and np.array_equal(n2, n[perm])
    o3, n3 = sample(dfl, dev, L[perm[:5]], d[perm[:5]], 1.0, 5, rid[perm[:5]], pos[perm[:5]])
    assert np.array_equal(o3, o[perm[:5]])
    og_, ng_ = dfl.verify_greedy(torch.from_numpy(L).to(dev), torch.from_numpy(d).to(dev))
    og2, _ = dfl.verify_greedy(torch.from_numpy(L[perm]).to(dev), torch.from_numpy(d[perm]).to(dev))
    assert np.array_equal(og2.cpu().numpy(), og_.cpu().numpy()[perm])


def test_sample_masked_logits(dfl, dev):
    """Masked vocabulary entries (-inf logits: weight 0) are never accepted or
    drawn, and the decisions equal the oracle's on the same logits.  NaN
    entries weigh 0 as well (the header's contract), so logits with NaN at
    those places give the same outputs as with -inf there."""
    rng = np.random.default_rng(77)
    B, T, V = 24, 8, 20000
    L = (rng.standard_normal((B, T, V)) * 4.0).astype(np.float32)
    mask = rng.random((B, T, V)) < 0.3
    mask[:, :, 0] = False                               # no row is masked whole
    g = np.argmax(np.where(mask, -np.inf, L), -1)
    d = g[:, :T - 1].astype(np.int32)                   # mostly acceptable drafts
    d[::2, 1] = np.argmax(mask[::2, 1], -1)             # half the requests draft a masked token at slot 2
    Linf = np.where(mask, np.float32(-np.inf), L).astype(np.float32)
    Lnan = np.where(mask, np.float32(np.nan), L).astype(np.float32)
    rid = np.arange(B) * 5 + 2
    pos = np.full(B, 40)
    o1, n1 = sample(dfl, dev, Linf, d, 1.0, 9, rid, pos)
    o0, n0, margin = osamp(Linf, d, 1.0, 9, rid, pos, return_margins=True)
    ok = (o1 == o0).all(1) & (n1 == n0)
    assert np.all(ok | (margin < 1e-12)) and (~ok).sum() <= 1, (np.nonzero(~ok), margin[~ok])
    for b in range(B):
        for t in range(n1[b]):
            assert not mask[b, t, o1[b, t]], (b, t)     # every emitted token has weight > 0
    assert np.all(n1[::2] <= 2)                          # a masked draft is rejected
    o2, n2 = sample(dfl, dev, Lnan, d, 1.0, 9, rid, pos)
    assert np.array_equal(o2, o1) and np.array_equal(n2, n1)
