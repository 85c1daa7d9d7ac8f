"""GPU parity of dflash_verify_sample_topkp against the oracle: exact tokens
and lengths per Philox counter (over shapes spanning several chunks with a
ragged tail, tie-heavy rows that overflow the candidate buffers, V below
top_k), its single-token limit equal to greedy verification, and the
filtered target distribution by chi-square."""

import numpy as np
import pytest
import torch
from scipy import stats

from oracle.verify import filtered_set, verify_greedy as og, verify_sample_topkp as otk

pytestmark = pytest.mark.gpu


def run(dfl, dev, L, d, tau, k, p, seed, rid, pos):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    o, n = dfl.verify_sample_topkp(t(L), t(d), tau, k, p, seed, t(rid.astype(np.int64)), t(pos.astype(np.int64)))
    torch.cuda.synchronize()
    return o.cpu().numpy(), n.cpu().numpy()


def case(seed, B, T, V, scale, quantize=False):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((B, T, V)) * scale
    if quantize:
        L = np.round(L)                      # many exact ties
    L = L.astype(np.float32)
    g = np.argmax(L, -1)
    d = g[:, :T - 1].astype(np.int32)
    d[::3, T // 2 - 1] = rng.integers(0, V, len(d[::3]))
    d[1::4, 0] = V + 5                       # an id outside the vocabulary: p = 0
    rid = rng.integers(0, 2**62, B)
    pos = rng.integers(0, 2**40, B)
    return L, d, rid, pos


@pytest.mark.parametrize("B,T,V,scale,tau,k,p,quant", [
    (16, 8, 4096, 3.0, 1.0, 20, 0.95, False),
    (8, 8, 151936, 4.0, 1.0, 20, 0.95, False),
    (32, 8, 4097, 2.0, 0.7, 64, 0.5, False),
    (12, 16, 20000, 1.0, 1.3, 7, 0.9, False),
    (20, 2, 3, 1.0, 1.0, 64, 1.0, False),
    (6, 4, 1, 1.0, 1.0, 20, 0.95, False),
    (10, 8, 9000, 1.0, 1.0, 20, 0.95, True),
    (10, 8, 70000, 0.3, 1.0, 64, 1.0, True),
])
def test_topkp_matches_oracle_per_counter(dfl, dev, B, T, V, scale, tau, k, p, quant):
    L, d, rid, pos = case(B * 7 + V, B, T, V, scale, quant)
    o, n = run(dfl, dev, L, d, tau, k, p, 99, rid, pos)
    o0, n0, margin = otk(L, d, tau, k, p, 99, rid, pos, return_margins=True)
    ok = (o == o0).all(1) & (n == n0)
    # a mismatch is only admissible for a decision within 1e-12 of its boundary
    assert np.all(ok | (margin < 1e-12)), (np.nonzero(~ok), margin[~ok])
    assert (~ok).sum() <= 1


def test_topkp_constant_rows(dfl, dev):
    """Every logit equal: the kept set is the lowest ids, ranked by id."""
    B, T, V = 4, 8, 20000
    L = np.zeros((B, T, V), np.float32)
    d = np.array([[3, 1, 0, 2, 5, 4, 9]] * B, np.int32)
    rid, pos = np.arange(B), np.full(B, 100)
    o, n = run(dfl, dev, L, d, 1.0, 10, 0.95, 3, rid, pos)
    o0, n0 = otk(L, d, 1.0, 10, 0.95, 3, rid, pos)
    assert np.array_equal(o, o0) and np.array_equal(n, n0)


@pytest.mark.parametrize("k,p", [(1, 0.95), (64, 1e-9)])
def test_topkp_single_token_is_greedy(dfl, dev, k, p):
    L, d, rid, pos = case(5, 24, 8, 30000, 3.0)
    o, n = run(dfl, dev, L, d, 1.0, k, p, 7, rid, pos)
    o0, n0 = og(L, d)
    assert np.array_equal(o, o0) and np.array_equal(n, n0)


def test_topkp_distribution_chi_square(dfl, dev):
    rng = np.random.default_rng(31)
    V, N = 5000, 1 << 17
    row0 = (rng.standard_normal(V) * 2.0).astype(np.float32)
    ids, w, Z = filtered_set(row0, 1.0, 20, 0.8)
    L = np.broadcast_to(np.stack([row0, rng.standard_normal(V).astype(np.float32)])[None], (N, 2, V))
    d = np.full((N, 1), int(ids[np.argsort(-w)[1]]), np.int32)
    o, _ = run(dfl, dev, L, d, 1.0, 20, 0.8, 5, np.arange(N), np.full(N, 11))
    obs = np.bincount(o[:, 0], minlength=V)
    assert obs.sum() == N and obs[np.setdiff1d(np.arange(V), ids)].sum() == 0
    chi = stats.chisquare(obs[ids], N * w / Z)
    assert chi.pvalue > 1e-4, chi


@pytest.mark.parametrize("V,period,k,p", [(262144, 512, 64, 1.0), (262144, 512, 20, 0.95), (9000, 1024, 64, 0.9)])
def test_topkp_periodic_rows_overflow_the_candidate_buffers(dfl, dev, V, period, k, p):
    """Rows repeating every `period` ids put hundreds of tied entries at or
    above each bound, so both kernels take their one-at-a-time paths."""
    rng = np.random.default_rng(period + k)
    B, T = 3, 8
    base = rng.standard_normal((B, T, period)).astype(np.float32)
    L = np.ascontiguousarray(np.tile(base, (1, 1, V // period + 1))[:, :, :V])
    d = np.argmax(L, -1)[:, :T - 1].astype(np.int32)
    d[:, 2] = (d[:, 2] + period) % V         # the same value under a larger id
    rid, pos = np.arange(B) * 17, np.full(B, 3)
    o, n = run(dfl, dev, L, d, 1.0, k, p, 21, rid, pos)
    o0, n0 = otk(L, d, 1.0, k, p, 21, rid, pos)
    assert np.array_equal(o, o0) and np.array_equal(n, n0)
