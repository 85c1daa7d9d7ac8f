"""GPU tests of the head's exactness certificate (dflash_head_weight_bound,
dflash_head_topk_certify): the row bounds against float64 numpy, certified
rows equal to the oracle's exact top-16, rows with wide margins certified,
exact ties at the 16th place left uncertified."""

import numpy as np
import pytest
import torch

from oracle.head import head_topk as oracle_topk

pytestmark = pytest.mark.gpu


def bf16(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(dev)


def test_weight_bound_matches_float64(dfl, dev):
    rng = np.random.default_rng(5)
    for V, D in [(1000, 320), (37, 8), (5000, 5120)]:
        W = bf16(rng.standard_normal((V, D)) * rng.uniform(0.01, 2.0, (V, 1)), dev)
        b = dfl.head_weight_bound(W).cpu().numpy().astype(np.float64)
        w = W.float().cpu().numpy().astype(np.float64)
        n2 = np.sqrt((w * w).sum(1)).max()
        n1 = np.abs(w).sum(1).max()
        assert n2 <= b[0] <= n2 * (1 + 1e-6), (b[0], n2)
        assert n1 <= b[1] <= n1 * (1 + 1e-6), (b[1], n1)


@pytest.mark.parametrize("M,D,V", [(7, 256, 4096), (56, 512, 20000), (65, 320, 3000), (224, 256, 8192)])
def test_certified_rows_are_the_exact_top16(dfl, dev, M, D, V):
    rng = np.random.default_rng(M + D + V)
    h = bf16(rng.standard_normal((M, D)), dev)
    W = bf16(rng.standard_normal((V, D)) * 0.05, dev)
    bound = dfl.head_weight_bound(W)
    tv, ti, cert = dfl.head_topk_certified(h, W, bound)
    ov, oi, _ = oracle_topk(h.cpu(), W.cpu())
    cert = cert.cpu().numpy()
    assert set(np.unique(cert)) <= {0, 1}
    ok = cert == 1
    assert np.array_equal(ti.cpu().numpy()[ok], oi[ok])
    assert np.array_equal(tv.cpu().numpy()[ok], ov[ok])


def test_wide_margins_are_certified(dfl, dev):
    """Sixteen planted vocabulary rows per request score 10 to 25, far above
    the rest (~N(0, 0.5)): rows whose exact 16th value clears the next logit
    by more than 1 must be certified."""
    rng = np.random.default_rng(9)
    M, D, V = 48, 512, 30000
    h = rng.standard_normal((M, D))
    W = rng.standard_normal((V, D)) * 0.02
    for m in range(M):
        ids = rng.choice(V, 16, replace=False)
        W[ids] = h[m][None, :] * ((10.0 + np.arange(16)) / (h[m] @ h[m]))[:, None]
    hd, Wd = bf16(h, dev), bf16(W, dev)
    tv, ti, cert = dfl.head_topk_certified(hd, Wd, dfl.head_weight_bound(Wd))
    ov, oi, _ = oracle_topk(hd.cpu(), Wd.cpu())
    assert np.array_equal(ti.cpu().numpy(), oi)
    z = hd.float().cpu().numpy().astype(np.float64) @ Wd.float().cpu().numpy().astype(np.float64).T
    zs = -np.sort(-z, axis=1)
    wide = (zs[:, 15] - zs[:, 16]) > 1.0
    assert wide.sum() >= M // 2
    assert np.all(cert.cpu().numpy()[wide] == 1)


def test_ties_at_the_sixteenth_place_are_not_certified(dfl, dev):
    """Forty identical vocabulary rows hold every request's largest logit: the
    16 returned (the lowest tied ids) are exact, but no bound separates them
    from the other 24, so the rows are left uncertified."""
    rng = np.random.default_rng(11)
    M, D, V = 16, 256, 5000
    sign = np.sign(rng.standard_normal(D))
    h = np.abs(rng.standard_normal((M, D))) * sign          # h_m . u > 0 for the shared row u
    W = rng.standard_normal((V, D)) * 0.02
    tied = np.sort(rng.choice(V, 40, replace=False))
    W[tied] = 0.5 * sign                                     # logit ~ 0.5 * sum |h_m| ~ 100
    hd, Wd = bf16(h, dev), bf16(W, dev)
    tv, ti, cert = dfl.head_topk_certified(hd, Wd, dfl.head_weight_bound(Wd))
    ov, oi, _ = oracle_topk(hd.cpu(), Wd.cpu())
    assert np.array_equal(ti.cpu().numpy(), oi)
    assert np.all(ti.cpu().numpy() == tied[:16][None, :])
    assert np.all(cert.cpu().numpy() == 0)


def test_full_size_certificate(dfl, dev):
    """The batch-32 head (M = 224, D = 5120, V = 151936): certified rows on
    sampled rows equal the oracle; the fraction certified is reported."""
    g = torch.Generator(device=dev).manual_seed(3)
    M, D, V = 224, 5120, 151936
    h = torch.randn(M, D, device=dev, generator=g).to(torch.bfloat16)
    W = (0.02 * torch.randn(V, D, device=dev, generator=g)).to(torch.bfloat16)
    tv, ti, cert = dfl.head_topk_certified(h, W, dfl.head_weight_bound(W))
    cert = cert.cpu().numpy()
    print(f"certified rows: {cert.sum()} of {M}", flush=True)
    rows = [int(r) for r in np.nonzero(cert == 1)[0][:3]] + [int(r) for r in np.nonzero(cert == 0)[0][:2]]
    if rows:
        ov, oi, _ = oracle_topk(h.cpu(), W.cpu(), rows=rows)
        assert np.array_equal(ti.cpu().numpy()[rows], oi)


def test_near_ties_clustered_in_one_list_are_exact_or_uncertified(dfl, dev):
    """Each request's 24 largest logits are near-ties (exact values within
    ~1e-6 of 20, below float32 resolution there) on 24 consecutive vocabulary
    ids, so one workgroup's partial list holds them and keeps only 16, in
    float32 order.  An exact top-16 entry dropped there is never re-scored;
    the certificate must then leave the row uncertified.  Every row is either
    equal to the oracle's exact top-16 or not certified."""
    rng = np.random.default_rng(21)
    M, D, V = 8, 512, 20000
    h = np.asarray(bf16(rng.standard_normal((M, D)), "cpu").float().numpy(), np.float64)
    W = rng.standard_normal((V, D)) * 0.02
    for m in range(M):
        base = h[m] * (20.0 / (h[m] @ h[m]))
        # variants of one row: two entries whose h values nearly agree swapped
        order = np.argsort(h[m])
        c0 = 1000 + 2000 * m
        for k in range(24):
            w = base.copy()
            if k:
                i, j = order[100 + 7 * k], order[101 + 7 * k]
                w[i], w[j] = base[j], base[i]
            W[c0 + k] = w
    hd, Wd = bf16(h, dev), bf16(W, dev)
    tv, ti, cert = dfl.head_topk_certified(hd, Wd, dfl.head_weight_bound(Wd))
    ov, oi, _ = oracle_topk(hd.cpu(), Wd.cpu())
    ti, cert = ti.cpu().numpy(), cert.cpu().numpy()
    z = hd.float().cpu().numpy().astype(np.float64) @ Wd.float().cpu().numpy().astype(np.float64).T
    for m in range(M):
        top = np.argsort(-z[m], kind="stable")[:24]
        assert np.all((top >= 1000 + 2000 * m) & (top < 1024 + 2000 * m)), m  # the planted cluster leads
        assert np.array_equal(ti[m], oi[m]) or cert[m] == 0, (m, ti[m], oi[m])
    assert np.all(cert == 0)  # no bound separates 16 of 24 near-ties
