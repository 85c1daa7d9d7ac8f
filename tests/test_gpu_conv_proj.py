"""GPU parity of dflash_conv2tap_proj (the conv with its taps projected in the
same call) against the oracle.

The kernel keeps the taps as float32 GEMM accumulators, whose summation order
is the hardware's; the oracle's taps are exact.  The bar, derived from that
arithmetic: every output equals the oracle's (the exact value rounded to
float32, then to bf16) except where the exact value lies within 1e-3 of its
magnitude scale (|a x_t| + |b x_t-1|, plus 1e-3 of the absolute sums inside
the taps, which bounds cancellation) of a bf16 rounding boundary; there the
two results are neighbours and the exact value lies between them.  Such
flips are rare (well under 2 % of outputs).  On integer grids, where every
float32 sum is exact, the outputs are identical."""

import numpy as np
import pytest
import torch

from oracle.conv import conv2tap as oracle_conv, conv2tap_proj as oracle_proj

pytestmark = pytest.mark.gpu


def rand_bf16(shape, seed, sd=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * sd).to(torch.bfloat16)


def check_admissible(y_gpu, x, w_tap, max_flip=0.02):
    y_ref, y64, scale = oracle_proj(x, w_tap, return_exact=True)
    g = y_gpu.float().numpy().astype(np.float64)
    r = y_ref.float().numpy().astype(np.float64)
    diff = g != r
    tol = 1e-3 * scale
    # the GPU value is the exact value up to one bf16 step and the tolerance
    assert np.all(np.abs(g - y64) <= 2.0 ** -7 * np.abs(y64) + tol)
    # every flip sits on a rounding boundary: the exact value is within the
    # tolerance of the midpoint of the two candidates
    mid = 0.5 * (g + r)
    bad = diff & (np.abs(y64 - mid) > tol)
    assert not bad.any(), (np.argwhere(bad)[:5], y64[bad][:5], g[bad][:5], r[bad][:5])
    assert diff.mean() <= max_flip, diff.mean()
    return diff.mean()


@pytest.mark.parametrize("S,T,D", [(1, 8, 64), (3, 8, 256), (5, 7, 512), (40, 8, 1024), (130, 8, 512),
                                   (2, 16, 5120), (3, 1, 128), (33, 16, 192)])
def test_conv_proj_matches_oracle(dfl, dev, S, T, D):
    """Shapes spanning one and several M-blocks (64 and 128 rows) with ragged
    last blocks, block lengths 1, 7, 8 and 16, and D from 64 to 5120."""
    x = rand_bf16((S, T, D), S * 31 + T)
    w = rand_bf16((2 * D, D), S * 31 + T + 1, sd=0.02)
    y = dfl.conv2tap_proj(x.to(dev), w.to(dev))
    torch.cuda.synchronize()
    check_admissible(y.cpu(), x, w)


@pytest.mark.parametrize("S,T,D", [(3, 8, 256), (140, 8, 320)])
def test_conv_proj_integer_grid_bit_exact(dfl, dev, S, T, D):
    """Small integers: every product and float32 sum is exact, so the outputs
    are bit-identical to the oracle's, and, with the taps exact in bf16, to
    the plain conv on those taps."""
    rng = np.random.default_rng(S + D)
    x = torch.tensor(rng.integers(-4, 5, (S, T, D)), dtype=torch.bfloat16)
    w = torch.tensor(rng.integers(-1, 2, (2 * D, D)), dtype=torch.bfloat16)
    y = dfl.conv2tap_proj(x.to(dev), w.to(dev)).cpu().float()
    # (compared by value: the sign of an exact zero is the only freedom)
    assert torch.equal(y, oracle_proj(x, w).float())
    taps = (x.double().reshape(-1, D) @ w.double().T).reshape(S, T, 2 * D)
    assert taps.abs().max() <= 256  # exact in bf16
    assert torch.equal(y, oracle_conv(x, taps.to(torch.bfloat16)).float())


def test_conv_proj_diagonal_projection(dfl, dev):
    """W_tap = [I; 0] makes y = x^2 and W_tap = [0; I] makes y[t] = x[t] x[t-1]
    (each one rounding from the exact product)."""
    S, T, D = 4, 8, 128
    x = rand_bf16((S, T, D), 5)
    eye, zero = torch.eye(D), torch.zeros(D, D)
    y1 = dfl.conv2tap_proj(x.to(dev), torch.cat([eye, zero]).to(torch.bfloat16).to(dev)).cpu()
    y2 = dfl.conv2tap_proj(x.to(dev), torch.cat([zero, eye]).to(torch.bfloat16).to(dev)).cpu()
    xf = x.float()
    assert torch.equal(y1, (xf * xf).to(torch.bfloat16))
    prev = torch.cat([torch.zeros(S, 1, D), xf[:, :-1]], 1)
    assert torch.equal(y2, (xf * prev).to(torch.bfloat16))


@pytest.mark.parametrize("S,T", [(160, 8), (160, 16)])
def test_conv_proj_full_size_sampled(dfl, dev, S, T):
    """The five-layer, batch-32 shapes at D = 5120 (block 8: 1280 token rows,
    block 16: 2560), in the launch configuration the benchmark times; the
    oracle checks 12 sampled sequences, first and last included."""
    D = 5120
    x = rand_bf16((S, T, D), 40 + T)
    w = rand_bf16((2 * D, D), 41 + T, sd=0.02)
    y = dfl.conv2tap_proj(x.to(dev), w.to(dev)).cpu()
    torch.cuda.synchronize()
    rng = np.random.default_rng(T)
    seqs = np.unique(np.concatenate([[0, S - 1], rng.choice(S, 10, replace=False)]))
    check_admissible(y[seqs], x[seqs], w)


def test_conv_proj_repeat_calls_identical(dfl, dev):
    """Run-to-run determinism: the same inputs give the same bits."""
    x = rand_bf16((40, 8, 1024), 7).to(dev)
    w = rand_bf16((2048, 1024), 8, sd=0.02).to(dev)
    y1 = dfl.conv2tap_proj(x, w)
    y2 = dfl.conv2tap_proj(x, w)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
