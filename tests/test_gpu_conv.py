"""GPU parity of dflash_conv2tap against the oracle: bit-exact bf16 outputs."""

import numpy as np
import pytest
import torch

from oracle import conv2tap as oracle_conv

pytestmark = pytest.mark.gpu


def rand_bf16(shape, seed, sd=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * sd).to(torch.bfloat16)


@pytest.mark.parametrize("S,T,D", [(1, 8, 256), (5, 8, 5120), (3, 1, 64), (2, 16, 136), (7, 3, 8),
                                   (4, 5, 2048), (9, 12, 520)])
def test_conv_matches_oracle(dfl, dev, S, T, D):
    x = rand_bf16((S, T, D), S * 100 + T)
    taps = rand_bf16((S, T, 2 * D), S * 100 + T + 1, sd=1.5)
    y = dfl.conv2tap(x.to(dev), taps.to(dev))
    torch.cuda.synchronize()
    ref = oracle_conv(x, taps)
    assert torch.equal(y.cpu().view(torch.int16), ref.view(torch.int16))


def test_conv_integer_grid_and_special_taps(dfl, dev):
    rng = np.random.default_rng(1)
    x = torch.tensor(rng.integers(-8, 9, (3, 8, 64)), dtype=torch.bfloat16)
    taps = torch.tensor(rng.integers(-4, 5, (3, 8, 128)), dtype=torch.bfloat16)
    y = dfl.conv2tap(x.to(dev), taps.to(dev)).cpu()
    assert torch.equal(y.view(torch.int16), oracle_conv(x, taps).view(torch.int16))
    ident = torch.cat([torch.ones(3, 8, 64), torch.zeros(3, 8, 64)], -1).to(torch.bfloat16)
    assert torch.equal(dfl.conv2tap(x.to(dev), ident.to(dev)).cpu(), x)


def test_conv_five_layer_batch32_shape(dfl, dev):
    """The block-8, batch-32 layer shape: [32][8][5120] per call, five calls."""
    for layer in range(5):
        x = rand_bf16((32, 8, 5120), 40 + layer)
        taps = rand_bf16((32, 8, 10240), 50 + layer, sd=1.43)
        y = dfl.conv2tap(x.to(dev), taps.to(dev)).cpu()
        assert torch.equal(y.view(torch.int16), oracle_conv(x, taps).view(torch.int16))


def test_conv_rejects_aliasing(dfl, dev):
    x = rand_bf16((1, 8, 64), 3).to(dev)
    taps = rand_bf16((1, 8, 128), 4).to(dev)
    with pytest.raises(dfl.DFlashError):
        dfl.conv2tap(x, taps, out=x)


@pytest.mark.parametrize("S,T,D", [(160, 16, 5120), (301, 7, 4096), (130, 13, 5120), (2100, 1, 4096),
                                   (132, 16, 5000)])
def test_conv_large_calls_four_rows_per_thread(dfl, dev, S, T, D):
    """Calls of at least 2^20 threads take four token rows per thread; groups
    of four straddle sequence starts when T is not a multiple of four, and the
    last group is ragged."""
    x = rand_bf16((S, T, D), S + T)
    taps = rand_bf16((S, T, 2 * D), S + T + 1, sd=1.4)
    y = dfl.conv2tap(x.to(dev), taps.to(dev)).cpu()
    assert torch.equal(y.view(torch.int16), oracle_conv(x, taps).view(torch.int16))


@pytest.mark.parametrize("S,T,D", [(160, 8, 5120), (101, 7, 6144), (1025, 1, 4096), (93, 15, 4104)])
def test_conv_mid_calls_two_rows_per_thread(dfl, dev, S, T, D):
    """Calls of 2^19 to 2^20 threads (the five-layer block-8 batch-32 shape
    among them) take two token rows per thread; pairs straddle sequence
    starts when T is odd, and the last pair is ragged when S*T is odd."""
    n = S * T * D // 8
    assert (1 << 19) <= n < (1 << 20)
    x = rand_bf16((S, T, D), S + T + 7)
    taps = rand_bf16((S, T, 2 * D), S + T + 8, sd=1.4)
    y = dfl.conv2tap(x.to(dev), taps.to(dev)).cpu()
    assert torch.equal(y.view(torch.int16), oracle_conv(x, taps).view(torch.int16))
