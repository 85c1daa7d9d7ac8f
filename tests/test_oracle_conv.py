"""Pins for the oracle's two-tap conv: special cases with closed forms,
exact integer arithmetic on a grid, and the rounding rule on constructed ties."""

import numpy as np
import torch

from oracle import conv2tap


def bf16(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def rand_bf16(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16)


def test_identity_taps():
    x = rand_bf16((3, 8, 64), 0)
    taps = torch.cat([torch.ones(3, 8, 64), torch.zeros(3, 8, 64)], -1).to(torch.bfloat16)
    assert torch.equal(conv2tap(x, taps).view(torch.int16), x.view(torch.int16))


def test_shift_taps():
    x = rand_bf16((2, 5, 32), 1)
    taps = torch.cat([torch.zeros(2, 5, 32), torch.ones(2, 5, 32)], -1).to(torch.bfloat16)
    y = conv2tap(x, taps).float()
    assert torch.all(y[:, 0] == 0)
    assert torch.equal(y[:, 1:], x[:, :-1].float())


def test_zero_taps():
    x = rand_bf16((1, 4, 16), 2)
    assert torch.all(conv2tap(x, torch.zeros(1, 4, 32, dtype=torch.bfloat16)).float() == 0)


def test_integer_grid_exact():
    # small integers: every product and sum is an exact small integer
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, (4, 6, 40))
    a = rng.integers(-4, 5, (4, 6, 40))
    b = rng.integers(-4, 5, (4, 6, 40))
    y = conv2tap(bf16(x), bf16(np.concatenate([a, b], -1))).float().numpy()
    for s in range(4):
        for t in range(6):
            for c in range(40):
                prev = int(x[s, t - 1, c]) if t > 0 else 0
                assert y[s, t, c] == int(a[s, t, c]) * int(x[s, t, c]) + int(b[s, t, c]) * prev


def test_round_to_nearest_even():
    # bf16 keeps 8 significant bits: between 1 and 2 the spacing is 2^-7.
    # a*x = 1, b*x_prev chosen to land exactly on, just above, or just below halfway.
    cases = [
        (2.0 ** -8, 1.0),                        # 1 + 2^-8: tie -> even (1.0)
        (3 * 2.0 ** -8, 1.0 + 2.0 ** -6),        # 1 + 3*2^-8: tie -> even (1 + 2^-6)
        (2.0 ** -8 + 2.0 ** -15, 1.0 + 2.0 ** -7),  # just above half -> up
        (2.0 ** -8 - 2.0 ** -16, 1.0),           # just below half -> down
    ]
    for bx, want in cases:
        # b * x_prev = bx with x_prev = 1, b = bx (bx is bf16-exact in every case)
        x = bf16([[[1.0], [1.0]]])                      # S=1, T=2, D=1
        taps = bf16([[[1.0, 0.0], [1.0, bx]]])
        assert float(bf16([bx]).float()[0]) == bx
        y = conv2tap(x, taps).float().numpy()
        assert y[0, 1, 0] == want, (bx, y[0, 1, 0], want)


def test_linear_in_taps_on_grid():
    rng = np.random.default_rng(4)
    x = bf16(rng.integers(-4, 5, (2, 4, 24)))
    t1 = rng.integers(-3, 4, (2, 4, 48))
    t2 = rng.integers(-3, 4, (2, 4, 48))
    y1 = conv2tap(x, bf16(t1)).float()
    y2 = conv2tap(x, bf16(t2)).float()
    y12 = conv2tap(x, bf16(t1 + t2)).float()
    assert torch.equal(y1 + y2, y12)
