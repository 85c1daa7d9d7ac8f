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


# --- the conv on projected taps (oracle.conv.conv2tap_proj) ---

def test_proj_diagonal_projection_closed_form():
    """W_tap = [alpha I; beta I] gives a = alpha x, b = beta x, so
    y[t] = alpha x[t]^2 + beta x[t] x[t-1] (small integers: exact)."""
    from oracle.conv import conv2tap_proj
    rng = np.random.default_rng(11)
    S, T, D = 3, 6, 16
    x = rng.integers(-6, 7, (S, T, D)).astype(np.float32)
    alpha, beta = 2.0, -0.5
    w = np.concatenate([alpha * np.eye(D), beta * np.eye(D)]).astype(np.float32)
    y = conv2tap_proj(bf16(x), bf16(w)).float().numpy()
    prev = np.concatenate([np.zeros((S, 1, D)), x[:, :-1]], axis=1)
    assert np.array_equal(y, alpha * x * x + beta * x * prev)


def test_proj_equals_conv_on_exact_taps_brute_force():
    """Against pure-Python loops on a tiny case: taps t[s][t][j] = sum_k
    x[s][t][k] W[j][k] (j < D gives a, j >= D gives b), then the direct conv.
    Integer inputs keep every tap exactly representable in bf16, so the
    result also equals the plain conv on those taps."""
    from oracle.conv import conv2tap_proj
    rng = np.random.default_rng(12)
    S, T, D = 2, 4, 3
    x = rng.integers(-3, 4, (S, T, D))
    w = rng.integers(-2, 3, (2 * D, D))
    taps = np.zeros((S, T, 2 * D))
    for s in range(S):
        for t in range(T):
            for j in range(2 * D):
                taps[s, t, j] = sum(int(x[s, t, k]) * int(w[j, k]) for k in range(D))
    ref = np.zeros((S, T, D))
    for s in range(S):
        for t in range(T):
            for c in range(D):
                prev = x[s, t - 1, c] if t > 0 else 0
                ref[s, t, c] = taps[s, t, c] * x[s, t, c] + taps[s, t, D + c] * prev
    y = conv2tap_proj(bf16(x), bf16(w))
    assert np.array_equal(y.float().numpy(), ref)
    assert torch.equal(y.view(torch.int16), conv2tap(bf16(x), bf16(taps)).view(torch.int16))


def test_proj_exact_value_and_scale():
    """The unrounded value rounds to the returned bf16, and the scale bounds
    the value (|y| <= |a x| + |b x_prev| <= scale)."""
    from oracle.conv import conv2tap_proj
    x = rand_bf16((2, 8, 32), 13)
    w = (0.05 * torch.randn(64, 32, generator=torch.Generator().manual_seed(14))).to(torch.bfloat16)
    y, y64, scale = conv2tap_proj(x, w, return_exact=True)
    assert torch.equal(y.view(torch.int16), bf16(y64.astype(np.float32)).view(torch.int16))
    assert np.all(np.abs(y64) <= scale)
    assert np.all(np.isfinite(y64))


def test_proj_scale_hand_computed():
    """S = 1, T = 2, D = 2 by hand: x_0 = (1, 2), x_1 = (3, -1); W_tap rows
    (1, 0), (0, 1) give a = x, rows (2, 1), (1, -1) give b = (2 x_0 + x_1,
    x_0 - x_1).  y_0 = a_0 x_0 = (1, 4) (no history); y_1 = a_1 x_1 + b_1 x_0 =
    (9 + 5, 1 + 8).  scale = |a x| + |b x_prev| + 1e-3 (|x||W_a| |x| +
    |x||W_b| |x_prev|)."""
    from oracle.conv import conv2tap_proj
    x = bf16([[[1, 2], [3, -1]]])
    w = bf16([[1, 0], [0, 1], [2, 1], [1, -1]])
    y, y64, scale = conv2tap_proj(x, w, return_exact=True)
    assert np.array_equal(y64[0], [[1.0, 4.0], [14.0, 9.0]])
    assert np.array_equal(y.float().numpy()[0], [[1.0, 4.0], [14.0, 9.0]])
    np.testing.assert_allclose(scale[0], [[1.0 + 1e-3 * 1, 4.0 + 1e-3 * 4],
                                          [14.0 + 1e-3 * (9 + 7), 9.0 + 1e-3 * (1 + 8)]], rtol=1e-15)


def _proj_f32(x, w, reverse):
    """The conv on projected taps evaluated in float32 with sequential sums in
    a chosen order (the worst case for rounding), as a float32 kernel might."""
    x32 = x.float().numpy().astype(np.float32)
    w32 = w.float().numpy().astype(np.float32)
    S, T, D = x32.shape
    xr = x32.reshape(S * T, D)
    acc = np.zeros((S * T, 2 * D), np.float32)
    for d in (range(D - 1, -1, -1) if reverse else range(D)):
        acc = (acc + xr[:, d:d + 1] * w32[:, d][None, :]).astype(np.float32)
    a, b = acc[:, :D].reshape(S, T, D), acc[:, D:].reshape(S, T, D)
    xp = np.zeros_like(x32)
    xp[:, 1:] = x32[:, :-1]
    return (a * x32 + b * xp).astype(np.float32).astype(np.float64)


def test_proj_scale_bounds_float32_evaluation():
    """Sequential float32 sums in either order stay within 1e-3 of the scale
    of the exact value (the tolerance the GPU parity test uses)."""
    from oracle.conv import conv2tap_proj
    x = rand_bf16((3, 8, 512), 15)
    w = (0.02 * torch.randn(1024, 512, generator=torch.Generator().manual_seed(16))).to(torch.bfloat16)
    _, y64, scale = conv2tap_proj(x, w, return_exact=True)
    for rev in (False, True):
        err = np.abs(_proj_f32(x, w, rev) - y64)
        assert np.all(err <= 1e-3 * scale)
        assert err.max() > 0  # float32 really rounds here


def test_proj_scale_covers_cancellation_inside_the_taps():
    """a = 2^20 + 2^-8 - 2^20 cancels: float32 loses the 2^-8 entirely, so the
    error is as large as the value itself; only the scale's second term (the
    absolute sums inside the taps) covers it."""
    from oracle.conv import conv2tap_proj
    x = bf16([[[1, 1, 1], [1, 1, 1]]])
    w = bf16([[2.0 ** 20, 2.0 ** -8, -2.0 ** 20], [0, 0, 0], [0, 0, 0],
              [0, 0, 0], [0, 0, 0], [0, 0, 0]])
    _, y64, scale = conv2tap_proj(x, w, return_exact=True)
    assert y64[0, 0, 0] == 2.0 ** -8
    err = np.abs(_proj_f32(x, w, False) - y64)
    assert err[0, 0, 0] == 2.0 ** -8                       # float32 gives 0
    first = np.abs(y64)                                     # |a x| + |b x_prev| (b = 0 here)
    assert err[0, 0, 0] > 1e-3 * first[0, 0, 0]
    assert np.all(err <= 1e-3 * scale)
