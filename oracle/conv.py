"""Two-tap dynamic depthwise causal convolution on draft hidden states.

Source: tamsi.dev "DFlash 2 — 3× plus de tokens…", § "L'idée, sans le papier"
(a two-tap conv in the Canon / short-conv style placed around each attention
and MLP block against suffix decay); myaiexp.com "DFlash 2", § 主な機能
(two-tap *dynamic* convolution); 0xbakeer.com sources list, § "Prior art
referenced by DFlash 2" (Canon layers, dynamic short convolutions).

Reading taken (the pages give no equation): causal taps over block slots
(t, t-1), one pair of taps per token and per channel ("dynamic", "depthwise"),
zero history before slot 0, no activation and no residual:

    y[s, t, c] = a[s, t, c] * x[s, t, c] + b[s, t, c] * x[s, t-1, c],
    x[s, -1, c] = 0,  a = taps[..., :D],  b = taps[..., D:].

Precision: inputs and output are bf16; the sum is formed exactly (float64
holds both bf16 x bf16 products and their sum exactly for these magnitudes),
rounded once to float32, then to bf16 (nearest-even).
"""

import numpy as np

from ._arrays import f64, f32_to_bf16


def conv2tap(x, taps):
    """x: [S][T][D] bf16 values, taps: [S][T][2D] -> y: torch.bfloat16 [S][T][D]."""
    x64 = f64(x)
    t64 = f64(taps)
    S, T, D = x64.shape
    assert t64.shape == (S, T, 2 * D)
    a = t64[:, :, :D]
    b = t64[:, :, D:]
    x_prev = np.zeros_like(x64)
    x_prev[:, 1:, :] = x64[:, :-1, :]
    y64 = a * x64 + b * x_prev
    return f32_to_bf16(y64.astype(np.float32))


def tap_projection(x, w_tap):
    """The drafter's per-token taps, exact: [a | b] = x W_tap^T in float64.
    x: [S][T][D] bf16 values, w_tap: [2D][D] -> (a, b), each float64 [S][T][D].

    Reading (the pages call the taps dynamic, i.e. per token, and give no
    producer): a linear projection of the token's own hidden state, rows
    0..D-1 of W_tap giving a and rows D..2D-1 giving b.  Every bf16 x bf16
    product is exact in float64; the sums carry float64 rounding only."""
    x64 = f64(x)
    w64 = f64(w_tap)
    S, T, D = x64.shape
    assert w64.shape == (2 * D, D)
    taps = x64.reshape(S * T, D) @ w64.T
    return taps[:, :D].reshape(S, T, D), taps[:, D:].reshape(S, T, D)


def conv2tap_proj(x, w_tap, return_exact=False):
    """The conv on taps projected from x (``tap_projection``), kept unrounded:
    y = a * x[t] + b * x[t-1] (x[-1] = 0), rounded to float32, then to bf16.

    With return_exact=True also returns the float64 y before rounding and the
    per-element magnitude scale |a x[t]| + |b x[t-1]| + 1e-3 (|x| |W_a|^T |x[t]| +
    |x| |W_b|^T |x[t-1]|), against which a float32 evaluation's deviation is
    measured (the second term bounds what cancellation inside the taps' sums
    can cost)."""
    x64 = f64(x)
    a, b = tap_projection(x, w_tap)
    x_prev = np.zeros_like(x64)
    x_prev[:, 1:, :] = x64[:, :-1, :]
    y64 = a * x64 + b * x_prev
    y = f32_to_bf16(y64.astype(np.float32))
    if not return_exact:
        return y
    S, T, D = x64.shape
    ab = np.abs(x64.reshape(S * T, D)) @ np.abs(f64(w_tap)).T
    aa, bb = ab[:, :D].reshape(S, T, D), ab[:, D:].reshape(S, T, D)
    scale = np.abs(a * x64) + np.abs(b * x_prev) + 1e-3 * (aa * np.abs(x64) + bb * np.abs(x_prev))
    return y, y64, scale
