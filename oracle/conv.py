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
