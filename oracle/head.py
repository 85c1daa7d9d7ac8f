"""Draft LM head and per-position top-16 candidate retention.

Source: tamsi.dev "DFlash 2 — 3× plus de tokens…", § "L'idée, sans le papier"
(the right token is in the drafter's top 16 at 99.5 % although top-1 is right
only 85.4 % of the time, so 16 candidates are kept per position);
myaiexp.com "DFlash 2", § 主な機能 (the path selector keeps each position's top
16 candidates over the vocabulary).

Definition: z[m, v] = sum_d h[m, d] * W[v, d] (the exact real value; float64
holds every bf16 x bf16 product exactly and the sums here to ~1e-16 relative).
Per row, candidates are ordered by value descending, ties to the lower vocab
id, and the first K are kept.  Values returned are float32(z).
"""

import numpy as np

from ._arrays import f64


def head_logits(h, W, rows=None, chunk=8192):
    """Exact logits z = h W^T in float64, streamed over vocab chunks.

    h: [M][D] bf16 values, W: [V][D] bf16 values (torch tensors or arrays).
    rows: optional list of row indices of h to evaluate.  Returns [R][V] f64.
    """
    h64 = f64(h)
    if rows is not None:
        h64 = h64[np.asarray(rows)]
    V = W.shape[0]
    out = np.empty((h64.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, chunk):
        w64 = f64(W[v0:v0 + chunk])
        out[:, v0:v0 + chunk] = h64 @ w64.T
    return out


def topk_from_logits(z, K=16):
    """Stable full sort of each row by value descending (ties: lower index)."""
    z = np.asarray(z, dtype=np.float64)
    order = np.argsort(-z, axis=-1, kind="stable")[..., :K]
    vals = np.take_along_axis(z, order, axis=-1)
    return vals.astype(np.float32), order.astype(np.int32), vals


def head_topk(h, W, K=16, rows=None, chunk=8192):
    """Top-K of h W^T per row -> (vals f32 [R][K], idx i32 [R][K], exact f64 vals)."""
    return topk_from_logits(head_logits(h, W, rows=rows, chunk=chunk), K)
