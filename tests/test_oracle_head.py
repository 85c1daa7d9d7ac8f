"""Pins for the oracle's LM head + top-16: exact integer arithmetic, a full
sort by Python's own sorted(), planted maxima with a known answer, and ties."""

import numpy as np
import torch

from oracle.head import head_logits, head_topk, topk_from_logits


def bf16(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def test_logits_exact_on_integer_grid():
    rng = np.random.default_rng(0)
    hi = rng.integers(-8, 9, (5, 96))
    wi = rng.integers(-16, 17, (300, 96))
    z = head_logits(bf16(hi / 8.0), bf16(wi / 256.0), chunk=64)
    exact = (hi.astype(object) @ wi.T.astype(object))  # python ints
    assert np.array_equal(z * 2048, exact.astype(np.float64))


def test_topk_matches_python_sorted():
    rng = np.random.default_rng(1)
    h = bf16(rng.standard_normal((4, 64)))
    W = bf16(0.02 * rng.standard_normal((1000, 64)))
    vals, idx, ex = head_topk(h, W, K=16)
    z = head_logits(h, W)
    for m in range(4):
        ref = sorted(range(1000), key=lambda v: (-z[m, v], v))[:16]
        assert list(idx[m]) == ref
        assert np.array_equal(vals[m], z[m, ref].astype(np.float32))


def test_ties_go_to_lower_id():
    # {-1, 0, 1} grid: many equal logits
    rng = np.random.default_rng(2)
    h = bf16(rng.integers(-1, 2, (6, 8)))
    W = bf16(rng.integers(-1, 2, (500, 8)))
    vals, idx, _ = head_topk(h, W)
    z = head_logits(h, W)
    for m in range(6):
        ref = sorted(range(500), key=lambda v: (-z[m, v], v))[:16]
        assert list(idx[m]) == ref
        # within a run of equal values the ids ascend
        for k in range(15):
            if vals[m, k] == vals[m, k + 1]:
                assert idx[m, k] < idx[m, k + 1]


def test_planted_maxima():
    # h = e_0 makes z[v] = W[v, 0]; plant 16 distinct large values at known ids
    V, D = 5000, 32
    rng = np.random.default_rng(3)
    W = 0.01 * np.round(rng.standard_normal((V, D)) * 8) / 8
    planted = rng.choice(V, 16, replace=False)
    W[planted, 0] = np.arange(16, 0, -1)  # 16, 15, ..., 1 (bf16-exact)
    h = np.zeros((1, D)); h[0, 0] = 1.0
    vals, idx, _ = head_topk(bf16(h), bf16(W))
    assert list(idx[0]) == list(planted)
    assert list(vals[0]) == list(np.arange(16, 0, -1, dtype=np.float32))


def test_topk_from_logits_negative_zero_and_tail():
    z = np.array([[0.0, -0.0, 1.0, -1.0] + [-5.0] * 20])
    vals, idx, _ = topk_from_logits(z, K=16)
    assert list(idx[0][:4]) == [2, 0, 1, 3]
