"""GPU parity of dflash_head_topk against the oracle.

Indices and values are compared exactly: the library re-scores its float32
candidates in float64 and orders them by the exact value, as the oracle does."""

import numpy as np
import pytest
import torch

from oracle.head import head_logits, head_topk as oracle_topk, topk_from_logits
from workload import get_config, make_cycle_inputs

pytestmark = pytest.mark.gpu


def bf16(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def check(dfl, dev, h, W, rows=None):
    tv, ti = dfl.head_topk(h.to(dev) if not h.is_cuda else h, W.to(dev) if not W.is_cuda else W)
    torch.cuda.synchronize()
    tv, ti = tv.cpu().numpy(), ti.cpu().numpy()
    hc, Wc = h.cpu(), W.cpu()
    rv, ri, _ = oracle_topk(hc, Wc, rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    assert np.array_equal(ti[sel], ri), (ti[sel][:2], ri[:2])
    assert np.array_equal(tv[sel], rv)


@pytest.mark.parametrize("M,D,V", [(1, 256, 4096), (7, 256, 4096), (7, 264, 4133), (16, 512, 1000),
                                   (17, 256, 5003), (56, 256, 4096), (65, 320, 3000), (128, 256, 2000),
                                   (224, 256, 8192), (257, 256, 2048), (480, 128, 4096), (300, 264, 3001),
                                   (3, 8, 40)])
def test_gaussian_shapes(dfl, dev, M, D, V):
    g = torch.Generator().manual_seed(M * 7 + D + V)
    h = torch.randn(M, D, generator=g).to(torch.bfloat16)
    W = (0.02 * torch.randn(V, D, generator=g)).to(torch.bfloat16)
    check(dfl, dev, h, W)


def test_integer_grid_with_ties(dfl, dev):
    rng = np.random.default_rng(5)
    h = bf16(rng.integers(-1, 2, (33, 64)))
    W = bf16(rng.integers(-1, 2, (3000, 64)))
    check(dfl, dev, h, W)


def test_integer_grid_fine(dfl, dev):
    rng = np.random.default_rng(6)
    h = bf16(rng.integers(-8, 9, (20, 512)) / 8.0)
    W = bf16(rng.integers(-16, 17, (7000, 512)) / 256.0)
    check(dfl, dev, h, W)


def test_vocab_exactly_k_and_constant_rows(dfl, dev):
    g = torch.Generator().manual_seed(3)
    check(dfl, dev, torch.randn(5, 64, generator=g).to(torch.bfloat16),
          torch.randn(16, 64, generator=g).to(torch.bfloat16))
    # all logits equal: ids 0..15 in order
    check(dfl, dev, torch.zeros(4, 32, dtype=torch.bfloat16), torch.ones(100, 32, dtype=torch.bfloat16))


def test_increasing_logits_stress_candidate_overflow(dfl, dev):
    """Strictly increasing logits z[v] = v / 256 (exact: W[v] = (v // 256,
    v % 256), h = (1, 1/256)): every element beats the running threshold, which
    exercises the bounded candidate buffers' retry path."""
    V, D = 6000, 16
    W = torch.zeros(V, D)
    v = torch.arange(V)
    W[:, 0] = (v // 256).float()
    W[:, 1] = (v % 256).float()
    h = torch.zeros(3, D)
    h[:, 0] = 1.0
    h[:, 1] = 1.0 / 256
    check(dfl, dev, h.to(torch.bfloat16), W.to(torch.bfloat16))


def test_rounded_ramp_heavy_ties(dfl, dev):
    """A ramp rounded to bf16 (v / 64): long runs of equal logits at the top,
    so the lower ids must win among equals across strips and retries."""
    V, D = 6000, 16
    W = torch.zeros(V, D)
    W[:, 0] = torch.arange(V, dtype=torch.float32) / 64.0
    h = torch.zeros(3, D)
    h[:, 0] = 1.0
    check(dfl, dev, h.to(torch.bfloat16), W.to(torch.bfloat16))


def test_planted_maxima(dfl, dev):
    V, D = 9000, 64
    rng = np.random.default_rng(7)
    W = 0.01 * np.round(rng.standard_normal((V, D)) * 8) / 8
    h = np.zeros((2, D)); h[0, 0] = 1.0; h[1, 1] = 1.0
    planted = rng.choice(V, 32, replace=False)
    W[planted[:16], 0] = np.arange(16, 0, -1)
    W[planted[16:], 1] = np.arange(16, 0, -1)
    tv, ti = dfl.head_topk(bf16(h).to(dev), bf16(W).to(dev))
    assert list(ti[0].cpu().numpy()) == list(planted[:16])
    assert list(ti[1].cpu().numpy()) == list(planted[16:])


@pytest.mark.parametrize("name,rows", [("c2_b1", None), ("c4_b32", [0, 1, 100, 223]),
                                       ("c5_stress", [0, 127, 128, 239, 240, 383, 384, 479])])
def test_full_size_configs(dfl, dev, name, rows):
    cfg = get_config(name)
    g = torch.Generator(device=dev).manual_seed(11)
    W = (0.02 * torch.randn(cfg.V, cfg.D, generator=g, device=dev)).to(torch.bfloat16)
    h = torch.randn(cfg.M, cfg.D, generator=g, device=dev).to(torch.bfloat16)
    check(dfl, dev, h, W, rows=rows)
