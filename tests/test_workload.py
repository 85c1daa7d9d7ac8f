"""CPU checks of the seeded workload generator and of one oracle cycle on the
tiny configuration (block 8, hidden 256, vocab 4096)."""

import numpy as np
import torch

from oracle.cycle import run_cycle
from workload import get_config, make_cycle_inputs


def test_tiny_inputs_shapes_and_determinism():
    cfg = get_config("c1_tiny")
    a = make_cycle_inputs(cfg)
    b = make_cycle_inputs(cfg)
    assert a["x"].shape == (5, 1, 8, 256) and a["taps"].shape == (5, 1, 8, 512)
    assert a["h"].shape == (7, 256) and a["W"].shape == (4096, 256)
    assert a["F_l"].shape == (4096, 32) and a["target"].shape == (1, 8, 4096)
    for k in ("x", "taps", "h", "W", "F_l", "F_r", "target"):
        assert torch.equal(a[k], b[k])
    other = make_cycle_inputs(get_config("c1_tiny", seed=1))
    assert not torch.equal(a["W"], other["W"])


def test_planted_margin_makes_token_top1():
    cfg = get_config("c1_tiny", plant_alpha=8.0, name="plant_probe")
    inp = make_cycle_inputs(cfg)
    z = inp["h"].float() @ inp["W"].float().T
    assert torch.all(torch.argmax(z, dim=1) == inp["planted"])


def test_context_copy_agreement_is_exact():
    cfg = get_config("c5_stress", B=2, T=6, D=64, V=2048, r=8, name="cc_probe")
    inp = make_cycle_inputs(cfg)
    t = inp["target"]
    P = cfg.P
    agree = sum(int(torch.argmax(t[m // P, m % P])) == int(inp["planted"][m]) for m in range(cfg.M))
    assert agree == round(cfg.agree_frac * cfg.M)


def test_tiny_cycle_runs_in_oracle():
    cfg = get_config("c1_tiny")
    inp = make_cycle_inputs(cfg)
    res = run_cycle(inp, cfg.B, cfg.T)
    assert len(res["y"]) == 5
    n = int(res["n_emit"][0])
    assert 1 <= n <= 8
    g = np.argmax(inp["target"][0].numpy(), -1)
    assert list(res["out_tok"][0, :n]) == list(g[:n])
