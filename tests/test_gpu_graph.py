"""HIP-graph capture of a whole cycle through the C-ABI.

Every call only enqueues kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a cycle can be captured once and replayed,
also with the greedy and sampled halves of a batch verified on two streams
(as the benchmark's graph does).  Each replay, with eager work and
synchronisations in between, must give exactly the outputs of the eager
cycle.
"""

import numpy as np
import pytest
import torch

from workload import get_config, make_cycle_inputs

pytestmark = pytest.mark.gpu


def _cycle(dfl, g, cfg, bufs, bound, fused=False, side=None):
    """fused: the conv projects its own taps, and verification runs from the
    target's hidden states through the LM head.  side: a second stream on
    which the greedy half verifies, forked after the selector and joined at
    the end (the two halves touch disjoint requests, outputs and
    workspaces)."""
    B, P, T = cfg.B, cfg.P, cfg.T
    calls = []
    for l in range(cfg.L):
        if fused:
            calls.append(bound.bind_conv2tap_proj(g["x"][l], g["w_tap"], bufs["y"][l]))
        else:
            calls.append(bound.bind_conv2tap(g["x"][l], g["taps"][l], bufs["y"][l]))
    calls.append(bound.bind_head_topk(g["h"], g["W"], bufs["tv"], bufs["ti"], bufs["ws_h"]))
    calls.append(bound.bind_select_path(bufs["tv"].view(B, P, 16), bufs["ti"].view(B, P, 16), g["F_l"], g["F_r"],
                                        bufs["rank"], bufs["tok"], bufs["score"], bufs["ws_s"]))
    h = B // 2

    def greedy():
        if fused:
            return bound.bind_verify_greedy_fused(g["h_target"][:h * T], g["W"], bufs["tok"][:h], bufs["out"][:h],
                                                  bufs["n"][:h], bufs["ws_g"])
        return bound.bind_verify_greedy(g["target"][:h], bufs["tok"][:h], bufs["out"][:h], bufs["n"][:h],
                                        bufs["ws_g"])

    def sample():
        if fused:
            return bound.bind_verify_sample_fused(g["h_target"][h * T:], g["W"], bufs["tok"][h:], 1.0, 7,
                                                  g["request_id"][h:], g["pos0"][h:], bufs["out"][h:],
                                                  bufs["n"][h:], bufs["ws_v"])
        return bound.bind_verify_sample(g["target"][h:], bufs["tok"][h:], 1.0, 7, g["request_id"][h:],
                                        g["pos0"][h:], bufs["out"][h:], bufs["n"][h:], bufs["ws_v"])

    for c in calls:
        c()
    if side is None:
        greedy()()
        sample()()
    else:
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            greedy()()  # bound to, and enqueued on, the side stream
        sample()()
        main.wait_stream(side)


def _snapshot(bufs):
    return {k: (v.clone() if isinstance(v, torch.Tensor) else [t.clone() for t in v])
            for k, v in bufs.items() if not k.startswith("ws")}


def _same(a, b):
    for k in a:
        if isinstance(a[k], list):
            if not all(torch.equal(x, y) for x, y in zip(a[k], b[k])):
                return False
        elif not torch.equal(a[k], b[k]):
            return False
    return True


@pytest.mark.parametrize("two_streams", [False, True])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name, overrides", [("c1_tiny", {"B": 4, "name": "c1_graph_b4"}),
                                              ("c1_tiny", {"B": 8, "D": 1024, "V": 20000, "name": "c1_graph_b8"})])
def test_graph_replays_equal_eager(dfl, dev, name, overrides, fused, two_streams):
    cfg = get_config(name, **overrides)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in make_cycle_inputs(cfg).items()}
    B, T, P, M = cfg.B, cfg.T, cfg.P, cfg.M
    u8 = torch.uint8
    bufs = {
        "y": [torch.empty_like(g["x"][l]) for l in range(cfg.L)],
        "tv": torch.empty((M, 16), dtype=torch.float32, device=dev),
        "ti": torch.empty((M, 16), dtype=torch.int32, device=dev),
        "rank": torch.empty((B, P), dtype=torch.int32, device=dev),
        "tok": torch.empty((B, P), dtype=torch.int32, device=dev),
        "score": torch.empty((B,), dtype=torch.float32, device=dev),
        "out": torch.empty((B, T), dtype=torch.int32, device=dev),
        "n": torch.empty((B,), dtype=torch.int32, device=dev),
        "ws_h": torch.empty(dfl.workspace_bytes("head_topk", M, cfg.D, cfg.V), dtype=u8, device=dev),
        "ws_s": torch.empty(dfl.workspace_bytes("select_path", B, P), dtype=u8, device=dev),
        "ws_g": torch.empty(dfl.workspace_bytes("verify_greedy_fused", B // 2, T, cfg.D, cfg.V) if fused else
                            dfl.workspace_bytes("verify_greedy", B // 2, T, cfg.V), dtype=u8, device=dev),
        "ws_v": torch.empty(dfl.workspace_bytes("verify_sample_fused", B - B // 2, T, cfg.D, cfg.V) if fused else
                            dfl.workspace_bytes("verify_sample", B - B // 2, T, cfg.V), dtype=u8, device=dev),
    }
    _cycle(dfl, g, cfg, bufs, dfl, fused)
    torch.cuda.synchronize()
    eager = _snapshot(bufs)

    side = torch.cuda.Stream() if two_streams else None  # default priority
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _cycle(dfl, g, cfg, bufs, dfl, fused, side)
    for rep in range(3):
        for v in bufs.values():  # scribble over the outputs between replays
            for t in (v if isinstance(v, list) else [v]):
                if t.dtype == torch.uint8:
                    continue
                t.fill_(-7) if t.dtype != torch.bfloat16 else t.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert _same(_snapshot(bufs), eager), f"replay {rep} differs from the eager cycle"
        _cycle(dfl, g, cfg, bufs, dfl, fused)  # eager work between replays
        torch.cuda.synchronize()
        assert _same(_snapshot(bufs), eager)
