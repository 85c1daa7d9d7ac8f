#!/usr/bin/env python3
"""Draft-verify cycles/s of the DFlash 2 cycle tail on one MI355X.

One step = one cycle tail over one batch of synthetic inputs resident in HBM:
the two-tap conv over the five drafter layers' hidden states (one call: the
layers' sequences are contiguous), the LM head with top-16, the pair
selector, and verification (greedy, sampled, or half of each), each a C-ABI
call on one stream.  Inputs rotate over enough copies to exceed the
256 MB Infinity Cache, so every step streams its inputs from HBM.  The cycles
are timed twice: launched eagerly (with per-stage events) and replayed from
one captured HIP graph per input set (the reported value; the replayed outputs
are checked to equal the eager ones).

By default the headline is the batch-32 workload (c4_b32); batch 1 (c2_b1)
and batch 8 (c3_b8) follow as sub-records of the same line, each with its own
roofline, oracle timing and parity.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "head_topk_traffic.json")
# the head kernels' sources: the kernel file and the key-sort header it includes
HEAD_SRC = [os.path.join(ROOT, "block_draft_verification_amd", "csrc", f) for f in ("head_topk.hip", "keysort.hpp")]
WORKLOAD_TEXT = {
    "c1_tiny": "batch 1, block 8, hidden 256, vocab 4096, top-16, selector rank 32, greedy",
    "c2_b1": "batch 1, block 8, hidden 5120, vocab 151936, top-16, selector rank 192, greedy",
    "c3_b8": "batch 8, block 8, hidden 5120, vocab 151936, top-16, rank 192, rejection sampling tau=1",
    "c4_b32": "batch 32, block 8, hidden 5120, vocab 151936, top-16, rank 192, half greedy / half sampled",
    "c5_stress": "batch 32, block 16, hidden 5120, vocab 262144, top-16, rank 192, greedy, context copy",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="c4_b32", choices=sorted(WORKLOAD_TEXT),
                    help="the headline workload (default c4_b32: batch 32)")
    ap.add_argument("--sub-configs", default=None,
                    help="comma-separated workloads measured after the headline and reported in its "
                         "'sub_records' key (default: c2_b1,c3_b8 with the default headline, none otherwise; "
                         "'none' for none)")
    ap.add_argument("--sub-steps", type=int, default=200, help="timed steps of each sub-record")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="bound on the oracle's timed CPU work")
    ap.add_argument("--max-sets", type=int, default=64)
    ap.add_argument("--sample-top-k", type=int, default=0,
                    help="sampled requests: filter the target to its top-k, then top-p (0 = full softmax)")
    ap.add_argument("--sample-top-p", type=float, default=1.0)
    ap.add_argument("--anchored", action="store_true",
                    help="selector anchored on each block's slot-0 token")
    ap.add_argument("--sampled-path", action="store_true",
                    help="sampled requests draw their path from the lattice's chain distribution and are "
                         "verified against the proposals that drew it")
    ap.add_argument("--fused-target-head", action="store_true",
                    help="requests are verified from the target's hidden states through the shared LM head "
                         "(argmax or softmax statistics in the GEMM epilogue, no target logits)")
    ap.add_argument("--fused-tap-proj", action="store_true",
                    help="the conv call projects its taps from the hidden states itself "
                         "(dflash_conv2tap_proj: the tap GEMM with the conv in its epilogue)")
    ap.add_argument("--copy-probe", type=float, default=None, metavar="GIB",
                    help="only copy a GIB-sized device buffer 3 times (calibrates rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE against known bytes) and exit")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="only time, at each workload's head shape, the vendor GEMM of the logits "
                         "(torch.mm, bf16 inputs, bf16 and fp32 outputs, no top-k) and a torch.topk "
                         "over its fp32 logits, beside dflash_head_topk (GEMM and top-16), and exit")
    return ap.parse_args()


def copy_probe(gib):
    import torch
    n = int(gib * (1 << 30))
    a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy probe: 3 copies of {n} bytes")


def gemm_probe():
    """The head's GEMM at each workload's shape through the vendor library
    (torch.mm on ROCm: hipBLASLt), which materialises the logits and keeps no
    top-k, timed beside dflash_head_topk on the same operands: a reference for
    what the bf16 GEMM of this shape reaches on the chip."""
    import torch
    import block_draft_verification_amd as dfl
    from workload.configs import get_config
    dev = torch.device("cuda:0")

    def timed(fn, reps=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / reps

    W_by_v = {}
    for name in ("c2_b1", "c3_b8", "c4_b32", "c5_stress"):
        cfg = get_config(name)
        M, V, D = cfg.M, cfg.V, cfg.D
        if V not in W_by_v:
            W_by_v.clear()
            g = torch.Generator(device=dev).manual_seed(1)
            W_by_v[V] = (0.02 * torch.randn(V, D, device=dev, generator=g)).to(torch.bfloat16)
        W = W_by_v[V]
        g = torch.Generator(device=dev).manual_seed(2)
        h = torch.randn(M, D, device=dev, generator=g).to(torch.bfloat16)
        flops = 2.0 * M * V * D
        rec = {"probe": "head GEMM", "workload": name, "M": M, "V": V, "D": D,
               "torch_mm_bf16_out_us": round(timed(lambda: torch.mm(h, W.t())), 1),
               "torch_mm_fp32_out_us": round(timed(lambda: torch.mm(h, W.t(), out_dtype=torch.float32)), 1),
               "dflash_head_topk_us": round(timed(lambda: dfl.head_topk(h, W)), 1)}
        z = torch.mm(h, W.t(), out_dtype=torch.float32)
        rec["torch_topk16_of_fp32_logits_us"] = round(timed(lambda: torch.topk(z, 16, dim=1)), 1)
        del z
        for k in ("torch_mm_bf16_out_us", "torch_mm_fp32_out_us", "dflash_head_topk_us"):
            rec[k.replace("_us", "_tflops")] = round(flops / rec[k] / 1e6, 1)
        print(json.dumps(rec), flush=True)


class CycleRunner:
    """Pre-bound C-ABI calls for every rotating input set."""

    def __init__(self, dfl, torch, cfg, sets, W, F_l, F_r, w_tap=None):
        self.dfl = dfl
        dev = W.device
        B, T, P, L = cfg.B, cfg.T, cfg.P, cfg.L
        self.cfg = cfg
        self.torch = torch
        # the L drafter layers' sequences are contiguous ([L][B][T][D]), so one
        # conv call covers all of them (S = L * B sequences)
        self.y_all = torch.empty_like(sets[0]["x"])
        self.y = [self.y_all[l] for l in range(L)]
        self.tv = torch.empty((cfg.M, 16), dtype=torch.float32, device=dev)
        self.ti = torch.empty((cfg.M, 16), dtype=torch.int32, device=dev)
        self.rank = torch.empty((B, P), dtype=torch.int32, device=dev)
        self.tok = torch.empty((B, P), dtype=torch.int32, device=dev)
        self.score = torch.empty((B,), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, T), dtype=torch.int32, device=dev)
        self.n = torch.empty((B,), dtype=torch.int32, device=dev)
        g = {"greedy": B, "sample": 0, "mixed": B // 2}[cfg.verify]
        self.g = g
        u8 = torch.uint8
        self.ws_head = torch.empty(dfl.workspace_bytes("head_topk", cfg.M, cfg.D, cfg.V), dtype=u8, device=dev)
        self.ws_sel = torch.empty(dfl.workspace_bytes("select_path_anchored" if cfg.anchored else "select_path", B, P),
                                  dtype=u8, device=dev)
        if cfg.sampled_path:  # the sampled requests' selector and their proposals
            self.ws_sel_s = torch.empty(dfl.workspace_bytes("select_path_sampled", max(B - g, 1), P, cfg.anchored),
                                        dtype=u8, device=dev)
            self.q = torch.empty((max(B - g, 1), P, 16), dtype=torch.float64, device=dev)
        if cfg.fused_target_head:
            self.ws_g = torch.empty(dfl.workspace_bytes("verify_greedy_fused", max(g, 1), T, cfg.D, cfg.V), dtype=u8,
                                    device=dev)
        else:
            self.ws_g = torch.empty(dfl.workspace_bytes("verify_greedy", max(g, 1), T, cfg.V), dtype=u8,
                                    device=dev)
        if cfg.fused_target_head:
            self.ws_s = torch.empty(dfl.workspace_bytes("verify_sample_fused", max(B - g, 1), T, cfg.D, cfg.V),
                                    dtype=u8, device=dev)
        elif cfg.top_k > 0:
            self.ws_s = torch.empty(dfl.workspace_bytes("verify_sample_topkp", max(B - g, 1), T, cfg.V, cfg.top_k),
                                    dtype=u8, device=dev)
        else:
            self.ws_s = torch.empty(dfl.workspace_bytes("verify_sample", max(B - g, 1), T, cfg.V), dtype=u8,
                                    device=dev)
        self.F_l, self.F_r, self.W, self.w_tap = F_l, F_r, W, w_tap
        self.sets = sets
        self.calls = [self.bind_set(s) for s in sets]

    def bind_set(self, s):
        """The cycle's C-ABI calls on input set s, bound to the current stream."""
        dfl, cfg, B, L, g = self.dfl, self.cfg, self.cfg.B, self.cfg.L, self.g
        tv3, ti3 = self.tv.view(B, cfg.P, 16), self.ti.view(B, cfg.P, 16)
        if cfg.fused_tap_proj:
            conv = [dfl.bind_conv2tap_proj(s["x"], self.w_tap, self.y_all)]
        else:
            conv = [dfl.bind_conv2tap(s["x"], s["taps"], self.y_all)]
        head = dfl.bind_head_topk(s["h"], self.W, self.tv, self.ti, self.ws_head)
        anchor = s["anchor"] if cfg.anchored else None
        if cfg.sampled_path and g < B:
            sel = []
            if g > 0:
                sel.append(dfl.bind_select_path(tv3[:g], ti3[:g], self.F_l, self.F_r, self.rank[:g], self.tok[:g],
                                                self.score[:g], self.ws_sel,
                                                anchor=None if anchor is None else anchor[:g]))
            sel.append(dfl.bind_select_path_sampled(tv3[g:], ti3[g:], self.F_l, self.F_r, cfg.seed, s["rid_s"],
                                                    s["pos_s"], self.rank[g:], self.tok[g:], self.q, self.ws_sel_s,
                                                    anchor=None if anchor is None else anchor[g:]))
        else:
            sel = [dfl.bind_select_path(tv3, ti3, self.F_l, self.F_r, self.rank, self.tok, self.score, self.ws_sel,
                                        anchor=anchor)]
        ver = []
        if g > 0 and cfg.fused_target_head:
            ver.append(dfl.bind_verify_greedy_fused(s["h_target_g"], self.W, self.tok[:g], self.out[:g], self.n[:g],
                                                    self.ws_g))
        elif g > 0:
            ver.append(dfl.bind_verify_greedy(s["target_g"], self.tok[:g], self.out[:g], self.n[:g], self.ws_g))
        if g < B:
            if cfg.fused_target_head:
                ver.append(dfl.bind_verify_sample_fused(s["h_target_s"], self.W, self.tok[g:], cfg.temperature,
                                                        cfg.seed, s["rid_s"], s["pos_s"], self.out[g:], self.n[g:],
                                                        self.ws_s))
            elif cfg.sampled_path:
                ver.append(dfl.bind_verify_sample_q(s["target_s"], self.tok[g:], ti3[g:], self.q, cfg.temperature,
                                                    cfg.seed, s["rid_s"], s["pos_s"], self.out[g:], self.n[g:],
                                                    self.ws_s))
            elif cfg.top_k > 0:
                ver.append(dfl.bind_verify_sample_topkp(s["target_s"], self.tok[g:], cfg.temperature, cfg.top_k,
                                                        cfg.top_p, cfg.seed, s["rid_s"], s["pos_s"], self.out[g:],
                                                        self.n[g:], self.ws_s))
            else:
                ver.append(dfl.bind_verify_sample(s["target_s"], self.tok[g:], cfg.temperature, cfg.seed,
                                                  s["rid_s"], s["pos_s"], self.out[g:], self.n[g:], self.ws_s))
        return conv, head, sel, ver

    def capture(self):
        """One HIP graph per input set holding that set's whole cycle.  In a
        batch that mixes greedy and sampled requests, the two verifications
        read and write disjoint requests, outputs and workspaces, so the graph
        runs them side by side on two streams (both at the default priority),
        joined before the graph ends."""
        torch = self.torch
        side = torch.cuda.Stream()
        graphs = []
        for s in self.sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                main = torch.cuda.current_stream()
                conv, head, sel, ver = self.bind_set(s)
                for c in conv:
                    c()
                head()
                for c in sel:
                    c()
                if len(ver) == 2:
                    side.wait_stream(main)
                    with torch.cuda.stream(side):
                        greedy_on_side = self.bind_set(s)[3][0]  # bound to the side stream
                        greedy_on_side()
                    ver[1]()
                    main.wait_stream(side)
                else:
                    for v in ver:
                        v()
            graphs.append(g)
        return graphs

    def outputs(self):
        return {"y": [y.cpu() for y in self.y], "ti": self.ti.cpu().numpy(), "tv": self.tv.cpu().numpy(),
                "tok": self.tok.cpu().numpy(), "out": self.out.cpu().numpy(), "n": self.n.cpu().numpy()}

    def run(self, i, ev=None):
        conv, head, sel, ver = self.calls[i % len(self.calls)]
        if ev is not None:
            ev[0].record()
        for c in conv:
            c()
        if ev is not None:
            ev[1].record()
        head()
        if ev is not None:
            ev[2].record()
        for c in sel:
            c()
        if ev is not None:
            ev[3].record()
        for v in ver:
            v()
        if ev is not None:
            ev[4].record()


def make_sets(torch, cfg, inp, max_sets):
    B, g = cfg.B, {"greedy": cfg.B, "sample": 0, "mixed": cfg.B // 2}[cfg.verify]
    fused = cfg.fused_target_head
    base = {
        "x": inp["x"], "taps": None if cfg.fused_tap_proj else inp["taps"], "h": inp["h"], "anchor": inp["anchor"],
        "target_g": inp["target"][:g].contiguous() if g > 0 and not fused else None,
        "h_target_g": inp["h_target"][:g * cfg.T].contiguous() if g > 0 and fused else None,
        "target_s": inp["target"][g:].contiguous() if g < B and not fused else None,
        "h_target_s": inp["h_target"][g * cfg.T:].contiguous() if g < B and fused else None,
        "rid_s": inp["request_id"][g:].contiguous(), "pos_s": inp["pos0"][g:].contiguous(),
    }
    per_set = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    n_sets = max(2, min(max_sets, math.ceil(512e6 / per_set)))
    sets = [base]
    for _ in range(n_sets - 1):
        sets.append({k: (v.clone() if v is not None else None) for k, v in base.items()})
    return sets, per_set


def head_kernels(cfg):
    if cfg.M <= 16:
        gemm = "head_skinny2_kernel"
    elif cfg.M <= 64:
        gemm = "head_wide_kernel"
    else:
        gemm = "head_mfma_kernel"
    return f"dflash_head_topk call = {gemm} + head_merge_kernel (HIP events around the call)"


def head_roofline(cfg, head_us):
    flops = 2.0 * cfg.M * cfg.V * cfg.D
    bytes_ = cfg.V * cfg.D * 2 + cfg.M * cfg.D * 2 + cfg.M * 16 * 8
    ai = flops / bytes_
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    t = head_us * 1e-6
    traffic = stored_traffic(cfg)
    # batched heads (M > 64 rows: the MFMA kernel) are reported against the
    # bf16 MFMA peak, with the byte-side fraction beside it
    if ai < ridge and cfg.M <= 64:
        ach = bytes_ / t / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": head_kernels(cfg), "algorithmic_bytes": int(bytes_), "flops": int(flops),
                "mfma_frac": round(flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    ach = flops / t / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
            "kernel": head_kernels(cfg), "algorithmic_bytes": int(bytes_), "flops": int(flops),
            "hbm_frac": round(bytes_ / t / 1e9 / HBM_PEAK_GBS, 4)}


def cycle_roofline(cfg, ms_cycle):
    fl = cycle_floor(cfg)
    floor_us = sum(fl.values())
    return {"floor_us": round(floor_us, 2), "measured_us": round(ms_cycle * 1e3, 2),
            "frac": round(floor_us / (ms_cycle * 1e3), 4), "floor_us_by_step": {k: round(v, 2) for k, v in fl.items()},
            "note": "sum of the steps' roofline floors (HBM 8 TB/s; the head at max(bytes, bf16 MFMA 2.5 PFLOP/s)) "
                    "over the measured cycle"}


def cycle_floor(cfg):
    """Roofline floor of one cycle: every step's algorithmic bytes at the HBM
    peak, the head at the larger of its byte and MFMA times.  conv: x, both
    taps and y per token; head: W once, h, the lists; selector: the table rows
    it gathers; verify: the target logits once."""
    hbm = HBM_PEAK_GBS * 1e9
    conv = 8.0 * cfg.L * cfg.B * cfg.T * cfg.D / hbm
    if cfg.fused_tap_proj:  # x and y per token plus W_tap once, or the projection's MFMA time
        conv = max((4.0 * cfg.L * cfg.B * cfg.T * cfg.D + 4.0 * cfg.D * cfg.D) / hbm,
                   4.0 * cfg.L * cfg.B * cfg.T * cfg.D * cfg.D / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    head_bytes = cfg.V * cfg.D * 2 + cfg.M * cfg.D * 2 + cfg.M * 16 * 8
    head = max(head_bytes / hbm, 2.0 * cfg.M * cfg.V * cfg.D / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    sel = cfg.B * max(cfg.P - 1, 0) * 2 * 16 * cfg.r * 4 / hbm
    g = {"greedy": cfg.B, "sample": 0, "mixed": cfg.B // 2}[cfg.verify]
    if cfg.fused_target_head:  # the target head over the block's rows instead of their logits
        ver = 0.0
        for mt in (g * cfg.T, (cfg.B - g) * cfg.T):  # one head call per verification kind
            if mt > 0:
                ver += max((cfg.V * cfg.D * 2 + mt * cfg.D * 2) / hbm,
                           2.0 * mt * cfg.V * cfg.D / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    else:
        ver = 4.0 * cfg.B * cfg.T * cfg.V / hbm
    return {"conv": conv * 1e6, "head_topk": head * 1e6, "select_path": sel * 1e6, "verify": ver * 1e6}


def head_source_sha():
    h = hashlib.sha256()
    for path in HEAD_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(cfg):
    """HBM bytes per head launch from committed rocprofv3 --pmc counters, if
    they were taken on the current head kernel source and this workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(cfg.name)
    if not entry or entry.get("head_source_sha") != head_source_sha():
        return None
    return entry.get("bytes_per_launch")


def conv_proj_parity(torch, cfg, host, gpu_res, n_seq=8):
    """The fused conv's outputs on n_seq sampled sequences of every layer
    against the oracle's exact result: identical except on a bf16 rounding
    boundary (the exact value within 1e-3 of its magnitude scale of the
    midpoint of the two results), and such flips under 2 %."""
    import numpy as np
    from oracle.conv import conv2tap_proj
    rng = np.random.default_rng(0)
    flips = total = 0
    for l in range(cfg.L):
        seqs = rng.choice(cfg.B, min(n_seq, cfg.B), replace=False)
        y_ref, y64, scale = conv2tap_proj(host["x"][l][seqs], host["w_tap"], return_exact=True)
        g = gpu_res["y"][l][seqs].float().numpy().astype(np.float64)
        r = y_ref.float().numpy().astype(np.float64)
        diff = g != r
        if np.any(diff & (np.abs(y64 - 0.5 * (g + r)) > 1e-3 * scale)):
            return False
        flips += int(diff.sum())
        total += diff.size
    return flips <= 0.02 * total


def conv_proj_roofline(cfg, conv_us):
    """The fused tap projection + conv against its roofline (HIP events around
    the conv call): bf16 MFMA peak above the ridge, else HBM (W_tap once, x
    read and y written)."""
    rows = cfg.L * cfg.B * cfg.T
    flops = 2.0 * rows * 2 * cfg.D * cfg.D
    bytes_ = 4.0 * cfg.D * cfg.D + 4.0 * rows * cfg.D
    t = conv_us * 1e-6
    out = {"kernel": "conv_proj_kernel (dflash_conv2tap_proj)", "flops": int(flops),
           "algorithmic_bytes": int(bytes_), "conv_us": round(conv_us, 2)}
    if flops / bytes_ < MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        ach = bytes_ / t / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), **out}
    ach = flops / t / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), **out}


def cpu_baseline(torch, cfg, inp, gpu_res, seconds):
    """The oracle, as it stands, on the host's cores, on this run's inputs."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle.cycle import run_cycle

    host = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    t0 = time.perf_counter()
    ref = run_cycle(host, cfg.B, cfg.T, verify=cfg.verify, top_k=cfg.top_k, top_p=cfg.top_p, anchored=cfg.anchored,
              sampled_path=cfg.sampled_path, fused_target_head=cfg.fused_target_head,
              fused_tap_proj=cfg.fused_tap_proj)
    t1 = time.perf_counter() - t0
    n, total = 1, t1
    while total + t1 <= seconds and n < 200:
        t0 = time.perf_counter()
        run_cycle(host, cfg.B, cfg.T, verify=cfg.verify, top_k=cfg.top_k, top_p=cfg.top_p, anchored=cfg.anchored,
              sampled_path=cfg.sampled_path, fused_target_head=cfg.fused_target_head,
              fused_tap_proj=cfg.fused_tap_proj)
        total += time.perf_counter() - t0
        n += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    if cfg.fused_tap_proj:
        conv_ok = conv_proj_parity(torch, cfg, host, gpu_res)
    else:
        conv_ok = all(torch.equal(gpu_res["y"][l].view(torch.int16), ref["y"][l].view(torch.int16))
                      for l in range(cfg.L))
    parity = {
        "conv_bits" if not cfg.fused_tap_proj else "conv_admissible": conv_ok,
        "top_idx": bool(np.array_equal(gpu_res["ti"], ref["top_idx"].reshape(-1, 16))),
        "path_tok": bool(np.array_equal(gpu_res["tok"], ref["path_tok"])),
        "out_tok": bool(np.array_equal(gpu_res["out"], ref["out_tok"])),
        "n_emit": bool(np.array_equal(gpu_res["n"], ref["n_emit"])),
    }
    return {"value": round(n / total, 4), "unit": "cycles/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} full {cfg.name} cycle(s) of the float64 numpy oracle on the inputs of "
                      f"set 0 ({total:.1f} s)",
            "host_cpus": len(os.sched_getaffinity(0))}, parity


def main():
    args = parse()
    if args.copy_probe is not None:
        copy_probe(args.copy_probe)
        return
    if args.gemm_probe:
        gemm_probe()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_draft_verification_amd as dfl

    dfl.lib()
    subs = args.sub_configs
    if subs is None:
        subs = "c2_b1,c3_b8" if args.config == "c4_b32" and not variant_flags(args) else "none"
    subs = [] if subs == "none" else [c for c in subs.split(",") if c]
    for c in subs:
        if c not in WORKLOAD_TEXT:
            sys.exit(f"unknown sub-config {c}")
    rec = run_config(args, torch, dfl, args.config, args.steps, args.cpu_seconds)
    if subs:
        rec["sub_records"] = {}
        for c in subs:
            torch.cuda.empty_cache()
            sub = run_config(args, torch, dfl, c, args.sub_steps, min(args.cpu_seconds, 10.0))
            rec["sub_records"][c] = {k: sub[k] for k in ("value", "unit", "ms_per_step", "steps", "config",
                                                         "roofline", "cycle_roofline", "stages_us",
                                                         "eager_cycles_per_s", "mean_n_emit", "cpu_baseline")
                                     if k in sub}
            if "parity_vs_oracle" in sub:
                rec["sub_records"][c]["parity_vs_oracle"] = sub["parity_vs_oracle"]
    print(json.dumps(rec), flush=True)


def variant_flags(args):
    return (args.sample_top_k > 0 or args.anchored or args.sampled_path or args.fused_target_head
            or args.fused_tap_proj)


def run_config(args, torch, dfl, name, steps, cpu_seconds):
    """Measure one workload; returns its JSON record."""
    import numpy as np
    from workload import get_config, make_cycle_inputs

    dev = torch.device("cuda:0")
    cfg = get_config(name, top_k=args.sample_top_k, top_p=args.sample_top_p, anchored=args.anchored,
                     sampled_path=args.sampled_path, fused_target_head=args.fused_target_head,
                     fused_tap_proj=args.fused_tap_proj)
    if cfg.fused_target_head and (cfg.sampled_path or cfg.top_k > 0):
        print("--fused-target-head verifies against the unfiltered target with the max-sum path", file=sys.stderr)
        sys.exit(2)
    if cfg.sampled_path and (cfg.top_k > 0 or cfg.verify == "greedy"):
        print("--sampled-path needs sampled verification without a top-k / top-p filter", file=sys.stderr)
        sys.exit(2)
    log(f"[bench] config {cfg.name}: generating inputs on {dev}")
    inp = make_cycle_inputs(cfg, device=dev)
    sets, per_set = make_sets(torch, cfg, inp, args.max_sets)
    log(f"[bench] {len(sets)} rotating input sets of {per_set / 1e6:.1f} MB")
    runner = CycleRunner(dfl, torch, cfg, sets, inp["W"], inp["F_l"], inp["F_r"], inp["w_tap"])

    # warmup (untimed)
    for i in range(args.warmup):
        runner.run(i)
    torch.cuda.synchronize()

    # per-stage events on the stream the kernels run on
    stream = torch.cuda.current_stream(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        runner.run(i, evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / steps
    stage = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(4)] for e in evs]) * 1e3  # us
    cycle_us = np.array([e[0].elapsed_time(e[4]) for e in evs]) * 1e3
    head_us = float(stage[:, 1].mean())
    log(f"[bench] {steps} cycles in {ms_total:.2f} ms (wall {wall * 1e3:.1f} ms): "
        f"{ms_per_step * 1e3:.1f} us/cycle; head {head_us:.1f} us")

    # outputs of one eager cycle on set 0, for the parity check
    runner.run(0)
    torch.cuda.synchronize()
    gpu_res = runner.outputs()

    # the same cycles replayed from HIP graphs (one graph per input set)
    graphs = runner.capture()
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    g_start = torch.cuda.Event(enable_timing=True)
    g_end = torch.cuda.Event(enable_timing=True)
    g_start.record(stream)
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    g_end.record(stream)
    torch.cuda.synchronize()
    ms_graph = g_start.elapsed_time(g_end) / steps
    graphs[0].replay()
    torch.cuda.synchronize()
    g_res = runner.outputs()
    graph_same = (all(torch.equal(a, b) for a, b in zip(g_res["y"], gpu_res["y"])) and
                  all(np.array_equal(g_res[k], gpu_res[k]) for k in ("ti", "tv", "tok", "out", "n")))
    log(f"[bench] graph replay: {ms_graph * 1e3:.1f} us/cycle (eager {ms_per_step * 1e3:.1f}); "
        f"outputs identical to eager: {graph_same}")
    if not graph_same:
        sys.exit("graph replay outputs differ from the eager cycle")

    rec = {
        "metric": "draft-verify cycles/sec at block 8, batch 1/8/32; % of HBM/MFMA roofline",
        "value": round(1e3 / ms_graph, 2),
        "unit": "cycles/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_graph, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {WORKLOAD_TEXT[cfg.name]}", "batch": cfg.B, "block": cfg.T,
                   "hidden": cfg.D, "vocab": cfg.V, "top_k": 16, "selector_rank": cfg.r,
                   "conv_layers": cfg.L, "verify": cfg.verify, "rotating_input_sets": len(sets),
                   **({"sample_filter": {"top_k": cfg.top_k, "top_p": cfg.top_p}} if cfg.top_k > 0 else {}),
                   **({"selector": "anchored on slot 0"} if cfg.anchored else {}),
                   **({"draft_path": "sampled from the lattice (proposal q verified)"} if cfg.sampled_path else {}),
                   **({"target": "hidden states through the shared LM head (argmax or softmax statistics in "
                                 "the GEMM epilogue, no target logits)"} if cfg.fused_target_head else {}),
                   **({"conv_taps": "projected from x in the conv call (5120 -> 10240 GEMM, conv in its "
                                    "epilogue, taps never written)"} if cfg.fused_tap_proj else {})},
        "roofline": head_roofline(cfg, head_us),
        "cycle_roofline": cycle_roofline(cfg, ms_graph),
        **({"conv_roofline": conv_proj_roofline(cfg, float(stage[:, 0].mean()))} if cfg.fused_tap_proj else {}),
        "stages_us": {"conv": round(float(np.median(stage[:, 0])), 2),
                      "head_topk": round(float(np.median(stage[:, 1])), 2),
                      "select_path": round(float(np.median(stage[:, 2])), 2),
                      "verify": round(float(np.median(stage[:, 3])), 2)},
        "launch": "one HIP graph per input set, replayed (eager launches measured as well); "
                  "greedy and sampled requests of one batch verify on two streams inside the graph",
        "eager_cycles_per_s": round(1e3 / ms_per_step, 2),
        "eager_cycle_us_p10_p50_p90": [round(float(np.percentile(cycle_us, q)), 2) for q in (10, 50, 90)],
        "mean_n_emit": round(float(gpu_res["n"].mean()), 3),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on the same inputs")
        cb, parity = cpu_baseline(torch, cfg, inp, gpu_res, cpu_seconds)
        rec["cpu_baseline"] = cb
        rec["parity_vs_oracle"] = parity
        log(f"[bench] oracle {cb['value']} cycles/s on {cb['cores']} threads; parity {parity}")
    else:
        rec["cpu_baseline"] = None
    return rec


if __name__ == "__main__":
    main()
