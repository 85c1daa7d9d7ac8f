"""Seeded input synthesis for one draft-verify cycle.

Recipe (all draws standard normal unless stated; bf16 tensors are drawn in
float32 and rounded to nearest-even):

* conv inputs: x [L][B][T][D] ~ N(0, 1); a shared tap projection
  W_tap [2D][D] ~ N(0, w_sd^2); taps = x W_tap^T (the drafter's own per-token
  tap projection, 2D outputs per token: a = taps[..., :D], b = taps[..., D:]).
* LM head: W [V][D] ~ N(0, w_sd^2); draft hiddens h [B*(T-1)][D] ~ N(0, 1).
  With plant_alpha > 0 a random token c per row gets a margin:
  h += plant_alpha * W[c] / |W[c]|^2, which lifts that row's logit at c by
  about plant_alpha (the literal "draft + N(0,1) noise" recipe on random
  weights would otherwise accept almost nothing).
* selector tables: P, Q [r][D] ~ N(0, w_sd^2) (2 r D parameters);
  F_l = W P^T, F_r = W Q^T, float32 [V][r] (a once-per-weight-load table).
* target logits [B][T][V] float32:
  - "draft_plus_noise": row t < T-1 is the draft row t's logits h_t W^T plus
    N(0, noise_sd^2); row T-1 is a fresh hidden's logits plus the same noise.
  - "context_copy": every row ~ N(0, 2.048 + 1); for exactly
    round(agree_frac * B * (T-1)) seeded (request, slot) pairs the planted
    draft token is raised to the row maximum + 1, and on the others it is
    pushed 1 below the best other token when it happened to be the argmax.
* target hidden states h_target [B*T][D] bf16, the same block in hidden
  space (for greedy verification fused into the shared LM head):
  - "draft_plus_noise": row t < T-1 is draft hidden t plus N(0, s^2) with
    s = noise_sd / (w_sd sqrt(D)), so that its logits carry noise of about
    noise_sd; row T-1 is the fresh hidden plus the same noise;
  - "context_copy": rows ~ N(0, 1) planted (plant_alpha) toward the draft's
    planted token on the agreeing (request, slot) pairs and toward another
    random token on the others; row T-1 ~ N(0, 1).
* request ids 0..B-1 (uint64 semantics), anchor positions 4096 + 64 b.

Every tensor has its own generator, seeded from (seed, config name, tensor
name); large tensors are drawn in fixed 16384-row chunks so the stream does not
depend on memory limits.  The same device gives the same values.
"""

import zlib

import numpy as np
import torch

CHUNK = 16384


def make_generator(device, seed, *names):
    words = [int(seed)] + [zlib.crc32(str(n).encode()) for n in names]
    s = int(np.random.SeedSequence(words).generate_state(1, np.uint64)[0]) & ((1 << 63) - 1)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _randn(shape, g, device, sd=1.0):
    """float32 N(0, sd^2), drawn in CHUNK-row pieces along dim 0."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    for r0 in range(0, shape[0], CHUNK):
        r1 = min(shape[0], r0 + CHUNK)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                                 device=device, dtype=torch.float32)
    if sd != 1.0:
        out.mul_(sd)
    return out


def _rows_times_wt(rows_f32, W_bf16):
    """rows [R][D] float32 times W^T -> [R][V] float32, chunked over V."""
    V = W_bf16.shape[0]
    out = torch.empty((rows_f32.shape[0], V), dtype=torch.float32, device=rows_f32.device)
    for v0 in range(0, V, CHUNK):
        out[:, v0:v0 + CHUNK] = rows_f32 @ W_bf16[v0:v0 + CHUNK].float().T
    return out


def make_cycle_inputs(cfg, device="cpu"):
    dev = torch.device(device)
    seed, nm = cfg.seed, cfg.name
    B, T, D, V, r, L = cfg.B, cfg.T, cfg.D, cfg.V, cfg.r, cfg.L
    P, M = cfg.P, cfg.M

    def gen(tensor):
        return make_generator(dev, seed, nm, tensor)

    # conv: inputs and the drafter's tap projection
    x = _randn((L * B * T, D), gen("x"), dev).to(torch.bfloat16)
    w_tap = _randn((2 * D, D), gen("w_tap"), dev, cfg.w_sd).to(torch.bfloat16)
    taps = torch.empty((L * B * T, 2 * D), dtype=torch.bfloat16, device=dev)
    for r0 in range(0, L * B * T, CHUNK):
        taps[r0:r0 + CHUNK] = (x[r0:r0 + CHUNK].float() @ w_tap.float().T).to(torch.bfloat16)
    x = x.view(L, B, T, D)
    taps = taps.view(L, B, T, 2 * D)

    # head weights and draft hiddens (with a planted margin)
    W = _randn((V, D), gen("W"), dev, cfg.w_sd).to(torch.bfloat16)
    h32 = _randn((M, D), gen("h"), dev)
    planted = torch.randint(0, V, (M,), generator=gen("planted"), device=dev, dtype=torch.int64)
    if cfg.plant_alpha > 0:
        wc = W[planted].float()
        h32 += cfg.plant_alpha * wc / (wc * wc).sum(dim=1, keepdim=True)
    h = h32.to(torch.bfloat16)

    # selector tables from the low-rank factors
    Psel = _randn((r, D), gen("P_sel"), dev, cfg.w_sd)
    Qsel = _randn((r, D), gen("Q_sel"), dev, cfg.w_sd)
    F_l = torch.empty((V, r), dtype=torch.float32, device=dev)
    F_r = torch.empty((V, r), dtype=torch.float32, device=dev)
    for v0 in range(0, V, CHUNK):
        wf = W[v0:v0 + CHUNK].float()
        F_l[v0:v0 + CHUNK] = wf @ Psel.T
        F_r[v0:v0 + CHUNK] = wf @ Qsel.T

    # target block logits
    target = torch.empty((B, T, V), dtype=torch.float32, device=dev)
    if cfg.logits == "draft_plus_noise":
        hb = h.float().view(B, P, D)
        fresh = _randn((B, D), gen("h_bonus"), dev)
        noise = gen("target_noise")
        for b in range(B):
            rows = torch.cat([hb[b], fresh[b:b + 1]], dim=0)  # [T][D]
            target[b] = _rows_times_wt(rows, W)
            target[b] += _randn((T, V), noise, dev, cfg.noise_sd)
        sd_h = cfg.noise_sd / (cfg.w_sd * float(np.sqrt(D)))
        ht_rows = hb + _randn((B, P, D), gen("h_target_noise"), dev, sd_h)
        ht_bonus = fresh + _randn((B, D), gen("h_target_bonus"), dev, sd_h)
    elif cfg.logits == "context_copy":
        sd = float(np.sqrt(cfg.w_sd ** 2 * D + 1.0))
        g = gen("target")
        for b in range(B):
            target[b] = _randn((T, V), g, dev, sd)
        n_agree = int(round(cfg.agree_frac * B * P))
        perm = torch.randperm(B * P, generator=make_generator("cpu", seed, nm, "agree"))
        agree = torch.zeros(B * P, dtype=torch.bool)
        agree[perm[:n_agree]] = True
        pl = planted.to("cpu").tolist()
        for m in range(B * P):
            b, t = divmod(m, P)
            row = target[b, t]
            c = pl[m]
            if agree[m]:
                row[c] = row.max() + 1.0
            elif int(torch.argmax(row)) == c:
                row[c] = -float("inf")
                row[c] = row.max() - 1.0
        ht_rows = _randn((B * P, D), gen("h_target"), dev)
        alt = torch.randint(0, V, (B * P,), generator=gen("h_target_alt"), device=dev, dtype=torch.int64)
        toward = torch.where(agree.to(dev), planted, alt)
        wt = W[toward].float()
        ht_rows = (ht_rows + cfg.plant_alpha * wt / (wt * wt).sum(dim=1, keepdim=True)).view(B, P, D)
        ht_bonus = _randn((B, D), gen("h_target_bonus"), dev)
    else:
        raise ValueError(cfg.logits)

    # the blocks' slot-0 tokens (the last verified token of each request), for
    # the anchored selector
    anchor = torch.randint(0, V, (B,), generator=gen("anchor"), device=dev, dtype=torch.int64).to(torch.int32)
    request_id = torch.arange(B, dtype=torch.int64, device=dev)
    pos0 = 4096 + 64 * torch.arange(B, dtype=torch.int64, device=dev)
    h_target = torch.cat([ht_rows, ht_bonus.view(B, 1, D)], dim=1).reshape(B * T, D).to(torch.bfloat16)
    return {
        "x": x, "taps": taps, "w_tap": w_tap, "h": h, "W": W, "F_l": F_l, "F_r": F_r,
        "target": target, "h_target": h_target, "request_id": request_id, "pos0": pos0, "anchor": anchor,
        "planted": planted, "temperature": float(cfg.temperature),
        "seed": int(cfg.seed),
    }
