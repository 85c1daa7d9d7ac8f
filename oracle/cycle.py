"""One whole draft-verify cycle tail in the oracle, step after step.

Order of a cycle (tamsi.dev "DFlash 2 — 3× plus de tokens…", § "L'idée, sans
le papier"; latenode.com "DFlash 2: un drafter de 3.43×…", opening section):
the drafter's convs (one call per drafter layer), the draft LM head with the
top-16 lists, the pair selector's path, then verification of that path against
the target's block logits.  "mixed" verification sends the first half of the
requests to the greedy rule and the second half to rejection sampling;
with top_k > 0 the sampled requests are verified against the top-k, then
top-p filtered target (latenode.com, FAQ: the published figures sample with
top-p 0.95 and top-k 20); with anchored=True the selector starts from each
block's slot-0 token; with sampled_path=True (a reading beyond the pages) the
sampled requests draw their path from the lattice's chain distribution and are
verified against the proposals that drew it; with fused_target_head=True
every request is verified from the target's hidden states through the shared
LM head; with fused_tap_proj=True the convs take their taps from the drafter's
tap projection of x (inp["w_tap"]), unrounded, instead of the given bf16 taps.
"""

import numpy as np

from .conv import conv2tap, conv2tap_proj
from .head import head_topk
from .selector import select_path, select_path_sampled
from .verify import (verify_greedy, verify_greedy_hidden, verify_sample, verify_sample_hidden, verify_sample_q,
                     verify_sample_topkp)


def run_cycle(inp, B, T, K=16, verify="greedy", head_chunk=8192, top_k=0, top_p=1.0, anchored=False,
              sampled_path=False, fused_target_head=False, fused_tap_proj=False):
    L = inp["x"].shape[0]
    if fused_tap_proj:
        ys = [conv2tap_proj(inp["x"][l], inp["w_tap"]) for l in range(L)]
    else:
        ys = [conv2tap(inp["x"][l], inp["taps"][l]) for l in range(L)]
    vals, idx, _ = head_topk(inp["h"], inp["W"], K=K, chunk=head_chunk)
    P = T - 1
    vals = vals.reshape(B, P, K)
    idx = idx.reshape(B, P, K)
    anchor = inp["anchor"] if anchored else None
    g = {"greedy": B, "sample": 0, "mixed": B // 2}[verify]
    if sampled_path and g < B:
        assert top_k == 0, "the sampled path is verified against the unfiltered target"
        rank = np.zeros((B, P), np.int32)
        tok = np.zeros((B, P), np.int32)
        score = np.zeros(B, np.float32)
        if g > 0:
            rank[:g], tok[:g], score[:g], _ = select_path(vals[:g], idx[:g], inp["F_l"], inp["F_r"],
                                                          anchor=None if anchor is None else anchor[:g])
        rank[g:], tok[g:], q = select_path_sampled(vals[g:], idx[g:], inp["F_l"], inp["F_r"], inp["seed"],
                                                   inp["request_id"][g:], inp["pos0"][g:],
                                                   anchor=None if anchor is None else anchor[g:])
    else:
        rank, tok, score, _ = select_path(vals, idx, inp["F_l"], inp["F_r"], anchor=anchor)
    logits = inp["target"]
    out = np.full((B, T), -1, np.int32)
    n = np.zeros(B, np.int32)
    if g > 0 and fused_target_head:
        out[:g], n[:g] = verify_greedy_hidden(inp["h_target"][:g * T], inp["W"], tok[:g], chunk=head_chunk)
    elif g > 0:
        out[:g], n[:g] = verify_greedy(logits[:g], tok[:g])
    if g < B and fused_target_head:
        out[g:], n[g:] = verify_sample_hidden(inp["h_target"][g * T:], inp["W"], tok[g:], inp["temperature"],
                                              inp["seed"], inp["request_id"][g:], inp["pos0"][g:], chunk=head_chunk)
    elif g < B and sampled_path:
        out[g:], n[g:] = verify_sample_q(logits[g:], tok[g:], idx[g:], q, inp["temperature"], inp["seed"],
                                         inp["request_id"][g:], inp["pos0"][g:])
    elif g < B and top_k > 0:
        out[g:], n[g:] = verify_sample_topkp(logits[g:], tok[g:], inp["temperature"], top_k, top_p, inp["seed"],
                                             inp["request_id"][g:], inp["pos0"][g:])
    elif g < B:
        out[g:], n[g:] = verify_sample(logits[g:], tok[g:], inp["temperature"], inp["seed"],
                                       inp["request_id"][g:], inp["pos0"][g:])
    return {"y": ys, "top_val": vals, "top_idx": idx, "path_rank": rank,
            "path_tok": tok, "path_score": score, "out_tok": out, "n_emit": n}
