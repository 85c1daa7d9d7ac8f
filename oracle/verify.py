"""Lossless verification of a drafted block against the target's block logits.

Source: tamsi.dev "DFlash 2 — 3× plus de tokens…", § "Les chiffres qui
comptent…" (greedy output is exactly the target's; sampling by rejection
sampling keeps the target distribution); latenode.com "DFlash 2: un drafter de
3.43×…", opening section and FAQ (same guarantee), § "El desacuerdo empieza…"
(acceptance length = tokens completed per verification step); myaiexp.com
"DFlash 2", § コツ (block size 8 means seven draft tokens).

Block layout (reading): T slots; slot 0 is the last verified token, slots
1..P = T-1 hold the drafts d[0..P-1].  Target row t (t = 0..T-1) is the
target's next-token distribution after slot t, so draft d[s-1] at slot s is
checked against row s-1 and row T-1 supplies the bonus token.

Outputs per request: out_tok[0..n] = accepted drafts then one target token,
-1 after; n_emit = n + 1 in [1, T].
"""

import math

import numpy as np

from ._arrays import f64, i64
from .philox import philox4x64_10

TWO_M53 = 2.0 ** -53
MASK64 = (1 << 64) - 1


def verify_greedy(logits, draft):
    """Greedy: g[t] = argmax_v logits[t][v] (lowest v on ties); accept the
    longest prefix with d[s-1] == g[s-1]; then emit g[n]."""
    L = f64(logits)
    d = i64(draft)
    B, T, V = L.shape
    P = T - 1
    assert d.shape == (B, P)
    out = np.full((B, T), -1, dtype=np.int32)
    n_emit = np.zeros(B, dtype=np.int32)
    for b in range(B):
        g = np.argmax(L[b], axis=-1)  # first maximum
        n = 0
        while n < P and d[b, n] == g[n]:
            out[b, n] = d[b, n]
            n += 1
        out[b, n] = g[n]
        n_emit[b] = n + 1
    return out, n_emit


def uniforms(seed, request_id, position):
    """Two 53-bit uniforms in [0, 1) for one decided slot.

    Philox4x64-10 keyed (seed, 0) on counter (1, request_id, position, 0);
    u_acc comes from output word 0 and u_res from word 1, each as
    (w >> 11) * 2^-53.  The counter depends on the request's id and the
    absolute position only, never on the batch slot, so a request's draws do
    not change with batch composition.
    """
    w = philox4x64_10((1, request_id & MASK64, position & MASK64, 0), (seed & MASK64, 0))
    return (w[0] >> 11) * TWO_M53, (w[1] >> 11) * TWO_M53


def row_weights(row, inv_tau):
    """e(v) = exp((l_v - m) * inv_tau), m = max_v l_v, all in float64."""
    row = np.asarray(row, dtype=np.float64)
    return np.exp((row - np.max(row)) * inv_tau)


def inverse_cdf(weights, target):
    """Smallest v with sum_{w <= v} weights[w] > target (ascending v).

    If rounding leaves no such v, the last v with non-zero weight."""
    c = np.cumsum(weights)
    hit = np.nonzero(c > target)[0]
    if hit.size:
        return int(hit[0])
    return int(np.nonzero(weights > 0)[0][-1])


def decide_slot(e, d, u_acc, u_res):
    """One draft slot: accept d iff u_acc * Z < e(d); otherwise draw from the
    residual max(0, p - onehot(d)) (p with d removed), renormalised.

    Returns (accepted, token).  With q = onehot(d) the emitted token has law
    p: P[d] = p(d), P[v != d] = (1 - p(d)) * p(v) / (1 - p(d)) = p(v).
    """
    Z = float(np.sum(e))
    if u_acc * Z < e[d]:
        return True, int(d)
    resid = e.copy()
    resid[d] = 0.0
    return False, inverse_cdf(resid, u_res * (Z - e[d]))


def decide_bonus(e, u_res):
    """Bonus token after a fully accepted block: draw from p by inverse CDF."""
    return inverse_cdf(e, u_res * float(np.sum(e)))


def verify_sample(logits, draft, temperature, seed, request_id, pos0,
                  return_margins=False):
    """Rejection-sampling verification with a deterministic draft.

    Readings taken (the pages give no algorithm):
    * p_t = softmax(logits[t] / tau) over the full vocabulary, as
      e_t(v) / Z_t with e_t(v) = exp((l - max) * (1 / tau)), float64.
    * The draft token is chosen by the selector, not sampled, so the proposal
      is q = one-hot(d) (``decide_slot``).
    * If all P drafts are accepted the bonus token comes from row T-1
      (``decide_bonus``).
    * Uniforms come from ``uniforms(seed, request_id, pos0 + s)`` for the slot
      s being decided (s = T for the bonus).
    Returns (out_tok, n_emit) and, if asked, per-request margins: the smallest
    distance, relative to the row's mass, of any decision from its boundary.
    """
    L = f64(logits)
    d = i64(draft)
    rid = i64(request_id)
    p0 = i64(pos0)
    B, T, V = L.shape
    P = T - 1
    inv_tau = 1.0 / float(np.float32(temperature))
    out = np.full((B, T), -1, dtype=np.int32)
    n_emit = np.zeros(B, dtype=np.int32)
    margins = np.full(B, np.inf)
    for b in range(B):
        n = 0
        for s in range(1, T + 1):
            u_acc, u_res = uniforms(int(seed), int(rid[b]), int(p0[b]) + s)
            if s <= P:
                e = row_weights(L[b, s - 1], inv_tau)
                tok = int(d[b, s - 1])
                if return_margins:
                    Z = float(np.sum(e))
                    margins[b] = min(margins[b], abs(u_acc * Z - e[tok]) / Z)
                    resid = e.copy()
                    resid[tok] = 0.0
                    margins[b] = min(margins[b], _edge_margin(resid, u_res * (Z - e[tok])))
                accepted, tok = decide_slot(e, tok, u_acc, u_res)
                out[b, n] = tok
                if accepted:
                    n += 1
                    continue
                break
            e = row_weights(L[b, T - 1], inv_tau)
            if return_margins:
                margins[b] = min(margins[b], _edge_margin(e, u_res * float(np.sum(e))))
            out[b, n] = decide_bonus(e, u_res)
        n_emit[b] = n + 1
    if return_margins:
        return out, n_emit, margins
    return out, n_emit


def _edge_margin(weights, target):
    """Distance, over the total mass, of an inverse-CDF target from the nearest
    point where ``inverse_cdf`` would return another token.

    Those points are the cumulative masses c[j] strictly between 0 and the
    total: targets are never negative, and a target at or past the total falls
    back to the last token of non-zero weight, which is also the token just
    below the total.  So 0 and the total are not boundaries, and a zero-weight
    bin adds none of its own (its c equals its predecessor's).  With no mass
    at all there is no draw (a residual is empty only when the drafted token
    holds all of the mass, and then it is always accepted): no boundary."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    if not c.size or not c[-1] > 0:
        return math.inf
    total = c[-1]
    k = inverse_cdf(w, target)                 # the landing bin: positive weight
    lo = c[k - 1] if k > 0 else 0.0            # its lower edge; c[k] its upper one
    d = math.inf
    if lo > 0.0:
        d = min(d, abs(target - lo))
    if c[k] < c[-1]:
        d = min(d, abs(c[k] - target))
    return d / total


# ------------------------------------------------- top-k / top-p (nucleus)
# Source: latenode.com "DFlash 2: un drafter de 3.43x...", FAQ (the published
# figures sample at temperature 1.0 with top-p 0.95 and top-k 20).  The page
# gives the parameters only; the readings below are the usual ones.

def filtered_set(row, inv_tau, top_k, top_p):
    """Tokens of one target row kept by top-k, then top-p, with their weights.

    Readings taken:
    * rank tokens by logit, descending, ties to the lower id; keep the first
      top_k (all of them if top_k >= V);
    * weights e(v) = exp((l_v - l_max) * inv_tau), float64; Zk = their sum
      accumulated in rank order;
    * nucleus: walk the kept tokens in rank order accumulating c; a token is
      kept while the mass before it is below top_p * Zk (the first token is
      always kept), i.e. the shortest rank prefix whose mass reaches
      top_p * Zk;
    * the filtered target is p'(v) = e(v) / Z' on the kept set, Z' = the
      accumulated mass of the kept prefix.
    Returns (ids ascending, their weights, Z')."""
    row = np.asarray(row, dtype=np.float64)
    V = row.size
    k = min(int(top_k), V)
    order = np.lexsort((np.arange(V), -row))[:k]
    e = np.exp((row[order] - row[order[0]]) * inv_tau)
    zk = 0.0
    for x in e:
        zk += float(x)
    bound = float(top_p) * zk
    kept, c = 0, 0.0
    for x in e:
        if kept > 0 and c >= bound:
            break
        c += float(x)
        kept += 1
    ids = order[:kept]
    w = e[:kept]
    by_id = np.argsort(ids, kind="stable")
    return ids[by_id].astype(np.int64), w[by_id], c


def _cut_margin(row, inv_tau, top_k, top_p):
    """Smallest distance, relative to Zk, of a nucleus accumulation from its
    top_p * Zk bound (a keep/drop decision that rounding could flip)."""
    row = np.asarray(row, dtype=np.float64)
    k = min(int(top_k), row.size)
    order = np.lexsort((np.arange(row.size), -row))[:k]
    e = np.exp((row[order] - row[order[0]]) * inv_tau)
    zk = float(np.sum(e))
    c = np.cumsum(e)[:-1]
    return float(np.min(np.abs(c - top_p * zk)) / zk) if c.size else math.inf


def decide_slot_filtered(ids, w, Z, d, u_acc, u_res):
    """decide_slot on the filtered target: a draft outside the kept set has
    p'(d) = 0 and is rejected; the residual max(0, p' - onehot(d)) is p' with
    d removed, drawn by inverse CDF over the kept ids in ascending order."""
    j = int(np.searchsorted(ids, d))
    inside = j < ids.size and ids[j] == d
    ed = float(w[j]) if inside else 0.0
    if u_acc * Z < ed:
        return True, int(d)
    resid = w.copy()
    if inside:
        resid[j] = 0.0
    return False, int(ids[inverse_cdf(resid, u_res * (Z - ed))])


def verify_sample_topkp(logits, draft, temperature, top_k, top_p, seed, request_id, pos0,
                        return_margins=False):
    """verify_sample with the target rows filtered by top-k then top-p
    (``filtered_set``); decisions, uniforms and outputs as in verify_sample,
    the bonus drawn from the filtered last row.  top_p is taken as float32,
    like the temperature."""
    L = f64(logits)
    d = i64(draft)
    rid = i64(request_id)
    p0 = i64(pos0)
    B, T, V = L.shape
    P = T - 1
    inv_tau = 1.0 / float(np.float32(temperature))
    tp = float(np.float32(top_p))
    out = np.full((B, T), -1, dtype=np.int32)
    n_emit = np.zeros(B, dtype=np.int32)
    margins = np.full(B, np.inf)
    for b in range(B):
        n = 0
        for s in range(1, T + 1):
            u_acc, u_res = uniforms(int(seed), int(rid[b]), int(p0[b]) + s)
            t = s - 1 if s <= P else T - 1
            ids, w, Z = filtered_set(L[b, t], inv_tau, top_k, tp)
            if return_margins:
                margins[b] = min(margins[b], _cut_margin(L[b, t], inv_tau, top_k, tp))
            if s <= P:
                tok = int(d[b, s - 1])
                if return_margins:
                    j = int(np.searchsorted(ids, tok))
                    ed = float(w[j]) if j < ids.size and ids[j] == tok else 0.0
                    margins[b] = min(margins[b], abs(u_acc * Z - ed) / Z)
                    resid = w.copy()
                    if ed > 0:
                        resid[j] = 0.0
                    margins[b] = min(margins[b], _edge_margin(resid, u_res * (Z - ed)))
                accepted, tok = decide_slot_filtered(ids, w, Z, tok, u_acc, u_res)
                out[b, n] = tok
                if accepted:
                    n += 1
                    continue
                break
            if return_margins:
                margins[b] = min(margins[b], _edge_margin(w, u_res * Z))
            out[b, n] = int(ids[inverse_cdf(w, u_res * Z)])
        n_emit[b] = n + 1
    if return_margins:
        return out, n_emit, margins
    return out, n_emit


# ---------------------------------------- general (sparse) proposal q (NEXT)
# Rejection sampling with a drawn draft (the sampled-path selector): draft
# d = d[s-1] was proposed with probability q(d) under a distribution q that
# is non-zero on at most K candidate ids.  Standard speculative sampling:
# accept with probability min(1, p(d) / q(d)), i.e. iff u_acc * q(d) * Z <
# e(d); otherwise draw from the residual max(0, p - q), renormalised.  With
# q = one-hot(d) this is ``decide_slot``.

def decide_slot_q(e, d, q_ids, q_prob, u_acc, u_res):
    """One draft slot with proposal q (ids q_ids, probabilities q_prob; ids
    outside the vocabulary carry no weight, repeated ids add up).  In weight
    units the residual of token v is max(0, e(v) - q(v) * Z)."""
    V = e.size
    Z = float(np.sum(e))
    qv = {}
    for v, w in zip(q_ids, q_prob):
        v = int(v)
        if 0 <= v < V:
            qv[v] = qv.get(v, 0.0) + float(w)
    qd = qv.get(int(d), 0.0)
    if 0 <= d < V and u_acc * qd * Z < e[d]:
        return True, int(d)
    resid = e.copy()
    for v, w in qv.items():
        resid[v] = max(0.0, e[v] - w * Z)
    return False, inverse_cdf(resid, u_res * float(np.sum(resid)))


def verify_sample_q(logits, draft, q_idx, q_prob, temperature, seed, request_id, pos0):
    """Rejection-sampling verification of drafts drawn from proposals q.

    q_idx i32 [B][P][K] and q_prob f64 [B][P][K] give the proposal the draft
    of slot s = p + 1 was drawn from.  Uniforms, rows and the bonus are those
    of ``verify_sample``."""
    L = f64(logits)
    d = i64(draft)
    qi = i64(q_idx)
    qp = f64(q_prob)
    rid = i64(request_id)
    p0 = i64(pos0)
    B, T, V = L.shape
    P = T - 1
    inv_tau = 1.0 / float(np.float32(temperature))
    out = np.full((B, T), -1, dtype=np.int32)
    n_emit = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = 0
        for s in range(1, T + 1):
            u_acc, u_res = uniforms(int(seed), int(rid[b]), int(p0[b]) + s)
            if s <= P:
                e = row_weights(L[b, s - 1], inv_tau)
                accepted, tok = decide_slot_q(e, int(d[b, s - 1]), qi[b, s - 1], qp[b, s - 1], u_acc, u_res)
                out[b, n] = tok
                if accepted:
                    n += 1
                    continue
                break
            e = row_weights(L[b, T - 1], inv_tau)
            out[b, n] = decide_bonus(e, u_res)
        n_emit[b] = n + 1
    return out, n_emit


# ------------------------------------ greedy from target hidden states (NEXT)
def verify_greedy_hidden(h_t, W, draft, chunk=8192):
    """Greedy verification when the target's block logits are given by its
    hidden states h_t [B*T][D] and the (shared) LM head W [V][D]: the logits
    are the exact z = h_t W^T (``head.head_logits``), then ``verify_greedy``.
    The GPU variant takes the argmax in the head GEMM's epilogue; the result
    is defined by the logits alone."""
    from .head import head_logits
    d = i64(draft)
    B, P = d.shape
    z = head_logits(h_t, W, chunk=chunk).reshape(B, P + 1, -1)
    return verify_greedy(z, d)


def verify_sample_hidden(h_t, W, draft, temperature, seed, request_id, pos0, chunk=8192, return_margins=False):
    """Rejection-sampling verification when the target's block logits are
    given by its hidden states h_t [B*T][D] and the shared LM head W [V][D]:
    the exact logits z = h_t W^T (``head.head_logits``), then ``verify_sample``.
    The GPU variant takes the row statistics in the head GEMM's epilogue from
    float32 logits; its decisions can differ from these only when a uniform
    falls within the float32 error of a decision boundary (see the margins)."""
    from .head import head_logits
    d = i64(draft)
    B, P = d.shape
    z = head_logits(h_t, W, chunk=chunk).reshape(B, P + 1, -1)
    return verify_sample(z, d, temperature, seed, request_id, pos0, return_margins=return_margins)
