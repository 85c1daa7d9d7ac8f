"""Low-rank bilinear pair selector and max-sum path through the top-16 lattice.

Source: tamsi.dev "DFlash 2 — 3× plus de tokens…", § "L'idée, sans le papier"
(the leak is choosing badly among good candidates; a pair selector of about
+2 M parameters picks a coherent path through the kept lists); myaiexp.com
"DFlash 2", § 主な機能 (keep the top 16 per position, score adjacent pairs so
the block is coherent); latenode.com "DFlash 2: un drafter de 3.43×…", opening
section (a light selector traces one coherent route through the candidates
kept at each position); postsingularityinstitute.com "Qwen 3.8 27B + DFlash2",
§ Résumé (candidates chosen by a bilinear attention).

Readings taken (the pages give no formula):

* pair(c, c') = <F_l[c], F_r[c']> with F_l = E P^T, F_r = E Q^T, E the tied
  LM-head rows and P, Q in R^{r x D}: 2 r D parameters (1.97 M at r = 192,
  D = 5120, matching "+2 M").  The tables F_l, F_r ([V][r] float32) are
  prepared once per weight load; per cycle the selector gathers rows.
* Edges join adjacent draft positions only; the unary term of candidate i at
  position p is its draft logit val[p][i] with weight 1.
* Max-sum dynamic programme (Viterbi):
      delta_0[i]     = val[0][i]
      delta_{p+1}[j] = val[p+1][j] + max_i (delta_p[i] + pair_p[i][j])
  with psi_{p+1}[j] the maximising i, the lowest i on ties; the path ends at
  the lowest i maximising delta_{P-1} and is read back through psi.
* Arithmetic is float64.  Each pair score is summed over k = 0..r-1 in index
  order (float32 x float32 products are exact in float64, so a fused or a
  separate multiply-add gives the same result at every step).
* Anchored variant (a NEXT item of the blueprint, reading): slot 0 of the
  block holds the last verified token a, known before drafting; it joins the
  lattice as a one-node column in front of position 0, so
      delta_0[i] = val[0][i] + pair(a, idx[0][i])
  and everything else is unchanged.  An anchor id outside [0, V) has a zero
  feature row (pair 0), like any other id.
"""

import numpy as np

from ._arrays import f64, i64


def pair_scores(idx_left, idx_right, F_l, F_r):
    """pair[i][j] = sum_k F_l[idx_left[i], k] * F_r[idx_right[j], k], k ascending."""
    A = f64(F_l[np.asarray(idx_left)])  # [K][r]
    Bm = f64(F_r[np.asarray(idx_right)])  # [K][r]
    K, r = A.shape
    acc = np.zeros((K, Bm.shape[0]), dtype=np.float64)
    for k in range(r):
        acc = acc + A[:, k, None] * Bm[None, :, k]
    return acc


def select_path(top_val, top_idx, F_l, F_r, anchor=None):
    """Max-sum path per request.

    top_val: [B][P][K] float32 draft logits of the candidates, top_idx: [B][P][K]
    vocab ids, anchor: optional [B] ids of the block's slot-0 tokens.  Returns
    (rank i32 [B][P], tok i32 [B][P], score f32 [B], score f64 [B]).
    """
    val = f64(top_val)
    idx = i64(top_idx)
    B, P, K = val.shape
    V = F_l.shape[0]
    rank = np.zeros((B, P), dtype=np.int32)
    tok = np.zeros((B, P), dtype=np.int32)
    score64 = np.zeros(B, dtype=np.float64)
    for b in range(B):
        delta = val[b, 0].copy()
        if anchor is not None:
            a = int(anchor[b])
            if 0 <= a < V:
                delta = delta + pair_scores([a], idx[b, 0], F_l, F_r)[0]
        psi = []
        for p in range(P - 1):
            pair = pair_scores(idx[b, p], idx[b, p + 1], F_l, F_r)
            cand = delta[:, None] + pair            # [i][j]
            best_i = np.argmax(cand, axis=0)        # first maximum: lowest i
            delta = val[b, p + 1] + cand[best_i, np.arange(K)]
            psi.append(best_i)
        end = int(np.argmax(delta))
        score64[b] = delta[end]
        path = [end]
        for p in range(P - 2, -1, -1):
            path.append(int(psi[p][path[-1]]))
        path.reverse()
        rank[b] = path
        tok[b] = idx[b, np.arange(P), path]
    return rank, tok, score64.astype(np.float32), score64


# ------------------------------------------------------ sampled path (NEXT)
# A reading beyond the pages (which choose the path by max-sum): the draft
# proposes a path drawn from the chain distribution over the lattice whose
# scores the max-sum selector maximises,
#     pi(i_0 .. i_{P-1}) ~ exp( sum_p u_p(i_p) + sum_{p < P-1} pair_p(i_p, i_{p+1}) ),
# u_p = val[p] (plus pair(anchor, .) at p = 0 with an anchor).  The verifier
# then needs the draft's proposal at each position given the drawn prefix,
# q_p(j) = pi(i_p = j | i_0 .. i_{p-1}), which is sparse over the vocabulary
# (16 candidates).  Standard chain inference gives it: backward messages
#     b_{P-1}(i) = u_{P-1}(i)
#     b_p(i)     = u_p(i) + logsumexp_j (pair_p(i, j) + b_{p+1}(j))
# and, in drafting order,
#     q_0(j) ~ exp(b_0(j)),   q_p(j) ~ exp(pair_{p-1}(i_{p-1}, j) + b_p(j)).
# Each position's draw uses word 2 of the Philox block of the slot it fills
# (counter (1, request_id, pos0 + p + 1, 0)); the verifier uses words 0 and 1
# of the same block.

TWO_M53 = 2.0 ** -53
MASK64 = (1 << 64) - 1


def path_uniform(seed, request_id, position):
    """u in [0, 1) for the draft position that fills slot `position`."""
    from .philox import philox4x64_10
    w = philox4x64_10((1, request_id & MASK64, position & MASK64, 0), (seed & MASK64, 0))
    return (w[2] >> 11) * TWO_M53


def _logsumexp(x):
    """m + log(sum_j exp(x_j - m)), m = max x, summed in index order."""
    m = float(np.max(x))
    s = 0.0
    for v in x:
        s += float(np.exp(float(v) - m))
    return m + float(np.log(s))


def _categorical(x, u):
    """Draw from q ~ exp(x): weights e_j = exp(x_j - max x), total in index
    order; the smallest j whose running sum exceeds u * total (the last j of
    non-zero weight if rounding leaves none).  Returns (j, q = e / total)."""
    m = float(np.max(x))
    e = np.array([float(np.exp(float(v) - m)) for v in x])
    tot = 0.0
    for v in e:
        tot += float(v)
    target = u * tot
    c = 0.0
    pick = -1
    for j, v in enumerate(e):
        c += float(v)
        if pick < 0 and c > target:
            pick = j
    if pick < 0:
        pick = int(np.nonzero(e > 0)[0][-1])
    return pick, e / tot


def select_path_sampled(top_val, top_idx, F_l, F_r, seed, request_id, pos0, anchor=None):
    """Draw one path per request from the chain distribution (see above).

    Returns (rank i32 [B][P], tok i32 [B][P], q f64 [B][P][K]): q[b][p] is the
    proposal over the K candidates of position p given the drawn prefix."""
    val = f64(top_val)
    idx = i64(top_idx)
    rid = i64(request_id)
    p0 = i64(pos0)
    B, P, K = val.shape
    V = F_l.shape[0]
    rank = np.zeros((B, P), dtype=np.int32)
    tok = np.zeros((B, P), dtype=np.int32)
    q = np.zeros((B, P, K), dtype=np.float64)
    for b in range(B):
        u = [val[b, p].copy() for p in range(P)]
        if anchor is not None:
            a = int(anchor[b])
            if 0 <= a < V:
                u[0] = u[0] + pair_scores([a], idx[b, 0], F_l, F_r)[0]
        pairs = [pair_scores(idx[b, p], idx[b, p + 1], F_l, F_r) for p in range(P - 1)]
        beta = [None] * P
        beta[P - 1] = u[P - 1]
        for p in range(P - 2, -1, -1):
            beta[p] = np.array([u[p][i] + _logsumexp(pairs[p][i] + beta[p + 1]) for i in range(K)])
        prev = -1
        for p in range(P):
            x = beta[0] if p == 0 else pairs[p - 1][prev] + beta[p]
            j, qp = _categorical(x, path_uniform(int(seed), int(rid[b]), int(p0[b]) + p + 1))
            rank[b, p] = j
            tok[b, p] = idx[b, p, j]
            q[b, p] = qp
            prev = j
    return rank, tok, q
