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
