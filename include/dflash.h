/*
 * dflash.h - C ABI of the DFlash 2 cycle-tail library for MI355X (gfx950).
 *
 * One draft-verify cycle of DFlash 2 block-parallel speculative decoding ends
 * with five steps, each one call here:
 *
 *   dflash_conv2tap       two-tap dynamic depthwise conv on draft hidden states
 *   dflash_head_topk      draft LM head fused with per-position top-16 retention
 *   dflash_select_path    low-rank bilinear pair scores + max-sum path (DP)
 *   dflash_verify_greedy  greedy longest-prefix acceptance
 *   dflash_verify_sample  rejection-sampling acceptance (Philox4x64-10 draws)
 *
 * and variants:
 *
 *   dflash_conv2tap_proj         the conv with its taps projected from the
 *                                hidden states inside the call (never written)
 *   dflash_select_path_anchored  the selector with the block's slot-0 token as
 *                                a fixed first column
 *   dflash_select_path_sampled   a path drawn from the lattice's chain
 *                                distribution, with the proposals that drew it
 *   dflash_verify_sample_q       rejection sampling of drawn drafts against a
 *                                general (sparse) proposal
 *   dflash_verify_greedy_fused   greedy verification from target hidden states,
 *                                the argmax taken in the LM-head GEMM epilogue
 *   dflash_verify_sample_fused   rejection sampling from target hidden states,
 *                                the softmax statistics taken in the LM-head
 *                                GEMM epilogue
 *   dflash_verify_sample_topkp   rejection sampling against a top-k / top-p
 *                                filtered target
 *
 * Sources (the pages describe the method in words only):
 *   tamsi.dev, "DFlash 2 - 3x plus de tokens sur Qwen3.8-27B, meme sortie",
 *     section "L'idee, sans le papier" (top-16 lists, pair selector, two-tap
 *     conv) and "Les chiffres qui comptent..." (greedy = target exactly,
 *     rejection sampling keeps the target distribution);
 *   myaiexp.com, "DFlash 2", section "main features" (path selector over the
 *     top 16 per position scoring adjacent pairs; two-tap dynamic conv;
 *     lossless verification);
 *   latenode.com, "DFlash 2: un drafter de 3.43x que cae a 1.45x bajo carga",
 *     opening section and FAQ (selector traces one coherent route; lossless);
 *   postsingularityinstitute.com, "Qwen 3.8 27B + DFlash2: 140 Token/Sec?",
 *     Resume (candidates chosen by a bilinear attention).
 *
 * Conventions shared by every entry point:
 *   - Array pointers are DEVICE pointers, allocated and owned by the caller,
 *     row-major and contiguous, 16-byte aligned.  bf16 arrays are passed as
 *     uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously on it; nothing allocates, frees or synchronises.  Outputs
 *     are valid once the stream reaches them.
 *   - Arguments are validated on the host before any HIP call; a failed check
 *     returns DFLASH_ERR_INVALID (or _UNSUPPORTED / _WORKSPACE) and enqueues
 *     nothing.  Validation makes no HIP call, so it can be exercised on a host
 *     without a GPU.
 *   - Workspace: where a call takes (workspace, workspace_bytes), passing
 *     workspace == NULL stores the bytes needed in *workspace_bytes and returns
 *     DFLASH_OK without launching; otherwise *workspace_bytes is the size of
 *     the caller's buffer and must be at least that.  Contents need no
 *     initialisation and are scratch after the call.
 *   - Floating-point inputs must be finite.  Index outputs lie in [0, V).
 *   - The library keeps no state between calls other than a per-device
 *     property cache filled on first use.  Calls on different streams may run
 *     concurrently if their workspaces differ.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DFLASH_OK = 0,
    DFLASH_ERR_INVALID = 1,     /* null pointer, bad size, misalignment, aliasing */
    DFLASH_ERR_UNSUPPORTED = 2, /* a size this library does not implement (K != 16) */
    DFLASH_ERR_WORKSPACE = 3,   /* workspace smaller than required */
    DFLASH_ERR_LAUNCH = 4,      /* HIP reported an error when enqueueing */
    DFLASH_ERR_DEVICE = 5       /* current device is not a gfx950 GPU */
};

/* Human-readable name of a status code (static string). */
const char* dflash_status_string(int status);

/* Library ABI version: (major << 16) | minor. */
int dflash_version(void);

/*
 * Two-tap dynamic depthwise causal conv over block slots.
 * Source: tamsi.dev "DFlash 2 - 3x plus de tokens...", section "L'idee, sans
 * le papier" (two-tap conv in the Canon / short-conv style around attention
 * and MLP against suffix decay); myaiexp.com "DFlash 2", main features (two-
 * tap dynamic convolution).  Reading: per token and per channel taps,
 *     y[s][t][c] = a[s][t][c] * x[s][t][c] + b[s][t][c] * x[s][t-1][c],
 *     x[s][-1][c] = 0,  a = taps[s][t][0:D],  b = taps[s][t][D:2D];
 * the sum is rounded once to float32, then to bf16 (nearest-even).
 *   x     bf16 [n_seq][T][D]     draft hidden states (one sequence = one block)
 *   taps  bf16 [n_seq][T][2*D]   per-token taps
 *   y     bf16 [n_seq][T][D]     output; must not overlap x or taps
 * Requires n_seq >= 1, 1 <= T <= 16, D >= 8, D % 8 == 0.
 */
int dflash_conv2tap(const uint16_t* x, const uint16_t* taps, uint16_t* y,
                    int64_t n_seq, int32_t T, int32_t D, void* stream);

/*
 * The two-tap dynamic conv with its taps produced in the same call by the
 * drafter's tap projection, so that the taps never reach memory.
 * Source: as dflash_conv2tap; "dynamic" taps are read as a linear function of
 * the token's own hidden state:
 *     [a | b][s][t] = x[s][t] W_tap^T  (float32 accumulation of exact bf16
 *                                       products; a = columns 0..D-1, b = D..2D-1)
 *     y[s][t][c] = bf16_rne(fmaf(a, x[s][t][c], b * x[s][t-1][c])),
 *     x[s][-1][c] = 0.
 * The taps keep float32 precision (they are never rounded to bf16), so y
 * differs from dflash_conv2tap on bf16-rounded taps; against the exact
 * result it differs only by the rounding of a float32 sum.
 *   x      bf16 [n_seq][T][D]   draft hidden states (one sequence = one block)
 *   w_tap  bf16 [2*D][D]        tap projection (rows 0..D-1 give a, D..2D-1 b)
 *   y      bf16 [n_seq][T][D]   output; must not overlap x or w_tap
 * Requires n_seq >= 1, 1 <= T <= 16, 64 <= D <= 65536, D % 64 == 0.
 */
int dflash_conv2tap_proj(const uint16_t* x, const uint16_t* w_tap, uint16_t* y,
                         int64_t n_seq, int32_t T, int32_t D, void* stream);

/*
 * Draft LM head fused with top-K retention per row.
 * Source: tamsi.dev, section "L'idee, sans le papier" (the right token is in
 * the top 16 far more often than at top-1, so 16 candidates are kept);
 * myaiexp.com "DFlash 2", main features (top 16 per position).
 *   z[m][v] = sum_d h[m][d] * W[v][d]; per row the K largest z, ordered by
 *   value descending, ties to the lower vocab id.  The candidates are found
 *   with a bf16 MFMA GEMM (float32 accumulation) and a running top-16 per row;
 *   the best 20 of them are then re-scored exactly (float64 dot products,
 *   in which every bf16 product is exact) and ordered by the exact value, so
 *   top_val[m][k] = float32 of the exact logit.
 *   h        bf16 [M][D]     draft hidden states of the draft positions
 *   W        bf16 [V][D]     LM-head rows (vocab entry v is row v)
 *   top_val  f32  [M][K]     output values, descending
 *   top_idx  i32  [M][K]     output vocab ids
 * Requires M >= 1, 8 <= D <= 65536, D % 8 == 0, K <= V < 2^31, M <= 2^24;
 * K == 16 (else UNSUPPORTED).
 * Workspace: partial candidate lists, see the workspace convention above.
 */
int dflash_head_topk(const uint16_t* h, const uint16_t* W, int64_t M, int32_t D,
                     int64_t V, int32_t K, float* top_val, int32_t* top_idx,
                     void* workspace, size_t* workspace_bytes, void* stream);

/*
 * dflash_head_topk without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and requirements as
 * dflash_head_topk; its scratch memory (the partial candidate lists) is a
 * 16 MiB device array inside the library, one per GPU, held from the first
 * use on that GPU until the process ends.  A size whose partial lists need
 * more than 16 MiB (dflash_head_topk's workspace query reports the bytes)
 * returns DFLASH_ERR_WORKSPACE before anything is enqueued; every M up to
 * 65536 fits at V <= 262144.  The first call on a device resolves the array's
 * address there (make it outside graph capture).  All calls on one GPU share
 * the array: calls that may overlap in time on one GPU race, so enqueue them
 * on one stream.  Allocates nothing, ever.
 */
int dflash_head_topk_noalloc(const uint16_t* h, const uint16_t* W, int64_t M,
                             int32_t D, int64_t V, int32_t K, float* top_val,
                             int32_t* top_idx, void* stream);

/*
 * Bounds on the rows of an LM head W, for dflash_head_topk_certify: bound[0]
 * >= max_v |W_v|_2 and bound[1] >= max_v |W_v|_1 (sums in float64, rounded
 * up to float32).  One pass over W; compute it once per weight matrix.
 *   W      bf16 [V][D] (16-byte aligned)
 *   bound  f32 [2] device, written on `stream`
 * Requires D % 8 == 0, 8 <= D <= 65536, 1 <= V < 2^31.
 */
int dflash_head_weight_bound(const uint16_t* W, int64_t V, int32_t D, float* bound,
                             void* stream);

/*
 * Certificate that dflash_head_topk's results are the exact top-16.
 * Source: the exactness contract of the head (top-k over exact logits, see
 * dflash_head_topk).  The head ranks its best 20 float32 candidates by their
 * exact values; an entry it did not re-score can only displace one of the 16
 * returned if its float32 logit erred by more than the gap.  Per row m:
 * certified[m] = 1 iff L16 > U + eps_m, where L16 is a lower bound of the
 * exact 16th value (top_val[m][15] minus half an ulp), U the largest float32
 * value among entries that were not re-scored (read from the partial lists
 * the head left in its workspace), and eps_m = gamma_D * min(|h_m|_2 *
 * bound[0], |h_m|_inf * bound[1]) with gamma_D = D u / (1 - D u), u = 2^-23
 * (an error of one unit in the last place per float32 addition, in any order
 * and rounding direction).  certified[m] = 0 does not mean the row is wrong,
 * only that this bound cannot show it; the caller may recompute such rows
 * (e.g. with the exact logits of their candidates).
 *   h          bf16 [M][D]      as given to dflash_head_topk
 *   bound      f32 [2]          from dflash_head_weight_bound on the same W
 *   top_val    f32 [M][16]      dflash_head_topk's output
 *   workspace  the workspace of that dflash_head_topk call (its partial
 *              lists), unchanged since; workspace_bytes its size
 *   certified  i32 [M]          1 certified exact, 0 not shown
 * Enqueue it on the same stream after dflash_head_topk.  Requires the same
 * M, D, V, K as that call; a smaller workspace than it needs returns
 * DFLASH_ERR_WORKSPACE.
 */
int dflash_head_topk_certify(const uint16_t* h, int64_t M, int32_t D, int64_t V, int32_t K,
                             const float* bound, const float* top_val,
                             const void* workspace, size_t workspace_bytes,
                             int32_t* certified, void* stream);

/*
 * Pair selector: one coherent path through the P x K candidate lattice.
 * Source: tamsi.dev, section "L'idee, sans le papier" (a pair selector of
 * about 2 M parameters chooses a coherent path among good candidates);
 * myaiexp.com "DFlash 2", main features (adjacent pairs scored);
 * postsingularityinstitute.com, Resume (bilinear attention over candidates).
 * Reading: pair(c, c') = <feat_l[c], feat_r[c']> with low-rank tables
 * feat_l = E P^T, feat_r = E Q^T ([V][r] float32, prepared by the caller once
 * per weight load); max-sum DP
 *     delta_0[i] = val[0][i],
 *     delta_{p+1}[j] = val[p+1][j] + max_i (delta_p[i] + pair_p[i][j]),
 * lowest i on ties, path ending at the lowest maximiser of delta_{P-1}.
 * Pair sums run over k = 0..r-1 in order and the DP in float64.
 *   top_val    f32 [B][P][K]   candidate draft logits (from dflash_head_topk)
 *   top_idx    i32 [B][P][K]   candidate vocab ids; ids outside [0, V) score 0
 *   feat_l/r   f32 [V][r]      16-byte aligned
 *   path_rank  i32 [B][P]      chosen candidate rank per position
 *   path_tok   i32 [B][P]      chosen vocab id per position (the draft tokens)
 *   path_score f32 [B]         float32 of the path's float64 score
 * Requires B >= 1, 1 <= P <= 15, V >= 1, 4 <= r <= 256, r % 4 == 0;
 * K == 16 (else UNSUPPORTED).  Workspace: the pair tiles (B*(P-1)*16*16
 * doubles), see the workspace convention above.
 */
int dflash_select_path(const float* top_val, const int32_t* top_idx,
                       const float* feat_l, const float* feat_r,
                       int32_t B, int32_t P, int32_t K, int64_t V, int32_t r,
                       int32_t* path_rank, int32_t* path_tok, float* path_score,
                       void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Pair selector anchored on the block's slot-0 token.
 * Source: as dflash_select_path (the pages describe scoring adjacent
 * positions so that the block is coherent; slot 0, the last verified token,
 * is the block's first position).  Reading: the anchor a = anchor[b] joins the
 * lattice as a one-node column before position 0,
 *     delta_0[i] = val[0][i] + pair(a, idx[0][i]),
 * everything else as dflash_select_path; an anchor outside [0, V) scores 0.
 *   anchor  i32 [B]   slot-0 token per request
 *   other arguments as for dflash_select_path.
 * Requires as dflash_select_path.  Workspace: B*P*16*16 doubles (the pair
 * tiles plus one anchor tile per request).
 */
int dflash_select_path_anchored(const float* top_val, const int32_t* top_idx,
                                const int32_t* anchor, const float* feat_l,
                                const float* feat_r, int32_t B, int32_t P, int32_t K,
                                int64_t V, int32_t r, int32_t* path_rank,
                                int32_t* path_tok, float* path_score, void* workspace,
                                size_t* workspace_bytes, void* stream);

/*
 * Sampled-path selector.  A reading beyond the pages, which pick the path by
 * max-sum (tamsi.dev, section "L'idee, sans le papier"): the path is drawn from
 * the chain distribution over the same lattice,
 *     pi(i_0..i_{P-1}) ~ exp(sum_p u_p(i_p) + sum_{p<P-1} pair_p(i_p, i_{p+1})),
 * u_p = val[p] plus, with an anchor, pair(anchor, .) at p = 0.  With backward
 * messages beta_{P-1} = u_{P-1}, beta_p(i) = u_p(i) + logsumexp_j(pair_p(i, j)
 * + beta_{p+1}(j)), position p draws from its proposal given the drawn prefix,
 *     q_0(j) ~ exp(beta_0(j)),  q_p(j) ~ exp(pair_{p-1}(i_{p-1}, j) + beta_p(j)),
 * the smallest j whose running sum exceeds u times the total, with u from word
 * 2 of Philox4x64-10 keyed (seed, 0) on counter (1, request_id[b],
 * pos0[b] + p + 1, 0) (words 0 and 1 of that block are the verifier's).
 * All float64.
 *   anchor      i32 [B] or NULL (no anchor column)
 *   request_id  u64 [B], pos0 i64 [B]   8-byte aligned
 *   path_q      f64 [B][P][16]   q_p over the position's 16 candidates (given
 *                                the drawn prefix), 8-byte aligned
 *   other arguments as for dflash_select_path (no path_score).
 * Requires as dflash_select_path.  Workspace as dflash_select_path, or as
 * dflash_select_path_anchored with an anchor.
 */
int dflash_select_path_sampled(const float* top_val, const int32_t* top_idx,
                               const int32_t* anchor, const float* feat_l,
                               const float* feat_r, int32_t B, int32_t P, int32_t K,
                               int64_t V, int32_t r, uint64_t seed,
                               const uint64_t* request_id, const int64_t* pos0,
                               int32_t* path_rank, int32_t* path_tok, double* path_q,
                               void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Greedy verification.
 * Source: tamsi.dev, section "Les chiffres qui comptent..." (greedy output is
 * exactly the target's); latenode.com, section "El desacuerdo empieza..."
 * (acceptance length = tokens completed per verify step).
 * Block of T slots: slot 0 is the last verified token, slot s = 1..T-1 holds
 * draft[b][s-1]; target row t is the distribution after slot t.
 * g[t] = argmax_v logits[b][t][v] (lowest v on ties); n = length of the
 * longest prefix with draft[b][s-1] == g[s-1]; out_tok[b][0..n-1] = drafts,
 * out_tok[b][n] = g[n], -1 after; n_emit[b] = n + 1.
 *   logits  f32 [B][T][V]   target block logits
 *   draft   i32 [B][T-1]
 *   out_tok i32 [B][T], n_emit i32 [B]
 * Requires B >= 1, 2 <= T <= 16, V >= 1, V < 2^31.
 */
int dflash_verify_greedy(const float* logits, const int32_t* draft, int32_t B,
                         int32_t T, int64_t V, int32_t* out_tok, int32_t* n_emit,
                         void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Greedy verification fused into the target LM head: the target's argmax per
 * row comes out of the head GEMM's epilogue, so target logits are never
 * written.  Source: as dflash_verify_greedy; the LM head is shared by target
 * and draft (the selector tables are built from its rows, see
 * dflash_select_path), so W is the draft head's matrix.
 * g[t] = argmax_v <h_t[b*T + t], W[v]> over exact products and sums (the
 * head's top-16 with exact re-scoring; lowest v on ties), then the prefix
 * rule of dflash_verify_greedy.
 *   h_t     bf16 [B*T][D]  target hidden states (row b*T + t: after slot t)
 *   W       bf16 [V][D]    LM head
 *   draft, out_tok, n_emit as for dflash_verify_greedy.
 * Requires B >= 1, 2 <= T <= 16, 8 <= D <= 65536, D % 8 == 0, 16 <= V < 2^31,
 * h_t and W 16-byte aligned.  Workspace: dflash_head_topk's for M = B*T plus
 * B*T*16*8 bytes.
 */
int dflash_verify_greedy_fused(const uint16_t* h_t, const uint16_t* W,
                               const int32_t* draft, int32_t B, int32_t T, int32_t D,
                               int64_t V, int32_t* out_tok, int32_t* n_emit,
                               void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Rejection-sampling verification fused into the target LM head: as
 * dflash_verify_sample on the logits z = h_t W^T, which are never written.
 * The head GEMM's epilogue keeps, per (row, 16-token tile), the tile maximum
 * and the tile sum of exp((z - m) / tau) from its float32 logits; the draft's
 * logit and the 16 logits of the tile an inverse CDF lands in are re-scored
 * exactly.  The decisions are those of dflash_verify_sample on the exact
 * logits except where a uniform falls within the float32 error (~1e-6 of the
 * row's mass) of a decision boundary.  If rounding leaves the inverse-CDF
 * target past the landing tile's exact mass, that tile's last token of
 * non-zero weight is emitted.
 *   h_t, W as for dflash_verify_greedy_fused; the other arguments as for
 *   dflash_verify_sample.
 * Requires as dflash_verify_greedy_fused plus temperature finite and > 0.
 * Workspace: B*T*ceil(V/16)*8 bytes.
 */
int dflash_verify_sample_fused(const uint16_t* h_t, const uint16_t* W,
                               const int32_t* draft, int32_t B, int32_t T, int32_t D,
                               int64_t V, float temperature, uint64_t seed,
                               const uint64_t* request_id, const int64_t* pos0,
                               int32_t* out_tok, int32_t* n_emit,
                               void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Rejection-sampling verification with a deterministic draft.
 * Source: tamsi.dev, section "Les chiffres qui comptent..." (sampling through
 * rejection sampling keeps the target distribution); latenode.com FAQ (same).
 * p_t(v) = e_t(v) / Z_t, e_t(v) = exp((l_t(v) - max_v l_t) * (1/tau)), float64.
 * For slot s = 1..T-1 with d = draft[b][s-1]: accept iff u_acc * Z_{s-1} <
 * e_{s-1}(d).  On the first rejection emit the smallest v with
 * sum_{w<=v, w!=d} e(w) > u_res * (Z - e(d)) (the residual max(0, p - q),
 * q = one-hot(d)) and stop; if every draft is accepted emit the bonus: the
 * smallest v with sum_{w<=v} e_{T-1}(w) > u_res * Z_{T-1}.
 * Uniforms for the slot s being decided (s = T for the bonus):
 * (w0, w1, w2, w3) = Philox4x64-10(counter = (1, request_id[b], pos0[b] + s, 0),
 * key = (seed, 0)) [Salmon et al., SC'11]; u_acc = (w0 >> 11) * 2^-53,
 * u_res = (w1 >> 11) * 2^-53.  Draws depend on (seed, request id, position)
 * only, so a request's outcome is the same in any batch.
 *   request_id u64 [B], pos0 i64 [B] (absolute position of slot 0)
 *   outputs as for dflash_verify_greedy.
 * Requires B >= 1, 2 <= T <= 16, 1 <= V < 2^31, temperature finite and > 0.
 * Logits must be finite or -inf (weight 0); a NaN logit also weighs 0.
 */
int dflash_verify_sample(const float* logits, const int32_t* draft, int32_t B,
                         int32_t T, int64_t V, float temperature, uint64_t seed,
                         const uint64_t* request_id, const int64_t* pos0,
                         int32_t* out_tok, int32_t* n_emit,
                         void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Rejection-sampling verification of drafts drawn from a proposal q (the
 * output of dflash_select_path_sampled).  Standard speculative sampling: slot
 * s accepts d = draft[b][s-1] iff u_acc * q(d) * Z_{s-1} < e_{s-1}(d)
 * (probability min(1, p(d) / q(d))); on the first rejection it emits the
 * smallest v whose running sum of residual weights max(0, e(v) - q(v) * Z)
 * exceeds u_res times their total, and stops; the bonus and the uniforms are
 * those of dflash_verify_sample.  q of slot s is the support q_idx[b][s-1][k]
 * with probabilities q_prob[b][s-1][k], k < 16; repeated ids add up, ids
 * outside [0, V) weigh nothing.  A one-hot q at d gives exactly
 * dflash_verify_sample.
 *   q_idx   i32 [B][T-1][16], q_prob f64 [B][T-1][16] (8-byte aligned)
 *   other arguments as for dflash_verify_sample.
 * Requires as dflash_verify_sample.  Workspace as dflash_verify_sample.
 */
int dflash_verify_sample_q(const float* logits, const int32_t* draft,
                           const int32_t* q_idx, const double* q_prob, int32_t B,
                           int32_t T, int64_t V, float temperature, uint64_t seed,
                           const uint64_t* request_id, const int64_t* pos0,
                           int32_t* out_tok, int32_t* n_emit,
                           void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Rejection-sampling verification against a filtered target.
 * Source: latenode.com "DFlash 2: un drafter de 3.43x...", FAQ (the published
 * figures sample at temperature 1.0 with top-p 0.95 and top-k 20).
 * Each target row t is filtered before the test: rank tokens by logit,
 * descending, ties to the lower id, and keep the first top_k; weights
 * e(v) = exp((l_t(v) - max_v l_t) * (1/tau)) in float64; Zk = their sum in rank
 * order; keep, in rank order, every token whose preceding mass is below
 * top_p * Zk (the first always), giving the set N_t with mass Z'_t.  Then as
 * dflash_verify_sample with p'_t = e / Z'_t on N_t (0 elsewhere): accept
 * d = draft[b][s-1] iff d is in N_{s-1} and u_acc * Z' < e(d); on the first
 * rejection emit the smallest id v in N with sum over ids w <= v in N, w != d,
 * of e(w) > u_res * (Z' - e'(d)) (e'(d) = e(d) if d is in N, else 0) and stop;
 * if every draft is accepted draw the bonus from N_{T-1} the same way with
 * target u_res * Z'.  Uniforms as for dflash_verify_sample.
 *   top_k   1..64 tokens kept per row before the nucleus cut
 *   top_p   nucleus mass in (0, 1]
 *   other arguments and outputs as for dflash_verify_sample.
 * Requires B >= 1, 2 <= T <= 16, 1 <= V < 2^31, temperature finite and > 0,
 * 1 <= top_k <= 64, 0 < top_p <= 1.  Logits must not be NaN.
 */
int dflash_verify_sample_topkp(const float* logits, const int32_t* draft, int32_t B,
                               int32_t T, int64_t V, float temperature, int32_t top_k,
                               float top_p, uint64_t seed, const uint64_t* request_id,
                               const int64_t* pos0, int32_t* out_tok, int32_t* n_emit,
                               void* workspace, size_t* workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
