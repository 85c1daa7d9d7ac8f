// Pair selector: low-rank bilinear pair scores + max-sum path (gfx950).
//
// Source: tamsi.dev "DFlash 2 - 3x plus de tokens...", section "L'idee, sans le
// papier" (a ~2 M-parameter pair selector picks one coherent path through the
// kept top-16 lists); myaiexp.com "DFlash 2", main features (adjacent pairs are
// scored over the 16 candidates per position); postsingularityinstitute.com
// "Qwen 3.8 27B + DFlash2: 140 Token/Sec?", Resume (bilinear attention).
//
// Reading: pair_p[i][j] = <F_l[idx[p][i]], F_r[idx[p+1][j]]> with float32 tables
// [V][r]; max-sum DP  delta_{p+1}[j] = val[p+1][j] + max_i(delta_p[i] + pair_p[i][j]),
// lowest i on ties, path ending at the lowest maximiser and read back.
//
// Kernel 1 (select_pairs_kernel), one 256-thread workgroup per (request,
// adjacent position pair): gathers the 16 left rows and the 16 right rows of
// the tables into LDS (vectorised loads, all issued first; k-major with a
// pitch of 17 floats so that both the transposing stores and the reads are
// free of bank conflicts), then thread (i, j) sums over k = 0..r-1 in order in
// float64 (each float32 product is exact in float64, so the fused
// multiply-add rounds exactly like an add of the exact product) and writes the
// 16x16 tile to the workspace.
// Kernel 2 (select_dp_kernel), one workgroup per request: it reads the
// request's tiles, values and ids into LDS in one round trip; then one
// wavefront runs the DP over the P positions (lane j holds delta[j]; every
// lane scans the sixteen predecessors of its column in order, with the
// others' delta values read lane by lane) with the back-pointers in LDS, and
// one lane reads the path back.  All DP arithmetic is float64.
// (A single-workgroup variant that also computes the tiles was measured
// slower: one CU then gathers every table row and forms every product.)

#include "common.hpp"
#include "keysort.hpp"
#include "philox.hpp"

namespace dflash {

constexpr int kMaxP = 15;
constexpr int kMaxVec = 4;         // float4s per thread per table: 16 rows x r <= 256 floats / 256 threads
constexpr int kPitch = kTopK + 1;  // floats per k in the staged tables

// Tiles p < P-1: pairs (p, p+1).  With an anchor, tile P-1 scores the
// request's anchor token (every row) against position 0's candidates.
__global__ __launch_bounds__(256) void select_pairs_kernel(const int32_t* __restrict__ top_idx,
                                                           const int32_t* __restrict__ anchor,
                                                           const float* __restrict__ feat_l,
                                                           const float* __restrict__ feat_r, int P, int64_t V,
                                                           int r, int n_tiles, double* __restrict__ pairs) {
    __shared__ float sl[256 * kPitch];
    __shared__ float sr[256 * kPitch];
    __shared__ int il_s[kTopK], ir_s[kTopK];
    const int p = blockIdx.x;   // tile
    const int b = blockIdx.y;   // request
    const int lt = threadIdx.x;
    if (lt < kTopK) {
        if (p == P - 1) {  // the anchor tile (only launched with an anchor)
            il_s[lt] = anchor[b];
            ir_s[lt] = top_idx[(int64_t)b * P * kTopK + lt];
        } else {
            il_s[lt] = top_idx[((int64_t)b * P + p) * kTopK + lt];
            ir_s[lt] = top_idx[((int64_t)b * P + p + 1) * kTopK + lt];
        }
    }
    __syncthreads();
    const int r4 = r >> 2;
    floatx4 ql[kMaxVec], qr[kMaxVec];
#pragma unroll
    for (int u = 0; u < kMaxVec; ++u) {
        const int e = lt + 256 * u;
        ql[u] = floatx4{0.f, 0.f, 0.f, 0.f};
        qr[u] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (e < kTopK * r4) {
            const int row = e / r4, k4 = e - row * r4;
            const int il = il_s[row], ir = ir_s[row];
            // ids outside [0, V) contribute a zero feature row
            if (il >= 0 && il < V) ql[u] = *reinterpret_cast<const floatx4*>(feat_l + (int64_t)il * r + 4 * k4);
            if (ir >= 0 && ir < V) qr[u] = *reinterpret_cast<const floatx4*>(feat_r + (int64_t)ir * r + 4 * k4);
        }
    }
#pragma unroll
    for (int u = 0; u < kMaxVec; ++u) {
        const int e = lt + 256 * u;
        if (e < kTopK * r4) {
            const int row = e / r4, k = 4 * (e - row * r4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                sl[(k + q) * kPitch + row] = ql[u][q];
                sr[(k + q) * kPitch + row] = qr[u][q];
            }
        }
    }
    __syncthreads();
    const int i = lt >> 4, j = lt & 15;
    double acc = 0.0;
#pragma unroll 16
    for (int k = 0; k < r; ++k) acc = fma((double)sl[k * kPitch + i], (double)sr[k * kPitch + j], acc);
    pairs[(((int64_t)b * n_tiles + p) * kTopK + i) * kTopK + j] = acc;
}

// The double held by lane l (l wavefront-uniform), in every lane.
__device__ __forceinline__ double readlane_f64(double x, int l) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__global__ __launch_bounds__(256) void select_dp_kernel(const float* __restrict__ top_val,
                                                        const int32_t* __restrict__ top_idx,
                                                        const double* __restrict__ pairs, int P, int n_tiles,
                                                        bool anchored, int32_t* __restrict__ path_rank,
                                                        int32_t* __restrict__ path_tok,
                                                        float* __restrict__ path_score) {
    __shared__ double pair_s[kMaxP][kTopK * kTopK];
    __shared__ double val_s[kMaxP][kTopK];
    __shared__ int idx_s[kMaxP][kTopK];
    __shared__ unsigned char psi[kMaxP][kTopK];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    {  // one round trip: the request's tiles, values and ids
        const double* pb = pairs + (int64_t)b * n_tiles * kTopK * kTopK;
        double pr[kMaxP];
#pragma unroll
        for (int u = 0; u < kMaxP; ++u) pr[u] = u < n_tiles ? pb[u * kTopK * kTopK + tid] : 0.0;
        const bool has = tid < P * kTopK;
        const float v = has ? top_val[(int64_t)b * P * kTopK + tid] : 0.0f;
        const int id = has ? top_idx[(int64_t)b * P * kTopK + tid] : 0;
#pragma unroll
        for (int u = 0; u < kMaxP; ++u)
            if (u < n_tiles) pair_s[u][tid] = pr[u];
        if (has) {
            val_s[tid / kTopK][tid % kTopK] = (double)v;
            idx_s[tid / kTopK][tid % kTopK] = id;
        }
    }
    __syncthreads();
    if (tid >= 64) return;
    // one wavefront: lane j (mod 16) holds delta[j]; every lane reads the
    // others' values lane by lane and scans i = 0..15 in order
    const int j = tid & 15;
    double dl = val_s[0][j] + (anchored ? pair_s[P - 1][j] : 0.0);
    for (int p = 0; p + 1 < P; ++p) {
        const double* pp = pair_s[p];
        double cv[kTopK];
#pragma unroll
        for (int i = 0; i < kTopK; ++i) cv[i] = pp[i * kTopK + j];
        double best = readlane_f64(dl, 0) + cv[0];
        int bi = 0;
#pragma unroll
        for (int i = 1; i < kTopK; ++i) {
            const double c = readlane_f64(dl, i) + cv[i];
            if (c > best) {
                best = c;
                bi = i;
            }
        }
        if (tid < kTopK) psi[p + 1][j] = (unsigned char)bi;
        dl = val_s[p + 1][j] + best;
    }
    wave_sync();
    if (tid == 0) {
        int end = 0;
        double best = readlane_f64(dl, 0);
        for (int i = 1; i < kTopK; ++i) {
            const double di = readlane_f64(dl, i);
            if (di > best) {
                best = di;
                end = i;
            }
        }
        int cur = end;
        for (int p = P - 1; p >= 0; --p) {
            path_rank[(int64_t)b * P + p] = cur;
            path_tok[(int64_t)b * P + p] = idx_s[p][cur];
            if (p > 0) cur = psi[p][cur];
        }
        path_score[b] = (float)best;
    }
}

// ---------------------------------------------------------- sampled path
// A reading beyond the pages, which choose the path by max-sum: the draft
// proposes a path drawn from the chain distribution whose scores the max-sum
// selector maximises, pi(path) ~ exp(sum_p u_p(i_p) + sum_p pair_p(i_p, i_{p+1})),
// u_p = val[p] (plus the anchor pair at p = 0).  Backward messages
// beta_{P-1} = u_{P-1}, beta_p(i) = u_p(i) + logsumexp_j(pair_p(i, j) +
// beta_{p+1}(j)) give the drafting-order proposals q_0 ~ exp(beta_0),
// q_p(j) ~ exp(pair_{p-1}(i_{p-1}, j) + beta_p(j)), from which each position
// draws with word 2 of the Philox block of the slot it fills (counter
// (1, request_id, pos0 + p + 1, 0); the verifier uses words 0 and 1).
// One workgroup per request: the tiles, values and ids in one round trip;
// the backward messages with one thread per (i, j) and 16-lane reductions;
// then one wavefront draws the positions in order (16-lane maximum and prefix
// sums with DPP row moves; the smallest j whose prefix sum exceeds u times the
// total).  All float64.
// 16-lane (one DPP row) butterflies: every lane of the row gets the result,
// bit-identical across the row (each step adds or compares the same two
// numbers in every lane).
__device__ __forceinline__ double as_f64(uint64_t u) { return __longlong_as_double((long long)u); }
__device__ __forceinline__ uint64_t as_u64(double x) { return (uint64_t)__double_as_longlong(x); }
__device__ __forceinline__ double max16(double x, int li) {
    x = fmax(x, as_f64(dpp_u64<kDppX1>(as_u64(x))));
    x = fmax(x, as_f64(dpp_u64<kDppX2>(as_u64(x))));
    x = fmax(x, as_f64(xor4_u64(as_u64(x), li)));
    x = fmax(x, as_f64(dpp_u64<kDppX8>(as_u64(x))));
    return x;
}
__device__ __forceinline__ double sum16(double x, int li) {
    x += as_f64(dpp_u64<kDppX1>(as_u64(x)));
    x += as_f64(dpp_u64<kDppX2>(as_u64(x)));
    x += as_f64(xor4_u64(as_u64(x), li));
    x += as_f64(dpp_u64<kDppX8>(as_u64(x)));
    return x;
}
// Lane l of the row gets x of lane l - n (n = 1, 2, 4, 8), 0 below the row start.
template <int CTRL>
__device__ __forceinline__ double shr_row_f64(double x) {
    const uint64_t u = as_u64(x);
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return as_f64(((uint64_t)hi << 32) | lo);
}

__global__ __launch_bounds__(256) void select_sample_kernel(
    const float* __restrict__ top_val, const int32_t* __restrict__ top_idx, const double* __restrict__ pairs, int P,
    int n_tiles, bool anchored, uint64_t seed, const uint64_t* __restrict__ request_id,
    const int64_t* __restrict__ pos0, int32_t* __restrict__ path_rank, int32_t* __restrict__ path_tok,
    double* __restrict__ path_q) {
    __shared__ double pair_s[kMaxP][kTopK * kTopK];
    __shared__ double val_s[kMaxP][kTopK];
    __shared__ int idx_s[kMaxP][kTopK];
    __shared__ double beta[kMaxP][kTopK];
    __shared__ double u_s[kMaxP];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    {  // one round trip: the request's tiles, values and ids
        const double* pb = pairs + (int64_t)b * n_tiles * kTopK * kTopK;
        double pr[kMaxP];
#pragma unroll
        for (int u = 0; u < kMaxP; ++u) pr[u] = u < n_tiles ? pb[u * kTopK * kTopK + tid] : 0.0;
        const bool has = tid < P * kTopK;
        const float v = has ? top_val[(int64_t)b * P * kTopK + tid] : 0.0f;
        const int id = has ? top_idx[(int64_t)b * P * kTopK + tid] : 0;
#pragma unroll
        for (int u = 0; u < kMaxP; ++u)
            if (u < n_tiles) pair_s[u][tid] = pr[u];
        if (has) {
            val_s[tid / kTopK][tid % kTopK] = (double)v;
            idx_s[tid / kTopK][tid % kTopK] = id;
        }
    }
    if (tid < P) {
        const Philox4 r = philox4x64_10(1ull, request_id[b], (uint64_t)(pos0[b] + tid + 1), 0ull, seed, 0ull);
        u_s[tid] = (double)(r.w[2] >> 11) * 0x1p-53;
    }
    __syncthreads();
    auto unary = [&](int p, int i) -> double {
        return val_s[p][i] + ((anchored && p == 0) ? pair_s[P - 1][i] : 0.0);
    };
    if (tid < kTopK) beta[P - 1][tid] = unary(P - 1, tid);
    __syncthreads();
    for (int p = P - 2; p >= 0; --p) {
        const int i = tid >> 4, j = tid & 15;
        const double x = pair_s[p][i * kTopK + j] + beta[p + 1][j];
        const double mx = max16(x, j);
        const double sm = sum16(exp(x - mx), j);
        if (j == 0) beta[p][i] = unary(p, i) + (mx + log(sm));
        __syncthreads();
    }
    if (tid >= 64) return;
    const int j = tid & 15;
    int prev = 0;
    for (int p = 0; p < P; ++p) {
        const double x = p == 0 ? beta[0][j] : pair_s[p - 1][prev * kTopK + j] + beta[p][j];
        const double e = exp(x - max16(x, j));
        double c = e;  // inclusive prefix sum over j (row shifts)
        c += shr_row_f64<0x111>(c);
        c += shr_row_f64<0x112>(c);
        c += shr_row_f64<0x114>(c);
        c += shr_row_f64<0x118>(c);
        const double tot = as_f64(readlane_u64(as_u64(c), 15));
        const uint64_t hit = __ballot(tid < kTopK && c > u_s[p] * tot);
        int pick;
        if (hit) {
            pick = __builtin_ctzll(hit);
        } else {  // rounding left no prefix above the target: the last candidate of non-zero weight
            const uint64_t pos = __ballot(tid < kTopK && e > 0.0);
            pick = 63 - __builtin_clzll(pos);
        }
        if (tid < kTopK) path_q[((int64_t)b * P + p) * kTopK + j] = e / tot;
        if (tid == 0) {
            path_rank[(int64_t)b * P + p] = pick;
            path_tok[(int64_t)b * P + p] = idx_s[p][pick];
        }
        prev = pick;
    }
}

size_t select_workspace_bytes(int B, int P, bool anchored) {
    const int n_tiles = P - 1 + (anchored ? 1 : 0);
    return (size_t)B * (n_tiles > 0 ? n_tiles : 1) * kTopK * kTopK * 8;
}

int launch_select_path(const float* top_val, const int32_t* top_idx, const int32_t* anchor, const float* feat_l,
                       const float* feat_r, int B, int P, int64_t V, int r, int32_t* path_rank,
                       int32_t* path_tok, float* path_score, void* ws, hipStream_t stream) {
    double* pairs = reinterpret_cast<double*>(ws);
    const int n_tiles = P - 1 + (anchor ? 1 : 0);
    if (n_tiles > 0) {
        hipLaunchKernelGGL(select_pairs_kernel, dim3(n_tiles, B), dim3(256), 0, stream, top_idx, anchor, feat_l,
                           feat_r, P, V, r, n_tiles, pairs);
        const int st = launch_status();
        if (st != DFLASH_OK) return st;
    }
    hipLaunchKernelGGL(select_dp_kernel, dim3(B), dim3(256), 0, stream, top_val, top_idx, pairs, P, n_tiles,
                       anchor != nullptr, path_rank, path_tok, path_score);
    return launch_status();
}

int launch_select_path_sampled(const float* top_val, const int32_t* top_idx, const int32_t* anchor,
                               const float* feat_l, const float* feat_r, int B, int P, int64_t V, int r,
                               uint64_t seed, const uint64_t* request_id, const int64_t* pos0, int32_t* path_rank,
                               int32_t* path_tok, double* path_q, void* ws, hipStream_t stream) {
    double* pairs = reinterpret_cast<double*>(ws);
    const int n_tiles = P - 1 + (anchor ? 1 : 0);
    if (n_tiles > 0) {
        hipLaunchKernelGGL(select_pairs_kernel, dim3(n_tiles, B), dim3(256), 0, stream, top_idx, anchor, feat_l,
                           feat_r, P, V, r, n_tiles, pairs);
        const int st = launch_status();
        if (st != DFLASH_OK) return st;
    }
    hipLaunchKernelGGL(select_sample_kernel, dim3(B), dim3(256), 0, stream, top_val, top_idx, pairs, P, n_tiles,
                       anchor != nullptr, seed, request_id, pos0, path_rank, path_tok, path_q);
    return launch_status();
}

}  // namespace dflash
