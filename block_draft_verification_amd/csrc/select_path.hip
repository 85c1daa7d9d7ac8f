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
// One workgroup per request of up to four groups of 256 threads.  Group g owns
// the pair tiles p = g, g+groups, ...: it gathers the 16 left rows and 16 right rows
// of the tables into LDS (transposed, k-major, pitch 17, so the 16 lanes of a
// tile row read consecutive words), then thread (i, j) sums over k = 0..r-1 in order in
// float64 (each float32 product is exact in float64, so the fused multiply-add
// rounds exactly like an add of the exact product).  All tiles stay in LDS;
// sixteen lanes then run the DP over the P positions with the back-pointers in
// LDS, and one lane reads the path back.

#include "common.hpp"

namespace dflash {

constexpr int kSelMaxGroups = 4;
constexpr int kSelThreads = 256 * kSelMaxGroups;
constexpr int kMaxP = 15;
constexpr int kMaxVec = 4;  // float4s per thread per table: 16 rows x r <= 256 floats / 256 threads
constexpr int kPitch = kTopK + 1;  // floats per k in the staged tables

__global__ __launch_bounds__(kSelThreads) void select_path_kernel(
    const float* __restrict__ top_val, const int32_t* __restrict__ top_idx,
    const float* __restrict__ feat_l, const float* __restrict__ feat_r, int P, int64_t V, int r,
    int32_t* __restrict__ path_rank, int32_t* __restrict__ path_tok,
    float* __restrict__ path_score) {
    extern __shared__ float stage[];  // [groups][2][r][kPitch], groups = blockDim.x / 256
    __shared__ double pair[kMaxP - 1][kTopK][kTopK];
    __shared__ double val_s[kMaxP][kTopK];
    __shared__ int idx_s[kMaxP][kTopK];
    __shared__ unsigned char psi[kMaxP][kTopK];
    __shared__ double delta[kTopK];

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int groups = nthreads >> 8;
    for (int e = tid; e < P * kTopK; e += nthreads) {
        val_s[e / kTopK][e % kTopK] = (double)top_val[(int64_t)b * P * kTopK + e];
        idx_s[e / kTopK][e % kTopK] = top_idx[(int64_t)b * P * kTopK + e];
    }
    __syncthreads();

    const int g = tid >> 8;
    const int lt = tid & 255;
    float* sl = stage + (size_t)g * 2 * r * kPitch;
    float* sr = sl + (size_t)r * kPitch;
    const int rounds = (P - 1 + groups - 1) / groups;
    for (int round = 0; round < rounds; ++round) {
        const int p = round * groups + g;
        const bool active = p < P - 1;
        if (active) {
            // 16 rows x r floats per table = 4*r float4s; thread lt takes float4s
            // lt, lt+256, ... (at most kMaxVec of them), all loads issued first.
            // LDS layout is k-major with a row pitch of 17 floats, so both the
            // transposing stores and the (i, j) reads are free of bank conflicts.
            const int r4 = r >> 2;
            floatx4 ql[kMaxVec], qr[kMaxVec];
#pragma unroll
            for (int u = 0; u < kMaxVec; ++u) {
                const int e = lt + 256 * u;
                ql[u] = floatx4{0.f, 0.f, 0.f, 0.f};
                qr[u] = floatx4{0.f, 0.f, 0.f, 0.f};
                if (e < kTopK * r4) {
                    const int row = e / r4, k4 = e - row * r4;
                    const int il = idx_s[p][row], ir = idx_s[p + 1][row];
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
        }
        __syncthreads();
        if (active) {
            const int i = lt >> 4, j = lt & 15;
            double acc = 0.0;
#pragma unroll 16
            for (int k = 0; k < r; ++k)
                acc = fma((double)sl[k * kPitch + i], (double)sr[k * kPitch + j], acc);
            pair[p][i][j] = acc;
        }
        __syncthreads();
    }

    // max-sum DP over positions (16 lanes), back-pointers in LDS
    if (tid < kTopK) delta[tid] = val_s[0][tid];
    __syncthreads();
    for (int p = 0; p + 1 < P; ++p) {
        double nd = 0.0;
        if (tid < kTopK) {
            const int j = tid;
            double best = delta[0] + pair[p][0][j];
            int bi = 0;
            for (int i = 1; i < kTopK; ++i) {
                const double c = delta[i] + pair[p][i][j];
                if (c > best) {
                    best = c;
                    bi = i;
                }
            }
            nd = val_s[p + 1][j] + best;
            psi[p + 1][j] = (unsigned char)bi;
        }
        __syncthreads();
        if (tid < kTopK) delta[tid] = nd;
        __syncthreads();
    }
    if (tid == 0) {
        int end = 0;
        double best = delta[0];
        for (int i = 1; i < kTopK; ++i)
            if (delta[i] > best) {
                best = delta[i];
                end = i;
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

int launch_select_path(const float* top_val, const int32_t* top_idx, const float* feat_l,
                       const float* feat_r, int B, int P, int64_t V, int r, int32_t* path_rank,
                       int32_t* path_tok, float* path_score, hipStream_t stream) {
    // as many concurrent tile groups as the tiles and 96 KiB of staging allow
    int groups = kSelMaxGroups;
    while (groups > 1 && (size_t)groups * 2 * r * kPitch * sizeof(float) > 96 * 1024) groups >>= 1;
    while (groups > 1 && groups / 2 >= P - 1) groups >>= 1;
    const size_t shmem = (size_t)groups * 2 * r * kPitch * sizeof(float);
    static bool attr_done = false;
    if (!attr_done) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&select_path_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
        attr_done = true;
    }
    hipLaunchKernelGGL(select_path_kernel, dim3(B), dim3(256 * groups), shmem, stream, top_val, top_idx,
                       feat_l, feat_r, P, V, r, path_rank, path_tok, path_score);
    return launch_status();
}

}  // namespace dflash
