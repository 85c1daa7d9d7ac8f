// Draft LM head fused with per-row top-16 retention (gfx950, bf16 MFMA).
//
// Source: tamsi.dev "DFlash 2 - 3x plus de tokens...", section "L'idee, sans le
// papier" (the right token is far more often in the top 16 than at top-1, so
// 16 candidates per draft position are kept); myaiexp.com "DFlash 2", main
// features (top 16 per position over the vocabulary).
//
// z = h W^T is never materialised.  Kernel 1 (head_topk_kernel) streams W once:
//  * a workgroup of NWAVES wavefronts owns an M-block of 16*MT rows of h and
//    walks vocabulary strips of NWAVES*NT*16 rows (strip = slot, slot+S, ...);
//  * per 32*KS-wide chunk of the hidden dimension, h[M-block][chunk] is staged
//    in LDS (double-buffered) and every wavefront loads its own NT*16 rows of
//    W straight into registers (double-buffered), 8*KS contiguous bf16 per
//    lane, then issues MT*NT*KS v_mfma_f32_16x16x32_bf16.  The hidden
//    dimension is permuted identically for both operands (lane group g holds
//    the g-th quarter of the chunk), which leaves the dot products unchanged
//    and makes each W row segment one contiguous run per lane;
//  * after a strip, the float32 logits still in the accumulators are filtered
//    against each row's running 16th-best value; the few survivors are merged
//    into the row's sorted top-16 list in LDS by a 32-lane bitonic sort;
//  * the workgroup's lists are written as partial lists [M][S][16].
// Kernel 2 (head_merge_kernel), one workgroup per row: keeps the entries of the
// partial lists whose heads rank in the top 20, ranks them, re-scores the best
// 20 exactly (float64 dot products; bf16 x bf16 products are exact in float64)
// and writes the 16 best by exact value, ties to the lower vocab id.

#include "common.hpp"

namespace dflash {

constexpr int kCap = 16;        // candidate slots per row between merges
constexpr int kRescore = 20;    // float32 candidates re-scored exactly per row
constexpr int kMergeThreads = 256;

template <int MT, int NT, int KS, int NWAVES>
struct HeadCfg {
    static constexpr int MB = 16 * MT;           // rows of h per workgroup
    static constexpr int KC = 32 * KS;           // hidden-dim chunk
    static constexpr int LDS_ROW = KC + 8;       // bf16 per LDS row (16 B pad)
    static constexpr int THREADS = 64 * NWAVES;
    static constexpr int STRIP = NWAVES * NT * 16;
    static constexpr int H_PIECES = MB * KC / 8; // 16-byte pieces per chunk
    static constexpr int H_PER_THREAD = (H_PIECES + THREADS - 1) / THREADS;
    static constexpr size_t LDS_H = (size_t)2 * MB * LDS_ROW * 2;
    static constexpr size_t LDS_LIST = (size_t)MB * kTopK * 8;
    static constexpr size_t LDS_CAND = (size_t)MB * kCap * 8;
    static constexpr size_t LDS_MISC = (size_t)MB * 8;  // thr + count
    static constexpr size_t LDS = LDS_H + LDS_LIST + LDS_CAND + LDS_MISC;
};

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// 32-lane bitonic sort, descending in ranks_before order, within each half of
// the wavefront (lane index li = lane & 31).
__device__ __forceinline__ void bitonic32_desc(float& v, int& ix) {
    const int li = threadIdx.x & 31;
#pragma unroll
    for (int k = 2; k <= 32; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const float pv = __shfl_xor(v, j);
            const int pi = __shfl_xor(ix, j);
            const bool desc_block = (li & k) == 0 || k == 32;
            const bool lower = (li & j) == 0;
            const bool want_better = (lower == desc_block);
            const bool partner_better = ranks_before(pv, pi, v, ix);
            const bool partner_worse = ranks_before(v, ix, pv, pi);
            if (want_better ? partner_better : partner_worse) {
                v = pv;
                ix = pi;
            }
        }
    }
}

template <int MT, int NT, int KS, int NWAVES>
__global__ __launch_bounds__(64 * NWAVES) void head_topk_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int64_t M, int D,
    int64_t V, int n_strips, int S, int n_mb, float* __restrict__ part_val,
    int* __restrict__ part_idx) {
    using C = HeadCfg<MT, NT, KS, NWAVES>;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem);                       // [2][MB][LDS_ROW]
    float* lval = reinterpret_cast<float*>(smem + C::LDS_H);               // [MB][16]
    int* lidx = reinterpret_cast<int*>(smem + C::LDS_H + C::MB * kTopK * 4);
    float* cval = reinterpret_cast<float*>(smem + C::LDS_H + C::LDS_LIST);  // [MB][kCap]
    int* cidx = reinterpret_cast<int*>(smem + C::LDS_H + C::LDS_LIST + C::MB * kCap * 4);
    float* thr = reinterpret_cast<float*>(smem + C::LDS_H + C::LDS_LIST + C::LDS_CAND);  // [MB]
    int* ccnt = reinterpret_cast<int*>(smem + C::LDS_H + C::LDS_LIST + C::LDS_CAND + C::MB * 4);

    // workgroup -> (M-block, slot): the M-blocks of one slot are dispatched
    // back to back on the same XCD so they share each W strip through L2.
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int kq = L >> 3;
    const int mb = kq % n_mb;
    const int slot = (kq / n_mb) * 8 + xcd;
    if (slot >= S) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ln = lane & 15;   // row (A) / column (B) within a 16-tile
    const int lg = lane >> 4;   // quarter of the chunk this lane carries
    const int64_t m0 = (int64_t)mb * C::MB;
    const int mt_active = (int)min<int64_t>(MT, (M - m0 + 15) / 16);

    for (int e = tid; e < C::MB * kTopK; e += C::THREADS) {
        lval[e] = -INFINITY;
        lidx[e] = 0x7FFFFFFF;
    }
    for (int e = tid; e < C::MB; e += C::THREADS) {
        thr[e] = -INFINITY;
        ccnt[e] = 0;
    }

    const int n_chunks = (D + C::KC - 1) / C::KC;

    for (int strip = slot; strip < n_strips; strip += S) {
        const int64_t col0 = (int64_t)strip * C::STRIP + wave * NT * 16;
        const uint16_t* wrow[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            int64_t rr = col0 + nt * 16 + ln;
            if (rr > V - 1) rr = V - 1;
            wrow[nt] = W + rr * D + lg * 8 * KS;
        }
        floatx4 acc[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

        u32x4 wb0[NT][KS], wb1[NT][KS];
        u32x4 hreg[C::H_PER_THREAD];

        auto load_h = [&](int c) {
            const int kc0 = c * C::KC;
#pragma unroll
            for (int u = 0; u < C::H_PER_THREAD; ++u) {
                const int p = tid + u * C::THREADS;
                u32x4 val = u32x4{0u, 0u, 0u, 0u};
                if (p < C::H_PIECES) {
                    const int pr = p / (C::KC / 8), cp = p % (C::KC / 8);
                    const int64_t gr = m0 + pr;
                    const int k = kc0 + cp * 8;
                    if (gr < M && k < D) val = *reinterpret_cast<const u32x4*>(h + gr * D + k);
                }
                hreg[u] = val;
            }
        };
        auto store_h = [&](int buf) {
            uint16_t* dst = hs + buf * C::MB * C::LDS_ROW;
#pragma unroll
            for (int u = 0; u < C::H_PER_THREAD; ++u) {
                const int p = tid + u * C::THREADS;
                if (p < C::H_PIECES) {
                    const int pr = p / (C::KC / 8), cp = p % (C::KC / 8);
                    *reinterpret_cast<u32x4*>(dst + pr * C::LDS_ROW + cp * 8) = hreg[u];
                }
            }
        };
        auto load_w = [&](u32x4 (&wb)[NT][KS], int c) {
            const int kc0 = c * C::KC;
            const bool full = kc0 + C::KC <= D;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    if (full || kc0 + lg * 8 * KS + 8 * s < D)
                        wb[nt][s] = ldg16(wrow[nt] + kc0 + 8 * s);
                    else
                        wb[nt][s] = u32x4{0u, 0u, 0u, 0u};
                }
        };
        auto compute = [&](const u32x4 (&wb)[NT][KS], int buf) {
            const uint16_t* src = hs + buf * C::MB * C::LDS_ROW + ln * C::LDS_ROW + lg * 8 * KS;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt < mt_active) {
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const u32x4 a = *reinterpret_cast<const u32x4*>(src + mt * 16 * C::LDS_ROW + 8 * s);
                        const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                av, __builtin_bit_cast(bf16x8, wb[nt][s]), acc[mt][nt], 0, 0, 0);
                    }
                }
            }
        };

        // software pipeline over hidden-dim chunks (h loads issued before W)
        load_h(0);
        load_w(wb0, 0);
        store_h(0);
        __syncthreads();
        for (int c = 0; c < n_chunks; c += 2) {
            const bool has1 = c + 1 < n_chunks;
            if (has1) {
                load_h(c + 1);
                load_w(wb1, c + 1);
            }
            compute(wb0, 0);
            if (has1) store_h(1);
            __syncthreads();
            if (!has1) break;
            const bool has2 = c + 2 < n_chunks;
            if (has2) {
                load_h(c + 2);
                load_w(wb0, c + 2);
            }
            compute(wb1, 1);
            if (has2) store_h(0);
            __syncthreads();
        }

        // ---- epilogue: threshold filter + bounded candidate buffers
        uint32_t pending[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) pending[mt] = 0;
        bool first_pass = true;
        while (true) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt < mt_active) {
                    const int r0 = mt * 16 + 4 * lg;
                    const float4 t4 = *reinterpret_cast<const float4*>(thr + r0);
                    const float tq[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int64_t col = col0 + nt * 16 + ln;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t bit = 1u << (nt * 4 + q);
                            const bool live = first_pass ? (col < V && m0 + r0 + q < M)
                                                         : (pending[mt] & bit) != 0;
                            if (!first_pass) pending[mt] &= ~bit;
                            const float v = acc[mt][nt][q];
                            if (live && v > tq[q]) {
                                const int slotc = atomicAdd(&ccnt[r0 + q], 1);
                                if (slotc < kCap) {
                                    cval[(r0 + q) * kCap + slotc] = v;
                                    cidx[(r0 + q) * kCap + slotc] = (int)col;
                                } else {
                                    pending[mt] |= bit;
                                }
                            }
                        }
                    }
                }
            }
            first_pass = false;
            __syncthreads();
            // merge: one half-wavefront per row with candidates
            const int li = lane & 31;
            for (int r = wave * 2 + (lane >> 5); r < mt_active * 16; r += NWAVES * 2) {
                const int cnt = ccnt[r];
                if (cnt == 0) continue;
                float v;
                int ix;
                if (li < kTopK) {
                    v = lval[r * kTopK + li];
                    ix = lidx[r * kTopK + li];
                } else if (li - kTopK < min(cnt, kCap)) {
                    v = cval[r * kCap + li - kTopK];
                    ix = cidx[r * kCap + li - kTopK];
                } else {
                    v = -INFINITY;
                    ix = 0x7FFFFFFF;
                }
                bitonic32_desc(v, ix);
                if (li < kTopK) {
                    lval[r * kTopK + li] = v;
                    lidx[r * kTopK + li] = ix;
                }
                if (li == kTopK - 1) thr[r] = v;
                if (li == 0) ccnt[r] = 0;
            }
            __syncthreads();
            int any = 0;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) any |= (pending[mt] != 0);
            if (!__syncthreads_or(any)) break;
        }
    }

    // write this workgroup's lists
    for (int e = tid; e < mt_active * 16 * kTopK; e += C::THREADS) {
        const int r = e / kTopK, k = e % kTopK;
        const int64_t gr = m0 + r;
        if (gr < M) {
            const int64_t o = (gr * S + slot) * kTopK + k;
            part_val[o] = lval[e];
            part_idx[o] = lidx[e];
        }
    }
}

// ---------------------------------------------------------------- merge
__global__ __launch_bounds__(kMergeThreads) void head_merge_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int D, int S,
    const float* __restrict__ part_val, const int* __restrict__ part_idx,
    float* __restrict__ top_val, int32_t* __restrict__ top_idx) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* hv = reinterpret_cast<float*>(smem);      // [S] list heads
    int* hi = reinterpret_cast<int*>(hv + S);        // [S]
    __shared__ float cv[kRescore * kTopK];
    __shared__ int ci[kRescore * kTopK];
    __shared__ int ccount;
    __shared__ float bound_v;
    __shared__ int bound_i;
    __shared__ int sel_i[kRescore];
    __shared__ double sel_z[kRescore];
    __shared__ int n_sel;

    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const float* pv = part_val + m * S * kTopK;
    const int* pi = part_idx + m * S * kTopK;
    for (int s = tid; s < S; s += kMergeThreads) {
        hv[s] = pv[s * kTopK];
        hi[s] = pi[s * kTopK];
    }
    if (tid == 0) {
        ccount = 0;
        bound_v = -INFINITY;
        bound_i = 0x7FFFFFFF;
    }
    __syncthreads();
    // bound = the kRescore-th best list head (every top-kRescore entry ranks at
    // or before it, and so does the head of the list holding it)
    for (int s = tid; s < S; s += kMergeThreads) {
        int rank = 0;
        for (int t = 0; t < S; ++t) rank += ranks_before(hv[t], hi[t], hv[s], hi[s]) ? 1 : 0;
        if (rank == kRescore - 1) {
            bound_v = hv[s];
            bound_i = hi[s];
        }
    }
    __syncthreads();
    const float bv = bound_v;
    const int bi = bound_i;
    for (int s = tid; s < S; s += kMergeThreads) {
        if (!ranks_before(bv, bi, hv[s], hi[s])) {  // head ranks at or before bound
            for (int k = 0; k < kTopK; ++k) {
                const float v = pv[s * kTopK + k];
                const int ix = pi[s * kTopK + k];
                if (ranks_before(bv, bi, v, ix)) break;
                const int o = atomicAdd(&ccount, 1);
                if (o < kRescore * kTopK) {
                    cv[o] = v;
                    ci[o] = ix;
                }
            }
        }
    }
    __syncthreads();
    const int nc = min(ccount, kRescore * kTopK);
    // rank candidates; keep the best kRescore (sentinel entries excluded)
    for (int c = tid; c < nc; c += kMergeThreads) {
        int rank = 0;
        for (int t = 0; t < nc; ++t) rank += ranks_before(cv[t], ci[t], cv[c], ci[c]) ? 1 : 0;
        if (rank < kRescore) sel_i[rank] = ci[c];
    }
    if (tid == 0) {
        int n = 0;
        for (int c = 0; c < nc; ++c) n += (ci[c] != 0x7FFFFFFF) ? 1 : 0;
        n_sel = min(n, kRescore);
    }
    __syncthreads();
    const int ns = n_sel;
    // exact re-scoring: wavefront w handles candidates w, w+4, ...
    const int wave = tid >> 6, lane = tid & 63;
    const uint16_t* hr = h + m * D;
    for (int c = wave; c < ns; c += kMergeThreads / 64) {
        const uint16_t* wr = W + (int64_t)sel_i[c] * D;
        double acc = 0.0;
        for (int d0 = lane * 8; d0 < D; d0 += 64 * 8) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(hr + d0);
            const u32x4 b = *reinterpret_cast<const u32x4*>(wr + d0);
            const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
            const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = fma((double)bf16_to_f32(aw[q] & 0xFFFFu), (double)bf16_to_f32(bw[q] & 0xFFFFu), acc);
                acc = fma((double)bf16_to_f32(aw[q] >> 16), (double)bf16_to_f32(bw[q] >> 16), acc);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == 0) sel_z[c] = acc;
    }
    __syncthreads();
    if (tid < ns) {
        int rank = 0;
        for (int t = 0; t < ns; ++t) rank += ranks_before_d(sel_z[t], sel_i[t], sel_z[tid], sel_i[tid]) ? 1 : 0;
        if (rank < kTopK) {
            top_val[m * kTopK + rank] = (float)sel_z[tid];
            top_idx[m * kTopK + rank] = sel_i[tid];
        }
    }
}

// ------------------------------------------------------------------ host
struct HeadPlan {
    int variant;   // which instantiation
    int mb_rows;   // rows per M-block
    int strip;     // vocab rows per strip
    size_t lds;
};

static HeadPlan head_plan(int64_t M) {
    if (M <= 16) return {0, 16, HeadCfg<1, 2, 8, 4>::STRIP, HeadCfg<1, 2, 8, 4>::LDS};
    if (M <= 64) return {1, 64, HeadCfg<4, 2, 4, 4>::STRIP, HeadCfg<4, 2, 4, 4>::LDS};
    if (M <= 128) return {2, 128, HeadCfg<8, 2, 2, 4>::STRIP, HeadCfg<8, 2, 2, 4>::LDS};
    return {3, 256, HeadCfg<16, 2, 2, 4>::STRIP, HeadCfg<16, 2, 2, 4>::LDS};
}

static void head_grid(int64_t M, int64_t V, int& S, int& n_mb, int& n_strips) {
    const HeadPlan p = head_plan(M);
    n_mb = (int)((M + p.mb_rows - 1) / p.mb_rows);
    n_strips = (int)((V + p.strip - 1) / p.strip);
    // about two workgroups per CU in total, a multiple of 8 slots per M-block
    int target = (512 + n_mb - 1) / n_mb;
    if (p.variant == 3) target = (256 + n_mb - 1) / n_mb;
    int s = n_strips < target ? n_strips : target;
    S = (s + 7) / 8 * 8;
}

size_t head_workspace_bytes(int64_t M, int64_t V) {
    int S, n_mb, n_strips;
    head_grid(M, V, S, n_mb, n_strips);
    return (size_t)M * S * kTopK * 8;
}

size_t head_max_lds_bytes() { return HeadCfg<16, 2, 2, 4>::LDS; }

template <int MT, int NT, int KS, int NW>
static void set_lds_attr() {
    static bool done = false;
    if (!done) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&head_topk_kernel<MT, NT, KS, NW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)HeadCfg<MT, NT, KS, NW>::LDS);
        done = true;
    }
}

template <int MT, int NT, int KS, int NW>
static void launch_variant(const uint16_t* h, const uint16_t* W, int64_t M, int D, int64_t V,
                           int n_strips, int S, int n_mb, float* pv, int* pi, hipStream_t stream) {
    set_lds_attr<MT, NT, KS, NW>();
    constexpr size_t lds = HeadCfg<MT, NT, KS, NW>::LDS;
    hipLaunchKernelGGL((head_topk_kernel<MT, NT, KS, NW>), dim3(S * n_mb), dim3(64 * NW), lds, stream, h, W,
                       M, D, V, n_strips, S, n_mb, pv, pi);
}

int launch_head_topk(const uint16_t* h, const uint16_t* W, int64_t M, int D, int64_t V,
                     float* top_val, int32_t* top_idx, void* ws, hipStream_t stream) {
    int S, n_mb, n_strips;
    head_grid(M, V, S, n_mb, n_strips);
    float* pv = reinterpret_cast<float*>(ws);
    int* pi = reinterpret_cast<int*>(pv + (size_t)M * S * kTopK);
    switch (head_plan(M).variant) {
        case 0: launch_variant<1, 2, 8, 4>(h, W, M, D, V, n_strips, S, n_mb, pv, pi, stream); break;
        case 1: launch_variant<4, 2, 4, 4>(h, W, M, D, V, n_strips, S, n_mb, pv, pi, stream); break;
        case 2: launch_variant<8, 2, 2, 4>(h, W, M, D, V, n_strips, S, n_mb, pv, pi, stream); break;
        default: launch_variant<16, 2, 2, 4>(h, W, M, D, V, n_strips, S, n_mb, pv, pi, stream); break;
    }
    int st = launch_status();
    if (st != DFLASH_OK) return st;
    const size_t lds = (size_t)S * 8;
    hipLaunchKernelGGL(head_merge_kernel, dim3((unsigned)M), dim3(kMergeThreads), lds, stream, h, W, D, S,
                       pv, pi, top_val, top_idx);
    return launch_status();
}

}  // namespace dflash
