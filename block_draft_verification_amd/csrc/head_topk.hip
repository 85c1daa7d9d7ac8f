// Draft LM head fused with per-row top-16 retention (gfx950, bf16 MFMA).
//
// Source: tamsi.dev "DFlash 2 - 3x plus de tokens...", section "L'idee, sans le
// papier" (the right token is far more often in the top 16 than at top-1, so
// 16 candidates per draft position are kept); myaiexp.com "DFlash 2", main
// features (top 16 per position over the vocabulary).
//
// z = h W^T is never materialised.  W (the whole vocabulary, 1.5-2.7 GB) is
// streamed from HBM exactly once by one of two GEMM kernels, each ending every
// vocabulary tile with a fused top-16 filter; a merge kernel then combines the
// partial lists and re-scores the survivors exactly.
//
// Operand layout (both kernels): v_mfma_f32_16x16x32_bf16 with A = h rows and
// B = W rows; for k-step s of a chunk, lane (r = lane % 16, g = lane / 16)
// holds k = 32 s + 8 g .. +8 of row r, so one 16-byte load per lane reads 64
// contiguous bytes of each of 16 rows, and two consecutive k-steps complete
// every 128-byte line.  Accumulator lane layout: C[4 g + q][r], q = 0..3.
//
// * head_skinny2_kernel (M <= 16, the batch-1 case): every wavefront is
//   independent.  It owns a contiguous, equal-sized range of 16-row vocabulary
//   tiles (balanced to one tile across all wavefronts of the grid), reads its
//   W rows and the h rows row-contiguously with buffer loads (two chunks of
//   32*KS columns in flight), stages them in its private LDS tile, multiplies
//   from there, and keeps its own running top-16 per row in LDS.  No barrier
//   inside the stream.  At the end the four wavefronts of a workgroup merge
//   their lists.
// * head_wide_kernel (M > 16): a workgroup of WM x WN wavefronts owns an
//   M-block of 16*MW*WM rows of h and a contiguous range of vocabulary strips
//   of 16*NT*WN rows.  Per chunk of the hidden dimension, h is staged once in
//   LDS for all wavefronts, and W goes straight to registers, one chunk
//   ahead; wavefronts with the same N-group load the same W rows (shared
//   through L1).  The M-blocks of one strip range are dispatched next to each
//   other on the same XCD so that they share W through its L2.
// * The top-16 epilogue: after a tile, the float32 logits still in the
//   accumulators are compared with each row's running 16th-best entry (value,
//   then id); the few survivors go to a bounded per-row buffer and are merged
//   into the row's sorted list by a 32-lane bitonic sort, retrying anything
//   that overflowed the buffer.
// * head_merge_kernel: see below.

#include <algorithm>
#include <mutex>

#include "common.hpp"

namespace dflash {

constexpr int kCap = 16;        // candidate slots per row between merges
constexpr int kRescore = 20;    // float32 candidates re-scored exactly per row
constexpr int kMergeThreads = 64 * (kRescore / 2);  // one wavefront per two re-scored candidates

__device__ __forceinline__ u32x4 ldg_stream(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ldg(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bitonic sort over groups of WIDTH lanes (WIDTH = 32 or 64), descending in the
// ranks_before order.
template <int WIDTH>
__device__ __forceinline__ void bitonic_desc(float& v, int& ix) {
    const int li = threadIdx.x & (WIDTH - 1);
#pragma unroll
    for (int k = 2; k <= WIDTH; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const float pv = __shfl_xor(v, j);
            const int pi = __shfl_xor(ix, j);
            const bool desc_block = (li & k) == 0 || k == WIDTH;
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

// Running top-16 state of a set of rows in LDS.
struct TopkRows {
    float* lval;  // [rows][16], sorted
    int* lidx;
    float* cval;  // [rows][kCap] candidate buffer
    int* cidx;
    float* thr;   // [rows] 16th-best value and id
    int* thri;
    int* ccnt;    // [rows] candidates since the last merge
};

__device__ __forceinline__ void topk_init(TopkRows t, int rows, int tid, int nthreads) {
    for (int e = tid; e < rows * kTopK; e += nthreads) {
        t.lval[e] = -INFINITY;
        t.lidx[e] = 0x7FFFFFFF;
    }
    for (int e = tid; e < rows; e += nthreads) {
        t.thr[e] = -INFINITY;
        t.thri[e] = 0x7FFFFFFF;
        t.ccnt[e] = 0;
    }
}

// Filter an MW x NT block of 16x16 accumulator tiles into the rows' lists.
//   rbase: LDS row of the block's first row; grow0: its global row
//   col0: global vocabulary id of tile column 0 (lane r = 0)
//   merge rows [0, n_merge_rows) by half-wavefronts h = hw0, hw0 + hw_step, ...
// WG = true: state shared by the workgroup (barriers); false: wave-private.
template <int MW, int NT, bool WG>
__device__ __forceinline__ void topk_epilogue(const floatx4 (&acc)[MW][NT], TopkRows t, int rbase, int64_t grow0,
                              int64_t M, int64_t col0, int nt_act, int64_t V, int mw_act,
                              int n_merge_rows, int hw0, int hw_step) {
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15, lg = lane >> 4;
    uint32_t pending[MW];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) pending[mt] = 0;
    bool first = true;
    while (true) {
#pragma unroll
        for (int mt = 0; mt < MW; ++mt) {
            if (mt < mw_act) {
                const int r0 = rbase + mt * 16 + 4 * lg;
                const float4 t4 = *reinterpret_cast<const float4*>(t.thr + r0);
                const int4 i4 = *reinterpret_cast<const int4*>(t.thri + r0);
                const float tq[4] = {t4.x, t4.y, t4.z, t4.w};
                const int iq[4] = {i4.x, i4.y, i4.z, i4.w};
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int64_t col = col0 + nt * 16 + ln;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t bit = 1u << (nt * 4 + q);
                        const bool live = first ? (nt < nt_act && col < V && grow0 + mt * 16 + 4 * lg + q < M)
                                                : (pending[mt] & bit) != 0;
                        if (!first) pending[mt] &= ~bit;
                        const float v = acc[mt][nt][q];
                        if (live && ranks_before(v, (int)col, tq[q], iq[q])) {
                            const int r = r0 + q;
                            const int slot = atomicAdd(&t.ccnt[r], 1);
                            if (slot < kCap) {
                                t.cval[r * kCap + slot] = v;
                                t.cidx[r * kCap + slot] = (int)col;
                            } else {
                                pending[mt] |= bit;
                            }
                        }
                    }
                }
            }
        }
        first = false;
        if (WG) __syncthreads(); else wave_sync();
        const int li = lane & 31;
        for (int r = hw0 + (lane >> 5); r < n_merge_rows; r += hw_step) {
            const int cnt = t.ccnt[r];
            if (cnt == 0) continue;
            float v;
            int ix;
            if (li < kTopK) {
                v = t.lval[r * kTopK + li];
                ix = t.lidx[r * kTopK + li];
            } else if (li - kTopK < min(cnt, kCap)) {
                v = t.cval[r * kCap + li - kTopK];
                ix = t.cidx[r * kCap + li - kTopK];
            } else {
                v = -INFINITY;
                ix = 0x7FFFFFFF;
            }
            bitonic_desc<32>(v, ix);
            if (li < kTopK) {
                t.lval[r * kTopK + li] = v;
                t.lidx[r * kTopK + li] = ix;
            }
            if (li == kTopK - 1) {
                t.thr[r] = v;
                t.thri[r] = ix;
            }
            if (li == 0) t.ccnt[r] = 0;
        }
        int any = 0;
#pragma unroll
        for (int mt = 0; mt < MW; ++mt) any |= (pending[mt] != 0);
        if (WG) {
            if (!__syncthreads_or(any)) break;
        } else {
            wave_sync();
            if (__ballot(any) == 0) break;
        }
    }
}

// Loads in the streaming loops are unconditional: rows past the end are
// clamped to a valid row (their results are masked in the epilogue) and only a
// ragged last chunk of the hidden dimension takes a masked path, so the
// compiler can keep every prefetched load in flight across iterations.
template <int KS>
__device__ __forceinline__ void load_frag(u32x4& out, const uint16_t* row, int kc0, int s, int lg, int D,
                                          bool full, bool stream) {
    if (full) {
        const uint16_t* p = row + kc0 + 32 * s + lg * 8;
        out = stream ? ldg_stream(p) : ldg(p);
    } else {
        const int k = kc0 + 32 * s + lg * 8;
        const bool in = k < D;
        const uint16_t* p = row + (in ? k : 0);
        const u32x4 v = stream ? ldg_stream(p) : ldg(p);
        out = in ? v : u32x4{0u, 0u, 0u, 0u};
    }
}

// ------------------------------------------------- skinny GEMM, LDS-staged W
// The same wavefront-independent scheme, but W reaches the MFMAs through LDS
// so that its HBM reads are row-contiguous: per chunk the wavefront's 16*NT
// rows x KC columns are read as 512/KC rows per load instruction (64 lanes x
// 16 contiguous bytes), written to the wavefront's private LDS tile, and read
// back in the MFMA operand layout (row pitch KC*2+16 bytes, so the 16 rows of a
// fragment read fall on disjoint bank groups).  Contiguous runs of 2*KC bytes
// per row instead of 64-byte pieces keep HBM pages open.
template <int NT, int KS>
struct Skinny2Cfg {
    static constexpr int KC = 32 * KS;
    static constexpr int R = 16 * NT;                 // W rows per wavefront tile
    static constexpr int ROWB = KC * 2 + 16;          // LDS bytes per staged row
    static constexpr int PIECES = KC / 8;             // 16-byte pieces per row
    static constexpr int ROWS_PER_LOAD = 64 / PIECES;
    static constexpr int LOADS = R / ROWS_PER_LOAD;   // W load instructions per chunk
    static constexpr int ALOADS = 16 / ROWS_PER_LOAD; // h load instructions per chunk
    static constexpr size_t LDS_W = (size_t)(R + 16) * ROWB;  // per wavefront: W rows then 16 h rows
};

// Buffer resource over [base, base + bytes): loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
constexpr int kBufNT = 2;                 // cache policy: non-temporal (streamed once)
constexpr int kOffNone = 0x7FFFFFF0;      // a lane offset outside every resource: loads 0

// Both operands are read row-contiguously into registers (two chunks in
// flight), staged in the wavefront's LDS tile, and read back as MFMA
// fragments.  h rows past M and W rows past V come back as zeros.
template <int NTX, int KS>
__device__ __forceinline__ void skinny2_tiles(__amdgpu_buffer_rsrc_t hsrc, const uint16_t* __restrict__ W,
                                              int64_t M, int D, int64_t V, int64_t t0, TopkRows tk,
                                              unsigned char* __restrict__ wl) {
    using C = Skinny2Cfg<NTX, KS>;
    constexpr int KC = C::KC;
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15, lg = lane >> 4;
    const int ri = lane / C::PIECES, pj = lane % C::PIECES;
    const int64_t row0 = t0 * 16;
    const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(W + row0 * D, (V - row0) * D * 2);
    const int voff = ri * D * 2 + pj * 16;  // + q * ROWS_PER_LOAD * D * 2 + kc0 * 2 (scalar)
    unsigned char* hl = wl + C::R * C::ROWB;
    floatx4 acc[1][NTX];
#pragma unroll
    for (int nt = 0; nt < NTX; ++nt) acc[0][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    u32x4 w0[C::LOADS], w1[C::LOADS], h0[C::ALOADS], h1[C::ALOADS];
    const int n_full = D / KC;
    const bool tail = n_full * KC < D;

    auto load = [&](u32x4 (&w)[C::LOADS], u32x4 (&hh)[C::ALOADS], int c, bool full) {
        const int kc0 = c * KC;
        const int vo = (full || kc0 + pj * 8 < D) ? voff : kOffNone;
#pragma unroll
        for (int q = 0; q < C::ALOADS; ++q)
            hh[q] = __builtin_amdgcn_raw_buffer_load_b128(hsrc, vo, (q * C::ROWS_PER_LOAD * D + kc0) * 2, 0);
#pragma unroll
        for (int q = 0; q < C::LOADS; ++q)
            w[q] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, vo, (q * C::ROWS_PER_LOAD * D + kc0) * 2, kBufNT);
    };
    auto stage = [&](const u32x4 (&w)[C::LOADS], const u32x4 (&hh)[C::ALOADS]) {
#pragma unroll
        for (int q = 0; q < C::ALOADS; ++q)
            *reinterpret_cast<u32x4*>(hl + (q * C::ROWS_PER_LOAD + ri) * C::ROWB + pj * 16) = hh[q];
#pragma unroll
        for (int q = 0; q < C::LOADS; ++q)
            *reinterpret_cast<u32x4*>(wl + (q * C::ROWS_PER_LOAD + ri) * C::ROWB + pj * 16) = w[q];
        wave_sync();
    };
    auto compute = [&]() {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(hl + ln * C::ROWB + (32 * s + 8 * lg) * 2);
            const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
            for (int nt = 0; nt < NTX; ++nt) {
                const u32x4 b = *reinterpret_cast<const u32x4*>(wl + (nt * 16 + ln) * C::ROWB + (32 * s + 8 * lg) * 2);
                acc[0][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b), acc[0][nt],
                                                                    0, 0, 0);
            }
        }
        wave_sync();  // all fragment reads done before the tile is overwritten
    };
    // steady state: chunks c+1 and c+2 in flight while chunk c is staged and
    // multiplied; the loads of the steady-state loop are unconditional
    if (n_full > 0) {
        load(w0, h0, 0, true);
        if (n_full > 1) load(w1, h1, 1, true);
        int c = 0;
        for (; c + 3 < n_full; c += 2) {
            stage(w0, h0);
            load(w0, h0, c + 2, true);
            compute();
            stage(w1, h1);
            load(w1, h1, c + 3, true);
            compute();
        }
        // remaining 1..3 full chunks
        if (c + 2 < n_full) {  // three left: c, c+1, c+2
            stage(w0, h0);
            load(w0, h0, c + 2, true);
            compute();
            stage(w1, h1);
            compute();
            stage(w0, h0);
            compute();
        } else if (c + 1 < n_full) {  // two left
            stage(w0, h0);
            compute();
            stage(w1, h1);
            compute();
        } else {
            stage(w0, h0);
            compute();
        }
    }
    if (tail) {
        load(w0, h0, n_full, false);
        stage(w0, h0);
        compute();
    }
    topk_epilogue<1, NTX, false>(acc, tk, 0, 0, M, t0 * 16, NTX, V, 1, (int)min<int64_t>(M, 16), 0, 2);
}

template <int NT, int KS>
__global__ __launch_bounds__(256) void head_skinny2_kernel(const uint16_t* __restrict__ h,
                                                           const uint16_t* __restrict__ W, int64_t M,
                                                           int D, int64_t V, int64_t n_tiles,
                                                           float* __restrict__ part_val,
                                                           int* __restrict__ part_idx) {
    using C = Skinny2Cfg<NT, KS>;
    __shared__ __align__(16) unsigned char s_w[4][C::LDS_W];
    __shared__ float s_lval[4][16 * kTopK];
    __shared__ int s_lidx[4][16 * kTopK];
    __shared__ float s_cval[4][16 * kCap];
    __shared__ int s_cidx[4][16 * kCap];
    __shared__ __align__(16) float s_thr[4][16];
    __shared__ __align__(16) int s_thri[4][16];
    __shared__ int s_ccnt[4][16];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    TopkRows tk{s_lval[wave], s_lidx[wave], s_cval[wave], s_cidx[wave], s_thr[wave], s_thri[wave], s_ccnt[wave]};
    topk_init(tk, 16, lane, 64);
    wave_sync();

    const int64_t nw = (int64_t)gridDim.x * 4;
    const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
    const int64_t t_begin = gw * n_tiles / nw, t_end = (gw + 1) * n_tiles / nw;
    const __amdgpu_buffer_rsrc_t hsrc = make_rsrc(h, M * D * 2);

    int64_t t0 = t_begin;
    for (; t0 + NT <= t_end; t0 += NT) skinny2_tiles<NT, KS>(hsrc, W, M, D, V, t0, tk, s_w[wave]);
    for (; t0 < t_end; ++t0) skinny2_tiles<1, KS>(hsrc, W, M, D, V, t0, tk, s_w[wave]);

    __syncthreads();
    const int S = gridDim.x;
    for (int r = wave; r < min<int64_t>(M, 16); r += 4) {
        const int src = lane >> 4, k = lane & 15;
        float v = s_lval[src][r * kTopK + k];
        int ix = s_lidx[src][r * kTopK + k];
        bitonic_desc<64>(v, ix);
        if (lane < kTopK) {
            const int64_t o = ((int64_t)r * S + blockIdx.x) * kTopK + lane;
            part_val[o] = v;
            part_idx[o] = ix;
        }
    }
}

// --------------------------------------------------------------- wide GEMM
template <int MW, int NT, int WM, int WN, int KS>
struct WideCfg {
    static constexpr int MB = 16 * MW * WM;
    static constexpr int KC = 32 * KS;
    static constexpr int LDS_ROW = KC + 8;  // bf16, 16-byte pad against bank conflicts
    static constexpr int THREADS = 64 * WM * WN;
    static constexpr int STRIP = 16 * NT * WN;
    static constexpr int H_PIECES = MB * KC / 8;
    static constexpr int H_PER_THREAD = (H_PIECES + THREADS - 1) / THREADS;
    static constexpr size_t LDS_H = (size_t)MB * LDS_ROW * 2;
    static constexpr size_t LDS_TOPK = (size_t)MB * (kTopK + kCap) * 8 + (size_t)MB * 12;
    static constexpr size_t LDS = LDS_H + LDS_TOPK;
};

template <int MW, int NT, int WM, int WN, int KS>
__global__ __launch_bounds__(64 * WM * WN) void head_wide_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int64_t M, int D, int64_t V,
    int n_strips, int S, int n_mb, float* __restrict__ part_val, int* __restrict__ part_idx) {
    using C = WideCfg<MW, NT, WM, WN, KS>;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
    unsigned char* tp = smem + C::LDS_H;
    TopkRows tk;
    tk.lval = reinterpret_cast<float*>(tp);
    tk.lidx = reinterpret_cast<int*>(tp + C::MB * kTopK * 4);
    tk.cval = reinterpret_cast<float*>(tp + C::MB * kTopK * 8);
    tk.cidx = reinterpret_cast<int*>(tp + C::MB * kTopK * 8 + C::MB * kCap * 4);
    tk.thr = reinterpret_cast<float*>(tp + C::MB * (kTopK + kCap) * 8);
    tk.thri = reinterpret_cast<int*>(tk.thr + C::MB);
    tk.ccnt = tk.thri + C::MB;

    // workgroup -> (M-block, slot): the M-blocks of one slot are dispatched
    // back to back on the same XCD so they share the slot's W rows in L2.
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int kq = L >> 3;
    const int mb = kq % n_mb;
    const int slot = (kq / n_mb) * 8 + xcd;
    if (slot >= S) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ln = lane & 15, lg = lane >> 4;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t m0 = (int64_t)mb * C::MB;
    const int rows_blk = (int)min<int64_t>(C::MB, M - m0);
    const int mw_act = max(0, min(MW, (rows_blk - wm * 16 * MW + 15) / 16));
    topk_init(tk, C::MB, tid, C::THREADS);
    __syncthreads();

    const int s_begin = (int)((int64_t)slot * n_strips / S);
    const int s_end = (int)((int64_t)(slot + 1) * n_strips / S);
    const int n_chunks = (D + C::KC - 1) / C::KC;
    const int n_full = D / C::KC;  // chunks without a ragged end
    u32x4 hreg[C::H_PER_THREAD];

    // rows past the block repeat its last row (never read back); only a ragged
    // last chunk masks k
    auto load_h = [&](int c, bool full) {
        const int kc0 = c * C::KC;
#pragma unroll
        for (int u = 0; u < C::H_PER_THREAD; ++u) {
            const int p = min(tid + u * C::THREADS, C::H_PIECES - 1);
            const int pr = p / (C::KC / 8), cp = p % (C::KC / 8);
            const uint16_t* row = h + (m0 + min(pr, rows_blk - 1)) * D;
            const int k = kc0 + cp * 8;
            if (full) {
                hreg[u] = ldg(row + k);
            } else {
                const u32x4 v = ldg(row + (k < D ? k : 0));
                hreg[u] = k < D ? v : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_h = [&]() {
#pragma unroll
        for (int u = 0; u < C::H_PER_THREAD; ++u) {
            const int p = tid + u * C::THREADS;
            if (p < C::H_PIECES) {
                const int pr = p / (C::KC / 8), cp = p % (C::KC / 8);
                *reinterpret_cast<u32x4*>(hs + pr * C::LDS_ROW + cp * 8) = hreg[u];
            }
        }
    };

    for (int strip = s_begin; strip < s_end; ++strip) {
        const int64_t col0 = (int64_t)strip * C::STRIP + wn * NT * 16;
        const int nt_act = (int)max<int64_t>(0, min<int64_t>(NT, (V - col0 + 15) / 16));
        const uint16_t* wrow[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            int64_t rr = col0 + nt * 16 + ln;
            if (rr > V - 1) rr = V - 1;
            wrow[nt] = W + rr * D;
        }
        floatx4 acc[MW][NT];
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
        u32x4 wa[NT][KS], wb[NT][KS];

        auto load_w = [&](u32x4 (&w)[NT][KS], int c, bool full) {
            const int kc0 = c * C::KC;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int s = 0; s < KS; ++s) load_frag<KS>(w[nt][s], wrow[nt], kc0, s, lg, D, full, true);
        };
        // A fragments of M-tile mt+1 are read from LDS while tile mt's MFMAs
        // issue; the scheduling barrier keeps the compiler from hoisting all
        // MW*KS fragments at once (register pressure).
        auto compute = [&](const u32x4 (&w)[NT][KS]) {
            const uint16_t* src = hs + (wm * 16 * MW + ln) * C::LDS_ROW + lg * 8;
            u32x4 a_cur[KS], a_nxt[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) a_cur[s] = *reinterpret_cast<const u32x4*>(src + 32 * s);
#pragma unroll
            for (int mt = 0; mt < MW; ++mt) {
                if (mt < mw_act) {
                    if (mt + 1 < MW && mt + 1 < mw_act) {
#pragma unroll
                        for (int s = 0; s < KS; ++s)
                            a_nxt[s] = *reinterpret_cast<const u32x4*>(src + (mt + 1) * 16 * C::LDS_ROW + 32 * s);
                    }
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const bf16x8 av = __builtin_bit_cast(bf16x8, a_cur[s]);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    av, __builtin_bit_cast(bf16x8, w[nt][s]), acc[mt][nt], 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int s = 0; s < KS; ++s) a_cur[s] = a_nxt[s];
                }
            }
        };
        // one chunk: h(c+1) to registers, W(c+1) in flight, MFMAs on chunk c,
        // then h(c+1) into LDS (h loads are issued before the W loads so that
        // waiting for them leaves the W loads outstanding)
        // steady state over the full chunks: chunk c+1 is always loaded while
        // chunk c computes, so the loads are unconditional; a ragged last
        // chunk of the hidden dimension follows with masked loads
        auto step = [&](const u32x4 (&cur)[NT][KS], u32x4 (&ahead)[NT][KS], int c) {
            load_h(c + 1, true);
            load_w(ahead, c + 1, true);
            compute(cur);
            __syncthreads();
            store_h();
            __syncthreads();
        };
        if (n_full > 0) {
            load_h(0, true);
            load_w(wa, 0, true);
            store_h();
            __syncthreads();
            int c = 0;
            for (; c + 2 < n_full; c += 2) {
                step(wa, wb, c);
                step(wb, wa, c + 1);
            }
            if (c + 1 < n_full) {
                step(wa, wb, c);
                compute(wb);
            } else {
                compute(wa);
            }
            __syncthreads();
        }
        if (n_full < n_chunks) {
            load_h(n_full, false);
            load_w(wa, n_full, false);
            store_h();
            __syncthreads();
            compute(wa);
            __syncthreads();
        }
        topk_epilogue<MW, NT, true>(acc, tk, wm * 16 * MW, m0 + wm * 16 * MW, M, col0, nt_act, V, mw_act,
                                    rows_blk, wave * 2, WM * WN * 2);
    }

    for (int e = tid; e < rows_blk * kTopK; e += C::THREADS) {
        const int r = e / kTopK, k = e % kTopK;
        const int64_t o = ((m0 + r) * S + slot) * kTopK + k;
        part_val[o] = tk.lval[e];
        part_idx[o] = tk.lidx[e];
    }
}

// ---------------------------------------------------------------- merge
// One workgroup of 10 wavefronts per row.
// (1) The row's S sorted partial lists (S <= kMaxLists) are copied to LDS.
// (2) k-way extraction: a wavefront takes 64 lists (one per lane), and 20
//     times pops the best of the 64 list heads (wavefront arg-max; the winning
//     lane advances in its list) -> a sorted top-20 per group of 64 lists.
// (3) One wavefront extracts the top 20 of the group results the same way.
// (4) Each wavefront re-scores two of those 20 exactly: all loads of the h
//     row and both W rows are issued before any arithmetic (one HBM round
//     trip); bf16 products are exact in float64 and summed in float64.
// (5) Rank by the exact value (ties: lower id) and write the best 16.
constexpr int kMaxLists = 1024;
constexpr int kMergeSeg = 10;  // 16-byte pieces per lane per pass over D

// Wavefront arg-max of (v, i) in ranks_before order; returns the winning lane.
__device__ __forceinline__ int wave_argmax_lane(float& v, int& i) {
    int who = threadIdx.x & 63;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float v2 = __shfl_xor(v, off);
        const int i2 = __shfl_xor(i, off);
        const int w2 = __shfl_xor(who, off);
        if (ranks_before(v2, i2, v, i) || (v2 == v && i2 == i && w2 < who)) {
            v = v2;
            i = i2;
            who = w2;
        }
    }
    return who;
}

// Pop the kRescore best entries of up to 64 sorted lists of length len held
// in LDS (list l of lane l at lv/li + l * len); results to ov/oi.
__device__ __forceinline__ void extract_top(const float* lv, const int* li, int len, int nlists, float* ov,
                                            int* oi) {
    const int lane = threadIdx.x & 63;
    int pos = 0;
    float hv = lane < nlists ? lv[lane * len] : -INFINITY;
    int hi = lane < nlists ? li[lane * len] : 0x7FFFFFFF;
    for (int k = 0; k < kRescore; ++k) {
        float bv = hv;
        int bi = hi;
        const int who = wave_argmax_lane(bv, bi);
        if (lane == 0) {
            ov[k] = bv;
            oi[k] = bi;
        }
        if (lane == who) {
            ++pos;
            hv = pos < len ? lv[lane * len + pos] : -INFINITY;
            hi = pos < len ? li[lane * len + pos] : 0x7FFFFFFF;
        }
    }
}

__global__ __launch_bounds__(kMergeThreads) void head_merge_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int D, int S,
    const float* __restrict__ part_val, const int* __restrict__ part_idx,
    float* __restrict__ top_val, int32_t* __restrict__ top_idx) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* lv = reinterpret_cast<float*>(smem);              // [S][16]
    int* li = reinterpret_cast<int*>(lv + (size_t)S * kTopK);  // [S][16]
    __shared__ float gv[kMaxLists / 64][kRescore];
    __shared__ int gi[kMaxLists / 64][kRescore];
    __shared__ float sel_v[kRescore];
    __shared__ int sel_i[kRescore];
    __shared__ double sel_z[kRescore];

    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const float4* pv4 = reinterpret_cast<const float4*>(part_val + m * S * kTopK);
    const int4* pi4 = reinterpret_cast<const int4*>(part_idx + m * S * kTopK);
    for (int e = tid; e < S * kTopK / 4; e += kMergeThreads) {
        reinterpret_cast<float4*>(lv)[e] = pv4[e];
        reinterpret_cast<int4*>(li)[e] = pi4[e];
    }
    __syncthreads();
    const int ng = (S + 63) / 64;
    for (int g = wave; g < ng; g += kMergeThreads / 64)
        extract_top(lv + g * 64 * kTopK, li + g * 64 * kTopK, kTopK, min(64, S - g * 64), gv[g], gi[g]);
    __syncthreads();
    if (wave == 0) extract_top(&gv[0][0], &gi[0][0], kRescore, ng, sel_v, sel_i);
    __syncthreads();
    int ns = 0;
    for (int c = 0; c < kRescore; ++c) ns += (sel_i[c] != 0x7FFFFFFF) ? 1 : 0;

    // exact re-scoring, two candidates per wavefront
    const uint16_t* hr = h + m * D;
    const int c0 = 2 * wave, c1 = 2 * wave + 1;
    if (c0 < ns) {
        const bool has1 = c1 < ns;
        const uint16_t* w0 = W + (int64_t)sel_i[c0] * D;
        const uint16_t* w1 = W + (int64_t)sel_i[has1 ? c1 : c0] * D;
        double acc0 = 0.0, acc1 = 0.0;
        for (int seg = 0; seg < D; seg += kMergeSeg * 512) {
            u32x4 ha[kMergeSeg], wa[kMergeSeg], wb[kMergeSeg];
#pragma unroll
            for (int j = 0; j < kMergeSeg; ++j) {
                const int d = min(seg + (j * 64 + lane) * 8, D - 8);
                ha[j] = *reinterpret_cast<const u32x4*>(hr + d);
                wa[j] = *reinterpret_cast<const u32x4*>(w0 + d);
                wb[j] = *reinterpret_cast<const u32x4*>(w1 + d);
            }
#pragma unroll
            for (int j = 0; j < kMergeSeg; ++j) {
                if (seg + (j * 64 + lane) * 8 < D) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const double a0 = (double)bf16_to_f32(ha[j][q] & 0xFFFFu);
                        const double a1 = (double)bf16_to_f32(ha[j][q] >> 16);
                        acc0 = fma(a0, (double)bf16_to_f32(wa[j][q] & 0xFFFFu), acc0);
                        acc0 = fma(a1, (double)bf16_to_f32(wa[j][q] >> 16), acc0);
                        acc1 = fma(a0, (double)bf16_to_f32(wb[j][q] & 0xFFFFu), acc1);
                        acc1 = fma(a1, (double)bf16_to_f32(wb[j][q] >> 16), acc1);
                    }
                }
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            acc0 += __shfl_xor(acc0, off);
            acc1 += __shfl_xor(acc1, off);
        }
        if (lane == 0) {
            sel_z[c0] = acc0;
            if (has1) sel_z[c1] = acc1;
        }
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
namespace {

enum HeadVariant { kSkinny = 0, kWide64 = 1, kWide128 = 2, kWide256 = 3 };

struct HeadPlan {
    HeadVariant variant;
    int mb_rows;    // rows per M-block (wide) / 16 (skinny)
    int strip;      // vocabulary rows per strip (wide)
    int S;          // partial lists per row (= workgroups per M-block)
    int n_mb;
    int n_strips;
};

using Wide64 = WideCfg<4, 2, 1, 4, 4>;
using Wide128 = WideCfg<8, 2, 1, 4, 4>;
using Wide256 = WideCfg<8, 2, 2, 4, 4>;
constexpr int kSkinnyNT = 2, kSkinnyKS = 4, kSkinnyWG = 512;  // 2 workgroups (8 wavefronts) per CU

HeadPlan head_plan(int64_t M, int64_t V) {
    HeadPlan p{};
    if (M <= 16) {
        p.variant = kSkinny;
        p.mb_rows = 16;
        p.n_mb = 1;
        const int64_t n_tiles = (V + 15) / 16;
        const int64_t want = (n_tiles + 3) / 4;  // at least one tile per wavefront
        p.S = (int)std::min<int64_t>(kSkinnyWG, want);
        p.strip = 16;
        p.n_strips = (int)n_tiles;
        return p;
    }
    int slots;
    if (M <= 64) {
        p.variant = kWide64;
        p.mb_rows = Wide64::MB;
        p.strip = Wide64::STRIP;
        slots = 512;
    } else if (M <= 128) {
        p.variant = kWide128;
        p.mb_rows = Wide128::MB;
        p.strip = Wide128::STRIP;
        slots = 512;
    } else {
        p.variant = kWide256;
        p.mb_rows = Wide256::MB;
        p.strip = Wide256::STRIP;
        slots = 256;  // one 8-wavefront workgroup per CU
    }
    p.n_mb = (int)((M + p.mb_rows - 1) / p.mb_rows);
    p.n_strips = (int)((V + p.strip - 1) / p.strip);
    int s = std::max(1, slots / p.n_mb);
    s = std::min(s, p.n_strips);
    p.S = std::min((s + 7) / 8 * 8, kMaxLists);  // whole XCD rounds of slots
    return p;
}

template <typename Cfg, typename K>
void set_lds(K kernel) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)Cfg::LDS);
}

std::once_flag g_head_attr_once;

}  // namespace

size_t head_workspace_bytes(int64_t M, int64_t V) {
    const HeadPlan p = head_plan(M, V);
    return (size_t)M * p.S * kTopK * 8;
}

int launch_head_topk(const uint16_t* h, const uint16_t* W, int64_t M, int D, int64_t V,
                     float* top_val, int32_t* top_idx, void* ws, hipStream_t stream) {
    std::call_once(g_head_attr_once, []() {
        set_lds<Wide64>(&head_wide_kernel<4, 2, 1, 4, 4>);
        set_lds<Wide128>(&head_wide_kernel<8, 2, 1, 4, 4>);
        set_lds<Wide256>(&head_wide_kernel<8, 2, 2, 4, 4>);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&head_merge_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLists * kTopK * 8);
    });
    const HeadPlan p = head_plan(M, V);
    float* pv = reinterpret_cast<float*>(ws);
    int* pi = reinterpret_cast<int*>(pv + (size_t)M * p.S * kTopK);
    const dim3 grid(p.S * p.n_mb);
    switch (p.variant) {
        case kSkinny:
            hipLaunchKernelGGL((head_skinny2_kernel<kSkinnyNT, kSkinnyKS>), dim3(p.S), dim3(256), 0, stream, h, W, M,
                               D, V, (int64_t)p.n_strips, pv, pi);
            break;
        case kWide64:
            hipLaunchKernelGGL((head_wide_kernel<4, 2, 1, 4, 4>), grid, dim3(Wide64::THREADS), Wide64::LDS, stream,
                               h, W, M, D, V, p.n_strips, p.S, p.n_mb, pv, pi);
            break;
        case kWide128:
            hipLaunchKernelGGL((head_wide_kernel<8, 2, 1, 4, 4>), grid, dim3(Wide128::THREADS), Wide128::LDS, stream,
                               h, W, M, D, V, p.n_strips, p.S, p.n_mb, pv, pi);
            break;
        default:
            hipLaunchKernelGGL((head_wide_kernel<8, 2, 2, 4, 4>), grid, dim3(Wide256::THREADS), Wide256::LDS, stream,
                               h, W, M, D, V, p.n_strips, p.S, p.n_mb, pv, pi);
            break;
    }
    int st = launch_status();
    if (st != DFLASH_OK) return st;
    const size_t lds = (size_t)p.S * kTopK * 8;
    hipLaunchKernelGGL(head_merge_kernel, dim3((unsigned)M), dim3(kMergeThreads), lds, stream, h, W, D, p.S, pv,
                       pi, top_val, top_idx);
    return launch_status();
}

}  // namespace dflash
