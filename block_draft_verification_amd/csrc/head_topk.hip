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
//   inside the stream.  At the end the wavefronts of a workgroup merge their
//   lists.
// * head_wide_kernel (M > 16): a workgroup of 2 x WN wavefronts owns an
//   M-block of 32*MW rows of h and a contiguous range of vocabulary tiles,
//   walked in strips of 16*NT*WN rows.  Per chunk of the hidden dimension the
//   whole workgroup stages the h rows and the strip's W rows in LDS
//   (row-contiguous buffer loads, several chunks ahead in registers) and every
//   wavefront multiplies its 16*MW x 16*NT tile from there.  The M-blocks of
//   one range are dispatched next to each other on the same XCD so that they
//   share W through its L2.
// * The top-16 epilogue: after a tile, the float32 logits still in the
//   accumulators are compared with each row's running 16th-best entry (value,
//   then id); the few survivors go to a bounded per-row buffer and are merged
//   into the row's sorted list by a 32-lane bitonic sort, retrying anything
//   that overflowed the buffer.
// * head_merge_kernel: see below.

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "keysort.hpp"

namespace dflash {

// LDS row padding of the staged tiles.  A fragment read (lane l: row l % 16,
// 16 bytes at column granule l / 16) is serviced by gfx950 for lanes 0-7 and
// 16-23 together (then 8-15 with 24-31, ...), i.e. rows 0..7 at two adjacent
// 16-byte granules.  With a pitch of p granules those fall on bank groups
// {p r, p r + 1 : r < 8} mod 16, all distinct iff p = 2 (mod 4); the data part
// (KC*2 bytes, KC a multiple of 32) is 0 (mod 4) granules, so 2 granules of
// padding.  (Measured: 16 bytes of padding doubles the cost of every fragment
// read; 32 bytes reaches the contiguous rate.)
constexpr int kPitchPad = 32;

constexpr int kCap = 16;        // candidate slots per row between merges
static_assert(kCap == 16, "one buffered candidate per lane of a 16-lane row");
constexpr int kRescore = 20;    // float32 candidates re-scored exactly per row
constexpr int kMergeThreads = 64 * (kRescore / 2);  // one wavefront per two re-scored candidates

__device__ __forceinline__ u32x4 ldg_stream(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ldg(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

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
    uint32_t* seed;  // [rows][16] first-strip threshold seeds (workgroup-shared lists only)
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
//   col0: global vocabulary id of fragment 0's column 0; fragment nt starts
//         col_step ids further on
//   merge rows [0, n_merge_rows) by 16-lane rows of wavefronts: row group
//   g = q0, q0 + q_step, ... (lane >> 4 is the group within a wavefront)
// Candidates (ranking before the row's 16th-best entry) go to a kCap-slot
// buffer; each row with candidates then sorts them ascending across 16 lanes,
// takes the lane-wise maximum with its descending list (the top 16 of both,
// as a bitonic sequence) and sorts that descending.  Candidates that found
// the buffer full are retried in another round.
// WG = true: state shared by the workgroup (barriers); false: wave-private.
template <int MW, int NT, bool WG>
__device__ __forceinline__ void topk_epilogue(const floatx4 (&acc)[MW][NT], TopkRows t, int rbase, int64_t grow0,
                              int64_t M, int64_t col0, int col_step, int nt_act, int64_t V, int mw_act,
                              int n_merge_rows, int q0, int q_step, bool seed = false) {
    // The empty asm statements make lane, M and rbase opaque at each call, so
    // that nothing derived from them is hoisted out of the caller's tile loop
    // (where it would stay live through the streaming loop and spill).
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    asm volatile("" : "+s"(M));
    asm volatile("" : "+v"(rbase));
    const int ln = lane & 15, lg = lane >> 4;
    // pending[mt] bit nt * 4 + q: value acc[mt][nt][q] still has to be
    // offered (initially: every value of a real row and vocabulary id)
    uint32_t pending[MW];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
        uint32_t p = 0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const bool col_ok = nt < nt_act && col0 + (int64_t)nt * col_step + ln < V;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (col_ok && mt < mw_act && grow0 + mt * 16 + 4 * lg + q < M) p |= 1u << (nt * 4 + q);
        }
        pending[mt] = p;
    }
    if (WG && seed) {
        // Threshold seed for lists that are still empty: for each row and lane
        // position ln, the largest of the values the wavefronts hold there
        // (distinct columns); the smallest of those 16 maxima is a value that
        // at least 16 distinct entries of the row reach, hence no greater than
        // the row's 16th best.  Rows start with it as threshold (id INT_MAX:
        // any value at least that large stays a candidate), which keeps most of
        // the first strip out of the merge rounds.
        for (int e = threadIdx.x; e < n_merge_rows * 16; e += blockDim.x) t.seed[e] = 0u;
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < MW; ++mt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float m = -INFINITY;
                bool any = false;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    if (pending[mt] & (1u << (nt * 4 + q))) {
                        m = any ? fmaxf(m, acc[mt][nt][q]) : acc[mt][nt][q];
                        any = true;
                    }
                if (any) atomicMax(&t.seed[(rbase + mt * 16 + 4 * lg + q) * 16 + ln], (uint32_t)(rank_key(m, 0) >> 32));
            }
        }
        __syncthreads();
        const int li = lane & 15;
        for (int r = q0 + (lane >> 4); r < n_merge_rows; r += q_step) {
            uint32_t k = t.seed[r * 16 + li];
            k = min(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, kDppX1, 0xF, 0xF, true));
            k = min(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, kDppX2, 0xF, 0xF, true));
            k = min(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, kDppX7, 0xF, 0xF, true));
            k = min(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, kDppX15, 0xF, 0xF, true));
            // key 0: some lane position held no value, so no bound
            if (li == 0 && k > (uint32_t)(kEmptyKey >> 32)) {
                t.thr[r] = key_value((uint64_t)k << 32);
                t.thri[r] = 0x7FFFFFFF;
            }
        }
        __syncthreads();
    }
    while (true) {
        // Per 16-row tile: compare every pending value with its row's
        // threshold, then (only if some lane has a candidate) reserve the
        // slots with all atomics in flight together, then store.
#pragma unroll
        for (int mt = 0; mt < MW; ++mt) {
            if (__ballot(pending[mt] != 0) == 0) continue;
            const int r0 = rbase + mt * 16 + 4 * lg;
            const float4 t4 = *reinterpret_cast<const float4*>(t.thr + r0);
            const int4 i4 = *reinterpret_cast<const int4*>(t.thri + r0);
            const float tq[4] = {t4.x, t4.y, t4.z, t4.w};
            const int iq[4] = {i4.x, i4.y, i4.z, i4.w};
            uint32_t cf = 0;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int col = (int)(col0 + (int64_t)nt * col_step + ln);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t bit = 1u << (nt * 4 + q);
                    if ((pending[mt] & bit) && ranks_before(acc[mt][nt][q], col, tq[q], iq[q])) cf |= bit;
                }
            }
            uint32_t pend = 0;
            if (__ballot(cf != 0) != 0) {
                int slot[NT * 4];
#pragma unroll
                for (int b = 0; b < NT * 4; ++b) {
                    slot[b] = kCap;
                    if (cf & (1u << b)) slot[b] = atomicAdd(&t.ccnt[r0 + (b & 3)], 1);
                }
#pragma unroll
                for (int b = 0; b < NT * 4; ++b) {
                    if (cf & (1u << b)) {
                        const int nt = b >> 2, q = b & 3, r = r0 + q;
                        if (slot[b] < kCap) {
                            t.cval[r * kCap + slot[b]] = acc[mt][nt][q];
                            t.cidx[r * kCap + slot[b]] = (int)(col0 + (int64_t)nt * col_step + ln);
                        } else {
                            pend |= 1u << b;
                        }
                    }
                }
            }
            pending[mt] = pend;
        }
        if (WG) __syncthreads(); else wave_sync();
        const int li = lane & 15;
        for (int r = q0 + (lane >> 4); r < n_merge_rows; r += q_step) {
            const int cnt = min(t.ccnt[r], kCap);
            if (cnt == 0) continue;
            const uint64_t kl = rank_key(t.lval[r * kTopK + li], t.lidx[r * kTopK + li]);
            const uint64_t kc = li < cnt ? rank_key(t.cval[r * kCap + li], t.cidx[r * kCap + li]) : kEmptyKey;
            uint64_t m = sort16<false>(kc, li);
            m = m > kl ? m : kl;
            m = merge16_desc(m, li);
            const float v = key_value(m);
            const int ix = key_id(m);
            t.lval[r * kTopK + li] = v;
            t.lidx[r * kTopK + li] = ix;
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

// ------------------------------------------- softmax-statistics epilogue
// For the sampling verifier fused into the target's LM head: instead of
// top-16 lists, the head kernels write, per (row, 16-column vocabulary tile),
// the tile's maximum logit m and s = sum over its columns of
// exp((z - m) / tau), from the float32 accumulators (s in float32 through
// v_exp_f32, so relative errors of ~1e-7 on top of the logits' own).
struct TileStats {
    float2* rec;      // [M][n16]
    int64_t n16;      // tiles per row, ceil(V / 16)
    float k2;         // (1 / tau) * log2(e)
};

__device__ __forceinline__ float dpp_f32(float x, int li, int which) {
    const uint32_t u = __float_as_uint(x);
    uint32_t r;
    switch (which) {
        case 1: r = (uint32_t)__builtin_amdgcn_mov_dpp((int)u, kDppX1, 0xF, 0xF, true); break;
        case 2: r = (uint32_t)__builtin_amdgcn_mov_dpp((int)u, kDppX2, 0xF, 0xF, true); break;
        case 8: r = (uint32_t)__builtin_amdgcn_mov_dpp((int)u, kDppX8, 0xF, 0xF, true); break;
        default: {  // lane ^ 4 inside the row
            const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x104, 0xF, 0xF, true);
            const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x114, 0xF, 0xF, true);
            r = (li & 4) ? dn : up;
        }
    }
    return __uint_as_float(r);
}

// acc[mt][nt][q] holds row grow0 + 16 mt + 4 (lane / 16) + q and column
// col0 + nt * col_step + lane % 16 (tiles start at multiples of 16).
template <int MW, int NT>
__device__ __forceinline__ void stats_epilogue(const floatx4 (&acc)[MW][NT], const TileStats& st, int64_t grow0,
                                               int64_t M, int64_t col0, int col_step, int nt_act, int64_t V,
                                               int mw_act) {
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
        if (mt >= mw_act) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt >= nt_act) continue;
            const int64_t tc = col0 + (int64_t)nt * col_step;  // the tile's first column
            const bool cok = tc + ln < V;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float z = acc[mt][nt][q];
                float m = cok ? z : -INFINITY;
                m = fmaxf(m, dpp_f32(m, ln, 1));
                m = fmaxf(m, dpp_f32(m, ln, 2));
                m = fmaxf(m, dpp_f32(m, ln, 4));
                m = fmaxf(m, dpp_f32(m, ln, 8));
                float e = cok ? __builtin_amdgcn_exp2f((z - m) * st.k2) : 0.0f;
                e += dpp_f32(e, ln, 1);
                e += dpp_f32(e, ln, 2);
                e += dpp_f32(e, ln, 4);
                e += dpp_f32(e, ln, 8);
                const int64_t row = grow0 + mt * 16 + 4 * lg + q;
                if (ln == 0 && row < M) st.rec[row * st.n16 + tc / 16] = make_float2(m, e);
            }
        }
    }
}

// ------------------------------------------------- skinny GEMM, LDS-staged W
// The same wavefront-independent scheme, but W reaches the MFMAs through LDS
// so that its HBM reads are row-contiguous: per chunk the wavefront's 16*NT
// rows x KC columns are read as 512/KC rows per load instruction (64 lanes x
// 16 contiguous bytes), written to the wavefront's private LDS tile, and read
// back in the MFMA operand layout (row pitch KC*2 + kPitchPad bytes).
// Contiguous runs of 2*KC bytes per row instead of 64-byte pieces keep HBM
// pages open.
template <int NT, int KS>
struct Skinny2Cfg {
    static constexpr int KC = 32 * KS;
    static constexpr int R = 16 * NT;                 // W rows per wavefront tile
    static constexpr int ROWB = KC * 2 + kPitchPad;   // LDS bytes per staged row
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
template <int NTX, int KS, bool STATS = false>
__device__ __forceinline__ void skinny2_tiles(__amdgpu_buffer_rsrc_t hsrc, const uint16_t* __restrict__ W,
                                              int64_t M, int D, int64_t V, int64_t row0, TopkRows tk,
                                              unsigned char* __restrict__ wl, const TileStats& st) {
    using C = Skinny2Cfg<NTX, KS>;
    constexpr int KC = C::KC;
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15, lg = lane >> 4;
    const int ri = lane / C::PIECES, pj = lane % C::PIECES;
    const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(W + row0 * D, (V - row0) * D * 2);
    // The row goes into the lane offset (range-checked against the resource),
    // the chunk's column offset into the scalar offset.
    const int voff = ri * D * 2 + pj * 16;
    const int qstride = C::ROWS_PER_LOAD * D * 2;
    unsigned char* hl = wl + C::R * C::ROWB;
    floatx4 acc[1][NTX];
#pragma unroll
    for (int nt = 0; nt < NTX; ++nt) acc[0][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    u32x4 w0[C::LOADS], w1[C::LOADS], h0[C::ALOADS], h1[C::ALOADS];
    const int n_full = D / KC;
    const bool tail = n_full * KC < D;

    auto load = [&](u32x4 (&w)[C::LOADS], u32x4 (&hh)[C::ALOADS], int c, bool full) {
        const int kc0 = c * KC;
        const bool in = full || kc0 + pj * 8 < D;
#pragma unroll
        for (int q = 0; q < C::ALOADS; ++q)
            hh[q] = __builtin_amdgcn_raw_buffer_load_b128(hsrc, in ? voff + q * qstride : kOffNone, kc0 * 2, 0);
#pragma unroll
        for (int q = 0; q < C::LOADS; ++q)
            w[q] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, in ? voff + q * qstride : kOffNone, kc0 * 2, kBufNT);
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
    auto compute = [&]() __attribute__((always_inline)) {
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
    if constexpr (STATS)
        stats_epilogue<1, NTX>(acc, st, 0, M, row0, 16, NTX, V, 1);
    else
        topk_epilogue<1, NTX, false>(acc, tk, 0, 0, M, row0, 16, NTX, V, 1, (int)min<int64_t>(M, 16), 0, 4);
}

// WAVES wavefronts per workgroup (4 or 8).
template <int NT, int KS, int WAVES>
struct SkinnyLds {
    using C = Skinny2Cfg<NT, KS>;
    static constexpr size_t TILES = (size_t)WAVES * C::LDS_W;
    static constexpr size_t LISTS = (size_t)WAVES * 16 * (kTopK * 8 + kCap * 8 + 12);
    static constexpr size_t BYTES = TILES + LISTS;
    static_assert(BYTES <= 160 * 1024, "LDS per workgroup");
};

template <int NT, int KS, int WAVES, bool STATS = false>
__global__ __launch_bounds__(64 * WAVES) void head_skinny2_kernel(const uint16_t* __restrict__ h,
                                                                 const uint16_t* __restrict__ W, int64_t M,
                                                                 int D, int64_t V,
                                                                 float* __restrict__ part_val,
                                                                 int* __restrict__ part_idx, TileStats st) {
    using C = Skinny2Cfg<NT, KS>;
    using Lds = SkinnyLds<NT, KS, WAVES>;
    extern __shared__ __align__(16) unsigned char smem[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    unsigned char* s_w = smem + (size_t)wave * C::LDS_W;
    // per-wavefront list state: lval, lidx [16][16]; cval, cidx [16][kCap]; thr, thri, ccnt [16]
    auto lists = [&](int w) { return smem + Lds::TILES + (size_t)w * 16 * (kTopK * 8 + kCap * 8 + 12); };
    auto make_rows = [&](int w) {
        unsigned char* b = lists(w);
        TopkRows t;
        t.lval = reinterpret_cast<float*>(b);
        t.lidx = reinterpret_cast<int*>(b + 16 * kTopK * 4);
        t.cval = reinterpret_cast<float*>(b + 16 * kTopK * 8);
        t.cidx = reinterpret_cast<int*>(b + 16 * kTopK * 8 + 16 * kCap * 4);
        t.thr = reinterpret_cast<float*>(b + 16 * kTopK * 8 + 16 * kCap * 8);
        t.thri = reinterpret_cast<int*>(t.thr + 16);
        t.ccnt = t.thri + 16;
        t.seed = nullptr;
        return t;
    };
    TopkRows tk = make_rows(wave);
    topk_init(tk, 16, lane, 64);
    wave_sync();

    // Each wavefront owns a contiguous range of vocabulary rows, balanced to
    // within one row (not whole 16-row tiles, whose count per wavefront would
    // differ by one tile): its last tile may be partial, and the range end
    // bounds both the buffer resource (rows past it load as zeros, without
    // memory traffic) and the ids the epilogue admits.
    const int64_t nw = (int64_t)gridDim.x * WAVES;
    const int64_t gw = (int64_t)blockIdx.x * WAVES + wave;
    const __amdgpu_buffer_rsrc_t hsrc = make_rsrc(h, M * D * 2);
    if constexpr (STATS) {
        // whole 16-row tiles (the statistics are kept per vocabulary tile)
        const int64_t n_tiles = (V + 15) / 16;
        const int64_t t_begin = gw * n_tiles / nw, t_end = (gw + 1) * n_tiles / nw;
        int64_t t = t_begin;
        for (; t + NT <= t_end; t += NT) skinny2_tiles<NT, KS, true>(hsrc, W, M, D, V, t * 16, tk, s_w, st);
        for (; t < t_end; ++t) skinny2_tiles<1, KS, true>(hsrc, W, M, D, V, t * 16, tk, s_w, st);
        return;
    }
    const int64_t r_begin = gw * V / nw, r_end = (gw + 1) * V / nw;

    int64_t row = r_begin;
    for (; row + 16 * NT <= r_end; row += 16 * NT) skinny2_tiles<NT, KS>(hsrc, W, M, D, r_end, row, tk, s_w, st);
    for (; row < r_end; row += 16) skinny2_tiles<1, KS>(hsrc, W, M, D, r_end, row, tk, s_w, st);

    // workgroup list per row: the wavefronts' lists merged in groups of four
    // (a 64-lane sort each), then the groups' leaders (a 32-lane sort)
    __syncthreads();
    static_assert(WAVES == 4 || WAVES == 8, "4 or 8 wavefronts");
    const int S = gridDim.x;
    for (int r = wave; r < min<int64_t>(M, 16); r += WAVES) {
        const int src = lane >> 4, k = lane & 15;
        TopkRows ta = make_rows(src);
        float v = ta.lval[r * kTopK + k];
        int ix = ta.lidx[r * kTopK + k];
        bitonic_desc<64>(v, ix);
        if (WAVES == 8) {
            TopkRows tb = make_rows(4 + src);
            float vb = tb.lval[r * kTopK + k];
            int ib = tb.lidx[r * kTopK + k];
            bitonic_desc<64>(vb, ib);
            const float vs = __shfl(vb, lane & 15);
            const int is = __shfl(ib, lane & 15);
            if (lane >= 16 && lane < 32) {
                v = vs;
                ix = is;
            }
            bitonic_desc<32>(v, ix);
        }
        if (lane < kTopK) {
            const int64_t o = ((int64_t)r * S + blockIdx.x) * kTopK + lane;
            part_val[o] = v;
            part_idx[o] = ix;
        }
    }
}

// ------------------------------------------------ wide GEMM, LDS-staged W and h
// head_wide_kernel (M > 16): a workgroup of 2 x 4 wavefronts (two per SIMD)
// computes logits for an M-block of 32*MW rows of h against its contiguous,
// balanced range of 16-row vocabulary tiles, in strips of 64*NT rows.
// Wavefront (wm, wn) owns rows [16*MW*wm, 16*MW*(wm+1)) of the block and the
// strip's tiles wn, wn+4, wn+8, ... (interleaved, so that a partial last strip
// still spreads over all four SIMDs).  Per KC-wide chunk of the hidden
// dimension all 512 threads read the h rows and the strip's W rows
// row-contiguously with buffer loads DEPTH chunks ahead in registers, then
// store one chunk into an LDS tile (row pitch KC*2 + kPitchPad bytes, free of
// bank conflicts for fragment reads); with DBUF the tile is double
// buffered and each chunk costs one barrier instead of two.  Fragments come
// from LDS and the accumulators stay in registers.  A strip as wide as the
// M-block makes re-reading h from L2 cost no more than streaming W.  The
// top-16 epilogue's candidate buffers reuse the chunk tile's LDS.
template <int MW, int NT, int KS, int DEPTH, bool DBUF, int WN>
struct WideCfg {
    static constexpr int THREADS = 128 * WN;          // 2 x WN wavefronts
    static constexpr int KC = 32 * KS;
    static constexpr int MB = 32 * MW;                // rows of h per workgroup
    static constexpr int NB = 16 * WN * NT;           // W rows per strip
    static constexpr int ROWB = KC * 2 + kPitchPad;
    static constexpr int PIECES = KC / 8;             // 16-byte pieces per row and chunk
    static constexpr int RPL = THREADS / PIECES;      // rows per workgroup-wide load
    static constexpr int HLOADS = (MB + RPL - 1) / RPL;
    static constexpr int WLOADS = NB / RPL;
    static constexpr size_t TILE = (size_t)(MB + NB) * ROWB;
    static constexpr size_t LDS_BUF = TILE * (DBUF ? 2 : 1);
    static constexpr size_t LDS_LIST = (size_t)MB * kTopK * 8 + (size_t)MB * 12;
    static constexpr size_t LDS = LDS_BUF + LDS_LIST;
    static_assert((size_t)MB * (kCap * 8 + 16 * 4) <= LDS_BUF, "candidate buffers and seeds must fit in the chunk tile");
    static_assert(NB % RPL == 0 && WLOADS > 0, "whole W loads");
    static_assert(LDS <= 160 * 1024, "LDS per workgroup");
};

// Calls f(std::integral_constant<int, j>) for j = k (0 <= k < N), so that
// register arrays are indexed by a compile-time constant.
template <int N, int J = 0, class F>
__device__ __forceinline__ void with_slot(int k, F&& f) {
    if constexpr (J < N) {
        if (k == J) f(std::integral_constant<int, J>{});
        else with_slot<N, J + 1>(k, f);
    }
}

template <int MW, int NT, int KS, int DEPTH, bool DBUF, int WN, bool STATS = false>
__global__ __launch_bounds__(128 * WN) __attribute__((amdgpu_waves_per_eu(WN / 2, WN / 2)))
void head_wide_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int64_t M, int D,
                      int64_t V, int64_t n_tiles, int S, int n_mb, float* __restrict__ part_val,
                      int* __restrict__ part_idx, TileStats st) {
    using C = WideCfg<MW, NT, KS, DEPTH, DBUF, WN>;
    constexpr int KC = C::KC;
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* lp = smem + C::LDS_BUF;
    TopkRows tk;
    tk.lval = reinterpret_cast<float*>(lp);
    tk.lidx = reinterpret_cast<int*>(lp + C::MB * kTopK * 4);
    tk.thr = reinterpret_cast<float*>(lp + C::MB * kTopK * 8);
    tk.thri = reinterpret_cast<int*>(tk.thr + C::MB);
    tk.ccnt = tk.thri + C::MB;
    tk.cval = reinterpret_cast<float*>(smem);  // aliases the chunk tile (epilogue only)
    tk.cidx = reinterpret_cast<int*>(smem + C::MB * kCap * 4);
    tk.seed = reinterpret_cast<uint32_t*>(smem + C::MB * kCap * 8);  // also in the chunk tile

    // workgroup -> (M-block, slot): the M-blocks of one slot are dispatched
    // back to back on the same XCD so they share the slot's W rows in L2.
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int kq = L >> 3;
    const int mb = kq % n_mb;
    const int slot = (kq / n_mb) * 8 + xcd;
    if (slot >= S) return;

    const int tid = threadIdx.x;
    // wave-uniform (scalar) so that per-wavefront tile bounds become scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int ln = lane & 15, lg = lane >> 4;
    const int wm = wave / WN, wn = wave % WN;
    const int ri = tid / C::PIECES, pj = tid % C::PIECES;  // workgroup-wide load mapping
    const int64_t m0 = (int64_t)mb * C::MB;
    const int rows_blk = (int)min<int64_t>(C::MB, M - m0);
    const int mw_act = max(0, min(MW, (rows_blk - wm * 16 * MW + 15) / 16));
    topk_init(tk, C::MB, tid, C::THREADS);
    __syncthreads();

    // Rows go into the lane offset (range-checked: rows past the block or the
    // range read as zero), the chunk's column offset into the scalar offset.
    const __amdgpu_buffer_rsrc_t hsrc = make_rsrc(h + m0 * D, (int64_t)rows_blk * D * 2);
    const int voff = ri * D * 2 + pj * 16;
    const int qstride = C::RPL * D * 2;
    const int64_t t_begin = (int64_t)slot * n_tiles / S, t_end = (int64_t)(slot + 1) * n_tiles / S;
    const int n_full = D / KC;
    const bool ktail = n_full * KC < D;
    // Rows of h and W lie D*2 bytes apart, so the rows of one chunk fall on
    // few memory channels; each workgroup starts its walk over the full
    // chunks at a different chunk so that the grid spreads over all of them.
    const int rot = n_full > 0 ? (int)(((int64_t)slot * 7 + mb * 3) % n_full) : 0;

    for (int64_t t0 = t_begin; t0 < t_end; t0 += C::NB / 16) {
        // declared per strip: nothing in them lives across the epilogue
        u32x4 hq[DEPTH][C::HLOADS], wq[DEPTH][C::WLOADS];
        const int64_t col0 = t0 * 16;
        const int tiles_here = (int)min<int64_t>(C::NB / 16, t_end - t0);
        const int64_t rows_here = min<int64_t>((int64_t)tiles_here * 16, V - col0);
        const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(W + col0 * D, rows_here * D * 2);
        const int nt_act = max(0, min(NT, (tiles_here - wn + WN - 1) / WN));
        const bool active = nt_act > 0 && mw_act > 0;
        floatx4 acc[MW][NT];
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

        auto load = [&](auto J, int c, bool full) __attribute__((always_inline)) {
            constexpr int j = decltype(J)::value;
            const int kc0 = (full ? (c + rot) % n_full : c) * KC;
            const bool in = full || kc0 + pj * 8 < D;
#pragma unroll
            for (int q = 0; q < C::HLOADS; ++q)
                hq[j][q] = __builtin_amdgcn_raw_buffer_load_b128(hsrc, in ? voff + q * qstride : kOffNone, kc0 * 2, 0);
#pragma unroll
            for (int q = 0; q < C::WLOADS; ++q)
                wq[j][q] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, in ? voff + q * qstride : kOffNone, kc0 * 2,
                                                                 kBufNT);
        };
        auto store = [&](auto J, int c) __attribute__((always_inline)) {
            constexpr int j = decltype(J)::value;
            unsigned char* tb = smem + (DBUF ? (size_t)(c & 1) * C::TILE : 0);
#pragma unroll
            for (int q = 0; q < C::HLOADS; ++q) {
                const int row = q * C::RPL + ri;
                if (C::MB % C::RPL == 0 || row < C::MB)
                    *reinterpret_cast<u32x4*>(tb + row * C::ROWB + pj * 16) = hq[j][q];
            }
            unsigned char* wb = tb + C::MB * C::ROWB;
#pragma unroll
            for (int q = 0; q < C::WLOADS; ++q)
                *reinterpret_cast<u32x4*>(wb + (q * C::RPL + ri) * C::ROWB + pj * 16) = wq[j][q];
        };
        auto mfma_chunk = [&](int c, auto FULL) __attribute__((always_inline)) {
            constexpr bool full = decltype(FULL)::value;
            const unsigned char* tb = smem + (DBUF ? (size_t)(c & 1) * C::TILE : 0);
            const unsigned char* ha = tb + (wm * 16 * MW + ln) * C::ROWB;
            const unsigned char* wbp = tb + (C::MB + wn * 16 + ln) * C::ROWB;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int po = (4 * s + lg) * 16;
                // all of the k-step's fragments first, then its MFMAs
                u32x4 b[NT], a[MW];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    if (full || nt < nt_act) b[nt] = *reinterpret_cast<const u32x4*>(wbp + nt * 16 * WN * C::ROWB + po);
#pragma unroll
                for (int mt = 0; mt < MW; ++mt) a[mt] = *reinterpret_cast<const u32x4*>(ha + mt * 16 * C::ROWB + po);
#pragma unroll
                for (int mt = 0; mt < MW; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        if (full || nt < nt_act)
                            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, a[mt]), __builtin_bit_cast(bf16x8, b[nt]), acc[mt][nt],
                                0, 0, 0);
            }
        };
        auto compute = [&](int c) __attribute__((always_inline)) {
            if (nt_act == NT && mw_act > 0) mfma_chunk(c, std::true_type{});
            else if (active) mfma_chunk(c, std::false_type{});
        };
        // Chunk c: multiply the staged chunk c, then stage chunk c+1 from its
        // register slot and refill that slot with chunk c+1+DEPTH.
        auto step = [&](auto J, int c, bool st, bool ld) __attribute__((always_inline)) {
            compute(c);
            if (!DBUF) __syncthreads();
            if (st) store(J, c + 1);
            if (ld) load(J, c + 1 + DEPTH, true);
            __syncthreads();
        };
        if (n_full > 0) {
#pragma unroll
            for (int j = 0; j < DEPTH; ++j)
                if (j < n_full) with_slot<DEPTH>(j, [&](auto J) __attribute__((always_inline)) { load(J, j, true); });
            store(std::integral_constant<int, 0>{}, 0);
            if (DEPTH < n_full) load(std::integral_constant<int, 0>{}, DEPTH, true);
            __syncthreads();
            int c = 0;
            for (; c + 2 * DEPTH <= n_full; c += DEPTH) {
#pragma unroll
                for (int j = 0; j < DEPTH; ++j)
                    with_slot<DEPTH>((j + 1) % DEPTH,
                                     [&](auto J) __attribute__((always_inline)) { step(J, c + j, true, true); });
            }
            for (; c < n_full; ++c)
                with_slot<DEPTH>((c + 1) % DEPTH, [&](auto J) __attribute__((always_inline)) {
                    step(J, c, c + 1 < n_full, c + 1 + DEPTH < n_full);
                });
            if (!DBUF) __syncthreads();
        }
        if (ktail) {
            const auto J0 = std::integral_constant<int, 0>{};
            load(J0, n_full, false);
            store(J0, n_full);
            __syncthreads();
            compute(n_full);
            __syncthreads();
        }
        if constexpr (STATS)
            stats_epilogue<MW, NT>(acc, st, m0 + wm * 16 * MW, M, col0 + wn * 16, 16 * WN, nt_act, V, mw_act);
        else
            topk_epilogue<MW, NT, true>(acc, tk, wm * 16 * MW, m0 + wm * 16 * MW, M, col0 + wn * 16, 16 * WN,
                                        nt_act, V, mw_act, rows_blk, wave * 4, 8 * WN, t0 == t_begin);
    }
    if constexpr (STATS) return;

    for (int e = tid; e < rows_blk * kTopK; e += C::THREADS) {
        const int r = e / kTopK, k = e % kTopK;
        const int64_t o = ((m0 + r) * S + slot) * kTopK + k;
        part_val[o] = tk.lval[e];
        part_idx[o] = tk.lidx[e];
    }
}

// ------------------------------------------- wide GEMM, W straight into registers
// head_mfma_kernel (M > 64): a workgroup of 4 wavefronts (one per SIMD, up to
// 512 registers each) owns an M-block of 16*MT rows of h and a contiguous,
// balanced range of 16-row vocabulary tiles, walked in strips of 64*NT rows.
// Wavefront w owns every row of the block and the strip's tiles w, w + 4,
// w + 8, ... (interleaved, so a partial last strip spreads over all four);
// its 16*MT x 16*NT float32 accumulators (4*MT*NT registers, at most 240) stay
// in AGPRs for the whole strip, updated in place by v_mfma_f32_16x16x32_bf16
// (register-only inline asm, so the accumulators are never renamed or copied).
//
// W is read by one wavefront only, so it goes straight from memory into
// registers.  Per 16-row tile and chunk of 64 hidden columns (one 128-byte
// line per row) two loads cover whole lines: load A rows 0-7, load B rows
// 8-15, lane (r, g) (r = lane % 16, g = lane / 16) taking 16-byte piece
// g + 4 (r >= 8) of row r % 8 (or 8 + r % 8).  Whole lines per load cut the
// requests the CU's memory pipeline must hold: with the two 64-byte halves
// of every line in two loads (the plain operand layout, 16 rows x 64 bytes)
// the loads stalled at issue for ~40 % of the loop at M = 224, and the loop
// ran ~7 % longer.  (Eight consecutive lanes per line would let the
// requests merge further, but the layout change back to the operand layout
// then costs 14 VALU operations per dword pair, more than it saves.)  At the
// chunk's start one row_ror:8 DPP move per dword (bank-masked to half of
// each 16-lane row) turns A and B into the MFMA operand layout: lane (r, g)
// then holds row r, piece g (k-step 0) and piece 4 + g (k-step 1).  Chunk
// c+3 is requested as chunk c starts, so three chunks are in flight beyond
// the one being multiplied: under a full streaming load HBM answers in
// ~3.5 us, which takes ~100 KB in flight per CU (an LDS ring that deep would
// not fit next to h).
// h is shared by the four wavefronts: per chunk its 16*MT rows x 128 bytes go
// straight into a 4-stage LDS ring with buffer_load_dwordx4 ... lds (no
// register staging; rows unpadded, 16-byte pieces permuted piece ^ (row & 6),
// which keeps fragment reads free of bank conflicts).  Each A fragment read
// from LDS feeds NT MFMAs; reads run R - 1 fragments ahead, the last ones of a
// chunk already reading the next chunk.  One barrier per chunk, between its
// two k-steps: h chunk c+1 has landed in every wavefront's part and chunk
// c-1's stage is no longer read, so it is refilled with chunk c+3 (two chunks
// of lookahead) while the second k-step runs.  The instruction order is
// fixed with scheduling barriers; the vmcnt waits count on it.
//
// After each strip the running top-16 lists (in LDS for the whole call)
// absorb the strip's logits (strip_topk).
// floats per lane in the epilogue's value rows (16 values; rows 16-byte
// aligned and spread over the LDS banks)
constexpr int kValsPitch = 20;

template <int MT, int NT>
struct MfmaCfg {
    static constexpr int MB = 16 * MT;            // rows of h per workgroup
    static constexpr int NB = 64 * NT;            // W rows per strip (4 wavefronts x 16 NT)
    static constexpr int KC = 64;                 // hidden columns per chunk (128 bytes per row)
    static constexpr int HST = 4;                 // h ring stages
    static constexpr int HSTAGE = MB * 128;
    static constexpr int HI = MB / 8;             // h DMA instructions (8 rows of 128 bytes) per chunk
    static constexpr int HPW = (HI + 3) / 4;      // per wavefront (extra ones fill a spare block)
    // A fragments in flight: a ring of R register sets, R dividing the 2 MT
    // fragments of a chunk (so a fragment's slot does not depend on the
    // chunk) and at least 5 (4 read ahead of the one multiplied)
    static constexpr int ring_size() {
        for (int r = 5; r <= 2 * MT; ++r)
            if ((2 * MT) % r == 0) return r;
        return 2 * MT;
    }
    static constexpr int R = ring_size();
    static constexpr int PF = R - 1;              // A fragments read ahead
    static constexpr size_t SPARE = (size_t)HST * HSTAGE;  // 1 KB target of the extra DMAs
    static constexpr size_t LISTS = SPARE + 1024;           // lists, thresholds, slot counters
    static constexpr size_t LDS = LISTS + (size_t)MB * (kTopK * 8 + 8);
    static constexpr int CAP = 32;                // candidate keys per row and round
    static_assert((size_t)MB * CAP * 8 + 256 * kValsPitch * 4 <= SPARE && (size_t)MB * 64 * 4 <= SPARE,
                  "candidates, value rows and seed lists fit in the drained ring");
    static_assert(LDS <= 160 * 1024, "LDS per workgroup");
    static_assert(MT * NT * 4 <= 240 && NT <= 8, "accumulators fit in the AGPRs");
    static_assert(PF <= MT && (2 * MT) % R == 0, "prefetch distance within a k-step");
};

// waitcnt with only vmcnt = n (0 <= n < 64); lgkmcnt and expcnt not waited
#define DFLASH_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (7 << 4) | (0xF << 8))

// One strip's K loop.  NTP <= NT: only the wavefront's first NTP column tiles
// are multiplied (a partial last strip; the others keep zeros and are not
// admitted); rows past M are multiplied as zeros and never admitted either.
template <int MT, int NT, int NTP, int WAUX>
__device__ __forceinline__ void mfma_strip(const __amdgpu_buffer_rsrc_t hsrc, const __amdgpu_buffer_rsrc_t wsrc,
                                           int D, int nK, int wave, int lane_in, floatx4 (&acc)[MT][NT]) {
    using C = MfmaCfg<MT, NT>;
    constexpr int HPW = C::HPW;
    extern __shared__ __align__(16) unsigned char smem[];
    // Per-lane offsets are computed here, per strip, from an opaque copy of
    // the lane id: kept live across the top-16 epilogue they would be spilled,
    // and every reload before a DMA would wait for all loads in flight.
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
    const int ln = lane & 15, lg = lane >> 4;
    int hoff[HPW], hdst[HPW], woff[NTP];
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        const int j = wave + 4 * u;  // h DMA instruction: rows 8 j .. 8 j + 7
        hoff[u] = j < C::HI ? (j * 8 + (lane >> 3)) * D * 2 + (((lane & 7) ^ ((lane >> 3) & 6)) * 16) : kOffNone;
        hdst[u] = j < C::HI ? j * 1024 : -1;
    }
#pragma unroll
    for (int t = 0; t < NTP; ++t) woff[t] = (16 * (wave + 4 * t) + (ln & 7)) * D * 2 + (lg + 4 * (ln >> 3)) * 16;
    // DMA: lane l writes bytes 16 l of its instruction's 1 KB (8 rows of 128
    // bytes): row l / 8, position l % 8, holding logical piece (l % 8) ^
    // ((l / 8) & 6); pieces past D (a ragged last chunk) load zeros
    const int dcol = ((lane & 7) ^ ((lane >> 3) & 6)) * 8;
    // fragment reads: row ln of a 16-row tile, logical piece 4 s + lg
    const int fo0 = ln * 128 + ((0 + lg) ^ (ln & 6)) * 16;
    const int fo1 = ln * 128 + ((4 + lg) ^ (ln & 6)) * 16;

    auto issue_h = [&](int c) __attribute__((always_inline)) {
        const bool live = c < nK && c * C::KC + dcol < D;
        const int soff = c < nK ? c * 128 : 0;
        const int st = (c % C::HST) * C::HSTAGE;
#pragma unroll
        for (int u = 0; u < HPW; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                hsrc, (__attribute__((address_space(3))) void*)(smem + (hdst[u] < 0 ? (int)C::SPARE : st + hdst[u])),
                16, live ? hoff[u] : kOffNone, soff, 0, 0);
    };
    u32x4 wq[4][NTP][2];  // W chunks in flight: slot c % 4
    auto issue_w = [&](u32x4 (&slot)[NTP][2], int c) __attribute__((always_inline)) {
        const int soff = c < nK ? c * 128 : 0;
        const bool live = c < nK && c * C::KC + 8 * (lg + 4 * (ln >> 3)) < D;  // the piece lies within D
#pragma unroll
        for (int s = 0; s < 2; ++s) {  // A: rows 0-7, B: rows 8-15 of the tile
#pragma unroll
            for (int t = 0; t < NTP; ++t)
                slot[t][s] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, live ? woff[t] + s * 8 * D * 2 : kOffNone,
                                                                   soff, WAUX);
        }
    };
    // A, B -> k-step 0, k-step 1 operands: lanes r >= 8 of each 16-lane row
    // take B from lane r - 8 (k-step 0), lanes r < 8 take A from lane r + 8
    // (k-step 1); the others keep what they loaded
    auto arrange = [&](u32x4 (&slot)[NTP][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NTP; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int a = (int)slot[t][0][j], b = (int)slot[t][1][j];
                slot[t][0][j] = (uint32_t)__builtin_amdgcn_update_dpp(a, b, 0x128, 0xF, 0xC, false);
                slot[t][1][j] = (uint32_t)__builtin_amdgcn_update_dpp(b, a, 0x128, 0xF, 0x3, false);
            }
        }
        // the MFMAs (inline asm, invisible to the hazard checks) read these
        // registers next: give the VALU writes their wait states
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 4" ::: "memory");
    };
    auto barrier = []() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // A fragment k of a chunk: k-step k / MT, tile k % MT
    auto frag = [&](int c, int k) __attribute__((always_inline)) {
        const int s = k / MT, i = k % MT;
        return *reinterpret_cast<const u32x4*>(smem + (c % C::HST) * C::HSTAGE + (16 * i) * 128 + (s ? fo1 : fo0));
    };
    u32x4 fa[C::R];
    // the MFMAs of A fragment k (in fa[k % R]) of a chunk with its W slot,
    // reading fragment k + PF (of this chunk or, past its end, of the next)
    // (past the last chunk the reads land in a stage that holds zeros or a
    // chunk already multiplied: in bounds, never used; reading them
    // unconditionally keeps the loop free of branches, whose joins would
    // drain the fragment reads in flight)
    auto frag_step = [&](const u32x4 (&slot)[NTP][2], int c, int k) __attribute__((always_inline)) {
        const int s = k / MT, i = k % MT;
        const u32x4 a = fa[k % C::R];
#pragma unroll
        for (int t = 0; t < NTP; ++t) {
            asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][t]) : "v"(a), "v"(slot[t][s]));
            if (t == 0) {
                const int kn = k + C::PF;
                fa[kn % C::R] = kn < 2 * MT ? frag(c, kn) : frag(c + 1, kn - 2 * MT);  // slot (kn - 2 MT) % R
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto chunk = [&](u32x4 (&slot)[NTP][2], u32x4 (&nslot)[NTP][2], int c) __attribute__((always_inline)) {
        // W chunk c+3 into the slot that chunk c-1 multiplied (its MFMAs have
        // read their operands long before the data returns)
        __builtin_amdgcn_sched_barrier(0);
        issue_w(nslot, c + 3);
        __builtin_amdgcn_sched_barrier(0);
        arrange(slot);  // (chunk c's loads have landed: h c, issued after them, was waited for)
        __builtin_amdgcn_sched_barrier(0);
        // k-step 0
#pragma unroll
        for (int k = 0; k < MT; ++k) frag_step(slot, c, k);
        // h chunk c+1 landed in every part (after it were issued W c+2, h c+2
        // and W c+3); chunk c-1's stage is no longer read
        DFLASH_WAIT_VM(4 * NTP + HPW);
        barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue_h(c + 3);
        __builtin_amdgcn_sched_barrier(0);
        // k-step 1 (its last reads are the next chunk's first fragments)
#pragma unroll
        for (int k = MT; k < 2 * MT; ++k) frag_step(slot, c, k);
    };
    // prologue: W0 h0 W1 h1 W2 h2 in flight (the steady-state order, every
    // group fenced); h chunk 0 landed everywhere; its first fragments read
    __builtin_amdgcn_sched_barrier(0);
    issue_w(wq[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    issue_h(0);
    __builtin_amdgcn_sched_barrier(0);
    issue_w(wq[1], 1);
    __builtin_amdgcn_sched_barrier(0);
    issue_h(1);
    __builtin_amdgcn_sched_barrier(0);
    issue_w(wq[2], 2);
    __builtin_amdgcn_sched_barrier(0);
    issue_h(2);
    __builtin_amdgcn_sched_barrier(0);
    DFLASH_WAIT_VM(4 * NTP + 2 * HPW);
    barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < C::PF; ++k) fa[k] = frag(0, k);
    for (int c = 0; c < nK; c += 4) {
        chunk(wq[0], wq[3], c);
        chunk(wq[1], wq[0], c + 1);
        chunk(wq[2], wq[1], c + 2);
        chunk(wq[3], wq[2], c + 3);
    }
    DFLASH_WAIT_VM(0);
    barrier();
    // the last MFMAs' results must be written before anything reads the AGPRs
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// The running top-16 lists of head_mfma_kernel (LDS).
struct StripLists {
    uint64_t* list;   // [MB][16] descending keys (kEmptyKey until filled), for the whole call
    float* thr;       // [MB] value of each row's 16th entry (-inf until 16 exist), or the seed
    int* cnt;         // [MB] candidate slots reserved this round (may pass CAP)
    uint64_t* cand;   // [MB][CAP] candidate keys (the drained ring)
    float* seed;      // [MB][4][16] per-wavefront sorted lane maxima (first strip; aliases cand)
    float* vals;      // [256][kValsPitch] each lane's values of one fragment row (after cand)
};

// One strip's logits, still in the accumulators, into the running lists.
// acc[i][t][q] is row 16 i + 4 (lane / 16) + q of the block and vocabulary
// column col0 + 16 (wave + 4 t) + lane % 16.
//  * First strip: each row's threshold starts at the 16th largest of its 64
//    lane maxima (4 wavefronts x 16 lanes): 64 distinct entries, so no more
//    than the row's 16th best.  Per wavefront the 16 lane maxima of a row are
//    sorted in its 16-lane group, then one group merges the four sorted lists.
//  * Filter: a value is a candidate iff it is at or above its row's threshold
//    (the 16th entry's value; ties at it are offered and sorted out by the
//    merge); values below it can never enter the list.  Candidates go to a
//    per-row buffer of CAP keys: each lane reserves a run of slots per row
//    with one LDS atomic (the reservations of a fragment row issued together,
//    so a round costs one LDS round trip per fragment row, not per value).
//  * Merge: 16-lane group g takes rows g, g + 16, ...; for each that received
//    candidates it sorts them 16 at a time and merges them into the row's
//    descending list (bitonic); the threshold becomes the new 16th value.
//    Candidates that found a full buffer stay pending for another round.
template <int MT, int NT>
__device__ __forceinline__ void strip_topk(const floatx4 (&acc)[MT][NT], const StripLists& sl, int wave, int lane_in,
                                           int rows_blk, int64_t col0, int nt_act, int64_t V, bool first) {
    constexpr int CAP = MfmaCfg<MT, NT>::CAP;
    static_assert(4 * NT <= kValsPitch, "a fragment row's values fit in the lane's value row");
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
    const int ln = lane & 15, lg = lane >> 4;
    // Per-lane LDS bases (local address space); everything else in an address
    // is a compile-time offset (a ds instruction's immediate), so no per-row
    // address lives in a register.  The empty asm keeps each base from being
    // folded back into per-row addresses.
    //  filter: rows 16 i + 4 lg + q;  merge: group g = 4 wave + lg, rows g + 16 j
    const int g = wave * 4 + lg;
    auto base = [](auto* p) __attribute__((always_inline)) {
        using T = std::remove_pointer_t<decltype(p)>;
        auto* q = (__attribute__((address_space(3))) T*)p;
        asm volatile("" : "+v"(q));
        return q;
    };
    auto* thr_l = base(sl.thr + 4 * lg);
    auto* cnt_l = base(sl.cnt + 4 * lg);
    auto* cand_l = base(sl.cand + 4 * lg * CAP);
    auto* cand_g = base(sl.cand + g * CAP + ln);
    auto* list_g = base(sl.list + g * kTopK + ln);
    auto* cnt_g = base(sl.cnt + g);
    auto* thr_g = base(sl.thr + g);
    auto* vals_l = base(sl.vals + (wave * 64 + lane) * kValsPitch);
    // accumulators are read where they are used, straight from their AGPRs:
    // copies kept in VGPRs across the rounds would not fit
    auto rd = [](const float& x) __attribute__((always_inline)) {
        float v;
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(x));
        return v;
    };
    auto thr_at = [&](int i) { return *(const __attribute__((address_space(3))) floatx4*)(thr_l + 16 * i); };
    auto cnt_at = [&](int i, int q) { return (int*)(cnt_l + 16 * i + q); };
    auto cand_at = [&](int i, int q) { return cand_l + (16 * i + q) * CAP; };

    // pending bits: bit 4 t + q of pend[i] <=> acc[i][t][q] is still to be offered
    uint32_t tbits = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t)
        if (t < nt_act && col0 + 16 * (wave + 4 * t) + ln < V) tbits |= 0xFu << (4 * t);
    uint32_t pend[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        uint32_t qb = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (16 * i + 4 * lg + q < rows_blk) qb |= 0x1111u << q;
        pend[i] = tbits & qb;
    }
    if (first) {
        // seeds: [row][wavefront][16] sorted lane maxima
        auto* seed_l = base(sl.seed + (4 * lg * 4 + wave) * 16 + ln);
        auto* seed_g = base(sl.seed + g * 64 + ln);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float m = -INFINITY;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    if (pend[i] & (1u << (4 * t + q))) m = fmaxf(m, rd(acc[i][t][q]));
                m = sort16_desc_f32(m, ln);
                seed_l[(16 * i + q) * 64] = m;
            }
            // one fragment row at a time: interleaved, the rows' sorting
            // networks would hold every accumulator in a register at once
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
#pragma unroll 2
        for (int j = 0; j < MT; ++j) {
            const auto* b = seed_g + j * 16 * 64;  // row g + 16 j, lane ln
            // the four lists reversed where a bitonic merge needs it: lane ln
            // reads entry 15 - ln of lists 1 and 3 (offset 15 - 2 ln from its own)
            float x = fmaxf(b[0], b[16 + 15 - 2 * ln]);  // top 16 of wavefronts 0 and 1 (bitonic)
            float y = fmaxf(b[32], b[48 + 15 - 2 * ln]);
            x = merge16_desc_f32(x, ln);
            y = merge16_desc_f32(y, ln);
            float z = fmaxf(x, dpp_f32v<kDppX15>(y));  // top 16 of all four (bitonic)
            z = fminf(z, dpp_f32v<kDppX1>(z));
            z = fminf(z, dpp_f32v<kDppX2>(z));
            z = fminf(z, xor4_f32(z, ln));
            z = fminf(z, dpp_f32v<kDppX8>(z));
            if (ln == 0) thr_g[16 * j] = z;
        }
        __syncthreads();  // the seeds are read; the candidates reuse their memory
    }
    while (true) {
        // thresholds read one fragment row ahead
        floatx4 tn = thr_at(0);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const floatx4 t4 = tn;
            if (i + 1 < MT) tn = thr_at(i + 1);
            if (__ballot(pend[i] != 0) == 0) continue;
            const float tq[4] = {t4[0], t4[1], t4[2], t4[3]};
            uint32_t m = 0;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (rd(acc[i][t][q]) >= tq[q]) m |= 1u << (4 * t + q);
            m &= pend[i];  // below the threshold: never again
            // one reservation per lane and row (row 16 i + 4 lg + q): a run of
            // slots as long as the lane's candidates for that row; the four
            // reservations are issued back to back
            int base[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = __builtin_popcount(m & (0x1111u << q));
                base[q] = n ? atomicAdd(cnt_at(i, q), n) : CAP;
            }
            // the four bases in 16-bit fields (a row takes at most 256
            // reservations per round), selected by a shift below
            uint64_t bases = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) bases |= (uint64_t)(uint32_t)base[q] << (16 * q);
            // The lane's 16 values go to its LDS scratch row, and the stores
            // visit only the set bits of m (a value is then read back by its
            // bit index; indexing the accumulators by it would go through
            // scratch memory).  A candidate's slot is its row's base plus
            // the lane's candidates of that row at lower bits; those past
            // the buffer stay pending.
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                floatx4 v4;
#pragma unroll
                for (int q = 0; q < 4; ++q) v4[q] = rd(acc[i][t][q]);
                *(__attribute__((address_space(3))) floatx4*)(vals_l + 4 * t) = v4;
            }
            uint32_t todo = m, left = m;
            while (todo) {
                const int b = __builtin_ctz(todo);
                todo &= todo - 1;
                const int q = b & 3;
                const int slot = (int)((bases >> (16 * q)) & 0xFFFFu) +
                                 __builtin_popcount(m & (0x1111u << q) & ((1u << b) - 1u));
                if (slot < CAP) {
                    cand_at(i, q)[slot] = rank_key(vals_l[b], (int)(col0 + 16 * (wave + 4 * (b >> 2)) + ln));
                    left &= ~(1u << b);
                }
            }
            pend[i] = left;
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        // 16-lane group g merges rows g, g + 16, ... that received
        // candidates, two rows at a time so that their sorting networks
        // interleave (with one wavefront per SIMD, a single network's
        // dependent steps would each wait out the full latency); the partner
        // of a row with candidates may merge only empty keys, which leave its
        // list as it is, and is not written back.
        int nrow[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) nrow[j] = cnt_g[16 * j];
#pragma unroll
        for (int j = 0; j < MT; j += 2) {
            const bool two = j + 1 < MT;
            const int n0 = min(nrow[j], CAP), n1 = two ? min(nrow[j + 1], CAP) : 0;
            if (n0 == 0 && n1 == 0) continue;
            auto* lst0 = list_g + 16 * kTopK * j;
            auto* lst1 = list_g + 16 * kTopK * (two ? j + 1 : j);
            const auto* cnd0 = cand_g + 16 * CAP * j;
            const auto* cnd1 = cand_g + 16 * CAP * (two ? j + 1 : j);
            uint64_t l0 = *lst0, l1 = *lst1;
            const int n = max(n0, n1);
            for (int c0 = 0; c0 < n; c0 += 16) {
                uint64_t k0 = c0 + ln < n0 ? cnd0[c0] : kEmptyKey;
                uint64_t k1 = c0 + ln < n1 ? cnd1[c0] : kEmptyKey;
                k0 = sort16<false>(k0, ln);
                k1 = sort16<false>(k1, ln);
                l0 = l0 > k0 ? l0 : k0;
                l1 = l1 > k1 ? l1 : k1;
                l0 = merge16_desc(l0, ln);
                l1 = merge16_desc(l1, ln);
            }
            if (n0 > 0) {
                *lst0 = l0;
                if (ln == kTopK - 1) thr_g[16 * j] = key_value(l0);
                if (ln == 0) cnt_g[16 * j] = 0;
            }
            if (n1 > 0) {
                *lst1 = l1;
                if (ln == kTopK - 1) thr_g[16 * (j + 1)] = key_value(l1);
                if (ln == 0) cnt_g[16 * (j + 1)] = 0;
            }
        }
        int any = 0;
#pragma unroll
        for (int i = 0; i < MT; ++i) any |= pend[i] != 0;
        if (!__syncthreads_or(any)) break;
    }
}

// The softmax statistics of one strip's logits, still in the accumulators
// (the target head of the fused sampler): per (row, 16-column vocabulary
// tile) the tile maximum m and the float32 sum of exp2((z - m) * k2), as
// stats_epilogue computes them, here from head_mfma_kernel's layout
// (acc[i][t][q]: row 16 i + 4 (lane / 16) + q of the block, tile wave + 4 t
// of the strip, column lane % 16 of the tile).
template <int MT, int NT>
__device__ __forceinline__ void mfma_stats_strip(const floatx4 (&acc)[MT][NT], const TileStats& st, int64_t m0,
                                                 int rows_blk, int64_t col0, int wave, int lane_in, int nt_act,
                                                 int64_t V) {
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
    const int ln = lane & 15, lg = lane >> 4;
    auto rd = [](const float& x) __attribute__((always_inline)) {
        float v;
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(x));
        return v;
    };
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t >= nt_act) continue;  // the wavefront's tiles past the strip's end
        const int64_t tc = col0 + 16 * (wave + 4 * t);  // the tile's first column (< V)
        const bool cok = tc + ln < V;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float z = rd(acc[i][t][q]);
                float m = cok ? z : -INFINITY;
                m = fmaxf(m, dpp_f32(m, ln, 1));
                m = fmaxf(m, dpp_f32(m, ln, 2));
                m = fmaxf(m, dpp_f32(m, ln, 4));
                m = fmaxf(m, dpp_f32(m, ln, 8));
                float e = cok ? __builtin_amdgcn_exp2f((z - m) * st.k2) : 0.0f;
                e += dpp_f32(e, ln, 1);
                e += dpp_f32(e, ln, 2);
                e += dpp_f32(e, ln, 4);
                e += dpp_f32(e, ln, 8);
                const int r = 16 * i + 4 * lg + q;
                if (ln == 0 && r < rows_blk) st.rec[(m0 + r) * st.n16 + tc / 16] = make_float2(m, e);
            }
            __builtin_amdgcn_sched_barrier(0);  // one fragment row at a time
        }
    }
}

// st.rec == nullptr: the top-16 lists into part_val / part_idx; otherwise the
// softmax statistics of every (row, tile) into st.rec (part_* unused).
template <int MT, int NT, int WAUX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void head_mfma_kernel(const uint16_t* h, const uint16_t* W, int64_t M, int D, int64_t V, int64_t n_tiles, int S,
                      int n_mb, float* __restrict__ part_val, int* __restrict__ part_idx, TileStats st) {
    // (h and W are deliberately not __restrict__: loads from restrict read-only
    // memory may be moved across the barrier asm, which would break the issue
    // order that the vmcnt waits count on)
    using C = MfmaCfg<MT, NT>;
    extern __shared__ __align__(16) unsigned char smem[];
    // workgroup -> (M-block, slot): the M-blocks of one slot are dispatched
    // back to back on the same XCD so they share the slot's W rows in L2.
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int kq = L >> 3;
    const int mb = kq % n_mb;
    const int slot = (kq / n_mb) * 8 + xcd;
    if (slot >= S) return;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int64_t m0 = (int64_t)mb * C::MB;
    const int rows_blk = (int)min<int64_t>(C::MB, M - m0);
    const int nK = (D + C::KC - 1) / C::KC;
    // Rows past the block or the strip read as zero (the resources end there).
    const __amdgpu_buffer_rsrc_t hsrc = make_rsrc(h + m0 * D, (int64_t)rows_blk * D * 2);

    StripLists sl;
    unsigned char* lp = smem + C::LISTS;
    sl.list = reinterpret_cast<uint64_t*>(lp);
    sl.thr = reinterpret_cast<float*>(lp + C::MB * kTopK * 8);
    sl.cnt = reinterpret_cast<int*>(sl.thr + C::MB);
    sl.cand = reinterpret_cast<uint64_t*>(smem);  // the drained ring (epilogue only)
    sl.seed = reinterpret_cast<float*>(smem);
    sl.vals = reinterpret_cast<float*>(smem + (size_t)C::MB * C::CAP * 8);
    for (int e = tid; e < C::MB * kTopK; e += 256) sl.list[e] = kEmptyKey;
    for (int e = tid; e < C::MB; e += 256) {
        sl.thr[e] = -INFINITY;
        sl.cnt[e] = 0;
    }
    __syncthreads();

    const int64_t t_begin = (int64_t)slot * n_tiles / S, t_end = (int64_t)(slot + 1) * n_tiles / S;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += C::NB / 16) {
        const int64_t col0 = t0 * 16;
        const int tiles_here = (int)min<int64_t>(C::NB / 16, t_end - t0);
        const int64_t rows_here = min<int64_t>((int64_t)tiles_here * 16, V - col0);
        const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(W + col0 * D, rows_here * D * 2);
        const int nt_act = max(0, min(NT, (tiles_here - wave + 3) / 4));
        floatx4 acc[MT][NT];
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
        // every wavefront runs the same loop (barriers); a partial strip
        // multiplies only as many column tiles as the busiest wavefront holds
        const int need = (tiles_here + 3) / 4;
        if (need > NT / 2)
            mfma_strip<MT, NT, NT, WAUX>(hsrc, wsrc, D, nK, wave, lane, acc);
        else if (need > 1)
            mfma_strip<MT, NT, NT / 2, WAUX>(hsrc, wsrc, D, nK, wave, lane, acc);
        else
            mfma_strip<MT, NT, 1, WAUX>(hsrc, wsrc, D, nK, wave, lane, acc);
        if (st.rec) {
            mfma_stats_strip<MT, NT>(acc, st, m0, rows_blk, col0, wave, lane, nt_act, V);
        } else {
            strip_topk<MT, NT>(acc, sl, wave, lane, rows_blk, col0, nt_act, V, t0 == t_begin);
            __syncthreads();  // the ring (epilogue scratch) is refilled by the next strip
        }
    }
    if (st.rec) return;
    for (int e = tid; e < rows_blk * kTopK; e += 256) {
        const int r = e / kTopK, k = e % kTopK;
        const int64_t o = ((m0 + r) * S + slot) * kTopK + k;
        part_val[o] = key_value(sl.list[e]);
        part_idx[o] = key_id(sl.list[e]);
    }
}

// ---------------------------------------------------------------- merge
// G workgroups of 10 wavefronts per row (G = 1 for many rows, up to 5 for a
// few, so that the exact re-scoring is spread over more CUs).
// (1) Each copies the row's S sorted partial lists (S <= kMaxLists) to LDS.
// (2) Threshold selection: the list heads fall into at most 64 buckets of b
//     consecutive lists; T = the 20th-best bucket maximum.  The maxima are
//     distinct entries, so at least 20 entries rank at or above T, and so do
//     all of the row's best 20.  The entries at or above T (a prefix of each
//     list, typically two dozen) are gathered and sorted in one wavefront.
//     (More than 64 of them: k-way extraction, where a wavefront takes 64
//     lists and 20 times pops the best list head, and one wavefront then pops
//     the best 20 of the group results.)
// (3) Workgroup g re-scores candidates g, g + G, ... exactly, one or two per
//     wavefront: all loads of the h row and the W rows are issued before any
//     arithmetic (one HBM round trip); bf16 products are exact in float64 and
//     summed in float64.
// (4) Rank by the exact value (ties: lower id) and write the best 16: in the
//     same workgroup when G = 1, else in head_rank_kernel, which reads the
//     candidates and their values from the workspace.
constexpr int kMaxLists = 1024;
constexpr int kMergeSeg = 10;  // 16-byte pieces per lane per pass over D
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMaxSplit = 5;  // workgroups per row at most



// Wavefront sum of a double (the result is complete in lane 63): row-level
// Hillis-Steele with DPP row shifts, then row broadcasts.  Lanes whose DPP
// source falls outside the row add zero.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_add_f64(double x) {
    const uint64_t u = __double_as_longlong(x);
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, CTRL, ROW_MASK, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), CTRL, ROW_MASK, 0xF, false);
    return x + __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_f64(double x) {
    x = dpp_add_f64<0x111, 0xF>(x);  // row_shr:1
    x = dpp_add_f64<0x112, 0xF>(x);  // row_shr:2
    x = dpp_add_f64<0x114, 0xF>(x);  // row_shr:4
    x = dpp_add_f64<0x118, 0xF>(x);  // row_shr:8
    x = dpp_add_f64<0x142, 0xA>(x);  // row_bcast:15
    x = dpp_add_f64<0x143, 0xC>(x);  // row_bcast:31
    return x;
}


// Wavefront maximum of a float (every lane gets it): DPP row shifts, row
// broadcasts and a read of lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_f32(float x) {
    return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(x), CTRL,
                                                               ROW_MASK, 0xF, false)));
}
__device__ __forceinline__ float wave_max_f32(float x) {
    x = dpp_max_f32<0x111, 0xF>(x);  // row_shr:1
    x = dpp_max_f32<0x112, 0xF>(x);  // row_shr:2
    x = dpp_max_f32<0x114, 0xF>(x);  // row_shr:4
    x = dpp_max_f32<0x118, 0xF>(x);  // row_shr:8
    x = dpp_max_f32<0x142, 0xA>(x);  // row_bcast:15
    x = dpp_max_f32<0x143, 0xC>(x);  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Pop the kRescore best entries of up to 64 sorted lists of length len held
// in LDS (list l of lane l at lv/li + l * len); results to ov/oi.  A pop
// takes the wavefront maximum of the list heads' values; when several lanes
// hold that value (ties, or only sentinels left) the lowest id among them
// wins, so the order is the ranks_before order.
__device__ __forceinline__ void extract_top(const float* lv, const int* li, int len, int nlists, float* ov,
                                            int* oi) {
    const int lane = threadIdx.x & 63;
    int pos = 0;
    float hv = lane < nlists ? lv[lane * len] : -INFINITY;
    int hi = lane < nlists ? li[lane * len] : 0x7FFFFFFF;
    for (int k = 0; k < kRescore; ++k) {
        const float best = wave_max_f32(hv);
        const uint64_t at = __ballot(hv == best);
        int win = __ffsll((unsigned long long)at) - 1;
        int wid = __shfl(hi, win);
        if (__popcll(at) > 1) {  // ties: lowest id among the lanes at the maximum
            int mid = hv == best ? hi : 0x7FFFFFFF;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mid = min(mid, __shfl_xor(mid, off));
            wid = mid;
            win = __ffsll((unsigned long long)__ballot(hv == best && hi == mid)) - 1;
        }
        if (lane == 0) {
            ov[k] = best;
            oi[k] = wid;
        }
        // only a lane that owns a list advances, and never past its end
        if (lane == win && lane < nlists && pos < len) {
            ++pos;
            hv = pos < len ? lv[lane * len + pos] : -INFINITY;
            hi = pos < len ? li[lane * len + pos] : 0x7FFFFFFF;
        }
    }
}

// Lane t < ns holds candidate t's exact value and id; its rank is the number
// of candidates that rank before it (larger value, then lower id).  The best
// 16 are written in rank order.
__device__ __forceinline__ void rank_and_write(double z, int id, int ns, float* __restrict__ out_val,
                                               int32_t* __restrict__ out_idx) {
    const int lane = threadIdx.x & 63;
    int rank = 0;
    for (int t = 0; t < ns; ++t) {
        const double zt = __longlong_as_double((long long)readlane_u64((uint64_t)__double_as_longlong(z), t));
        const int it = __builtin_amdgcn_readlane(id, t);
        rank += ranks_before_d(zt, it, z, id) ? 1 : 0;
    }
    if (lane < ns && rank < kTopK) {
        out_val[rank] = (float)z;
        out_idx[rank] = id;
    }
}

__global__ __launch_bounds__(kMergeThreads) void head_merge_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int D, int64_t V, int S, int G,
    const float* __restrict__ part_val, const int* __restrict__ part_idx, double* __restrict__ cand_z,
    int* __restrict__ cand_id, float* __restrict__ top_val, int32_t* __restrict__ top_idx) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* lv = reinterpret_cast<float*>(smem);              // [S][16]
    int* li = reinterpret_cast<int*>(lv + (size_t)S * kTopK);  // [S][16]
    __shared__ float gv[kMaxLists / 64][kRescore];
    __shared__ int gi[kMaxLists / 64][kRescore];
    __shared__ float sel_v[kRescore];
    __shared__ int sel_i[kRescore];
    __shared__ double sel_z[kRescore];
    __shared__ unsigned long long bucket_max[64];
    __shared__ unsigned long long cand[64];
    __shared__ int s_count;

    const int64_t m = blockIdx.x / G;
    const int g = blockIdx.x % G;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const float4* pv4 = reinterpret_cast<const float4*>(part_val + m * S * kTopK);
    const int4* pi4 = reinterpret_cast<const int4*>(part_idx + m * S * kTopK);
    {  // all loads of the copy are issued before any store
        constexpr int kIters = (kMaxLists * kTopK / 4 + kMergeThreads - 1) / kMergeThreads;
        const int n4 = S * kTopK / 4;
        float4 cv[kIters];
        int4 ci[kIters];
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int e = min(tid + it * kMergeThreads, n4 - 1);  // unconditional loads
            cv[it] = pv4[e];
            ci[it] = pi4[e];
        }
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int e = tid + it * kMergeThreads;
            if (e < n4) {
                reinterpret_cast<float4*>(lv)[e] = cv[it];
                reinterpret_cast<int4*>(li)[e] = ci[it];
            }
        }
    }
    if (tid == 0) s_count = 0;
    __syncthreads();
    // (2) The list heads in at most 64 buckets of b consecutive lists.
    const int b = S <= 64 ? 1 : S <= 128 ? 2 : S <= 256 ? 4 : S <= 512 ? 8 : 16;
    const int nb = (S + b - 1) / b;
    for (int base = 0; base < S; base += kMergeThreads) {  // every lane takes part in the group maxima
        const int t = base + tid;
        uint64_t k = t < S ? rank_key(lv[t * kTopK], li[t * kTopK]) : kEmptyKey;
        k = group_max_u64(k, b);
        if (t < S && t % b == 0) bucket_max[t / b] = k;
    }
    __syncthreads();
    // T = the kRescore-th best bucket maximum (every wavefront sorts the
    // maxima itself).  With fewer than kRescore buckets there is no bound: T
    // is the empty key and every entry is a candidate.
    uint64_t bk = lane < nb ? bucket_max[lane] : kEmptyKey;
    bk = sort64_desc(bk, lane);
    const uint64_t T = nb >= kRescore ? readlane_u64(bk, kRescore - 1) : kEmptyKey;
    for (int t = tid; t < S; t += kMergeThreads) {
        for (int c = 0; c < kTopK; ++c) {
            const unsigned long long k = rank_key(lv[t * kTopK + c], li[t * kTopK + c]);
            if (k < T) break;
            const int pos = atomicAdd(&s_count, 1);
            if (pos < 64) cand[pos] = k;
        }
    }
    __syncthreads();
    // lane c < kRescore of every wavefront: the c-th best candidate's key
    uint64_t ck;
    const int n_cand = s_count;
    if (n_cand <= 64) {
        ck = lane < n_cand ? cand[lane] : kEmptyKey;
        ck = sort64_desc(ck, lane);
    } else {
        const int ng = (S + 63) / 64;
        for (int gg = wave; gg < ng; gg += kMergeWaves)
            extract_top(lv + gg * 64 * kTopK, li + gg * 64 * kTopK, kTopK, min(64, S - gg * 64), gv[gg], gi[gg]);
        __syncthreads();
        if (wave == 0) extract_top(&gv[0][0], &gi[0][0], kRescore, ng, sel_v, sel_i);
        __syncthreads();
        ck = lane < kRescore ? rank_key(sel_v[lane], sel_i[lane]) : kEmptyKey;
    }
    // real entries precede the sentinels; an id outside [0, V) (none is
    // expected) ends the list rather than being dereferenced
    const int cid = key_id(ck);
    const uint64_t valid = __ballot(lane < kRescore && cid >= 0 && cid < V);
    const int ns = __builtin_ctzll(~valid);

    // (3) exact re-scoring: candidates g, g + G, ... of this workgroup, one
    // or two per wavefront
    const uint16_t* hr = h + m * D;
    const int c0 = g + G * wave, c1 = g + G * (wave + kMergeWaves);
    if (c0 < ns) {
        const bool has1 = c1 < ns;
        const int id0 = key_id(readlane_u64(ck, c0));
        const int id1 = has1 ? key_id(readlane_u64(ck, c1)) : id0;
        const uint16_t* w0 = W + (int64_t)id0 * D;
        const uint16_t* w1 = W + (int64_t)id1 * D;
        double acc0 = 0.0, acc1 = 0.0;
        for (int seg = 0; seg < D; seg += kMergeSeg * 512) {
            u32x4 ha[kMergeSeg], wa[kMergeSeg], wb[kMergeSeg];
#pragma unroll
            for (int j = 0; j < kMergeSeg; ++j) {
                const int d = min(seg + (j * 64 + lane) * 8, D - 8);
                ha[j] = *reinterpret_cast<const u32x4*>(hr + d);
                wa[j] = *reinterpret_cast<const u32x4*>(w0 + d);
                if (has1) wb[j] = *reinterpret_cast<const u32x4*>(w1 + d);
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
                        if (has1) {
                            acc1 = fma(a0, (double)bf16_to_f32(wb[j][q] & 0xFFFFu), acc1);
                            acc1 = fma(a1, (double)bf16_to_f32(wb[j][q] >> 16), acc1);
                        }
                    }
                }
            }
        }
        acc0 = wave_sum_f64(acc0);
        if (has1) acc1 = wave_sum_f64(acc1);
        if (lane == 63) {
            if (G == 1) {
                sel_z[c0] = acc0;
                if (has1) sel_z[c1] = acc1;
            } else {
                cand_z[m * kRescore + c0] = acc0;
                if (has1) cand_z[m * kRescore + c1] = acc1;
            }
        }
    }
    const int id = lane < ns ? cid : 0x7FFFFFFF;
    if (G > 1) {  // head_rank_kernel ranks
        if (g == 0 && wave == 0 && lane < kRescore) cand_id[m * kRescore + lane] = id;
        return;
    }
    __syncthreads();
    // (4) lane t < ns holds candidate t
    if (wave == 0) rank_and_write(lane < ns ? sel_z[lane] : 0.0, id, ns, top_val + m * kTopK, top_idx + m * kTopK);
}

// (4) for rows merged by several workgroups: one wavefront per row reads the
// row's candidates (ids in rank order of their float32 values, the sentinel
// id after the last) and their exact values.
constexpr int kRankRows = 4;  // rows per workgroup
__global__ __launch_bounds__(64 * kRankRows) void head_rank_kernel(int64_t M, int64_t V,
                                                                   const double* __restrict__ cand_z,
                                                                   const int* __restrict__ cand_id,
                                                                   float* __restrict__ top_val,
                                                                   int32_t* __restrict__ top_idx) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * kRankRows + (threadIdx.x >> 6);
    if (m >= M) return;
    // both loads in one round trip (the values of entries past the last
    // candidate are read but not used)
    const int id = lane < kRescore ? cand_id[m * kRescore + lane] : 0x7FFFFFFF;
    const double zr = lane < kRescore ? cand_z[m * kRescore + lane] : 0.0;
    const uint64_t valid = __ballot(lane < kRescore && id >= 0 && id < V);
    const int ns = __builtin_ctzll(~valid);
    rank_and_write(lane < ns ? zr : 0.0, lane < ns ? id : 0x7FFFFFFF, ns, top_val + m * kTopK, top_idx + m * kTopK);
}

// ------------------------------------------------------------------ host
namespace {

enum HeadVariant { kSkinny = 0, kWide64 = 1, kMfma128 = 2, kMfma224 = 3, kMfma240 = 4 };

struct HeadPlan {
    HeadVariant variant;
    int mb_rows;    // rows per M-block
    int S;          // partial lists per row (= workgroups per M-block)
    int n_mb;
    int64_t n_tiles;
    int G;          // merge workgroups per row
};

// One instantiation of head_wide_kernel with its launch.
template <int MW, int NT, int KS, int DEPTH, bool DBUF, int WN>
struct WideVariant {
    using Cfg = WideCfg<MW, NT, KS, DEPTH, DBUF, WN>;
    template <bool STATS>
    static const void* fn() {
        return reinterpret_cast<const void*>(&head_wide_kernel<MW, NT, KS, DEPTH, DBUF, WN, STATS>);
    }
    static void set_attr() {
        (void)hipFuncSetAttribute(fn<false>(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::LDS);
        (void)hipFuncSetAttribute(fn<true>(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::LDS);
    }
    template <bool STATS = false>
    static void launch(int S, int n_mb, const uint16_t* h, const uint16_t* W, int64_t M, int D, int64_t V,
                       int64_t n_tiles, float* pv, int* pi, hipStream_t stream, TileStats st = TileStats{}) {
        const int grid = (S + 7) / 8 * 8 * n_mb;
        hipLaunchKernelGGL((head_wide_kernel<MW, NT, KS, DEPTH, DBUF, WN, STATS>), dim3(grid), dim3(Cfg::THREADS),
                           Cfg::LDS, stream, h, W, M, D, V, n_tiles, S, n_mb, pv, pi, st);
    }
};

// One instantiation of head_mfma_kernel with its launch.
// W's loads are non-temporal when each W row is read by one workgroup (one
// M-block; measured 3-4 % faster at M = 128 and 224), and cached when the
// M-blocks of a slot share W rows through L2 (non-temporal there measured
// 1.5 % slower at M = 480).
template <int MT, int NT>
struct MfmaVariant {
    using Cfg = MfmaCfg<MT, NT>;
    template <int WAUX>
    static const void* fn() { return reinterpret_cast<const void*>(&head_mfma_kernel<MT, NT, WAUX>); }
    static void set_attr() {
        (void)hipFuncSetAttribute(fn<0>(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::LDS);
        (void)hipFuncSetAttribute(fn<kBufNT>(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::LDS);
    }
    // st.rec set: the statistics epilogue instead of the top-16 lists
    static void launch(int S, int n_mb, const uint16_t* h, const uint16_t* W, int64_t M, int D, int64_t V,
                       int64_t n_tiles, float* pv, int* pi, hipStream_t stream, TileStats st = TileStats{}) {
        const int grid = (S + 7) / 8 * 8 * n_mb;
        if (n_mb == 1)
            hipLaunchKernelGGL((head_mfma_kernel<MT, NT, kBufNT>), dim3(grid), dim3(256), Cfg::LDS, stream, h, W, M,
                               D, V, n_tiles, S, n_mb, pv, pi, st);
        else
            hipLaunchKernelGGL((head_mfma_kernel<MT, NT, 0>), dim3(grid), dim3(256), Cfg::LDS, stream, h, W, M, D, V,
                               n_tiles, S, n_mb, pv, pi, st);
    }
};
using Mfma128 = MfmaVariant<8, 4>;   // M-blocks of 128 rows, 256-row strips
using Mfma224 = MfmaVariant<14, 4>;  // M-blocks of 224 rows, 256-row strips
using Mfma240 = MfmaVariant<15, 4>;  // M-blocks of 240 rows, 256-row strips

// two workgroups of four wavefronts per CU (measured faster than one of eight)
constexpr int kSkinnyNT = 2, kSkinnyKS = 4, kSkinnyWaves = 4, kSkinnyWG = 512;
using SkinnyL = SkinnyLds<kSkinnyNT, kSkinnyKS, kSkinnyWaves>;
// at most 64 rows: 64-row blocks keep both wavefront rows busy (M = 56:
// 306 us against 321 us with a 128-row block, whose second wavefront row
// holds no rows; 256-row strips and deeper prefetch measured slower)
using Wide64 = WideVariant<2, 2, 2, 4, true, 4>;
constexpr int kCUs = 256;

// The same plan serves the top-16 head and the softmax-statistics GEMM of
// the fused sampler (the skinny and 64-row kernels take a template flag for
// the epilogue, head_mfma_kernel a run-time one).
HeadPlan head_plan(int64_t M, int64_t V) {
    HeadPlan p{};
    p.n_tiles = (V + 15) / 16;
    // merge workgroups per row: spread the re-scoring of few rows over more CUs
    p.G = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxSplit, kCUs / M));
    if (M <= 16) {
        p.variant = kSkinny;
        p.mb_rows = 16;
        p.n_mb = 1;
        const int64_t want = (p.n_tiles + kSkinnyWaves - 1) / kSkinnyWaves;  // at least one tile per wavefront
        p.S = (int)std::min<int64_t>(kSkinnyWG, want);
        return p;
    }
    if (M <= 64) {
        p.variant = kWide64;
        p.mb_rows = Wide64::Cfg::MB;
    } else {
        // the M-block size that pads M the least (larger blocks win ties:
        // fewer of them read W)
        const int64_t pad128 = (M + 127) / 128 * 128, pad224 = (M + 223) / 224 * 224, pad240 = (M + 239) / 240 * 240;
        if (pad240 <= pad224 && pad240 <= pad128) {
            p.variant = kMfma240;
            p.mb_rows = Mfma240::Cfg::MB;
        } else if (pad224 <= pad128) {
            p.variant = kMfma224;
            p.mb_rows = Mfma224::Cfg::MB;
        } else {
            p.variant = kMfma128;
            p.mb_rows = Mfma128::Cfg::MB;
        }
    }
    p.n_mb = (int)((M + p.mb_rows - 1) / p.mb_rows);
    // one workgroup per CU (the chunk tile takes most of the LDS)
    int s = std::max(1, kCUs / p.n_mb);
    s = (int)std::min<int64_t>(s, p.n_tiles);  // at least one tile each
    p.S = std::min(s, kMaxLists);
    return p;
}

std::once_flag g_head_attr_once;

}  // namespace

// Workspace: partial values [M][S][16] float, partial ids [M][S][16] int,
// then, when rows are merged by several workgroups, the re-scored candidates:
// exact values [M][20] double and ids [M][20] int.
size_t head_workspace_bytes(int64_t M, int64_t V) {
    const HeadPlan p = head_plan(M, V);
    size_t b = (size_t)M * p.S * kTopK * 8;
    if (p.G > 1) b += (size_t)M * kRescore * 12;
    return b;
}

static void set_head_attrs() {
    std::call_once(g_head_attr_once, []() {
        (void)hipFuncSetAttribute(
            reinterpret_cast<const void*>(&head_skinny2_kernel<kSkinnyNT, kSkinnyKS, kSkinnyWaves, false>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)SkinnyL::BYTES);
        (void)hipFuncSetAttribute(
            reinterpret_cast<const void*>(&head_skinny2_kernel<kSkinnyNT, kSkinnyKS, kSkinnyWaves, true>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)SkinnyL::BYTES);
        Wide64::set_attr();
        Mfma128::set_attr();
        Mfma224::set_attr();
        Mfma240::set_attr();
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&head_merge_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLists * kTopK * 8);
    });
}

int launch_head_topk(const uint16_t* h, const uint16_t* W, int64_t M, int D, int64_t V,
                     float* top_val, int32_t* top_idx, void* ws, hipStream_t stream) {
    set_head_attrs();
    const HeadPlan p = head_plan(M, V);
    float* pv = reinterpret_cast<float*>(ws);
    int* pi = reinterpret_cast<int*>(pv + (size_t)M * p.S * kTopK);
    double* cand_z = reinterpret_cast<double*>(pi + (size_t)M * p.S * kTopK);
    int* cand_id = reinterpret_cast<int*>(cand_z + (size_t)M * kRescore);
    switch (p.variant) {
        case kSkinny:
            hipLaunchKernelGGL((head_skinny2_kernel<kSkinnyNT, kSkinnyKS, kSkinnyWaves, false>), dim3(p.S),
                               dim3(64 * kSkinnyWaves), SkinnyL::BYTES, stream, h, W, M,
                               D, V, pv, pi, TileStats{});
            break;
        case kWide64:
            Wide64::launch(p.S, p.n_mb, h, W, M, D, V, p.n_tiles, pv, pi, stream);
            break;
        case kMfma128:
            Mfma128::launch(p.S, p.n_mb, h, W, M, D, V, p.n_tiles, pv, pi, stream);
            break;
        case kMfma224:
            Mfma224::launch(p.S, p.n_mb, h, W, M, D, V, p.n_tiles, pv, pi, stream);
            break;
        default:
            Mfma240::launch(p.S, p.n_mb, h, W, M, D, V, p.n_tiles, pv, pi, stream);
            break;
    }
    int st = launch_status();
    if (st != DFLASH_OK) return st;
    const size_t lds = (size_t)p.S * kTopK * 8;
    hipLaunchKernelGGL(head_merge_kernel, dim3((unsigned)(M * p.G)), dim3(kMergeThreads), lds, stream, h, W, D, V,
                       p.S, p.G, pv, pi, cand_z, cand_id, top_val, top_idx);
    if (p.G > 1) {
        st = launch_status();
        if (st != DFLASH_OK) return st;
        hipLaunchKernelGGL(head_rank_kernel, dim3((unsigned)((M + kRankRows - 1) / kRankRows)), dim3(64 * kRankRows),
                           0, stream, M, V, cand_z, cand_id, top_val, top_idx);
    }
    return launch_status();
}

// ------------------------------------------------ allocation-free variant
// For callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid hipMalloc): the partial lists live in a file-scope
// device array instead of a caller workspace.  Every GPU holds its own copy
// from module load until the process ends; calls on one GPU share it, so
// calls that overlap in time on one GPU race on it (enqueue them on one
// stream).  Nothing in it needs clearing: the GEMM writes every partial entry
// the merge reads, and the merge writes every candidate the rank step reads.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

size_t head_static_scratch_bytes() { return kStaticScratchBytes; }

namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];
}  // namespace

// The array's address on the current device, resolved once per device with
// that device current (the array's name in host code is only a stand-in).
static void* static_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev]() {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) {
            g_scratch_ptr[dev] = p;
        } else {
            (void)hipGetLastError();  // leave no sticky error for a later launch check
            g_scratch_ptr[dev] = nullptr;
        }
    });
    return g_scratch_ptr[dev];
}

// Caller has checked head_workspace_bytes(M, V) <= kStaticScratchBytes.
int launch_head_topk_static(const uint16_t* h, const uint16_t* W, int64_t M, int D, int64_t V, float* top_val,
                            int32_t* top_idx, hipStream_t stream) {
    if (head_workspace_bytes(M, V) > kStaticScratchBytes) return DFLASH_ERR_WORKSPACE;
    void* ws = static_scratch();
    if (!ws) return DFLASH_ERR_LAUNCH;
    return launch_head_topk(h, W, M, D, V, top_val, top_idx, ws, stream);
}

// The same GEMMs with the softmax-statistics epilogue: rec [M][ceil(V/16)]
// float2 (tile maximum, tile sum of exp((z - m) * inv_tau)); no merge.
size_t head_stats_bytes(int64_t M, int64_t V) { return (size_t)M * ((V + 15) / 16) * 8; }

int launch_head_stats(const uint16_t* h, const uint16_t* W, int64_t M, int D, int64_t V, double inv_tau,
                      float2* rec, hipStream_t stream) {
    set_head_attrs();
    const HeadPlan p = head_plan(M, V);
    const TileStats st{rec, (V + 15) / 16, (float)(inv_tau * 1.4426950408889634)};
    switch (p.variant) {
        case kSkinny:
            hipLaunchKernelGGL((head_skinny2_kernel<kSkinnyNT, kSkinnyKS, kSkinnyWaves, true>), dim3(p.S),
                               dim3(64 * kSkinnyWaves), SkinnyL::BYTES, stream, h, W, M, D, V, nullptr, nullptr, st);
            break;
        case kWide64:
            Wide64::launch<true>(p.S, p.n_mb, h, W, M, D, V, p.n_tiles, nullptr, nullptr, stream, st);
            break;
        case kMfma128:
            Mfma128::launch(p.S, p.n_mb, h, W, M, D, V, p.n_tiles, nullptr, nullptr, stream, st);
            break;
        case kMfma224:
            Mfma224::launch(p.S, p.n_mb, h, W, M, D, V, p.n_tiles, nullptr, nullptr, stream, st);
            break;
        default:
            Mfma240::launch(p.S, p.n_mb, h, W, M, D, V, p.n_tiles, nullptr, nullptr, stream, st);
            break;
    }
    return launch_status();
}

// ------------------------------------------------ exactness certificate
// The head returns the best 16 of its best kRescore float32 candidates by
// exact value.  An entry outside those candidates could still belong in the
// exact top-16 if its float32 logit erred by more than the gap.  For row m:
//  * every float32 logit f_v (the GEMM's float32 accumulation of D exact
//    bf16 products) satisfies |f_v - z_v| <= eps_m = gamma_D min(|h_m|_2 N2,
//    |h_m|_inf N1), with N2, N1 bounds on max_v |W_v|_2 and max_v |W_v|_1 and
//    gamma_D = D u / (1 - D u), u = 2^-23: one unit in the last place per
//    addition, whatever the order and the direction of rounding;
//  * U = the largest float32 value among entries that were not re-scored:
//    the best list head left once the re-scored keys are taken from the
//    partial lists, or the 16th entry of a list all of whose entries were
//    taken (its unseen entries are no larger);
//  * L16 = a lower bound of the exact 16th value (its float32 rounding minus
//    half a unit in the last place).
// L16 > U + eps_m means every entry outside the candidates has z_v < z_16:
// the 16 returned are the exact top-16.

// N2 and N1 (rounded up) over W's rows; out must be zeroed first.
__global__ __launch_bounds__(256) void head_weight_bound_kernel(const uint16_t* __restrict__ W, int64_t V, int D,
                                                                unsigned* __restrict__ out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    double best2 = 0.0, best1 = 0.0;
    for (int64_t v = (int64_t)blockIdx.x * 4 + wave; v < V; v += (int64_t)gridDim.x * 4) {
        const uint16_t* wr = W + v * D;
        double s2 = 0.0, s1 = 0.0;
        for (int k = lane * 8; k < D; k += 512) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(wr + k);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double a = bf16_to_f32(q[j] & 0xFFFFu), b = bf16_to_f32(q[j] >> 16);
                s2 = fma(a, a, fma(b, b, s2));
                s1 += fabs(a) + fabs(b);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            s2 += __shfl_xor(s2, off);
            s1 += __shfl_xor(s1, off);
        }
        best2 = fmax(best2, s2);
        best1 = fmax(best1, s1);
    }
    if (lane == 0) {
        // float64 sums of at most 65536 terms err by less than 2^-37 relative
        const float n2 = __double2float_ru(sqrt(best2) * (1.0 + 0x1p-30));
        const float n1 = __double2float_ru(best1 * (1.0 + 0x1p-30));
        atomicMax(out + 0, __float_as_uint(n2));  // non-negative floats order as their bits
        atomicMax(out + 1, __float_as_uint(n1));
    }
}

__global__ void head_bound_clear_kernel(unsigned* out) {
    if (threadIdx.x < 2) out[threadIdx.x] = 0u;
}

// One wavefront per row: the exact-top-16 certificate from the partial lists
// the head left in its workspace (pv, pi: [M][S][16], sorted per list).
__global__ __launch_bounds__(64) void head_certify_kernel(const uint16_t* __restrict__ h, int D, int S,
                                                          const float* __restrict__ pv, const int* __restrict__ pi,
                                                          const float* __restrict__ top_val,
                                                          const float* __restrict__ bound,
                                                          int32_t* __restrict__ certified) {
    const int64_t m = blockIdx.x;
    const int lane = threadIdx.x;
    const uint16_t* hr = h + m * D;
    double s2 = 0.0, mx = 0.0;
    for (int k = lane; k < D; k += 64) {
        const double x = bf16_to_f32(hr[k]);
        s2 = fma(x, x, s2);
        mx = fmax(mx, fabs(x));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        s2 += __shfl_xor(s2, off);
        mx = fmax(mx, __shfl_xor(mx, off));
    }
    // k-way extraction over the lists: lane l holds the heads of lists
    // l, l + 64, ...; 0 marks no list (below every key)
    constexpr int kPer = kMaxLists / 64;
    const float* rv = pv + m * S * kTopK;
    const int* ri = pi + m * S * kTopK;
    int ptr[kPer];
    uint64_t head[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int l = lane + 64 * j;
        ptr[j] = 0;
        head[j] = l < S ? rank_key(rv[l * kTopK], ri[l * kTopK]) : 0ull;
    }
    float exhausted = -INFINITY;  // 16th value of lists taken whole
    uint64_t next = 0ull;         // the best key left after the candidates
    for (int it = 0; it <= kRescore; ++it) {
        uint64_t best = 0ull;
#pragma unroll
        for (int j = 0; j < kPer; ++j) best = head[j] > best ? head[j] : best;
        uint64_t w = best;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t o = shfl_xor_u64(w, off);
            w = o > w ? o : w;
        }
        if (it == kRescore || w <= kEmptyKey) {  // past the candidates, or only empty entries left
            next = w;
            break;
        }
        if (best == w) {  // the list holding it (ids are unique) moves on
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                if (head[j] == w) {
                    const int l = lane + 64 * j;
                    if (++ptr[j] < kTopK) {
                        head[j] = rank_key(rv[l * kTopK + ptr[j]], ri[l * kTopK + ptr[j]]);
                    } else {
                        exhausted = fmaxf(exhausted, rv[l * kTopK + kTopK - 1]);
                        head[j] = 0ull;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) exhausted = fmaxf(exhausted, __shfl_xor(exhausted, off));
    const double U = fmax((double)(next > kEmptyKey ? key_value(next) : -INFINITY), (double)exhausted);
    const double u = 0x1p-23, Du = (double)D * u;
    const double gamma = Du / (1.0 - Du);
    const double eps = gamma * fmin(sqrt(s2) * (double)bound[0], mx * (double)bound[1]) * (1.0 + 0x1p-30);
    const double tv = (double)top_val[m * kTopK + kTopK - 1];
    const double L16 = tv - fabs(tv) * 0x1p-24 - 0x1p-149;
    if (lane == 0) certified[m] = L16 > U + eps ? 1 : 0;
}

int launch_head_weight_bound(const uint16_t* W, int64_t V, int D, float* bound, hipStream_t stream) {
    unsigned* out = reinterpret_cast<unsigned*>(bound);
    hipLaunchKernelGGL(head_bound_clear_kernel, dim3(1), dim3(64), 0, stream, out);
    int st = launch_status();
    if (st != DFLASH_OK) return st;
    const int64_t blocks = std::min<int64_t>((V + 3) / 4, 8 * kCUs);
    hipLaunchKernelGGL(head_weight_bound_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W, V, D, out);
    return launch_status();
}

int launch_head_certify(const uint16_t* h, int64_t M, int D, int64_t V, const float* bound, const float* top_val,
                        const void* ws, int32_t* certified, hipStream_t stream) {
    const HeadPlan p = head_plan(M, V);
    const float* pv = reinterpret_cast<const float*>(ws);
    const int* pi = reinterpret_cast<const int*>(pv + (size_t)M * p.S * kTopK);
    hipLaunchKernelGGL(head_certify_kernel, dim3((unsigned)M), dim3(64), 0, stream, h, D, p.S, pv, pi, top_val,
                       bound, certified);
    return launch_status();
}

}  // namespace dflash
