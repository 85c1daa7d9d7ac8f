// Two-tap dynamic conv fused with the projection that produces its taps
// (gfx950, bf16 MFMA).
//
// Source: tamsi.dev "DFlash 2 - 3x plus de tokens...", section "L'idee, sans le
// papier" (a two-tap conv in the Canon / short-conv style); myaiexp.com
// "DFlash 2", main features (two-tap *dynamic* convolution: the taps depend on
// the token).  Reading: each token's taps are a linear projection of its own
// hidden state, [a | b] = x W_tap^T with W_tap [2D][D]; then
//     y[s][t][c] = a[s][t][c] * x[s][t][c] + b[s][t][c] * x[s][t-1][c],
// x[s][-1][c] = 0.  The taps are never written: they stay in the float32
// accumulators of the projection GEMM, whose epilogue applies the conv.
//
// GEMM shape: M = n_seq * T token rows, N = 2D (a and b), K = D.  A workgroup
// owns an M-block of 64*WM rows and a block of 64 channels, i.e. the 64 rows
// c0.. of W_tap that give a and the 64 rows D+c0.. that give b, so that every
// lane ends with a and b of the same (token, channel) in registers.
// Per chunk of 64 hidden columns the workgroup stages the x rows and the 128
// W_tap rows in LDS (row-contiguous buffer loads, two chunks ahead in
// registers, double-buffered tile, 32-byte row padding against bank
// conflicts) and each of its 2*WM wavefronts multiplies a 16*MT-row x
// 64-column tile (MT x 4 v_mfma_f32_16x16x32_bf16; columns 0-31 are a, 32-63
// are b of the same 32 channels).  In the steady state the next chunk's LDS
// writes and global loads, and the next k-step's fragment reads, are
// scheduled between the MFMAs (scheduling-group hints over a branch-free
// region whose two LDS buffers are declared disjoint).  Operand and accumulator layouts as in the LM head: for
// k-step s lane (r = lane % 16, g = lane / 16) holds k = 32 s + 8 g .. +8 of
// row r; the accumulator lane holds C[4 g + q][r], q = 0..3.
// Workgroups are mapped XCD-aware: the M-blocks of one channel block run next
// to each other on one XCD (its W_tap rows are read from HBM once, then hit
// in that XCD's L2), and the channel blocks resident on one XCD at a time
// share their x rows there.

#include <mutex>
#include <type_traits>

#include "common.hpp"

namespace dflash {

namespace {

constexpr int kProjCh = 64;                     // channels per workgroup
constexpr int kProjDepth = 2;                   // chunks in flight in registers

// WM wavefront rows x 2 wavefront columns; each wavefront owns MT 16-row
// tiles; chunks of KC hidden columns.
template <int WM, int MT, int KC>
struct ProjCfg {
    static constexpr int THREADS = 128 * WM;
    static constexpr int MB = 16 * MT * WM;    // token rows per workgroup
    static constexpr int NB = 2 * kProjCh;     // W_tap rows per workgroup (a then b)
    // LDS pitch: data plus 32 bytes, an odd number of 32-byte granule pairs
    // (2 mod 4 granules of 16 bytes), which keeps fragment reads conflict-free
    static constexpr int ROWB = KC * 2 + 32;
    static constexpr int PIECES = KC / 8;      // 16-byte pieces per row and chunk
    static constexpr int RPL = THREADS / PIECES;  // rows per workgroup-wide load
    static constexpr int HLOADS = MB / RPL;
    static constexpr int WLOADS = NB / RPL;
    static constexpr size_t TILE = (size_t)(MB + NB) * ROWB;
    static constexpr size_t LDS = 2 * TILE;
    static_assert(KC % 32 == 0 && MB % RPL == 0, "whole loads");
    static_assert(WLOADS % 2 == 0 && (WLOADS / 2) * RPL == kProjCh, "a rows, then b rows");
    static_assert(LDS <= 160 * 1024, "LDS per workgroup");
};

// Buffer resource over [base, base + bytes): loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t proj_rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Calls f(std::integral_constant<int, j>) for j = k (0 <= k < N).
template <int N, int J = 0, class F>
__device__ __forceinline__ void proj_slot(int k, F&& f) {
    if constexpr (J < N) {
        if (k == J) f(std::integral_constant<int, J>{});
        else proj_slot<N, J + 1>(k, f);
    }
}

template <int WM, int MT, int KC>
__global__ __launch_bounds__(128 * WM) __attribute__((amdgpu_waves_per_eu(2, 2)))
void conv_proj_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wt, uint16_t* __restrict__ y,
                      int64_t M, int T, int D, int n_mb, int n_cb) {
    using C = ProjCfg<WM, MT, KC>;
    constexpr int kProjRowB = C::ROWB;
    constexpr int kProjPieces = C::PIECES;
    extern __shared__ __align__(16) unsigned char smem[];

    // workgroup -> (M-block, channel block); dispatch is round-robin over the
    // 8 XCDs, so workgroups L, L + 8, ... share an XCD
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int kq = L >> 3;
    const int mb = kq % n_mb;
    const int cb = (kq / n_mb) * 8 + xcd;
    if (cb >= n_cb) return;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int ln = lane & 15, lg = lane >> 4;
    const int wm = wave >> 1, wc = wave & 1;
    const int ri = tid / kProjPieces, pj = tid % kProjPieces;
    const int64_t m0 = (int64_t)mb * C::MB;
    const int c0 = cb * kProjCh;
    const int rows_blk = (int)min<int64_t>(C::MB, M - m0);

    // rows go into the lane offset (rows past the block read as zero), the
    // chunk's column offset into the scalar offset
    const __amdgpu_buffer_rsrc_t xsrc = proj_rsrc(x + m0 * D, (int64_t)rows_blk * D * 2);
    const __amdgpu_buffer_rsrc_t asrc = proj_rsrc(Wt + (int64_t)c0 * D, (int64_t)kProjCh * D * 2);
    const __amdgpu_buffer_rsrc_t bsrc = proj_rsrc(Wt + (int64_t)(D + c0) * D, (int64_t)kProjCh * D * 2);
    const int voff = ri * D * 2 + pj * 16;
    const int qstride = C::RPL * D * 2;
    const int n_ch = D / KC;

    u32x4 hq[kProjDepth][C::HLOADS], wq[kProjDepth][C::WLOADS];
    floatx4 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto load = [&](auto J, int c) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        const int kb = c * KC * 2;
#pragma unroll
        for (int q = 0; q < C::HLOADS; ++q)
            hq[j][q] = __builtin_amdgcn_raw_buffer_load_b128(xsrc, voff + q * qstride, kb, 0);
#pragma unroll
        for (int q = 0; q < C::WLOADS; ++q)
            wq[j][q] = __builtin_amdgcn_raw_buffer_load_b128(q < C::WLOADS / 2 ? asrc : bsrc,
                                                             voff + (q % (C::WLOADS / 2)) * qstride, kb, 0);
    };
    auto store = [&](auto J, unsigned char* __restrict__ tb) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
#pragma unroll
        for (int q = 0; q < C::HLOADS; ++q)
            *reinterpret_cast<u32x4*>(tb + (q * C::RPL + ri) * kProjRowB + pj * 16) = hq[j][q];
        unsigned char* wb = tb + C::MB * kProjRowB;
#pragma unroll
        for (int q = 0; q < C::WLOADS; ++q)
            *reinterpret_cast<u32x4*>(wb + (q * C::RPL + ri) * kProjRowB + pj * 16) = wq[j][q];
    };
    auto compute = [&](const unsigned char* __restrict__ tb) __attribute__((always_inline)) {
        const unsigned char* ha = tb + (wm * 16 * MT + ln) * kProjRowB;
        const unsigned char* wa = tb + (C::MB + wc * 32 + ln) * kProjRowB;   // a rows of this wave's channels
        const unsigned char* wbp = wa + kProjCh * kProjRowB;                 // their b rows
#pragma unroll
        for (int s = 0; s < KC / 32; ++s) {
            const int po = (4 * s + lg) * 16;
            u32x4 a[MT], b[4];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                b[j] = *reinterpret_cast<const u32x4*>(wa + j * 16 * kProjRowB + po);
                b[j + 2] = *reinterpret_cast<const u32x4*>(wbp + j * 16 * kProjRowB + po);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[mt] = *reinterpret_cast<const u32x4*>(ha + mt * 16 * kProjRowB + po);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, a[mt]), __builtin_bit_cast(bf16x8, b[j]), acc[mt][j], 0, 0, 0);
        }
    };
    auto buf = [&](int c) __attribute__((always_inline)) { return smem + (size_t)(c & 1) * C::TILE; };
    // Chunk c: multiply the staged chunk c, stage chunk c+1 from its register
    // slot into the other buffer and refill that slot with chunk c+1+depth.
    // One barrier per chunk: every wavefront has finished multiplying chunk
    // c-1 (the buffer being overwritten) before any passes the barrier of c-1.
    auto step = [&](auto J, int c) __attribute__((always_inline)) {
        compute(buf(c));
        if (c + 1 < n_ch) store(J, buf(c + 1));
        if (c + 1 + kProjDepth < n_ch) load(J, c + 1 + kProjDepth);
        __syncthreads();
    };
    // The same step where both the staging and the refill happen: one
    // branch-free region whose two buffers are declared disjoint, so that the
    // next chunk's LDS writes and global loads can be issued between this
    // chunk's MFMAs instead of after them.
    auto full_step = [&](auto J, int c, const unsigned char* __restrict__ rd, unsigned char* __restrict__ wr)
                         __attribute__((always_inline)) {
        compute(rd);
        store(J, wr);
        load(J, c + 1 + kProjDepth);
        {
            // the first k-step's fragments, then each k-step's MFMAs with the
            // next k-step's fragment reads, the LDS writes and the global
            // loads spread between them
            constexpr int KS = KC / 32;
            constexpr int NL = C::HLOADS + C::WLOADS;
            constexpr int NR = MT + 4;  // fragment reads per k-step
            __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int NW = NL * (s + 1) / KS - NL * s / KS;
                const int nr = s + 1 < KS ? NR : 0;
#pragma unroll
                for (int i = 0; i < 4 * MT; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    else if (i - nr < NW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                    else if (i - nr - NW < NW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
        }
        __syncthreads();
    };
#pragma unroll
    for (int j = 0; j < kProjDepth; ++j)
        if (j < n_ch) proj_slot<kProjDepth>(j, [&](auto J) __attribute__((always_inline)) { load(J, j); });
    store(std::integral_constant<int, 0>{}, buf(0));
    if (kProjDepth < n_ch) load(std::integral_constant<int, 0>{}, kProjDepth);
    __syncthreads();
    static_assert(kProjDepth == 2, "the steady-state loop alternates the two buffers");
    int c = 0;
    for (; c + 2 * kProjDepth < n_ch; c += 2) {
        full_step(std::integral_constant<int, 1>{}, c, smem, smem + C::TILE);
        full_step(std::integral_constant<int, 0>{}, c + 1, smem + C::TILE, smem);
    }
    for (; c < n_ch; ++c)
        proj_slot<kProjDepth>((c + 1) % kProjDepth, [&](auto J) __attribute__((always_inline)) { step(J, c); });

    // Conv epilogue: lane (r, g) holds, for rows 4g + q of each 16-row tile,
    // a (tiles 0, 1) and b (tiles 2, 3) of channels c0 + 32 wc + 16 j + r.
    // y = a x_t + b x_{t-1} in float32 (one fma over a rounded b x_{t-1}),
    // then nearest-even to bf16.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t rb = m0 + wm * 16 * MT + mt * 16 + 4 * lg;  // this lane's first row
        if (rb >= M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ch = c0 + wc * 32 + j * 16 + ln;
            float xv[5];  // rows rb-1 .. rb+3
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int64_t r = rb - 1 + i;
                xv[i] = (r >= 0 && r < M) ? bf16_to_f32(x[r * D + ch]) : 0.f;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t r = rb + q;
                if (r < M) {
                    const float xp = (r % T) != 0 ? xv[q] : 0.f;
                    const float v = fmaf(acc[mt][j][q], xv[q + 1], acc[mt][j + 2][q] * xp);
                    y[r * D + ch] = (uint16_t)f32_to_bf16_rne(v);
                }
            }
        }
    }
}

template <int WM, int MT, int KC>
int launch_proj(const uint16_t* x, const uint16_t* Wt, uint16_t* y, int64_t M, int T, int D, hipStream_t stream) {
    using C = ProjCfg<WM, MT, KC>;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute((const void*)conv_proj_kernel<WM, MT, KC>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
    });
    if (attr != hipSuccess) return DFLASH_ERR_LAUNCH;
    const int n_mb = (int)((M + C::MB - 1) / C::MB);
    const int n_cb = D / kProjCh;
    const int64_t grid = (int64_t)n_mb * ((n_cb + 7) / 8 * 8);
    hipLaunchKernelGGL((conv_proj_kernel<WM, MT, KC>), dim3((unsigned)grid), dim3(C::THREADS), C::LDS, stream, x, Wt, y, M, T,
                       D, n_mb, n_cb);
    return launch_status();
}

}  // namespace

// M = n_seq * T token rows; requires D % 64 == 0 (checked by the caller).
int launch_conv2tap_proj(const uint16_t* x, const uint16_t* Wt, uint16_t* y, int64_t n_seq, int T, int D,
                         hipStream_t stream) {
    const int64_t M = n_seq * T;
    // measured at D = 5120 (interleaved schedule): M = 40 takes 33 us with
    // 32-row, 4-wavefront blocks; M = 320 46 us with 32-row, 8-wavefront
    // blocks; M = 1280 and 2560 160 and 288 us with 64-row, 4-wavefront blocks
    if (M <= 128) return launch_proj<2, 2, 64>(x, Wt, y, M, T, D, stream);
    if (M <= 512) return launch_proj<4, 2, 64>(x, Wt, y, M, T, D, stream);
    return launch_proj<2, 4, 64>(x, Wt, y, M, T, D, stream);
}

}  // namespace dflash
