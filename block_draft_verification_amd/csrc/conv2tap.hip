// Two-tap dynamic depthwise causal conv over block slots (gfx950).
//
// Source: tamsi.dev "DFlash 2 - 3x plus de tokens...", section "L'idee, sans le
// papier" (a two-tap conv of the Canon / short-conv kind around each attention
// and MLP block); myaiexp.com "DFlash 2", main features (two-tap dynamic conv).
// Reading: y[s][t][c] = a*x[s][t][c] + b*x[s][t-1][c], x[s][-1][c] = 0, with a,
// b the token's own taps (taps[s][t][0:D] and taps[s][t][D:2D]).
//
// Layout and mapping: one thread per (token row, eight channels), i.e. every
// wavefront covers 1 KiB of contiguous channels of one token row, and a
// launch has S*T*D/8 threads, enough to keep the whole chip's memory queues
// full even for a single sequence.  A thread reads its row's x and taps and
// the previous row's x (the same bytes the neighbouring thread reads as its
// own x, so that read hits the cache).  Calls of 2^20 threads or more give each
// thread four consecutive rows instead (2^19 or more: two), keeping x[t-1] in
// registers inside the group.  Algorithmic HBM traffic per element: x 2 B + taps 4 B + y 2 B.
//
// Arithmetic: bf16 x bf16 products are exact in float32, so fmaf(a, x, b*xp)
// rounds the exact sum once; the result is rounded to bf16 nearest-even.

#include "common.hpp"

namespace dflash {

#ifndef CONV_R4_MIN
#define CONV_R4_MIN (1 << 20)
#endif

__device__ __forceinline__ uint32_t conv_pair(uint32_t xw, uint32_t aw, uint32_t bw,
                                              float& p0, float& p1) {
    const float x0 = bf16_to_f32(xw & 0xFFFFu), x1 = bf16_to_f32(xw >> 16);
    const float a0 = bf16_to_f32(aw & 0xFFFFu), a1 = bf16_to_f32(aw >> 16);
    const float b0 = bf16_to_f32(bw & 0xFFFFu), b1 = bf16_to_f32(bw >> 16);
    const float y0 = fmaf(a0, x0, b0 * p0);
    const float y1 = fmaf(a1, x1, b1 * p1);
    p0 = x0;
    p1 = x1;
    return f32_to_bf16_rne(y0) | (f32_to_bf16_rne(y1) << 16);
}

// R consecutive token rows per thread (same 8 channels): the previous row's x
// comes from a register except for the thread's first row.
template <int R>
__global__ __launch_bounds__(256) void conv2tap_kernel(const u32x4* __restrict__ x,
                                                       const u32x4* __restrict__ taps,
                                                       u32x4* __restrict__ y, int64_t n_rows, int T, int D8) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n_groups = (n_rows + R - 1) / R;
    if (gid >= n_groups * D8) return;
    const int64_t grp = gid / D8;
    const int c8 = (int)(gid - grp * D8);
    const int64_t row0 = grp * R;
    u32x4 xv[R], av[R], bv[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t row = min(row0 + i, n_rows - 1);  // rows past the end: loaded, not stored
        xv[i] = x[row * D8 + c8];
        av[i] = __builtin_nontemporal_load(taps + row * 2 * D8 + c8);
        bv[i] = __builtin_nontemporal_load(taps + row * 2 * D8 + D8 + c8);
    }
    const int t0 = (int)(row0 % T);
    const u32x4 pv = t0 > 0 ? x[(row0 - 1) * D8 + c8] : u32x4{0u, 0u, 0u, 0u};
    float p[8];
    p[0] = bf16_to_f32(pv.x & 0xFFFFu), p[1] = bf16_to_f32(pv.x >> 16);
    p[2] = bf16_to_f32(pv.y & 0xFFFFu), p[3] = bf16_to_f32(pv.y >> 16);
    p[4] = bf16_to_f32(pv.z & 0xFFFFu), p[5] = bf16_to_f32(pv.z >> 16);
    p[6] = bf16_to_f32(pv.w & 0xFFFFu), p[7] = bf16_to_f32(pv.w >> 16);
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t row = row0 + i;
        if (row >= n_rows) break;
        if (i > 0 && row % T == 0) {  // a new sequence starts inside the group
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = 0.f;
        }
        u32x4 o;
        o.x = conv_pair(xv[i].x, av[i].x, bv[i].x, p[0], p[1]);
        o.y = conv_pair(xv[i].y, av[i].y, bv[i].y, p[2], p[3]);
        o.z = conv_pair(xv[i].z, av[i].z, bv[i].z, p[4], p[5]);
        o.w = conv_pair(xv[i].w, av[i].w, bv[i].w, p[6], p[7]);
        __builtin_nontemporal_store(o, y + row * D8 + c8);
    }
}

int launch_conv2tap(const uint16_t* x, const uint16_t* taps, uint16_t* y, int64_t n_seq,
                    int T, int D, hipStream_t stream) {
    const int D8 = D / 8;
    const int64_t n_rows = n_seq * T;
    const int block = 256;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    const u32x4* tv = reinterpret_cast<const u32x4*>(taps);
    u32x4* yv = reinterpret_cast<u32x4*>(y);
    // large calls (the block-16, batch-32, five-layer shape: 105 MB, 20.2 ->
    // 17.4 us measured): four rows per thread, a quarter of the workgroups and
    // of the x[t-1] re-reads; mid-sized ones (block 8, batch 32, five layers:
    // 52 MB) two rows per thread (9.9 -> 8.5 us; four rows: 9.7 us); small
    // ones one row per thread, the most threads for the memory queues
    if (n_rows * D8 >= (int64_t)CONV_R4_MIN) {
        const int64_t grid = ((n_rows + 3) / 4 * D8 + block - 1) / block;
        hipLaunchKernelGGL(conv2tap_kernel<4>, dim3((unsigned)grid), dim3(block), 0, stream, xv, tv, yv, n_rows, T, D8);
    } else if (n_rows * D8 >= (int64_t)CONV_R4_MIN / 2) {
        const int64_t grid = ((n_rows + 1) / 2 * D8 + block - 1) / block;
        hipLaunchKernelGGL(conv2tap_kernel<2>, dim3((unsigned)grid), dim3(block), 0, stream, xv, tv, yv, n_rows, T, D8);
    } else {
        const int64_t grid = (n_rows * D8 + block - 1) / block;
        hipLaunchKernelGGL(conv2tap_kernel<1>, dim3((unsigned)grid), dim3(block), 0, stream, xv, tv, yv, n_rows, T, D8);
    }
    return launch_status();
}

}  // namespace dflash
