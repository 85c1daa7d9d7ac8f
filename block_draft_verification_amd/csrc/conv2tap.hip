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
// own x, so that read hits the cache).  Algorithmic HBM traffic per element:
// x 2 B + taps 4 B + y 2 B.
//
// Arithmetic: bf16 x bf16 products are exact in float32, so fmaf(a, x, b*xp)
// rounds the exact sum once; the result is rounded to bf16 nearest-even.

#include "common.hpp"

namespace dflash {

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

__global__ __launch_bounds__(256) void conv2tap_kernel(const u32x4* __restrict__ x,
                                                       const u32x4* __restrict__ taps,
                                                       u32x4* __restrict__ y, int64_t n_rows, int T, int D8) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_rows * D8) return;
    const int64_t row = gid / D8;  // s * T + t
    const int c8 = (int)(gid - row * D8);
    const int t = (int)(row % T);
    const u32x4 xv = x[row * D8 + c8];
    const u32x4 av = __builtin_nontemporal_load(taps + row * 2 * D8 + c8);
    const u32x4 bv = __builtin_nontemporal_load(taps + row * 2 * D8 + D8 + c8);
    const u32x4 pv = t > 0 ? x[(row - 1) * D8 + c8] : u32x4{0u, 0u, 0u, 0u};
    float p[8];
    p[0] = bf16_to_f32(pv.x & 0xFFFFu), p[1] = bf16_to_f32(pv.x >> 16);
    p[2] = bf16_to_f32(pv.y & 0xFFFFu), p[3] = bf16_to_f32(pv.y >> 16);
    p[4] = bf16_to_f32(pv.z & 0xFFFFu), p[5] = bf16_to_f32(pv.z >> 16);
    p[6] = bf16_to_f32(pv.w & 0xFFFFu), p[7] = bf16_to_f32(pv.w >> 16);
    u32x4 o;
    o.x = conv_pair(xv.x, av.x, bv.x, p[0], p[1]);
    o.y = conv_pair(xv.y, av.y, bv.y, p[2], p[3]);
    o.z = conv_pair(xv.z, av.z, bv.z, p[4], p[5]);
    o.w = conv_pair(xv.w, av.w, bv.w, p[6], p[7]);
    __builtin_nontemporal_store(o, y + row * D8 + c8);
}

int launch_conv2tap(const uint16_t* x, const uint16_t* taps, uint16_t* y, int64_t n_seq,
                    int T, int D, hipStream_t stream) {
    const int D8 = D / 8;
    const int64_t n_rows = n_seq * T;
    const int block = 256;
    const int64_t grid = (n_rows * D8 + block - 1) / block;
    hipLaunchKernelGGL(conv2tap_kernel, dim3((unsigned)grid), dim3(block), 0, stream,
                       reinterpret_cast<const u32x4*>(x), reinterpret_cast<const u32x4*>(taps),
                       reinterpret_cast<u32x4*>(y), n_rows, T, D8);
    return launch_status();
}

}  // namespace dflash
