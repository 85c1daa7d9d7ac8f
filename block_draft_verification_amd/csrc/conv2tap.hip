// Two-tap dynamic depthwise causal conv over block slots (gfx950).
//
// Source: tamsi.dev "DFlash 2 - 3x plus de tokens...", section "L'idee, sans le
// papier" (a two-tap conv of the Canon / short-conv kind around each attention
// and MLP block); myaiexp.com "DFlash 2", main features (two-tap dynamic conv).
// Reading: y[s][t][c] = a*x[s][t][c] + b*x[s][t-1][c], x[s][-1][c] = 0, with a,
// b the token's own taps (taps[s][t][0:D] and taps[s][t][D:2D]).
//
// Layout and mapping: one thread owns eight channels (one 16-byte vector) of
// one sequence and walks its T slots, so x is read from HBM exactly once and
// x[t-1] comes from a register.  Consecutive threads own consecutive 16-byte
// vectors of the same row: every load and store of a wavefront covers 1 KiB of
// contiguous memory.  All 3T loads of a thread are issued before any math.
// HBM traffic per element: x 2 B + taps 4 B + y 2 B.
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

template <int TMAX>
__global__ __launch_bounds__(256) void conv2tap_kernel(const u32x4* __restrict__ x,
                                                       const u32x4* __restrict__ taps,
                                                       u32x4* __restrict__ y,
                                                       int64_t n_seq, int T, int D8) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_seq * D8) return;
    const int64_t s = gid / D8;
    const int c8 = (int)(gid - s * D8);
    const u32x4* xs = x + s * T * D8 + c8;
    const u32x4* ts = taps + s * T * 2 * D8 + c8;
    u32x4* ys = y + s * T * D8 + c8;

    u32x4 xv[TMAX], av[TMAX], bv[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t < T) {
            xv[t] = __builtin_nontemporal_load(xs + (int64_t)t * D8);
            av[t] = __builtin_nontemporal_load(ts + (int64_t)t * 2 * D8);
            bv[t] = __builtin_nontemporal_load(ts + (int64_t)t * 2 * D8 + D8);
        }
    }
    float p[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t < T) {
            u32x4 o;
            o.x = conv_pair(xv[t].x, av[t].x, bv[t].x, p[0], p[1]);
            o.y = conv_pair(xv[t].y, av[t].y, bv[t].y, p[2], p[3]);
            o.z = conv_pair(xv[t].z, av[t].z, bv[t].z, p[4], p[5]);
            o.w = conv_pair(xv[t].w, av[t].w, bv[t].w, p[6], p[7]);
            __builtin_nontemporal_store(o, ys + (int64_t)t * D8);
        }
    }
}

int launch_conv2tap(const uint16_t* x, const uint16_t* taps, uint16_t* y, int64_t n_seq,
                    int T, int D, hipStream_t stream) {
    const int D8 = D / 8;
    const int64_t threads = n_seq * D8;
    const int block = 256;
    const int64_t grid = (threads + block - 1) / block;
    const u32x4* xp = reinterpret_cast<const u32x4*>(x);
    const u32x4* tp = reinterpret_cast<const u32x4*>(taps);
    u32x4* yp = reinterpret_cast<u32x4*>(y);
    if (T <= 4)
        hipLaunchKernelGGL(conv2tap_kernel<4>, dim3((unsigned)grid), dim3(block), 0, stream, xp, tp, yp, n_seq, T, D8);
    else if (T <= 8)
        hipLaunchKernelGGL(conv2tap_kernel<8>, dim3((unsigned)grid), dim3(block), 0, stream, xp, tp, yp, n_seq, T, D8);
    else
        hipLaunchKernelGGL(conv2tap_kernel<16>, dim3((unsigned)grid), dim3(block), 0, stream, xp, tp, yp, n_seq, T, D8);
    return launch_status();
}

}  // namespace dflash
