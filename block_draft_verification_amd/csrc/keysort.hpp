// Sortable 64-bit keys and wavefront bitonic networks on them (gfx950 DPP),
// shared by the top-16 kernels and the filtered sampler.
//
// A key packs (value, id) so that a larger key ranks first: larger value,
// then lower id.  Lanes exchange keys with DPP moves inside 16-lane rows
// (row shifts, mirrors, quad permutes) and with a permute across rows.
#pragma once

#include "common.hpp"

namespace dflash {

// 64-bit key ordered like ranks_before: larger value first, then lower id
// (-0 counts as +0, as in the float comparison).
__device__ __forceinline__ uint64_t rank_key(float v, int i) {
    uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    u ^= (u >> 31) ? 0xFFFFFFFFu : 0x80000000u;  // order-preserving map of floats to uint32
    return ((uint64_t)u << 32) | (uint32_t)(0x7FFFFFFF - i);
}
__device__ __forceinline__ float key_value(uint64_t k) {
    const uint32_t u = (uint32_t)(k >> 32);
    return __uint_as_float((u >> 31) ? (u ^ 0x80000000u) : ~u);
}
__device__ __forceinline__ int key_id(uint64_t k) { return 0x7FFFFFFF - (int)(uint32_t)k; }
constexpr uint64_t kEmptyKey = 0x007FFFFF00000000ull;  // rank_key(-inf, 0x7FFFFFFF)

// A 64-bit value from another lane of the same 16-lane row (DPP control CTRL;
// every source lane is inside the row, so no bound control is involved).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)x, CTRL, 0xF, 0xF, true);
    const uint32_t hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, true);
    return ((uint64_t)hi << 32) | lo;
}
// Lane ^ 4 within a row: row_shl:4 brings lane i+4, row_shr:4 lane i-4.
__device__ __forceinline__ uint64_t xor4_u64(uint64_t x, int li) {
    const uint64_t up = dpp_u64<0x104>(x);
    const uint64_t dn = dpp_u64<0x114>(x);
    return (li & 4) ? dn : up;
}
// Compare-exchange with the partner's key p: keep the larger key if keep_max.
__device__ __forceinline__ uint64_t cx(uint64_t k, uint64_t p, bool keep_max) {
    const bool take = (p > k) == keep_max;
    return take ? p : k;
}
// DPP controls: quad_perm [1,0,3,2] / [2,3,0,1] / [3,2,1,0] (lane ^ 1, ^ 2, ^ 3),
// row_half_mirror (^ 7), row_mirror (^ 15), row_ror:8 (^ 8).
constexpr int kDppX1 = 0xB1, kDppX2 = 0x4E, kDppX3 = 0x1B, kDppX7 = 0x141, kDppX15 = 0x140, kDppX8 = 0x128;

// Bitonic sort of one key per lane over each 16-lane row, descending if DESC.
// Every merge stage starts with the mirrored comparison (lane ^ (2s - 1)) so
// all blocks sort in the same direction; lane ^ 4 takes two row shifts.
template <bool DESC>
__device__ __forceinline__ uint64_t sort16(uint64_t k, int li) {
    k = cx(k, dpp_u64<kDppX1>(k), ((li & 1) == 0) == DESC);
    k = cx(k, dpp_u64<kDppX3>(k), ((li & 2) == 0) == DESC);
    k = cx(k, dpp_u64<kDppX1>(k), ((li & 1) == 0) == DESC);
    k = cx(k, dpp_u64<kDppX7>(k), ((li & 4) == 0) == DESC);
    k = cx(k, dpp_u64<kDppX2>(k), ((li & 2) == 0) == DESC);
    k = cx(k, dpp_u64<kDppX1>(k), ((li & 1) == 0) == DESC);
    k = cx(k, dpp_u64<kDppX15>(k), ((li & 8) == 0) == DESC);
    k = cx(k, xor4_u64(k, li), ((li & 4) == 0) == DESC);
    k = cx(k, dpp_u64<kDppX2>(k), ((li & 2) == 0) == DESC);
    k = cx(k, dpp_u64<kDppX1>(k), ((li & 1) == 0) == DESC);
    return k;
}
// Sort a bitonic sequence of 16 keys (one per lane of a row) descending.
__device__ __forceinline__ uint64_t merge16_desc(uint64_t k, int li) {
    k = cx(k, dpp_u64<kDppX8>(k), (li & 8) == 0);
    k = cx(k, xor4_u64(k, li), (li & 4) == 0);
    k = cx(k, dpp_u64<kDppX2>(k), (li & 2) == 0);
    k = cx(k, dpp_u64<kDppX1>(k), (li & 1) == 0);
    return k;
}

// The same networks on plain float32 values (no ids), for thresholds.
template <int CTRL>
__device__ __forceinline__ float dpp_f32v(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float xor4_f32(float x, int li) {
    const float up = dpp_f32v<0x104>(x);
    const float dn = dpp_f32v<0x114>(x);
    return (li & 4) ? dn : up;
}
__device__ __forceinline__ float cxf(float k, float p, bool keep_max) { return keep_max ? fmaxf(k, p) : fminf(k, p); }
// Descending bitonic sort of one value per lane over each 16-lane row.
__device__ __forceinline__ float sort16_desc_f32(float k, int li) {
    k = cxf(k, dpp_f32v<kDppX1>(k), (li & 1) == 0);
    k = cxf(k, dpp_f32v<kDppX3>(k), (li & 2) == 0);
    k = cxf(k, dpp_f32v<kDppX1>(k), (li & 1) == 0);
    k = cxf(k, dpp_f32v<kDppX7>(k), (li & 4) == 0);
    k = cxf(k, dpp_f32v<kDppX2>(k), (li & 2) == 0);
    k = cxf(k, dpp_f32v<kDppX1>(k), (li & 1) == 0);
    k = cxf(k, dpp_f32v<kDppX15>(k), (li & 8) == 0);
    k = cxf(k, xor4_f32(k, li), (li & 4) == 0);
    k = cxf(k, dpp_f32v<kDppX2>(k), (li & 2) == 0);
    k = cxf(k, dpp_f32v<kDppX1>(k), (li & 1) == 0);
    return k;
}
// Sort a bitonic sequence of 16 values (one per lane of a row) descending.
__device__ __forceinline__ float merge16_desc_f32(float k, int li) {
    k = cxf(k, dpp_f32v<kDppX8>(k), (li & 8) == 0);
    k = cxf(k, xor4_f32(k, li), (li & 4) == 0);
    k = cxf(k, dpp_f32v<kDppX2>(k), (li & 2) == 0);
    k = cxf(k, dpp_f32v<kDppX1>(k), (li & 1) == 0);
    return k;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, m);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}
// Lane ^ m for any m: DPP inside 16-lane rows where one exists, else a permute.
template <int M>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t k, int lane) {
    if constexpr (M == 1) return dpp_u64<kDppX1>(k);
    else if constexpr (M == 2) return dpp_u64<kDppX2>(k);
    else if constexpr (M == 3) return dpp_u64<kDppX3>(k);
    else if constexpr (M == 4) return xor4_u64(k, lane & 15);
    else if constexpr (M == 7) return dpp_u64<kDppX7>(k);
    else if constexpr (M == 8) return dpp_u64<kDppX8>(k);
    else if constexpr (M == 15) return dpp_u64<kDppX15>(k);
    else return shfl_xor_u64(k, M);
}
// Bitonic sort of one key per lane across the wavefront, descending: merge
// stages start with the mirrored comparison (lane ^ (2s - 1)), so every block
// sorts in the same direction.
template <int S2 = 1>
__device__ __forceinline__ uint64_t sort64_stage(uint64_t k, int lane) {
    if constexpr (S2 < 64) {
        k = cx(k, xor_lane_u64<2 * S2 - 1>(k, lane), (lane & S2) == 0);
        if constexpr (S2 >= 32) k = cx(k, xor_lane_u64<16>(k, lane), (lane & 16) == 0);
        if constexpr (S2 >= 16) k = cx(k, xor_lane_u64<8>(k, lane), (lane & 8) == 0);
        if constexpr (S2 >= 8) k = cx(k, xor_lane_u64<4>(k, lane), (lane & 4) == 0);
        if constexpr (S2 >= 4) k = cx(k, xor_lane_u64<2>(k, lane), (lane & 2) == 0);
        if constexpr (S2 >= 2) k = cx(k, xor_lane_u64<1>(k, lane), (lane & 1) == 0);
        return sort64_stage<S2 * 2>(k, lane);
    } else {
        return k;
    }
}
__device__ __forceinline__ uint64_t sort64_desc(uint64_t k, int lane) { return sort64_stage<1>(k, lane); }

// The key held by lane l (l wavefront-uniform), in every lane.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
// Largest key over aligned groups of b consecutive lanes (b = 1, 2, 4, 8 or
// 16, wavefront-uniform), in every lane of the group: quad permutes, then the
// half-row and row mirrors.
__device__ __forceinline__ uint64_t group_max_u64(uint64_t k, int b) {
    uint64_t p;
    if (b >= 2) p = dpp_u64<kDppX1>(k), k = p > k ? p : k;
    if (b >= 4) p = dpp_u64<kDppX2>(k), k = p > k ? p : k;
    if (b >= 8) p = dpp_u64<kDppX7>(k), k = p > k ? p : k;
    if (b >= 16) p = dpp_u64<kDppX15>(k), k = p > k ? p : k;
    return k;
}

}  // namespace dflash
