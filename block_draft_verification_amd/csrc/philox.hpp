// Philox4x64-10 counter-based generator (device side), shared by the
// sampling verifiers and the sampled-path selector.
#pragma once

#include "common.hpp"

namespace dflash {

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): counter words 0 and 2 are
// multiplied by two fixed odd constants; high/low product halves are xored with
// words 1, 3 and the round key; the key advances by two Weyl constants.
struct Philox4 {
    uint64_t w[4];
};

__device__ inline Philox4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                 uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
        const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
        const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    Philox4 out;
    out.w[0] = c0;
    out.w[1] = c1;
    out.w[2] = c2;
    out.w[3] = c3;
    return out;
}

}  // namespace dflash
