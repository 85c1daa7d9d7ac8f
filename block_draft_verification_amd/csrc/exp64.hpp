// float64 exponential for the sampler's weights (gfx950).
//
// Every weight the verifiers take is exp(x) with x = (l - m) / tau <= 0 (a
// logit below a maximum) or barely above 0, never near overflow.  For that
// range the general library exponential does more than needed (overflow and
// special-value paths, ~28 VALU instructions); this one takes 16:
//   k = rint(x log2 e),  r = x - k ln2  (Cody-Waite: ln2 in a high part whose
//   32 significant bits make k * LN2_HI exact for |k| < 2^21, and a low part),
//   exp(r) by a degree-10 polynomial on |r| <= ln2 / 2 (Chebyshev fit of exp,
//   fit error 2.2e-16), Horner with fused multiply-adds,
//   result = p * 2^k (ldexp: underflow to subnormals and to 0 rounds there).
// Relative error <= 4e-16 for x in [-708, 1] (measured against a 200-bit
// evaluation with each operation rounded to double as here); below -708 the
// subnormal result is exact to its last place.  x is clamped at -746 first,
// so -inf (an absent entry) weighs exactly 0.  NaN is not expected (logits
// must be finite) and also maps to 0.
#pragma once

#include <hip/hip_runtime.h>

namespace dflash {

__device__ __forceinline__ double exp64(double x) {
    constexpr double kLog2e = 1.4426950408889634;
    constexpr double kLn2Hi = 0.6931471803691238;      // 0x3FE62E42FEE00000
    constexpr double kLn2Lo = 1.9082149292705877e-10;  // ln 2 - kLn2Hi
    constexpr double c0 = 1.0;
    constexpr double c1 = 1.0000000000000067;
    constexpr double c2 = 0.5000000000000006;
    constexpr double c3 = 0.16666666666554314;
    constexpr double c4 = 0.041666666666573066;
    constexpr double c5 = 0.008333333385699212;
    constexpr double c6 = 0.001388888893251478;
    constexpr double c7 = 0.00019841170230570286;
    constexpr double c8 = 2.480150431378554e-05;
    constexpr double c9 = 2.764019739169484e-06;
    constexpr double c10 = 2.7626371065696354e-07;
    x = fmax(x, -746.0);
    const double k = __builtin_rint(x * kLog2e);
    double r = __builtin_fma(-k, kLn2Hi, x);
    r = __builtin_fma(-k, kLn2Lo, r);
    double p = c10;
    p = __builtin_fma(p, r, c9);
    p = __builtin_fma(p, r, c8);
    p = __builtin_fma(p, r, c7);
    p = __builtin_fma(p, r, c6);
    p = __builtin_fma(p, r, c5);
    p = __builtin_fma(p, r, c4);
    p = __builtin_fma(p, r, c3);
    p = __builtin_fma(p, r, c2);
    p = __builtin_fma(p, r, c1);
    p = __builtin_fma(p, r, c0);
    return __builtin_ldexp(p, (int)k);
}

}  // namespace dflash
