// recip_div.h -- a / b, correctly rounded (binary32, round to nearest), from a correctly rounded
// reciprocal y = RN(1 / b) and fused multiply-adds, for divisions that share their divisor.
//
// q0 = RN(a y) lies within 1.5 ulp of a / b.  One correction q1 = RN(q0 + r0 y), r0 = RN(a - b q0),
// brings it within (1/2 + 2^-22) ulp, i.e. within 1 ulp; then the remainder r1 = a - b q1 is exact
// (an FMA) and q2 = RN(q1 + r1 y) is the correctly rounded quotient (P. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990; the
// theorem as stated in Muller et al., "Handbook of Floating-Point Arithmetic", division by FMA with a
// correctly rounded reciprocal).  A quotient of binary32 numbers is never halfway between two
// binary32 numbers, so no tie arises.  The remainders are exact only without underflow and a y must
// not overflow: the callers keep b in [2^-75, 2^100] (y is then a normal number), |a| <= 2^126 and
// |a / b| <= 2^126 (their quotients are at most 1, or 2^91 for sqrt(v) / sqrt(1 - beta2^t)), and the
// result is exact whenever |a / b| >= 2^-28 (exponents of b and q add to >= -103, so b q1
// has no bits below 2^-149); below that it is within 2^-149 / b of the quotient.  (Checked on the
// host against binary64 division for every binary32 a and 13 divisors, and a sample of 200 more; the
// only failures were at |a| ~ 2^128 or overflowing quotients, where a y overflows.)  Host and device: the host checks compile
// this same function.
#pragma once

namespace qlora {

constexpr float kRecipDivMinB = 0x1p-75f, kRecipDivMaxB = 0x1p100f, kRecipDivMaxA = 0x1p126f;

__host__ __device__ inline float recip_div(float a, float b, float y) {
  const float q0 = a * y;
  const float r0 = __builtin_fmaf(-b, q0, a);
  const float q1 = __builtin_fmaf(r0, y, q0);
  const float r1 = __builtin_fmaf(-b, q1, a);
  return __builtin_fmaf(r1, y, q1);
}

}  // namespace qlora
