// dyn_code.h -- the dynamic 8-bit code books of the block-wise optimizer state, their encoding
// thresholds and a bucket index over them, all computed at compile time (plain C++17: no HIP).
//
// Code book (Dettmers et al., "8-bit Optimizers via Block-wise Quantization", ICLR 2022, the
// dynamic data type; named by "Module 08 - QLoRA & Quantization" (ainiketan.in), "4. QLoRA in
// code", as the paged_adamw_8bit optimizer): in a signed byte (first moment) bit 7 is the sign and,
// among the other 7 bits, E = the leading zeros, then an indicator bit, then F = 6 - E fraction
// bits f; the magnitude is fl32((0.1 + 0.9 ((f + 1) / 2^F)) / 10^E) (binary64, in that order) and
// all-zero bits mean 0.  An unsigned byte (second moment) counts E among 8 bits, F = 7 - E.
// Magnitudes grow with the bits' unsigned value, so the nearest code of a (ties to the smaller
// magnitude) is the number of thresholds below a, threshold i being the largest binary32 value not
// above the exact midpoint of magnitudes i-1 and i.
//
// Bucket index: the bits of a non-negative binary32 value, shifted right by kIxShift, number
// buckets of 64 per octave (the exponent and the top 6 fraction bits).  Entry j of a book's index
// holds the number of thresholds below the lower edge of bucket base + j; at most kCmp thresholds
// fall inside one bucket (checked below), so the code of a is that count plus kCmp comparisons
// with the next thresholds -- the same result as counting all thresholds, for every binary32 a.
#pragma once
#include <stdint.h>

namespace qlora {

constexpr float dyn_mag(int p, int bits) {
  if (p == 0) return 0.f;
  int top = 0;  // the indicator bit
  while ((p >> (top + 1)) != 0) ++top;
  const int E = bits - 1 - top, F = top, f = p - (1 << F);
  double p10 = 1.0;
  for (int i = 0; i < E; ++i) p10 *= 10.0;  // exact
  // each binary64 operation rounded once, in this order
  return (float)((0.1 + 0.9 * ((double)(f + 1) / (double)(1 << F))) / p10);
}
constexpr float below_mid(float lo, float hi) {  // largest binary32 not above (lo + hi) / 2
  const double mid = ((double)lo + (double)hi) * 0.5;  // exact
  float t = (float)mid;
  if ((double)t > mid) t = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, t) - 1u);  // t > 0 here
  return t;
}

// Magnitudes of the unsigned (um) and signed (sm) codes and thr[i] = below_mid(mag[i-1], mag[i])
// (entry 0 unused); the threshold arrays carry kCmp entries of +inf past the end, so that the
// comparisons after the last real threshold never count.
constexpr int kCmpU = 2, kCmpS = 1;
struct DynBooks {
  float um[256], sm[128], ut[256 + kCmpU], st[128 + kCmpS];
};
constexpr DynBooks make_dyn_books() {
  DynBooks b{};
  for (int i = 0; i < 256; ++i) b.um[i] = dyn_mag(i, 8);
  for (int i = 0; i < 128; ++i) b.sm[i] = dyn_mag(i, 7);
  for (int i = 1; i < 256; ++i) b.ut[i] = below_mid(b.um[i - 1], b.um[i]);
  for (int i = 1; i < 128; ++i) b.st[i] = below_mid(b.sm[i - 1], b.sm[i]);
  for (int k = 0; k < kCmpU; ++k) b.ut[256 + k] = __builtin_huge_valf();
  for (int k = 0; k < kCmpS; ++k) b.st[128 + k] = __builtin_huge_valf();
  return b;
}
constexpr DynBooks kBooks = make_dyn_books();

constexpr int kIxShift = 17;                                // 64 buckets per octave
constexpr int kIxTop = (int)(0x3f800000u >> kIxShift);     // bucket of 1.0, the largest normalized value
constexpr int bucket_of(float x) { return (int)(__builtin_bit_cast(uint32_t, x) >> kIxShift); }
constexpr int kIxBaseU = bucket_of(kBooks.ut[1]), kIxBaseS = bucket_of(kBooks.st[1]);  // smallest thresholds
constexpr int kIxLastU = kIxTop - kIxBaseU, kIxLastS = kIxTop - kIxBaseS;             // last entries
constexpr int kIxWordsU = (kIxLastU + 4) / 4, kIxWordsS = (kIxLastS + 4) / 4;        // entries packed 4 per word

struct DynIndex {
  uint32_t u[kIxWordsU], s[kIxWordsS];
  bool ok;  // thresholds strictly increasing and at most kCmp of them inside any bucket
};
// Fills one book's index: values below bucket base and above 1.0 are clamped to the first and last
// bucket, so the first bucket reaches down to 0 and the last up to +inf.
constexpr bool fill_index(uint32_t *w, const float *thr, int n, int base, int last, int ncmp) {
  bool ok = true;
  for (int i = 2; i < n; ++i) ok = ok && thr[i - 1] < thr[i];
  int i = 1;  // first threshold not below the current lower edge
  for (int j = 0; j <= last; ++j) {
    const float lo = j == 0 ? 0.f : __builtin_bit_cast(float, (uint32_t)(base + j) << kIxShift);
    const float hi = j == last ? __builtin_huge_valf() : __builtin_bit_cast(float, (uint32_t)(base + j + 1) << kIxShift);
    while (i < n && thr[i] < lo) ++i;
    int k = i;
    while (k < n && thr[k] < hi) ++k;
    ok = ok && k - i <= ncmp;
    w[j >> 2] |= (uint32_t)(i - 1) << (8 * (j & 3));
  }
  return ok;
}
constexpr DynIndex make_dyn_index() {
  DynIndex x{};
  const bool ok_u = fill_index(x.u, kBooks.ut, 256, kIxBaseU, kIxLastU, kCmpU);
  const bool ok_s = fill_index(x.s, kBooks.st, 128, kIxBaseS, kIxLastS, kCmpS);
  x.ok = ok_u && ok_s;
  return x;
}
constexpr DynIndex kIndex = make_dyn_index();
static_assert(kIndex.ok, "a bucket holds more thresholds than the encoder compares");

// The code of a: the number of thresholds thr[1 ..] below a.  ix: the book's bucket index read as
// bytes, base / last: its first bucket and last entry, thr: its thresholds with the +inf padding.
// NaN and negative inputs (which the optimizer never forms) give 0, as counting would.  constexpr,
// so that the same function serves device code and host checks.
template <int NCMP>
constexpr uint32_t dyn_code(float a, const uint8_t *ix, int base, int last, const float *thr) {
  const uint32_t u = __builtin_bit_cast(uint32_t, a);
  int j = (int)(u >> kIxShift) - base;
  j = j < 0 ? 0 : (j > last ? last : j);
  const int c0 = ix[j];
  int c = c0;
  for (int k = 1; k <= NCMP; ++k) c += a > thr[c0 + k] ? 1 : 0;
  return u > 0x7f800000u ? 0u : (uint32_t)c;
}

}  // namespace qlora
