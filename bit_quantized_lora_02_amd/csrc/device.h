// device.h -- device-side helpers shared by the gfx950 kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// The 16 NF4 levels (ascending) and the 15 encode thresholds, passed by value.
struct Levels {
  float v[16];
};
struct Thresholds {
  float v[15];
};

// Two binary32 values -> packed bf16 pair (lo in bits 0..15), round to nearest
// even.  On gfx950 this is one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float x) { return __builtin_bit_cast(bf16_t, (__bf16)x); }

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// D = A.B + C on a 32x32x16 bf16 tile.  Lane l holds A[m = l%32][k = 8(l/32) .. +7],
// B[k = 8(l/32) .. +7][n = l%32]; accumulator element j of lane l is
// C[m = 8(j/4) + 4(l/32) + j%4][n = l%32].
__device__ __forceinline__ f32x16_t mfma_32x32x16(const u32x4_t &a, const u32x4_t &b, const f32x16_t &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Copy the level table into LDS (first 16 threads); the selects keep the
// kernel-argument array out of private memory.
__device__ __forceinline__ void levels_to_lds(const Levels &lv, float *s_lv, int tid) {
  if (tid < 16) {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v = (tid == i) ? lv.v[i] : v;
    s_lv[tid] = v;
  }
}

// Level-pair table for byte-wise decode: entry b = (level[b & 15], level[b >> 4]),
// i.e. the levels of the low and the high nibble of code byte b.  Threads
// 0..255 write one entry each.
__device__ __forceinline__ void pair_levels_to_lds(const Levels &lv, float2 *tab, int tid) {
  if (tid < 256) {
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      lo = ((tid & 15) == i) ? lv.v[i] : lo;
      hi = ((tid >> 4) == i) ? lv.v[i] : hi;
    }
    tab[tid] = make_float2(lo, hi);
  }
}

// 8 codes of one 32-bit word -> 4 packed bf16 pairs of fl32(level * cq), from
// the level-pair table (entry b = levels of the low and high nibble of byte b;
// the address is the byte times 8, one v_lshlrev_b32 with a byte select).
__device__ __forceinline__ u32x4_t decode8_pairs(uint32_t w, float cq, const float2 *tab) {
  u32x4_t o;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float2 l = tab[(w >> (8 * b)) & 0xffu];
    o[b] = pack_bf16x2(__fmul_rn(l.x, cq), __fmul_rn(l.y, cq));
  }
  return o;
}

// Block constant of NF4 block b: fl32(q_b * d_{b/256}).
__device__ __forceinline__ float block_scale(const uint8_t *__restrict__ absmax_q, const float *__restrict__ step,
                                             int64_t b) {
  return __fmul_rn((float)absmax_q[b], step[b >> 8]);
}

// The two loads behind a block constant, kept raw so that a prefetch does not
// make the wave wait for them: the product is formed where it is used.
struct RawScale {
  uint32_t q;
  float d;
};
__device__ __forceinline__ RawScale load_scale(const uint8_t *__restrict__ absmax_q, const float *__restrict__ step,
                                               int64_t b) {
  return RawScale{(uint32_t)absmax_q[b], step[b >> 8]};
}
__device__ __forceinline__ float scale_of(const RawScale &r) { return __fmul_rn((float)r.q, r.d); }

// Decode the 8 nibbles of `codes` (element e in bits 4e..4e+3) into binary32
// products level * cq; each product is rounded once (no contraction).
__device__ __forceinline__ void decode8(uint32_t codes, float cq, const float *s_lv, float out[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = __fmul_rn(s_lv[(codes >> (4 * e)) & 15u], cq);
}

}  // namespace qlora
