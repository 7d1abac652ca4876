// quant.hip -- NF4 block quantization with double quantization, and dequant.
//
// Method ("What does QLoRA change compared with plain LoRA when fine-tuning
// Llama?", katajob.com, sections "NF4: 4-bit NormalFloat" and "Double
// quantization"): one absmax per 64 contiguous weights, each weight coded as
// the nearest of 16 levels after division by its block absmax, and the block
// constants themselves stored in 8 bits with a binary32 step per group of 256.
//
// gfx950 mapping: one 256-thread workgroup owns one group of 256 blocks
// (16384 weights, 64 KB of binary32).  Sixteen lanes cover one 64-weight block
// with a float4 each, so a wave reads 1 KB contiguous per load and the block
// absmax is a 16-lane butterfly.  The group maximum goes through LDS.  The
// weights stay in registers between the absmax pass and the encode pass, so W
// is read from HBM exactly once.
#include "device.h"
#include "launch.h"

namespace qlora {

__global__ __launch_bounds__(256) void k_quantize_nf4(const float *__restrict__ W, int64_t nblk,
                                                      uint8_t *__restrict__ codes, uint8_t *__restrict__ absmax_q,
                                                      float *__restrict__ absmax_step, Thresholds thr) {
  __shared__ float s_c[256];
  __shared__ float s_wmax[4];
  const int tid = threadIdx.x;
  const int sub = tid & 15;  // float4 slot inside the 64-weight block
  const int64_t g = blockIdx.x;
  const int64_t b0 = g * 256;
  const int nb = (int)((nblk - b0) < 256 ? (nblk - b0) : 256);

  float4 w[16];
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int lb = it * 16 + (tid >> 4);
    float m = 0.f;
    if (lb < nb) {
      w[it] = *reinterpret_cast<const float4 *>(W + (b0 + lb) * 64 + sub * 4);
      m = fmaxf(fmaxf(fabsf(w[it].x), fabsf(w[it].y)), fmaxf(fabsf(w[it].z), fabsf(w[it].w)));
    } else {
      w[it] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (sub == 0) s_c[lb] = m;  // exact: a maximum of absolute values
  }
  __syncthreads();

  // group maximum over the 256 block constants (zeros past the end of a partial group)
  float gm = s_c[tid];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) gm = fmaxf(gm, __shfl_xor(gm, o));
  if ((tid & 63) == 0) s_wmax[tid >> 6] = gm;
  __syncthreads();
  gm = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
  const float d = (gm == 0.f) ? 0.f : __fdiv_rn(gm, 255.0f);
  if (tid == 0) absmax_step[g] = d;
  if (tid < nb) {
    int q = 0;
    if (gm != 0.f) {
      const float r = __builtin_rintf(__fdiv_rn(s_c[tid], d));  // round half to even
      q = (int)fminf(fmaxf(r, 0.f), 255.f);
    }
    absmax_q[b0 + tid] = (uint8_t)q;
  }

  // encode with the exact binary32 block absmax: code = #{i : x > thr_i}
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int lb = it * 16 + (tid >> 4);
    if (lb < nb) {
      const float c = s_c[lb];
      const float e[4] = {w[it].x, w[it].y, w[it].z, w[it].w};
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t code = 7u;
        if (c != 0.f) {
          const float x = __fdiv_rn(e[i], c);
          code = 0u;
#pragma unroll
          for (int j = 0; j < 15; ++j) code += (x > thr.v[j]) ? 1u : 0u;
        }
        packed |= code << (4 * i);
      }
      *reinterpret_cast<uint16_t *>(codes + (b0 + lb) * 32 + sub * 2) = (uint16_t)packed;
    }
  }
}

// One thread expands 8 weights (one 32-bit word of codes) into one 16-byte store.
__global__ __launch_bounds__(256) void k_dequant(const uint32_t *__restrict__ codes, const uint8_t *__restrict__ absmax_q,
                                                 const float *__restrict__ step, int64_t n8, u32x4_t *__restrict__ out,
                                                 Levels lv) {
  __shared__ float s_lv[16];
  levels_to_lds(lv, s_lv, threadIdx.x);
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float cq = block_scale(absmax_q, step, i >> 3);
  float v[8];
  decode8(codes[i], cq, s_lv, v);
  u32x4_t o;
  o.x = pack_bf16x2(v[0], v[1]);
  o.y = pack_bf16x2(v[2], v[3]);
  o.z = pack_bf16x2(v[4], v[5]);
  o.w = pack_bf16x2(v[6], v[7]);
  out[i] = o;
}

hipError_t launch_quantize_nf4(const float *W, int64_t n_out, int64_t n_in, uint8_t *codes, uint8_t *absmax_q,
                               float *absmax_step, const Thresholds &thr, hipStream_t s) {
  const int64_t nblk = n_out * n_in / 64;
  const int64_t ngrp = (nblk + 255) / 256;
  if (ngrp == 0) return hipSuccess;
  launch(k_quantize_nf4, dim3((unsigned)ngrp), dim3(256), 0, s, W, nblk, codes, absmax_q, absmax_step, thr);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *codes, const uint8_t *absmax_q, const float *absmax_step, int64_t n_out,
                          int64_t n_in, bf16_t *out, const Levels &lv, hipStream_t s) {
  const int64_t n8 = n_out * n_in / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t grid = (n8 + 255) / 256;
  launch(k_dequant, dim3((unsigned)grid), dim3(256), 0, s, reinterpret_cast<const uint32_t *>(codes),
                     absmax_q, absmax_step, n8, reinterpret_cast<u32x4_t *>(out), lv);
  return hipGetLastError();
}

}  // namespace qlora
