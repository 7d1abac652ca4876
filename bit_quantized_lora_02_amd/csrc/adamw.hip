// adamw.hip -- one fused AdamW step over a list of adapter tensors.
//
// "What does QLoRA change compared with plain LoRA when fine-tuning Llama?"
// (katajob.com), "What stays in full precision": the adapters A and B are bf16
// tensors with ordinary AdamW state; "QLoRA: fine-tuning a large model on one
// GPU" (pranaymahendrakar), Developer level, "The walkthrough": about 8 bytes
// of Adam state per trainable parameter, i.e. two binary32 moments.  AdamW is
// Adam with the weight decay decoupled from the gradient (Loshchilov and
// Hutter, ICLR 2019), here with a constant schedule multiplier.
//
// Per element, in binary32 with every operation rounded once (no contraction):
//   m     = b1 m + (1 - b1) g
//   v     = b2 v + ((1 - b2) g) g
//   theta = theta decay - step_size (m / (sqrt(v) / sqrt_bc2 + eps))
// where the host forms decay = fl32(1 - lr wd), step_size = fl32(lr / (1 - b1^t))
// and sqrt_bc2 = fl32(sqrt(1 - b2^t)) in binary64.  theta is the binary32
// master copy when the caller keeps one, else the bf16 parameter widened; the
// parameter is stored as bf16_rne(theta).
//
// gfx950 mapping: the step is HBM-bound (22 bytes per element, 30 with a master
// copy) and short, so one launch covers up to 32 tensors, whose descriptors
// travel in the kernel arguments.  A 256-thread workgroup takes 2048
// consecutive elements of one tensor, 8 per thread: one 16-byte load of the
// parameter and of the gradient, two of each binary32 array.
#include "adamw.h"
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {

__device__ __forceinline__ float adam_elem(float &m, float &v, float theta, float g, const AdamParams &a) {
  m = __fadd_rn(__fmul_rn(a.b1, m), __fmul_rn(a.omb1, g));
  v = __fadd_rn(__fmul_rn(a.b2, v), __fmul_rn(__fmul_rn(a.omb2, g), g));
  const float denom = __fadd_rn(__fdiv_rn(__fsqrt_rn(v), a.sqrt_bc2), a.eps);
  return __fsub_rn(__fmul_rn(theta, a.decay), __fmul_rn(a.step_size, __fdiv_rn(m, denom)));
}

}  // namespace

__global__ __launch_bounds__(256) void k_adamw(AdamParams a) {
  // the tensor of this workgroup (uniform), picked with selects so that the
  // descriptors are read straight from the kernel arguments
  const int64_t blk = blockIdx.x;
  bf16_t *p = nullptr;
  const bf16_t *g = nullptr;
  float *m = nullptr, *v = nullptr, *master = nullptr;
  int64_t n = 0, b0 = 0;
#pragma unroll
  for (int i = 0; i < kAdamMaxTensors; ++i) {
    if (i < a.count && blk >= a.t[i].block0) {
      p = a.t[i].p;
      g = a.t[i].g;
      m = a.t[i].m;
      v = a.t[i].v;
      master = a.t[i].master;
      n = a.t[i].n;
      b0 = a.t[i].block0;
    }
  }
  const int64_t e0 = (blk - b0) * kAdamChunk + (int64_t)threadIdx.x * 8;
  if (e0 >= n) return;
  if (e0 + 8 <= n) {
    const u32x4_t pw = *reinterpret_cast<const u32x4_t *>(p + e0);
    const u32x4_t gw = *reinterpret_cast<const u32x4_t *>(g + e0);
    float4 mv[2], vv[2], tv[2];
    mv[0] = *reinterpret_cast<const float4 *>(m + e0);
    mv[1] = *reinterpret_cast<const float4 *>(m + e0 + 4);
    vv[0] = *reinterpret_cast<const float4 *>(v + e0);
    vv[1] = *reinterpret_cast<const float4 *>(v + e0 + 4);
    if (master) {
      tv[0] = *reinterpret_cast<const float4 *>(master + e0);
      tv[1] = *reinterpret_cast<const float4 *>(master + e0 + 4);
    }
    float mm[8], vs[8], th[8], gr[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      mm[4 * h] = mv[h].x, mm[4 * h + 1] = mv[h].y, mm[4 * h + 2] = mv[h].z, mm[4 * h + 3] = mv[h].w;
      vs[4 * h] = vv[h].x, vs[4 * h + 1] = vv[h].y, vs[4 * h + 2] = vv[h].z, vs[4 * h + 3] = vv[h].w;
      if (master) th[4 * h] = tv[h].x, th[4 * h + 1] = tv[h].y, th[4 * h + 2] = tv[h].z, th[4 * h + 3] = tv[h].w;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      gr[2 * w] = bf16_lo_to_f32(gw[w]);
      gr[2 * w + 1] = bf16_hi_to_f32(gw[w]);
      if (!master) {
        th[2 * w] = bf16_lo_to_f32(pw[w]);
        th[2 * w + 1] = bf16_hi_to_f32(pw[w]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) th[e] = adam_elem(mm[e], vs[e], th[e], gr[e], a);
    u32x4_t po;
#pragma unroll
    for (int w = 0; w < 4; ++w) po[w] = pack_bf16x2(th[2 * w], th[2 * w + 1]);
    *reinterpret_cast<u32x4_t *>(p + e0) = po;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<float4 *>(m + e0 + 4 * h) = make_float4(mm[4 * h], mm[4 * h + 1], mm[4 * h + 2], mm[4 * h + 3]);
      *reinterpret_cast<float4 *>(v + e0 + 4 * h) = make_float4(vs[4 * h], vs[4 * h + 1], vs[4 * h + 2], vs[4 * h + 3]);
      if (master)
        *reinterpret_cast<float4 *>(master + e0 + 4 * h) =
            make_float4(th[4 * h], th[4 * h + 1], th[4 * h + 2], th[4 * h + 3]);
    }
    return;
  }
  for (int64_t e = e0; e < n; ++e) {  // the ragged end of a tensor
    float mm = m[e], vs = v[e];
    const float theta = master ? master[e] : __builtin_bit_cast(float, (uint32_t)p[e] << 16);
    const float gr = __builtin_bit_cast(float, (uint32_t)g[e] << 16);
    const float t = adam_elem(mm, vs, theta, gr, a);
    m[e] = mm;
    v[e] = vs;
    if (master) master[e] = t;
    p[e] = f32_to_bf16(t);
  }
}

hipError_t launch_adamw(const AdamParams &a, int64_t blocks, hipStream_t s) {
  if (blocks == 0) return hipSuccess;
  launch(k_adamw, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qlora
