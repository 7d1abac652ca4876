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
#include "dyn_code.h"
#include "recip_div.h"
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {

// (sqrtf is the correctly rounded square root; __fsqrt_rn would be the native one here).  sqrt(v) /
// sqrt_bc2 divides by a constant of the launch: recip_div from the host's RN(1 / sqrt_bc2) gives the
// same correctly rounded quotient (sqrt(v) <= 2^64 unless v is infinite, which passes through).
template <class P>
__device__ __forceinline__ float adam_elem(float &m, float &v, float theta, float g, const P &a) {
  m = __fadd_rn(__fmul_rn(a.b1, m), __fmul_rn(a.omb1, g));
  v = __fadd_rn(__fmul_rn(a.b2, v), __fmul_rn(__fmul_rn(a.omb2, g), g));
  const float sv = sqrtf(v);
  const float sq = a.fast_bc2 ? (__builtin_isinf(sv) ? sv : recip_div(sv, a.sqrt_bc2, a.rbc2)) : __fdiv_rn(sv, a.sqrt_bc2);
  const float denom = __fadd_rn(sq, a.eps);
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

// ------------------------------------------------------------ 8-bit state
// "Module 08 - QLoRA & Quantization" (ainiketan.in), "4. QLoRA in code" and "5.
// Other memory-saving levers": paged_adamw_8bit keeps the state in 8 bits.
// Block-wise state quantization after Dettmers et al., "8-bit Optimizers via
// Block-wise Quantization" (ICLR 2022): per block of 2048 elements, 8-bit codes
// and one binary32 absmax for each moment, in the dynamic code books of
// dyn_code.h (nearest code, ties to the smaller magnitude).
// One workgroup owns one block: it decodes the moments (fl32(book * absmax)),
// runs the binary32 step of k_adamw, reduces the block's new absmax, and
// encodes x = fl32(value / absmax) through the bucket index: one table read
// and one or two threshold comparisons per code (the books, thresholds and
// index are compile-time constants, copied into LDS).
__constant__ const DynBooks kDynBooks = kBooks;
__constant__ const DynIndex kDynIndex = kIndex;

__global__ __launch_bounds__(256) void k_adamw8(Adam8Params a) {
  __shared__ float s_sm[128], s_um[256], s_st[128 + kCmpS], s_ut[256 + kCmpU];
  __shared__ uint32_t s_ixu[kIxWordsU], s_ixs[kIxWordsS];
  __shared__ float s_red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  s_um[tid] = kDynBooks.um[tid];
  s_ut[tid] = kDynBooks.ut[tid];
  if (tid < 128) {
    s_sm[tid] = kDynBooks.sm[tid];
    s_st[tid] = kDynBooks.st[tid];
  }
  if (tid < kCmpU) s_ut[256 + tid] = kDynBooks.ut[256 + tid];
  if (tid < kCmpS) s_st[128 + tid] = kDynBooks.st[128 + tid];
  for (int i = tid; i < kIxWordsU; i += 256) s_ixu[i] = kDynIndex.u[i];
  for (int i = tid; i < kIxWordsS; i += 256) s_ixs[i] = kDynIndex.s[i];

  const int64_t blk = blockIdx.x;
  uint16_t *p = nullptr;
  const uint16_t *g = nullptr;
  uint8_t *mq = nullptr, *vq = nullptr;
  float *ma = nullptr, *va = nullptr, *master = nullptr;
  int64_t n = 0, b0 = 0;
#pragma unroll
  for (int i = 0; i < kAdamMaxTensors; ++i) {
    if (i < a.count && blk >= a.t[i].block0) {
      p = a.t[i].p, g = a.t[i].g, mq = a.t[i].mq, ma = a.t[i].ma, vq = a.t[i].vq, va = a.t[i].va;
      master = a.t[i].master, n = a.t[i].n, b0 = a.t[i].block0;
    }
  }
  const int64_t lb = blk - b0;  // block of this tensor
  const int64_t e0 = lb * kAdam8Block + (int64_t)tid * 8;
  const int cnt = (int)((n - e0) < 0 ? 0 : ((n - e0) > 8 ? 8 : (n - e0)));
  const float m_abs = ma[lb], v_abs = va[lb];
  __syncthreads();  // books, thresholds and index visible

  float m[8], v[8], th[8];
  uint32_t mc[2] = {0u, 0u}, vc[2] = {0u, 0u};
  float gr[8];
  if (cnt == 8) {
    const u32x2_t mw = *reinterpret_cast<const u32x2_t *>(mq + e0), vw = *reinterpret_cast<const u32x2_t *>(vq + e0);
    mc[0] = mw.x, mc[1] = mw.y, vc[0] = vw.x, vc[1] = vw.y;
    const u32x4_t gw = *reinterpret_cast<const u32x4_t *>(g + e0);
    const u32x4_t pw = *reinterpret_cast<const u32x4_t *>(p + e0);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      gr[2 * w] = bf16_lo_to_f32(gw[w]), gr[2 * w + 1] = bf16_hi_to_f32(gw[w]);
      th[2 * w] = bf16_lo_to_f32(pw[w]), th[2 * w + 1] = bf16_hi_to_f32(pw[w]);
    }
    if (master) {
      const float4 t0 = *reinterpret_cast<const float4 *>(master + e0), t1 = *reinterpret_cast<const float4 *>(master + e0 + 4);
      th[0] = t0.x, th[1] = t0.y, th[2] = t0.z, th[3] = t0.w, th[4] = t1.x, th[5] = t1.y, th[6] = t1.z, th[7] = t1.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gr[e] = 0.f, th[e] = 0.f;
      if (e < cnt) {
        mc[e >> 2] |= (uint32_t)mq[e0 + e] << (8 * (e & 3));
        vc[e >> 2] |= (uint32_t)vq[e0 + e] << (8 * (e & 3));
        gr[e] = __builtin_bit_cast(float, (uint32_t)g[e0 + e] << 16);
        th[e] = master ? master[e0 + e] : __builtin_bit_cast(float, (uint32_t)p[e0 + e] << 16);
      }
    }
  }
  float mx = 0.f, vx = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t cm = (mc[e >> 2] >> (8 * (e & 3))) & 0xffu, cv = (vc[e >> 2] >> (8 * (e & 3))) & 0xffu;
    const float mag = s_sm[cm & 127u];
    m[e] = __fmul_rn((cm & 128u) ? -mag : mag, m_abs);
    v[e] = __fmul_rn(s_um[cv], v_abs);
    th[e] = adam_elem(m[e], v[e], th[e], gr[e], a);
    if (e < cnt) {
      mx = fmaxf(mx, fabsf(m[e]));
      vx = fmaxf(vx, v[e]);
    }
  }
  // block absmax of the new moments
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    vx = fmaxf(vx, __shfl_xor(vx, o));
  }
  if (lane == 0) s_red[0][wave] = mx, s_red[1][wave] = vx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  vx = fmaxf(fmaxf(s_red[1][0], s_red[1][1]), fmaxf(s_red[1][2], s_red[1][3]));
  if (tid == 0) ma[lb] = mx, va[lb] = vx;
  uint32_t om[2] = {0u, 0u}, ov[2] = {0u, 0u};
  // x / absmax through one reciprocal per block where recip_div is exact (|x| <= absmax <= 2^100)
  const bool fm = mx >= kRecipDivMinB && mx <= kRecipDivMaxB, fv = vx >= kRecipDivMinB && vx <= kRecipDivMaxB;
  const float ym = fm ? __fdiv_rn(1.f, mx) : 0.f, yv = fv ? __fdiv_rn(1.f, vx) : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t cm = 0u, cv = 0u;
    if (mx > 0.f) {
      const float x = fm ? recip_div(m[e], mx, ym) : __fdiv_rn(m[e], mx);
      cm = dyn_code<kCmpS>(fabsf(x), reinterpret_cast<const uint8_t *>(s_ixs), kIxBaseS, kIxLastS, s_st);
      if (x < 0.f && cm) cm |= 128u;
    }
    if (vx > 0.f)
      cv = dyn_code<kCmpU>(fv ? recip_div(v[e], vx, yv) : __fdiv_rn(v[e], vx), reinterpret_cast<const uint8_t *>(s_ixu),
                           kIxBaseU, kIxLastU, s_ut);
    om[e >> 2] |= cm << (8 * (e & 3));
    ov[e >> 2] |= cv << (8 * (e & 3));
  }
  if (cnt == 8) {
    *reinterpret_cast<u32x2_t *>(mq + e0) = u32x2_t{om[0], om[1]};
    *reinterpret_cast<u32x2_t *>(vq + e0) = u32x2_t{ov[0], ov[1]};
    u32x4_t po;
#pragma unroll
    for (int w = 0; w < 4; ++w) po[w] = pack_bf16x2(th[2 * w], th[2 * w + 1]);
    *reinterpret_cast<u32x4_t *>(p + e0) = po;
    if (master) {
      *reinterpret_cast<float4 *>(master + e0) = make_float4(th[0], th[1], th[2], th[3]);
      *reinterpret_cast<float4 *>(master + e0 + 4) = make_float4(th[4], th[5], th[6], th[7]);
    }
  } else {
    for (int e = 0; e < cnt; ++e) {
      mq[e0 + e] = (uint8_t)(om[e >> 2] >> (8 * (e & 3)));
      vq[e0 + e] = (uint8_t)(ov[e >> 2] >> (8 * (e & 3)));
      p[e0 + e] = f32_to_bf16(th[e]);
      if (master) master[e0 + e] = th[e];
    }
  }
}

hipError_t launch_adamw8(const Adam8Params &a, int64_t blocks, hipStream_t s) {
  if (blocks == 0) return hipSuccess;
  launch(k_adamw8, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamParams &a, int64_t blocks, hipStream_t s) {
  if (blocks == 0) return hipSuccess;
  launch(k_adamw, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qlora
