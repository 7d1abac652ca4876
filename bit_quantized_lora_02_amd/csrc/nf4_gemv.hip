// nf4_gemv.hip -- the forward for few tokens (T <= 64), where the layer is bound
// by streaming the 4-bit weight from HBM, not by arithmetic.
//
// Same computation as the tiled forward ("What does QLoRA change compared with
// plain LoRA when fine-tuning Llama?", katajob.com, "NF4: 4-bit NormalFloat":
// blocks expanded to bf16 inside the matmul), organised for bandwidth:
//   * a workgroup (4 waves) owns 64 weight rows and one K range; each wave
//     owns 16 rows and issues v_mfma_f32_16x16x32_bf16 with the tokens as the
//     M dimension (T padded to 16 * MT);
//   * each lane streams 16 bytes of codes (32 consecutive weights of one row,
//     one block constant) per 128-deep step and decodes them straight into
//     its four B operands, so the weight never touches LDS.  The four lane
//     groups of a wave take the four 32-wide slices of the 128-deep step; the
//     activation operand is loaded with the same slice mapping, which is a
//     consistent permutation of the reduction index;
//   * codes are prefetched two steps ahead to keep enough bytes in flight;
//   * K is split across workgroups so that every CU has several; the binary32
//     partial sums go to a workspace and a second kernel adds them in a fixed
//     order, adds the LoRA term s U B^T and rounds to bf16.
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
}  // namespace

// part[split][t][n] = sum over k in this workgroup's range of X[t, k] W'[n, k]
template <int MT>
__global__ __launch_bounds__(256) void k_nf4_gemv(const bf16_t *__restrict__ X, int64_t T, int64_t K,
                                                  const uint8_t *__restrict__ codes,
                                                  const uint8_t *__restrict__ absmax_q,
                                                  const float *__restrict__ step, int64_t N, int64_t kchunk,
                                                  float *__restrict__ part, Levels lv) {
  __shared__ float s_lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  levels_to_lds(lv, s_lv, tid);
  __syncthreads();
  const int g = lane >> 4;  // 32-wide slice of each 128-deep step
  const int64_t n = (int64_t)blockIdx.x * 64 + wave * 16 + (lane & 15);
  const bool nok = n < N;
  const int64_t kb = (int64_t)blockIdx.y * kchunk;
  const int64_t ke = (kb + kchunk < K) ? kb + kchunk : K;
  const int nsteps = (int)((ke - kb) / 128);
  const uint8_t *crow = codes + n * (K / 2);

  auto load_codes = [&](int s, u32x4_t &c, RawScale &cq) {
    const int64_t k = kb + (int64_t)s * 128 + 32 * g;
    if (nok && s < nsteps) {
      c = *reinterpret_cast<const u32x4_t *>(crow + k / 2);
      cq = load_scale(absmax_q, step, n * (K / 64) + k / 64);
    } else {
      c = u32x4_t{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
      cq = RawScale{0u, 0.f};
    }
  };

  f32x4_t acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t c0, c1;
  RawScale q0, q1;
  load_codes(0, c0, q0);
  load_codes(1, c1, q1);
  for (int s = 0; s < nsteps; ++s) {
    const int64_t k = kb + (int64_t)s * 128 + 32 * g;
    // activation operands: token t = 16 m + (lane & 15), the same 32-wide slice.
    // Rows past T read row T-1 (finite values) and only feed accumulator rows
    // that are never stored, so the loads need no branch.
    u32x4_t a[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      int64_t t = m * 16 + (lane & 15);
      t = t < T ? t : T - 1;
#pragma unroll
      for (int q = 0; q < 4; ++q) a[m][q] = *reinterpret_cast<const u32x4_t *>(X + t * K + k + 8 * q);
    }
    // prefetch two steps ahead, issued after the activation loads so that
    // waiting for those does not wait for the prefetch
    u32x4_t c2;
    RawScale q2;
    load_codes(s + 2, c2, q2);
    const float cq = scale_of(q0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[8];
      decode8(c0[q], cq, s_lv, v);
      u32x4_t b;
      b.x = pack_bf16x2(v[0], v[1]);
      b.y = pack_bf16x2(v[2], v[3]);
      b.z = pack_bf16x2(v[4], v[5]);
      b.w = pack_bf16x2(v[6], v[7]);
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = mfma_16x16x32(a[m][q], b, acc[m]);
    }
    c0 = c1;
    q0 = q1;
    c1 = c2;
    q1 = q2;
  }
  // accumulator element j of lane l holds token 16 m + 4 (l >> 4) + j, row n
  if (nok) {
    float *dst = part + (int64_t)blockIdx.y * T * N;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t t = m * 16 + 4 * g + j;
        if (t < T) dst[t * N + n] = acc[m][j];
      }
  }
}

// Y[t, n] = bf16( sum_p part[p][t][n] + sum_{j<r} V[t, j] B[n, j] ),  V = bf16(s U) with row stride rp
__global__ __launch_bounds__(256) void k_gemv_reduce(const float *__restrict__ part, int nsplit, int64_t T, int64_t N,
                                                     const bf16_t *__restrict__ V, int64_t rp,
                                                     const bf16_t *__restrict__ B, int64_t r,
                                                     bf16_t *__restrict__ Y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * N) return;
  const int64_t t = i / N, n = i - t * N;
  float acc = 0.f;
  for (int p = 0; p < nsplit; ++p) acc += part[(int64_t)p * T * N + i];
  float lora = 0.f;
  for (int64_t j = 0; j < r; ++j) lora += bf16_lo_to_f32(V[t * rp + j]) * bf16_lo_to_f32(B[n * r + j]);
  Y[i] = f32_to_bf16(acc + lora);
}

// Split of K for the small-token forward: aim at ~8 workgroups per CU, each
// K range a multiple of 128 and at least 512 deep, and keep the binary32
// partial sums (written and read once) below ~1/8 of the weight stream.
void nf4_gemv_plan(int64_t T, int64_t N, int64_t K, int *nsplit, int64_t *kchunk) {
  const int64_t tiles = (N + 63) / 64;
  int64_t ns = (2048 + tiles - 1) / tiles;
  const int64_t by_depth = K / 512 > 0 ? K / 512 : 1;
  // partial traffic 8 * ns * T * N bytes vs weight stream ~0.516 * N * K bytes: ns <= K / (128 T)
  const int64_t tt = T > 0 ? T : 1;
  const int64_t by_traffic = K / (128 * tt) > 0 ? K / (128 * tt) : 1;
  if (ns > by_depth) ns = by_depth;
  if (ns > by_traffic) ns = by_traffic;
  if (ns < 1) ns = 1;
  int64_t kc = (K + ns - 1) / ns;
  kc = (kc + 127) / 128 * 128;
  *kchunk = kc;
  *nsplit = (int)((K + kc - 1) / kc);
}

hipError_t launch_nf4_gemv(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                           const float *step, int64_t N, int nsplit, int64_t kchunk, float *part, const Levels &lv,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)nsplit);
  if (T <= 16)
    hipLaunchKernelGGL(k_nf4_gemv<1>, grid, dim3(256), 0, s, X, T, K, codes, absmax_q, step, N, kchunk, part, lv);
  else if (T <= 32)
    hipLaunchKernelGGL(k_nf4_gemv<2>, grid, dim3(256), 0, s, X, T, K, codes, absmax_q, step, N, kchunk, part, lv);
  else
    hipLaunchKernelGGL(k_nf4_gemv<4>, grid, dim3(256), 0, s, X, T, K, codes, absmax_q, step, N, kchunk, part, lv);
  return hipGetLastError();
}

hipError_t launch_gemv_reduce(const float *part, int nsplit, int64_t T, int64_t N, const bf16_t *V, int64_t rp,
                              const bf16_t *B, int64_t r, bf16_t *Y, hipStream_t s) {
  const int64_t total = T * N;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gemv_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, nsplit, T, N, V, rp,
                     B, r, Y);
  return hipGetLastError();
}

}  // namespace qlora
