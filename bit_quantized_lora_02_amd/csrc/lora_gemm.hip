// lora_gemm.hip -- the skinny rank-r contractions of the LoRA branch.
//
// "QLoRA: fine-tuning a large model on one GPU" (learn.pranaymahendrakar.com),
// Researcher level, "LoRA, stated once": the adapter adds (alpha/r) B A x with
// B of shape d x r and A of shape r x k.  Its gradients (same page, "What
// QLoRA adds"; katajob.com, "What stays in full precision") are
//   U = X A^T,  dU = s dY B,  dA = dU^T X,  dB = s dY^T U.
// Every one of them has one long reduction (over n_in, n_out or the T tokens)
// and a narrow output (r <= 128 on one side), so each is a split-K bf16 MFMA
// GEMM that writes binary32 partial sums; a finalize kernel then adds the
// splits in a fixed order (bitwise repeatable, no atomics), scales, and rounds
// to bf16 once.
//
// C[M, N] = sum_k A(m, k) B(k, n), 64x64 tile, reduction step 32, 4 waves in
// a 2x2 grid, one v_mfma_f32_32x32x16_bf16 tile per wave.  Operand storage:
//   LA = 0: A(m, k) at A[m*lda + k]   (reduction contiguous)
//   LA = 1: A(m, k) at A[k*lda + m]   (output index contiguous: transposed into LDS)
//   LB = 0: B(k, n) at B[n*ldb + k];   LB = 1: B(k, n) at B[k*ldb + n]
// lda and ldb are multiples of 8 and the bases 16-byte aligned.
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {
constexpr int TM = 64, TN = 64, TK = 32;

// LDS tiles are [64 rows][32] bf16, 64-byte rows; 16-byte chunks swizzled so
// that the 8 rows read by 8 consecutive lanes hit distinct banks.
__device__ __forceinline__ int soff(int row, int chunk) { return row * TK + ((chunk ^ ((row >> 1) & 3)) << 3); }

// Stage one operand tile into LDS as [row = output index][k].
template <int L>
__device__ __forceinline__ void stage_tile(const bf16_t *__restrict__ P, int64_t ld, int64_t r0, int64_t R,
                                           int64_t k0, int64_t kend, int tid, bf16_t *s) {
  if (L == 0) {
    // 64 rows x 4 chunks of 8 k: one chunk per thread
    const int row = tid >> 2, ch = tid & 3;
    const int64_t gr = r0 + row, gk = k0 + ch * 8;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (gr < R) {
      if (gk + 8 <= kend) {
        v = *reinterpret_cast<const u32x4_t *>(P + gr * ld + gk);
      } else {
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = (gk + i < kend) ? P[gr * ld + gk + i] : (uint16_t)0;
        v.x = e[0] | ((uint32_t)e[1] << 16);
        v.y = e[2] | ((uint32_t)e[3] << 16);
        v.z = e[4] | ((uint32_t)e[5] << 16);
        v.w = e[6] | ((uint32_t)e[7] << 16);
      }
    }
    *reinterpret_cast<u32x4_t *>(s + soff(row, ch)) = v;
  } else {
    // 32 k x 8 chunks of 8 output indices: one chunk per thread, scattered into [row][k]
    const int kk = tid >> 3, ch = tid & 7;
    const int64_t gk = k0 + kk, gr = r0 + ch * 8;
    uint16_t e[8];
    if (gk < kend && gr + 8 <= R) {
      u32x4_t v = *reinterpret_cast<const u32x4_t *>(P + gk * ld + gr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[2 * i] = (uint16_t)(v[i] & 0xffffu);
        e[2 * i + 1] = (uint16_t)(v[i] >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = (gk < kend && gr + i < R) ? P[gk * ld + gr + i] : (uint16_t)0;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = ch * 8 + i;
      s[soff(row, kk >> 3) + (kk & 7)] = e[i];
    }
  }
}
}  // namespace

template <int LA, int LB>
__global__ __launch_bounds__(256) void k_gemm_splitk(const bf16_t *__restrict__ A, int64_t lda,
                                                     const bf16_t *__restrict__ B, int64_t ldb, int64_t M, int64_t N,
                                                     int64_t Kred, int64_t kchunk, float *__restrict__ C) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[TM * TK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[TN * TK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  const int64_t kb = (int64_t)blockIdx.z * kchunk;
  const int64_t ke = (kb + kchunk < Kred) ? kb + kchunk : Kred;
  f32x16_t acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  for (int64_t k0 = kb; k0 < ke; k0 += TK) {
    stage_tile<LA>(A, lda, m0, M, k0, ke, tid, sA);
    stage_tile<LB>(B, ldb, n0, N, k0, ke, tid, sB);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      const u32x4_t a = *reinterpret_cast<const u32x4_t *>(sA + soff(wm * 32 + (lane & 31), ch));
      const u32x4_t b = *reinterpret_cast<const u32x4_t *>(sB + soff(wn * 32 + (lane & 31), ch));
      acc = mfma_32x32x16(a, b, acc);
    }
    __syncthreads();
  }
  float *Cs = C + (int64_t)blockIdx.z * M * N;
  const int64_t col = n0 + wn * 32 + (lane & 31);
  if (col < N) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = m0 + wm * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
      if (row < M) Cs[row * N + col] = acc[e];
    }
  }
}

// out1[m*ld1 + n] = bf16(scale1 * S) for n < n1;
// out2[m*ld2 + n] = n < nvalid2 ? bf16(scale2 * S) : 0 for n < n2;
// S = sum over splits p = 0 .. nsplit-1 (in that order) of part[p][m][n] (ld = N).
__global__ __launch_bounds__(256) void k_finalize(const float *__restrict__ part, int nsplit, int64_t M, int64_t N,
                                                  bf16_t *__restrict__ out1, int64_t ld1, int64_t n1, float scale1,
                                                  bf16_t *__restrict__ out2, int64_t ld2, int64_t n2, int64_t nvalid2,
                                                  float scale2) {
  const int64_t ncol = (n1 > n2) ? n1 : n2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * ncol) return;
  const int64_t m = i / ncol, n = i - m * ncol;
  float sum = 0.f;
  if (n < N)
    for (int p = 0; p < nsplit; ++p) sum += part[((int64_t)p * M + m) * N + n];
  if (out1 && n < n1) out1[m * ld1 + n] = f32_to_bf16(scale1 * sum);
  if (out2 && n < n2) out2[m * ld2 + n] = (n < nvalid2) ? f32_to_bf16(scale2 * sum) : (bf16_t)0;
}

// out[m*ldo + n] = n < ncols ? in[m*ldi + n] : 0, for n < ldo (zero-padded copy).
__global__ __launch_bounds__(256) void k_pad_copy(const bf16_t *__restrict__ in, int64_t ldi, int64_t ncols, int64_t M,
                                                  bf16_t *__restrict__ out, int64_t ldo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * ldo) return;
  const int64_t m = i / ldo, n = i - m * ldo;
  out[i] = (n < ncols) ? in[m * ldi + n] : (bf16_t)0;
}

hipError_t launch_gemm_splitk(int la, int lb, const bf16_t *A, int64_t lda, const bf16_t *B, int64_t ldb, int64_t M,
                              int64_t N, int64_t Kred, int64_t kchunk, int nsplit, float *C, hipStream_t s) {
  if (M == 0 || N == 0 || nsplit == 0) return hipSuccess;
  dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM), (unsigned)nsplit);
  if (la == 0 && lb == 0)
    hipLaunchKernelGGL((k_gemm_splitk<0, 0>), grid, dim3(256), 0, s, A, lda, B, ldb, M, N, Kred, kchunk, C);
  else if (la == 0 && lb == 1)
    hipLaunchKernelGGL((k_gemm_splitk<0, 1>), grid, dim3(256), 0, s, A, lda, B, ldb, M, N, Kred, kchunk, C);
  else if (la == 1 && lb == 0)
    hipLaunchKernelGGL((k_gemm_splitk<1, 0>), grid, dim3(256), 0, s, A, lda, B, ldb, M, N, Kred, kchunk, C);
  else
    hipLaunchKernelGGL((k_gemm_splitk<1, 1>), grid, dim3(256), 0, s, A, lda, B, ldb, M, N, Kred, kchunk, C);
  return hipGetLastError();
}

hipError_t launch_finalize(const float *part, int nsplit, int64_t M, int64_t N, bf16_t *out1, int64_t ld1, int64_t n1,
                           float scale1, bf16_t *out2, int64_t ld2, int64_t n2, int64_t nvalid2, float scale2,
                           hipStream_t s) {
  const int64_t ncol = (n1 > n2) ? n1 : n2;
  const int64_t total = M * ncol;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_finalize, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, nsplit, M, N, out1, ld1,
                     n1, scale1, out2, ld2, n2, nvalid2, scale2);
  return hipGetLastError();
}

hipError_t launch_pad_copy(const bf16_t *in, int64_t ldi, int64_t ncols, int64_t M, bf16_t *out, int64_t ldo,
                           hipStream_t s) {
  const int64_t total = M * ldo;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pad_copy, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, in, ldi, ncols, M, out, ldo);
  return hipGetLastError();
}

}  // namespace qlora
