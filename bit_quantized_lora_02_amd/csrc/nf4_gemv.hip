// nf4_gemv.hip -- the forward for few tokens (T <= 64), where the layer is bound
// by streaming the 4-bit weight from HBM, not by arithmetic.
//
// Same computation as the tiled forward ("What does QLoRA change compared with
// plain LoRA when fine-tuning Llama?", katajob.com, "NF4: 4-bit NormalFloat":
// blocks expanded to bf16 inside the matmul; "QLoRA: fine-tuning a large model
// on one GPU", learn.pranaymahendrakar.com, "LoRA, stated once": the adapter
// adds (alpha/r) B A x), organised for bandwidth in three launches:
//
// 1. k_lora_u_small: U = X A^T for all T rows (one workgroup per 16 tokens x
//    16 ranks, the four waves split n_in and reduce through LDS); writes U and
//    V = bf16(s U).
// 2. k_nf4_gemv: a workgroup (4 waves) owns 64 weight rows and one K range;
//    each wave owns 16 rows and issues v_mfma_f32_16x16x32_bf16 with the tokens
//    as the M dimension.  Each lane streams 16 bytes of codes (32 consecutive
//    weights of one row, one block constant) per 128-deep step and decodes them
//    straight into its four B operands, so the weight never touches LDS.  The
//    decode looks up both levels of a code byte at once in a 256-entry LDS table
//    of level pairs (two copies, one per half-wave, to spread bank traffic):
//    per byte one shift, one and-or (table offset), one 8-byte LDS read, two
//    binary32 multiplies by the block constant and one bf16 pack.
//    Codes are prefetched three steps ahead.  Each K range writes binary32
//    partial sums; the first also carries the LoRA term V B^T.  (A single
//    launch with a last-arriving-workgroup reduction needs device-scope
//    fences, which on this chip write back and invalidate the L2 in every
//    workgroup and cost far more than a third launch.)
// 3. k_gemv_reduce: Y = bf16(sum of the partials in split order), so the
//    result does not depend on the order in which workgroups finish.
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Two copies of the level-pair table: entry b = (level[b & 15], level[b >> 4]).
constexpr uint32_t kPairTableBytes = 256 * 8;

__device__ __forceinline__ void pair_table_to_lds(const Levels &lv, float2 *tab, int tid) {
  // 256 threads: thread t writes entry t of both copies
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    lo = ((tid & 15) == i) ? lv.v[i] : lo;
    hi = ((tid >> 4) == i) ? lv.v[i] : hi;
  }
  tab[tid] = make_float2(lo, hi);
  tab[256 + tid] = make_float2(lo, hi);
}

// 8 codes of one 32-bit word -> 4 packed bf16 pairs of fl32(level * cq).
// `copy` is the byte offset of this lane's table copy.
__device__ __forceinline__ u32x4_t decode8_pairs(uint32_t w, float cq, const char *tab, uint32_t copy) {
  u32x4_t o;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t sh = (b == 0) ? (w << 3) : (w >> (8 * b - 3));
    const float2 l = *reinterpret_cast<const float2 *>(tab + ((sh & 0x7f8u) | copy));
    o[b] = pack_bf16x2(__fmul_rn(l.x, cq), __fmul_rn(l.y, cq));
  }
  return o;
}
}  // namespace

// ------------------------------------------------------------- U for few tokens
// U[t, j] = sum_k X[t, k] A[j, k]; U_out (nullable, [T, r]) and V = bf16(s U) ([T, rp], zero past r).
// Workgroup (bx, by) covers tokens 16 bx .. +15 and ranks 16 by .. +15; wave w
// takes the k range [w K/4, (w+1) K/4) in 32-deep MFMA steps.
__global__ __launch_bounds__(256) void k_lora_u_small(const bf16_t *__restrict__ X, int64_t T, int64_t K,
                                                      const bf16_t *__restrict__ A, int64_t r, float s,
                                                      bf16_t *__restrict__ U_out, bf16_t *__restrict__ V, int64_t rp) {
  __shared__ f32x4_t red[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * 16, j0 = (int64_t)blockIdx.y * 16;
  int64_t t = t0 + (lane & 15);
  t = t < T ? t : T - 1;  // rows past T feed outputs that are not stored
  const int64_t j = j0 + (lane & 15);
  const bool jok = j < r;
  const int64_t kq = K / 4, kb = wave * kq;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k = kb + 8 * (lane >> 4); k < kb + kq; k += 32) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(X + t * K + k);
    const u32x4_t b = jok ? *reinterpret_cast<const u32x4_t *>(A + j * K + k) : u32x4_t{0u, 0u, 0u, 0u};
    acc = mfma_16x16x32(a, b, acc);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const f32x4_t sum = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
    // element i of lane l: token 16 bx + 4 (l >> 4) + i, rank 16 by + (l & 15)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tt = t0 + 4 * (lane >> 4) + i;
      if (tt >= T) continue;
      if (jok) {
        if (U_out) U_out[tt * r + j] = f32_to_bf16(sum[i]);
        V[tt * rp + j] = f32_to_bf16(s * sum[i]);
      } else if (j < rp) {
        V[tt * rp + j] = (bf16_t)0;
      }
    }
  }
}

// ------------------------------------------------------------------ the GEMV
template <int MT>
__global__ __launch_bounds__(256) void k_nf4_gemv(const bf16_t *__restrict__ X, int64_t T, int64_t K,
                                                  const uint8_t *__restrict__ codes,
                                                  const uint8_t *__restrict__ absmax_q,
                                                  const float *__restrict__ step, int64_t N, int64_t kchunk,
                                                  const bf16_t *__restrict__ V, int64_t rp,
                                                  const bf16_t *__restrict__ B, int64_t r, float *__restrict__ part,
                                                  bf16_t *__restrict__ Y, Levels lv) {
  __shared__ __attribute__((aligned(16))) float2 s_tab[512];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  pair_table_to_lds(lv, s_tab, tid);
  __syncthreads();
  const char *tab = reinterpret_cast<const char *>(s_tab);
  const uint32_t copy = (lane >> 5) ? kPairTableBytes : 0u;
  const int g = lane >> 4;  // 32-wide slice of each 128-deep step
  const int64_t n = (int64_t)blockIdx.x * 64 + wave * 16 + (lane & 15);
  const bool nok = n < N;
  const int64_t kb = (int64_t)blockIdx.y * kchunk;
  const int64_t ke = (kb + kchunk < K) ? kb + kchunk : K;
  const int nsteps = (int)((ke - kb) / 128);
  const uint8_t *cptr = codes + (nok ? n : 0) * (K / 2) + (kb + 32 * g) / 2;
  const int64_t bidx = (nok ? n : 0) * (K / 64) + (kb + 32 * g) / 64;

  auto load_codes = [&](int s, u32x4_t &c, RawScale &cq) {
    if (nok && s < nsteps) {
      c = *reinterpret_cast<const u32x4_t *>(cptr + (int64_t)s * 64);
      cq = load_scale(absmax_q, step, bidx + 2 * s);
    } else {
      c = u32x4_t{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
      cq = RawScale{0u, 0.f};
    }
  };
  const bf16_t *xrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    int64_t t = m * 16 + (lane & 15);
    t = t < T ? t : T - 1;  // rows past T read row T-1 and feed outputs that are never stored
    xrow[m] = X + t * K + kb + 32 * g;
  }

  f32x4_t acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // three fixed prefetch slots, unrolled so that no register holding a load in
  // flight is ever copied (a copy would make the wave wait for that load)
  u32x4_t c0, c1, c2;
  RawScale q0, q1, q2;
  load_codes(0, c0, q0);
  load_codes(1, c1, q1);
  load_codes(2, c2, q2);
  auto do_step = [&](int s, u32x4_t &c, RawScale &cq_raw) {
    u32x4_t a[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) a[m][q] = *reinterpret_cast<const u32x4_t *>(xrow[m] + (int64_t)s * 128 + 8 * q);
    const float cq = scale_of(cq_raw);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4_t b = decode8_pairs(c[q], cq, tab, copy);
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = mfma_16x16x32(a[m][q], b, acc[m]);
    }
    load_codes(s + 3, c, cq_raw);  // refill this slot three steps ahead
  };
  for (int s = 0; s < nsteps; s += 3) {
    do_step(s, c0, q0);
    if (s + 1 < nsteps) do_step(s + 1, c1, q1);
    if (s + 2 < nsteps) do_step(s + 2, c2, q2);
  }

  // the first K range also carries the LoRA term V[T, rp] . B[n, :r]^T
  if (blockIdx.y == 0) {
    for (int64_t j = 8 * g; j < rp; j += 32) {
      u32x4_t a[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        int64_t t = m * 16 + (lane & 15);
        t = t < T ? t : T - 1;
        a[m] = *reinterpret_cast<const u32x4_t *>(V + t * rp + j);
      }
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (nok && j + e < r) ? (uint32_t)B[n * r + j + e] : 0u;
      const u32x4_t b = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = mfma_16x16x32(a[m], b, acc[m]);
    }
  }

  // accumulator element i of lane l holds token 16 m + 4 (l >> 4) + i, row n
  const int nsplit = (int)gridDim.y;
  if (nsplit == 1) {
    if (nok)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t t = m * 16 + 4 * g + i;
          if (t < T) Y[t * N + n] = f32_to_bf16(acc[m][i]);
        }
    return;
  }
  if (nok) {
    float *dst = part + (int64_t)blockIdx.y * T * N;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = m * 16 + 4 * g + i;
        if (t < T) dst[t * N + n] = acc[m][i];
      }
  }
}

// Y[i] = bf16(sum over p = 0 .. nsplit-1, in that order, of part[p][i]), i over T * N
__global__ __launch_bounds__(256) void k_gemv_reduce(const float *__restrict__ part, int nsplit, int64_t total,
                                                     bf16_t *__restrict__ Y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  float sum = 0.f;
  for (int p = 0; p < nsplit; ++p) sum += part[(int64_t)p * total + i];
  Y[i] = f32_to_bf16(sum);
}

// Split of K for the small-token forward: aim at ~8 workgroups per CU, each
// K range a multiple of 128 and at least 512 deep, and keep the binary32
// partial sums (written and read once) below ~1/8 of the weight stream:
// 8 ns T N bytes <= 0.516 N K / 8  <=>  ns <= K / (128 T).
void nf4_gemv_plan(int64_t T, int64_t N, int64_t K, int *nsplit, int64_t *kchunk) {
  const int64_t tiles = (N + 63) / 64;
  int64_t ns = (2048 + tiles - 1) / tiles;
  const int64_t by_depth = K / 512 > 0 ? K / 512 : 1;
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

hipError_t launch_lora_u_small(const bf16_t *X, int64_t T, int64_t K, const bf16_t *A, int64_t r, float s,
                               bf16_t *U_out, bf16_t *V, int64_t rp, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((T + 15) / 16), (unsigned)((rp + 15) / 16));
  launch(k_lora_u_small, grid, dim3(256), 0, st, X, T, K, A, r, s, U_out, V, rp);
  return hipGetLastError();
}

hipError_t launch_nf4_gemv(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                           const float *step, int64_t N, int nsplit, int64_t kchunk, const bf16_t *V, int64_t rp,
                           const bf16_t *B, int64_t r, float *part, bf16_t *Y, const Levels &lv, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)nsplit);
  if (T <= 16)
    launch(k_nf4_gemv<1>, grid, dim3(256), 0, s, X, T, K, codes, absmax_q, step, N, kchunk, V, rp, B, r,
                       part, Y, lv);
  else if (T <= 32)
    launch(k_nf4_gemv<2>, grid, dim3(256), 0, s, X, T, K, codes, absmax_q, step, N, kchunk, V, rp, B, r,
                       part, Y, lv);
  else
    launch(k_nf4_gemv<4>, grid, dim3(256), 0, s, X, T, K, codes, absmax_q, step, N, kchunk, V, rp, B, r,
                       part, Y, lv);
  return hipGetLastError();
}

hipError_t launch_gemv_reduce(const float *part, int nsplit, int64_t T, int64_t N, bf16_t *Y, hipStream_t s) {
  const int64_t total = T * N;
  if (total == 0 || nsplit <= 1) return hipSuccess;
  launch(k_gemv_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, nsplit, total, Y);
  return hipGetLastError();
}

}  // namespace qlora
