// merge.hip -- fold a trained adapter into a 16-bit base for export.
//
// "Module 08 - QLoRA & Quantization" (ainiketan.in), "7. A subtle but important
// deployment note", and katajob.com, "What it costs" (3. Merging): for serving,
// the adapter is merged into a 16-bit base -- the reloaded original, or the
// dequantized NF4 base the adapter was trained against -- and the merged model
// may then be quantized again (here: binary32 output fed to the NF4 quantizer).
//   Wm = W + s B A,   W [N, K], B [N, r], A [r, K],  s = fl32(alpha / r)
// Arithmetic: P = B A in binary32 (exact bf16 products, binary32 MFMA sums),
// v = fl32(s P), m = fl32(w + v) with w the bf16 base value (the base decoded
// as bf16_rne(fl32(level * c')) when it is NF4); outputs bf16_rne(m) and/or m.
//
// gfx950 mapping: HBM-bound (0.52 B read per weight from NF4 or 2 B from bf16,
// 2 or 4 B written).  A workgroup owns a 64 x 128 output tile; B [64, r] and
// A [r, 128] go to LDS, four waves form P with 32x32x16 bf16 MFMAs (the rank is
// the reduction, rounded up to 16), park it in LDS, and then every thread
// combines 8 consecutive outputs of one row with their decoded base values and
// stores them with 16-byte writes.
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {
constexpr int MT = 64;          // output rows (n) per workgroup
constexpr int KT = 128;         // output columns (k) per workgroup
constexpr int LDA = KT + 32;    // row pitch (elements) of the A tile: transposing reads cover all 64 banks
constexpr int LDST = KT + 4;    // row pitch (floats) of the staged product

// 8 consecutive rank values of rows row0..row0+7 at one column, transposed: in
// each 16-lane group, lane i gets element (i & 3) of the 8 bytes addressed by
// lane 4m + (i >> 2) (ds_read_b64_tr_b16).
__device__ __forceinline__ u32x4_t read_tr8(const bf16_t *s, int ld, int row0, int col) {
  typedef short s4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4_t lds_s4;
  const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(s + row0 * ld + col));
  const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(s + (row0 + 4) * ld + col));
  const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{l2.x, l2.y, h2.x, h2.y};
}
}  // namespace

template <int RP>
__global__ __launch_bounds__(256) void k_merge(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ absmax_q,
                                               const float *__restrict__ step, const bf16_t *__restrict__ W_base,
                                               int64_t N, int64_t K, const bf16_t *__restrict__ A,
                                               const bf16_t *__restrict__ B, int r, float s, bf16_t *__restrict__ out,
                                               float *__restrict__ out_f32, Levels lv) {
  constexpr int LDB = RP + 8;  // row pitch of the B tile (16-byte aligned rows)
  constexpr int OPS = (RP * LDA + MT * LDB) * 2;
  constexpr int STAGE = MT * LDST * 4;
  __shared__ __attribute__((aligned(16))) char smem[OPS > STAGE ? OPS : STAGE];
  __shared__ float s_lv[16];
  bf16_t *sA = reinterpret_cast<bf16_t *>(smem);  // [RP][LDA]: A rows j, tile columns
  bf16_t *sB = sA + RP * LDA;                     // [MT][LDB]: tile rows n, ranks j
  float *st = reinterpret_cast<float *>(smem);    // [MT][LDST]: s-less product, after the MFMAs
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tiles_k = (K + KT - 1) / KT;  // one-dimensional grid, column tiles fastest
  const int64_t k0 = ((int64_t)blockIdx.x % tiles_k) * KT, n0 = ((int64_t)blockIdx.x / tiles_k) * MT;
  levels_to_lds(lv, s_lv, tid);

  // A tile: 16-byte chunks (K is a multiple of 64, so a chunk is all in or all out)
  for (int c = tid; c < RP * KT / 8; c += 256) {
    const int j = c / (KT / 8), col = (c % (KT / 8)) * 8;
    const bool ok = j < r && k0 + col < K;
    *reinterpret_cast<u32x4_t *>(sA + j * LDA + col) =
        ok ? *reinterpret_cast<const u32x4_t *>(A + (int64_t)j * K + k0 + col) : u32x4_t{0u, 0u, 0u, 0u};
  }
  // B tile: rows of r elements have no alignment to rely on, so element by element
  for (int c = tid; c < MT * RP; c += 256) {
    const int n = c / RP, j = c % RP;
    sB[n * LDB + j] = (j < r && n0 + n < N) ? B[(n0 + n) * r + j] : (bf16_t)0;
  }
  __syncthreads();

  // P tile: wave w owns rows 32 (w / 2) .., columns 64 (w % 2) .. (two 32x32 MFMA tiles)
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 64;
  f32x16_t acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  const int grp = lane >> 4, ai = lane & 15;
#pragma unroll
  for (int kk = 0; kk < RP / 16; ++kk) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(sB + (wr + (lane & 31)) * LDB + kk * 16 + 8 * (lane >> 5));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4_t b = read_tr8(sA, LDA, kk * 16 + 8 * (grp >> 1) + (ai >> 2), wc + t * 32 + 16 * (grp & 1) + 4 * (ai & 3));
      acc[t] = mfma_32x32x16(a, b, acc[t]);
    }
  }
  __syncthreads();  // operands no longer needed: the product takes their place
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      st[(wr + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3)) * LDST + wc + t * 32 + (lane & 31)] = acc[t][e];
  __syncthreads();

  // combine: 8 consecutive outputs of one row per thread and chunk
#pragma unroll
  for (int i = 0; i < MT * KT / 8 / 256; ++i) {
    const int c = tid + 256 * i;
    const int row = c / (KT / 8), col = (c % (KT / 8)) * 8;
    const int64_t n = n0 + row, k = k0 + col;
    if (n >= N || k >= K) continue;
    const int64_t e0 = n * K + k;
    float w[8];
    if (W_base) {
      const u32x4_t b = *reinterpret_cast<const u32x4_t *>(W_base + e0);
#pragma unroll
      for (int q = 0; q < 4; ++q) w[2 * q] = bf16_lo_to_f32(b[q]), w[2 * q + 1] = bf16_hi_to_f32(b[q]);
    } else {  // decoded NF4 base: bf16(level * c') as in every kernel of this library
      const uint32_t cw = *reinterpret_cast<const uint32_t *>(codes + e0 / 2);
      const float cq = block_scale(absmax_q, step, e0 / 64);
      float d[8];
      decode8(cw, cq, s_lv, d);
#pragma unroll
      for (int q = 0; q < 8; ++q) w[q] = __builtin_bit_cast(float, (uint32_t)f32_to_bf16(d[q]) << 16);
    }
    const float4 p0 = *reinterpret_cast<const float4 *>(st + row * LDST + col);
    const float4 p1 = *reinterpret_cast<const float4 *>(st + row * LDST + col + 4);
    const float p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float m[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) m[q] = __fadd_rn(w[q], __fmul_rn(s, p[q]));
    if (out)
      *reinterpret_cast<u32x4_t *>(out + e0) =
          u32x4_t{pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]), pack_bf16x2(m[4], m[5]), pack_bf16x2(m[6], m[7])};
    if (out_f32) {
      *reinterpret_cast<float4 *>(out_f32 + e0) = make_float4(m[0], m[1], m[2], m[3]);
      *reinterpret_cast<float4 *>(out_f32 + e0 + 4) = make_float4(m[4], m[5], m[6], m[7]);
    }
  }
}

hipError_t launch_merge(const uint8_t *codes, const uint8_t *absmax_q, const float *step, const bf16_t *W_base,
                        int64_t N, int64_t K, const bf16_t *A, const bf16_t *B, int r, float s, bf16_t *out,
                        float *out_f32, const Levels &lv, hipStream_t st) {
  if (N == 0 || K == 0) return hipSuccess;
  const dim3 grid((unsigned)(((K + KT - 1) / KT) * ((N + MT - 1) / MT)));
  if (r <= 16)
    launch(k_merge<16>, grid, dim3(256), 0, st, codes, absmax_q, step, W_base, N, K, A, B, r, s, out, out_f32, lv);
  else if (r <= 32)
    launch(k_merge<32>, grid, dim3(256), 0, st, codes, absmax_q, step, W_base, N, K, A, B, r, s, out, out_f32, lv);
  else if (r <= 64)
    launch(k_merge<64>, grid, dim3(256), 0, st, codes, absmax_q, step, W_base, N, K, A, B, r, s, out, out_f32, lv);
  else
    launch(k_merge<128>, grid, dim3(256), 0, st, codes, absmax_q, step, W_base, N, K, A, B, r, s, out, out_f32, lv);
  return hipGetLastError();
}

}  // namespace qlora
