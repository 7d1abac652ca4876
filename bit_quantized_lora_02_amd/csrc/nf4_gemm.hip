// nf4_gemm.hip -- bf16 MFMA GEMMs with the NF4 decode fused into the B operand.
//
// The method dequantizes each block of the 4-bit weight to bf16 inside the
// matmul and throws the expanded copy away ("What does QLoRA change compared
// with plain LoRA when fine-tuning Llama?", katajob.com, section "NF4: 4-bit
// NormalFloat"; "Module 08 -- QLoRA & Quantization", ainiketan.in, section 3):
//
//   forward   Y  = X . W'^T + V . Bp^T      V = bf16(s . X . A^T), Bp = B (padded)
//   backward  dX = dY . W'  + dUp . A       dUp = bf16(s . dY . B) (padded)
//
// Each workgroup computes a 128x128 output tile with 4 waves (2x2, 64x64 per
// wave, 2x2 tiles of v_mfma_f32_32x32x16_bf16).  The reduction runs in steps
// of 64: the A operand (activations) is copied global -> registers -> LDS, the
// B operand is decoded from nibbles in registers and written to LDS as bf16,
// so the dequantized weight exists only as one 128x64 tile in LDS.  The LoRA
// term is appended as extra reduction steps over the padded rank, so it lands
// in the same binary32 accumulators.  LDS is double buffered: the global loads
// for step s+1 are issued before the MFMAs of step s.
//
// LDS tiles are [row][64] bf16 (128-byte rows) with the 16-byte chunk index
// XOR-swizzled by (row & 7), so the 32 rows a wave reads per MFMA operand fall
// on distinct banks.
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int NT = 256;

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

// Copy a [128 x 64] bf16 tile of a row-major matrix (row stride ld elements)
// into registers: thread t takes rows (t>>3) + 32i, 16-byte chunk (t&7).  Rows
// at or past `rows` and columns at or past `cols` read as zero (cols % 8 == 0).
__device__ __forceinline__ void load_act_tile(const bf16_t *__restrict__ src, int64_t ld, int64_t row0, int64_t rows,
                                              int64_t col0, int64_t cols, int tid, u32x4_t r[4]) {
  const int chunk = tid & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + (tid >> 3) + 32 * i;
    const int64_t col = col0 + chunk * 8;
    if (row < rows && col < cols)
      r[i] = *reinterpret_cast<const u32x4_t *>(src + row * ld + col);
    else
      r[i] = u32x4_t{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_act_tile(bf16_t *s, int tid, const u32x4_t r[4]) {
  const int chunk = tid & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 3) + 32 * i;
    *reinterpret_cast<u32x4_t *>(s + lds_off(row, chunk)) = r[i];
  }
}

// 2x2 wave grid, 64x64 per wave: one 64-deep reduction step out of LDS.
__device__ __forceinline__ void mma_step(const bf16_t *sA, const bf16_t *sB, int wm, int wn, int lane,
                                         f32x16_t acc[2][2]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int chunk = kk * 2 + (lane >> 5);
    u32x4_t a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ra = wm * 64 + i * 32 + (lane & 31);
      a[i] = *reinterpret_cast<const u32x4_t *>(sA + lds_off(ra, chunk));
      const int rb = wn * 64 + i * 32 + (lane & 31);
      b[i] = *reinterpret_cast<const u32x4_t *>(sB + lds_off(rb, chunk));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16(a[i], b[j], acc[i][j]);
  }
}

__device__ __forceinline__ void store_tile_out(bf16_t *__restrict__ out, int64_t ld, int64_t m0, int64_t rows,
                                               int64_t n0, int64_t cols, int wm, int wn, int lane,
                                               const f32x16_t acc[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= cols) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (row < rows) out[row * ld + col] = f32_to_bf16(acc[i][j][e]);
      }
    }
}
}  // namespace

// ---------------------------------------------------------------- forward
// Y[T, N] = X[T, K] . W'[N, K]^T + V[T, rp] . Bp[N, rp]^T
__global__ __launch_bounds__(NT) void k_nf4_gemm_fwd(const bf16_t *__restrict__ X, int64_t T, int64_t K,
                                                     const uint8_t *__restrict__ codes,
                                                     const uint8_t *__restrict__ absmax_q,
                                                     const float *__restrict__ step, int64_t N,
                                                     const bf16_t *__restrict__ V, const bf16_t *__restrict__ Bp,
                                                     int64_t rp, bf16_t *__restrict__ Y, Levels lv) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * BK];
  __shared__ float s_lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  levels_to_lds(lv, s_lv, tid);

  const int nk = (int)(K / BK), nsteps = nk + (int)(rp / BK);
  // B-operand loader: row (tid >> 1) of the tile, 32 consecutive k from (tid & 1) * 32
  const int brow = tid >> 1, bhalf = tid & 1;
  const int64_t wrow = n0 + brow;
  const bool wrow_ok = wrow < N;

  u32x4_t ra[4], rb[4];
  uint32_t rc[4];
  float rcq = 0.f;

  auto load_step = [&](int s) {
    if (s < nk) {
      const int64_t k0 = (int64_t)s * BK;
      load_act_tile(X, K, m0, T, k0, K, tid, ra);
      if (wrow_ok) {
        u32x4_t c = *reinterpret_cast<const u32x4_t *>(codes + wrow * (K / 2) + k0 / 2 + bhalf * 16);
        rc[0] = c.x; rc[1] = c.y; rc[2] = c.z; rc[3] = c.w;
        rcq = block_scale(absmax_q, step, wrow * (K / BK) + s);
      } else {
        rc[0] = rc[1] = rc[2] = rc[3] = 0x77777777u;
        rcq = 0.f;
      }
    } else {
      const int64_t k0 = (int64_t)(s - nk) * BK;
      load_act_tile(V, rp, m0, T, k0, rp, tid, ra);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        rb[c] = wrow_ok ? *reinterpret_cast<const u32x4_t *>(Bp + wrow * rp + k0 + bhalf * 32 + c * 8)
                        : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_step = [&](int s, int buf) {
    store_act_tile(sA[buf], tid, ra);
    if (s < nk) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float v[8];
        decode8(rc[c], rcq, s_lv, v);
        u32x4_t o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        o.z = pack_bf16x2(v[4], v[5]);
        o.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<u32x4_t *>(sB[buf] + lds_off(brow, bhalf * 4 + c)) = o;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4_t *>(sB[buf] + lds_off(brow, bhalf * 4 + c)) = rb[c];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  load_step(0);
  __syncthreads();  // level table visible
  store_step(0, 0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load_step(s + 1);
    mma_step(sA[buf], sB[buf], wm, wn, lane, acc);
    if (s + 1 < nsteps) store_step(s + 1, buf ^ 1);
    __syncthreads();
  }
  store_tile_out(Y, N, m0, T, n0, N, wm, wn, lane, acc);
}

// --------------------------------------------------------------- backward
// dX[T, K] = dY[T, N] . W'[N, K] + dUp[T, rp] . A[r, K]   (rows of A past r read as 0)
// The reduction index is the weight row n, so the B operand is decoded in
// 4-row x 8-column micro-tiles and packed across rows: the transposition to
// [k_out][n] happens in the bf16 pack, at no extra cost.
__global__ __launch_bounds__(NT) void k_nf4_gemm_dx(const bf16_t *__restrict__ dY, int64_t T, int64_t N,
                                                    const uint8_t *__restrict__ codes,
                                                    const uint8_t *__restrict__ absmax_q,
                                                    const float *__restrict__ step, int64_t K,
                                                    const bf16_t *__restrict__ dUp, const bf16_t *__restrict__ A,
                                                    int64_t r, int64_t rp, bf16_t *__restrict__ dX, Levels lv) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * BK];
  __shared__ float s_lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;  // n0 indexes k_out (columns of W)
  levels_to_lds(lv, s_lv, tid);

  const int nk = (int)((N + BK - 1) / BK), nsteps = nk + (int)(rp / BK);
  // B loader: column chunk cc = tid & 15 (8 output columns), row group g = tid >> 4 (4 reduction rows)
  const int cc = tid & 15, g = tid >> 4;
  const int64_t kcol = n0 + cc * 8;
  const bool kcol_ok = kcol < K;

  u32x4_t ra[4];
  uint32_t rw[4];  // one 32-bit word (8 nibbles) per reduction row
  float rcq[4];
  u32x4_t rl[4];   // LoRA phase: 8 bf16 of A per row

  auto load_step = [&](int s) {
    if (s < nk) {
      const int64_t k0 = (int64_t)s * BK;
      load_act_tile(dY, N, m0, T, k0, N, tid, ra);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int64_t n = k0 + g * 4 + p;
        if (n < N && kcol_ok) {
          rw[p] = *reinterpret_cast<const uint32_t *>(codes + n * (K / 2) + kcol / 2);
          rcq[p] = block_scale(absmax_q, step, n * (K / BK) + kcol / BK);
        } else {
          rw[p] = 0x77777777u;
          rcq[p] = 0.f;
        }
      }
    } else {
      const int64_t k0 = (int64_t)(s - nk) * BK;
      load_act_tile(dUp, rp, m0, T, k0, rp, tid, ra);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int64_t j = k0 + g * 4 + p;
        rl[p] = (j < r && kcol_ok) ? *reinterpret_cast<const u32x4_t *>(A + j * K + kcol) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_step = [&](int s, int buf) {
    store_act_tile(sA[buf], tid, ra);
    // destination: LDS row (k_out) = cc*8 + e, reduction columns g*4 .. g*4+3 (8 bytes)
    if (s < nk) {
      float v[4][8];
#pragma unroll
      for (int p = 0; p < 4; ++p) decode8(rw[p], rcq[p], s_lv, v[p]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = cc * 8 + e;
        u32x2_t o;
        o.x = pack_bf16x2(v[0][e], v[1][e]);
        o.y = pack_bf16x2(v[2][e], v[3][e]);
        *reinterpret_cast<u32x2_t *>(sB[buf] + lds_off(row, g >> 1) + (g & 1) * 4) = o;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = cc * 8 + e;
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 of each word
        u32x2_t o;
        o.x = __builtin_amdgcn_perm(rl[1][w], rl[0][w], sel);
        o.y = __builtin_amdgcn_perm(rl[3][w], rl[2][w], sel);
        *reinterpret_cast<u32x2_t *>(sB[buf] + lds_off(row, g >> 1) + (g & 1) * 4) = o;
      }
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  load_step(0);
  __syncthreads();
  store_step(0, 0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load_step(s + 1);
    mma_step(sA[buf], sB[buf], wm, wn, lane, acc);
    if (s + 1 < nsteps) store_step(s + 1, buf ^ 1);
    __syncthreads();
  }
  store_tile_out(dX, K, m0, T, n0, K, wm, wn, lane, acc);
}

hipError_t launch_nf4_gemm_fwd(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                               const float *step, int64_t N, const bf16_t *V, const bf16_t *Bp, int64_t rp, bf16_t *Y,
                               const Levels &lv, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((T + BM - 1) / BM));
  hipLaunchKernelGGL(k_nf4_gemm_fwd, grid, dim3(NT), 0, s, X, T, K, codes, absmax_q, step, N, V, Bp, rp, Y, lv);
  return hipGetLastError();
}

hipError_t launch_nf4_gemm_dx(const bf16_t *dY, int64_t T, int64_t N, const uint8_t *codes, const uint8_t *absmax_q,
                              const float *step, int64_t K, const bf16_t *dUp, const bf16_t *A, int64_t r, int64_t rp,
                              bf16_t *dX, const Levels &lv, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((K + BN - 1) / BN), (unsigned)((T + BM - 1) / BM));
  hipLaunchKernelGGL(k_nf4_gemm_dx, grid, dim3(NT), 0, s, dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv);
  return hipGetLastError();
}

}  // namespace qlora
