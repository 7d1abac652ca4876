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
// A workgroup of WAVES_M x WAVES_N waves computes a BM x BN output tile; each
// wave owns WM x WN tiles of v_mfma_f32_32x32x16_bf16 (32x32 outputs each).
// The reduction runs in steps of 64 (one NF4 block per weight row): the A
// operand (activations) goes global -> registers -> LDS; the B operand is
// decoded from nibbles in registers and written to LDS as bf16, so the
// dequantized weight exists only as one BN x 64 tile in LDS.  LDS is double
// buffered and the global loads of step s+1 are issued before the MFMAs of
// step s, so one barrier per step separates the two.  The LoRA term follows as
// a few unpipelined extra reduction steps over the padded rank, landing in the
// same binary32 accumulators.
//
// LDS tiles are [row][64] bf16 (128-byte rows) with the 16-byte chunk index
// XOR-swizzled by (row & 7), so the 8 rows that 8 consecutive lanes read fall
// on distinct banks.
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int BK = 64;

template <int WAVES_M_, int WAVES_N_, int WM_, int WN_>
struct TileCfg {
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, WM = WM_, WN = WN_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int BM = WAVES_M * WM * 32;
  static constexpr int BN = WAVES_N * WN * 32;
  static constexpr int A_CH = BM * 8 / NT;   // 16-byte chunks of the A tile per thread and step
  // 16-byte chunks of codes (32 nibbles) per thread; with fewer chunks than
  // threads (C_SPARSE) only the first 2*BN threads load and decode
  static constexpr bool C_SPARSE = BN * 2 < NT;
  static constexpr int C_CH = C_SPARSE ? 1 : BN * 2 / NT;
  static constexpr int L_CH = BN * 8 / NT;   // 16-byte bf16 chunks of the LoRA B tile per thread (forward)
  static_assert(A_CH >= 1 && C_CH >= 1 && L_CH >= 1, "unsupported tile");
};

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

// Output tile of this workgroup.  Workgroups are dispatched round-robin over
// the 8 XCDs (linear id i runs on XCD i % 8), each with its own L2.  With
// xb_m, xb_n > 0 the tile grid (tiles_m x tiles_n) is cut into 8 blocks of
// xb_m x xb_n tiles and XCD j computes block j, so the activation rows and
// weight columns one XCD reads are shared by all its workgroups.  With 0 the
// tiles are taken in row-major order.
struct TileCoord {
  int64_t m, n;
};
__device__ __forceinline__ TileCoord tile_of(int64_t tiles_n, int xb_m, int xb_n) {
  const int64_t lin = blockIdx.x;
  if (xb_m <= 0) return TileCoord{lin / tiles_n, lin % tiles_n};
  const int64_t xcd = lin & 7, local = lin >> 3;
  const int64_t blocks_n = tiles_n / xb_n;
  const int64_t bm = xcd / blocks_n, bn = xcd % blocks_n;
  return TileCoord{bm * xb_m + local / xb_n, bn * xb_n + local % xb_n};
}

template <class C>
__device__ __forceinline__ void zero_acc(f32x16_t acc[C::WM][C::WN]) {
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// Rows [row0, row0+BM) x columns [col0, col0+64) of a row-major bf16 matrix
// into registers: chunk c = tid + NT*i covers row c>>3, 16-byte chunk c&7.
// Rows >= rows or columns >= cols read as zero (cols % 8 == 0).
template <class C>
__device__ __forceinline__ void load_a(const bf16_t *__restrict__ src, int64_t ld, int64_t row0, int64_t rows,
                                       int64_t col0, int64_t cols, int tid, u32x4_t r[C::A_CH]) {
#pragma unroll
  for (int i = 0; i < C::A_CH; ++i) {
    const int c = tid + C::NT * i;
    const int64_t row = row0 + (c >> 3), col = col0 + (c & 7) * 8;
    r[i] = (row < rows && col < cols) ? *reinterpret_cast<const u32x4_t *>(src + row * ld + col)
                                      : u32x4_t{0u, 0u, 0u, 0u};
  }
}

template <class C>
__device__ __forceinline__ void store_a(bf16_t *s, int tid, const u32x4_t r[C::A_CH]) {
#pragma unroll
  for (int i = 0; i < C::A_CH; ++i) {
    const int c = tid + C::NT * i;
    *reinterpret_cast<u32x4_t *>(s + lds_off(c >> 3, c & 7)) = r[i];
  }
}

// One 64-deep reduction step out of LDS for this wave's WM x WN MFMA tiles.
template <class C>
__device__ __forceinline__ void mma_step(const bf16_t *sA, const bf16_t *sB, int wm, int wn, int lane,
                                         f32x16_t acc[C::WM][C::WN]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int chunk = kk * 2 + (lane >> 5);
    u32x4_t a[C::WM], b[C::WN];
#pragma unroll
    for (int i = 0; i < C::WM; ++i) {
      const int ra = (wm * C::WM + i) * 32 + (lane & 31);
      a[i] = *reinterpret_cast<const u32x4_t *>(sA + lds_off(ra, chunk));
    }
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      const int rb = (wn * C::WN + j) * 32 + (lane & 31);
      b[j] = *reinterpret_cast<const u32x4_t *>(sB + lds_off(rb, chunk));
    }
#pragma unroll
    for (int i = 0; i < C::WM; ++i)
#pragma unroll
      for (int j = 0; j < C::WN; ++j) acc[i][j] = mfma_32x32x16(a[i], b[j], acc[i][j]);
  }
}

template <class C>
__device__ __forceinline__ void store_out(bf16_t *__restrict__ out, int64_t ld, int64_t m0, int64_t rows, int64_t n0,
                                          int64_t cols, int wm, int wn, int lane, const f32x16_t acc[C::WM][C::WN]) {
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      const int64_t col = n0 + (wn * C::WN + j) * 32 + (lane & 31);
      if (col >= cols) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + (wm * C::WM + i) * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (row < rows) out[row * ld + col] = f32_to_bf16(acc[i][j][e]);
      }
    }
}

}  // namespace

// ---------------------------------------------------------------- forward
// Y[T, N] = X[T, K] . W'[N, K]^T + V[T, rp] . B[N, :r]^T   (B row stride ldb, columns >= r read as 0)
template <class C>
__global__ __launch_bounds__(C::NT) void k_nf4_gemm_fwd(const bf16_t *__restrict__ X, int64_t T, int64_t K,
                                                        const uint8_t *__restrict__ codes,
                                                        const uint8_t *__restrict__ absmax_q,
                                                        const float *__restrict__ step, int64_t N,
                                                        const bf16_t *__restrict__ V, const bf16_t *__restrict__ Bp,
                                                        int64_t ldb, int64_t r, int64_t rp, bf16_t *__restrict__ Y,
                                                        Levels lv, int xb_m, int xb_n) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][C::BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][C::BN * BK];
  __shared__ float s_lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const TileCoord tc = tile_of((N + C::BN - 1) / C::BN, xb_m, xb_n);
  const int64_t m0 = tc.m * C::BM, n0 = tc.n * C::BN;
  levels_to_lds(lv, s_lv, tid);

  const int nk = (int)(K / BK);
  u32x4_t ra[C::A_CH];
  u32x4_t rc[C::C_CH];
  RawScale rcq[C::C_CH];

  auto load_main = [&](int s) {
    const int64_t k0 = (int64_t)s * BK;
    load_a<C>(X, K, m0, T, k0, K, tid, ra);
#pragma unroll
    for (int i = 0; i < C::C_CH; ++i) {
      const int c = tid + C::NT * i;
      const int64_t wrow = n0 + (c >> 1);
      if (wrow < N && (!C::C_SPARSE || c < 2 * C::BN)) {
        rc[i] = *reinterpret_cast<const u32x4_t *>(codes + wrow * (K / 2) + k0 / 2 + (c & 1) * 16);
        rcq[i] = load_scale(absmax_q, step, wrow * (K / BK) + s);
      } else {
        rc[i] = u32x4_t{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
        rcq[i] = RawScale{0u, 0.f};
      }
    }
  };
  auto store_main = [&](int buf) {
    store_a<C>(sA[buf], tid, ra);
#pragma unroll
    for (int i = 0; i < C::C_CH; ++i) {
      const int c = tid + C::NT * i;
      if (C::C_SPARSE && c >= 2 * C::BN) break;
      const int row = c >> 1, half = c & 1;
      const float cq = scale_of(rcq[i]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float v[8];
        decode8(rc[i][w], cq, s_lv, v);
        u32x4_t o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        o.z = pack_bf16x2(v[4], v[5]);
        o.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<u32x4_t *>(sB[buf] + lds_off(row, half * 4 + w)) = o;
      }
    }
  };

  f32x16_t acc[C::WM][C::WN];
  zero_acc<C>(acc);

  load_main(0);
  __syncthreads();  // level table visible
  store_main(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) load_main(s + 1);
    mma_step<C>(sA[buf], sB[buf], wm, wn, lane, acc);
    if (s + 1 < nk) store_main(buf ^ 1);
    __syncthreads();
  }
  // LoRA up-projection: V [T, rp] . Bp [N, rp]^T, one 64-deep step at a time
  for (int64_t k0 = 0; k0 < rp; k0 += BK) {
    {
      u32x4_t rv[C::A_CH], rb[C::L_CH];
      load_a<C>(V, rp, m0, T, k0, rp, tid, rv);
#pragma unroll
      for (int i = 0; i < C::L_CH; ++i) {
        const int c = tid + C::NT * i;
        const int64_t wrow = n0 + (c >> 3), col = k0 + (c & 7) * 8;  // r % 8 == 0 or B padded to ldb
        rb[i] = (wrow < N && col < r) ? *reinterpret_cast<const u32x4_t *>(Bp + wrow * ldb + col)
                                      : u32x4_t{0u, 0u, 0u, 0u};
      }
      store_a<C>(sA[0], tid, rv);
#pragma unroll
      for (int i = 0; i < C::L_CH; ++i) {
        const int c = tid + C::NT * i;
        *reinterpret_cast<u32x4_t *>(sB[0] + lds_off(c >> 3, c & 7)) = rb[i];
      }
    }
    __syncthreads();
    mma_step<C>(sA[0], sB[0], wm, wn, lane, acc);
    __syncthreads();
  }
  store_out<C>(Y, N, m0, T, n0, N, wm, wn, lane, acc);
}

// --------------------------------------------------------------- backward
// dX[T, K] = dY[T, N] . W'[N, K] + dUp[T, rp] . A[r, K]   (rows of A past r read as 0)
// The reduction index is the weight row n.  The B operand is decoded exactly as
// in the forward (16 bytes of codes = 32 consecutive columns of one weight
// row, one block constant) and stored in its natural [n][k_out] layout, rows
// padded by 32 bytes so that four consecutive rows start 32 bytes apart in
// the bank space.  The MFMA operand, which needs 8 consecutive n for one
// k_out, is read with ds_read_b64_tr_b16: in each 16-lane group, lane i gets
// element (i & 3) of the 8 bytes addressed by lane 4m + (i >> 2), m = 0..3, so
// lane a points at row base + (a >> 2), columns 4 (a & 3) .. +3, and two such
// reads (rows +0..3 and +4..7) give the 8 reduction values of the operand.
template <class C>
__global__ __launch_bounds__(C::NT) void k_nf4_gemm_dx(const bf16_t *__restrict__ dY, int64_t T, int64_t N,
                                                       const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ absmax_q,
                                                       const float *__restrict__ step, int64_t K,
                                                       const bf16_t *__restrict__ dUp, const bf16_t *__restrict__ A,
                                                       int64_t r, int64_t rp, bf16_t *__restrict__ dX, Levels lv,
                                                       int xb_m, int xb_n) {
  constexpr int LDB = C::BN + 16;  // padded row length (elements) of the [64][BN] B tile
  constexpr int PIECES = C::BN / 32;  // 32-column pieces per B-tile row
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][C::BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BK * LDB];
  __shared__ float s_lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const TileCoord tc = tile_of((K + C::BN - 1) / C::BN, xb_m, xb_n);
  const int64_t m0 = tc.m * C::BM, n0 = tc.n * C::BN;  // n0 indexes k_out
  levels_to_lds(lv, s_lv, tid);

  const int nk = (int)((N + BK - 1) / BK);
  u32x4_t ra[C::A_CH];
  u32x4_t rc[C::C_CH];
  RawScale rcq[C::C_CH];

  auto load_main = [&](int s) {
    const int64_t k0 = (int64_t)s * BK;
    load_a<C>(dY, N, m0, T, k0, N, tid, ra);
#pragma unroll
    for (int i = 0; i < C::C_CH; ++i) {
      const int c = tid + C::NT * i;
      const int64_t n = k0 + c / PIECES, kc = n0 + (c % PIECES) * 32;
      if (n < N && kc < K && (!C::C_SPARSE || c < 2 * C::BN)) {
        rc[i] = *reinterpret_cast<const u32x4_t *>(codes + n * (K / 2) + kc / 2);
        rcq[i] = load_scale(absmax_q, step, n * (K / BK) + kc / BK);
      } else {
        rc[i] = u32x4_t{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
        rcq[i] = RawScale{0u, 0.f};
      }
    }
  };
  auto store_main = [&](int buf) {
    store_a<C>(sA[buf], tid, ra);
#pragma unroll
    for (int i = 0; i < C::C_CH; ++i) {
      const int c = tid + C::NT * i;
      if (C::C_SPARSE && c >= 2 * C::BN) break;
      bf16_t *dst = sB[buf] + (c / PIECES) * LDB + (c % PIECES) * 32;
      const float cq = scale_of(rcq[i]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float v[8];
        decode8(rc[i][w], cq, s_lv, v);
        u32x4_t o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        o.z = pack_bf16x2(v[4], v[5]);
        o.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<u32x4_t *>(dst + w * 8) = o;
      }
    }
  };
  // this wave's B operands for one 16-deep substep, via two transposing reads each
  const int grp = lane >> 4, ai = lane & 15;
  auto mma = [&](const bf16_t *sa, const bf16_t *sb, f32x16_t (&acc)[C::WM][C::WN]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      u32x4_t a[C::WM], b[C::WN];
#pragma unroll
      for (int i = 0; i < C::WM; ++i) {
        const int ra_ = (wm * C::WM + i) * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const u32x4_t *>(sa + lds_off(ra_, chunk));
      }
#pragma unroll
      for (int j = 0; j < C::WN; ++j) {
        const int row = kk * 16 + 8 * (grp >> 1) + (ai >> 2);
        const int col = (wn * C::WN + j) * 32 + 16 * (grp & 1) + 4 * (ai & 3);
        typedef short s4_t __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s4_t lds_s4;
        const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(sb + row * LDB + col));
        const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(sb + (row + 4) * LDB + col));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        b[j] = u32x4_t{l2.x, l2.y, h2.x, h2.y};
      }
#pragma unroll
      for (int i = 0; i < C::WM; ++i)
#pragma unroll
        for (int j = 0; j < C::WN; ++j) acc[i][j] = mfma_32x32x16(a[i], b[j], acc[i][j]);
    }
  };

  f32x16_t acc[C::WM][C::WN];
  zero_acc<C>(acc);

  load_main(0);
  __syncthreads();
  store_main(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) load_main(s + 1);
    mma(sA[buf], sB[buf], acc);
    if (s + 1 < nk) store_main(buf ^ 1);
    __syncthreads();
  }
  // LoRA term: dUp [T, rp] . A [r, K], reduction over the rank (rows j of A)
  for (int64_t k0 = 0; k0 < rp; k0 += BK) {
    {
      constexpr int LCH = BK * C::BN / 8 / C::NT;  // 16-byte chunks of A per thread
      u32x4_t rv[C::A_CH], rl[LCH];
      load_a<C>(dUp, rp, m0, T, k0, rp, tid, rv);
#pragma unroll
      for (int i = 0; i < LCH; ++i) {
        const int c = tid + C::NT * i;
        const int64_t j = k0 + c / (C::BN / 8), kc = n0 + (c % (C::BN / 8)) * 8;
        rl[i] = (j < r && kc < K) ? *reinterpret_cast<const u32x4_t *>(A + j * K + kc) : u32x4_t{0u, 0u, 0u, 0u};
      }
      store_a<C>(sA[0], tid, rv);
#pragma unroll
      for (int i = 0; i < LCH; ++i) {
        const int c = tid + C::NT * i;
        *reinterpret_cast<u32x4_t *>(sB[0] + (c / (C::BN / 8)) * LDB + (c % (C::BN / 8)) * 8) = rl[i];
      }
    }
    __syncthreads();
    mma(sA[0], sB[0], acc);
    __syncthreads();
  }
  store_out<C>(dX, K, m0, T, n0, K, wm, wn, lane, acc);
}

// ---------------------------------------------------------------- dispatch
namespace {
using T128x128 = TileCfg<2, 2, 2, 2>;    // 4 waves, 64x64 per wave, two workgroups per CU
using T256x256w8 = TileCfg<2, 4, 4, 2>;  // 8 waves, 128x64 per wave, one workgroup per CU
using T256x128w8 = TileCfg<4, 2, 2, 2>;  // 8 waves, 64x64 per wave
using T128x256w8 = TileCfg<2, 4, 2, 2>;  // 8 waves, 64x64 per wave
using T128x128w8 = TileCfg<2, 4, 2, 1>;  // 8 waves, 64x32 per wave

// XCD blocking of a tiles_m x tiles_n grid: the 8-way split (xb_m x xb_n
// tiles per XCD) that minimises the modelled L2-miss traffic
//   8 * (xb_m / tiles_m * a_bytes + xb_n / tiles_n * b_bytes),
// where a_bytes is the activation operand and b_bytes the weight stream.
// Returns 0 x 0 (row-major order) when the grid does not split into 8 blocks.
void xcd_blocking(int64_t tiles_m, int64_t tiles_n, double a_bytes, double b_bytes, int *xb_m, int *xb_n) {
  *xb_m = *xb_n = 0;
  double best = 0.0;
  for (int64_t bm = 1; bm <= tiles_m; ++bm) {
    if (tiles_m % bm) continue;
    const int64_t blocks_m = tiles_m / bm;
    if (8 % blocks_m) continue;
    const int64_t blocks_n = 8 / blocks_m;
    if (tiles_n % blocks_n) continue;
    const int64_t bn = tiles_n / blocks_n;
    const double cost = 8.0 * ((double)bm / tiles_m * a_bytes + (double)bn / tiles_n * b_bytes);
    if (*xb_m == 0 || cost < best) {
      best = cost;
      *xb_m = (int)bm;
      *xb_n = (int)bn;
    }
  }
}

template <class C>
hipError_t fwd_with(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                    const float *step, int64_t N, const bf16_t *V, const bf16_t *Bp, int64_t ldb, int64_t r,
                    int64_t rp, bf16_t *Y, const Levels &lv, hipStream_t s) {
  const int64_t tm = (T + C::BM - 1) / C::BM, tn = (N + C::BN - 1) / C::BN;
  int xb_m, xb_n;
  xcd_blocking(tm, tn, 2.0 * T * K, 0.516 * N * K, &xb_m, &xb_n);
  hipLaunchKernelGGL(k_nf4_gemm_fwd<C>, dim3((unsigned)(tm * tn)), dim3(C::NT), 0, s, X, T, K, codes, absmax_q, step,
                     N, V, Bp, ldb, r, rp, Y, lv, xb_m, xb_n);
  return hipGetLastError();
}

template <class C>
hipError_t dx_with(const bf16_t *dY, int64_t T, int64_t N, const uint8_t *codes, const uint8_t *absmax_q,
                   const float *step, int64_t K, const bf16_t *dUp, const bf16_t *A, int64_t r, int64_t rp,
                   bf16_t *dX, const Levels &lv, hipStream_t s) {
  const int64_t tm = (T + C::BM - 1) / C::BM, tn = (K + C::BN - 1) / C::BN;
  int xb_m, xb_n;
  xcd_blocking(tm, tn, 2.0 * T * N, 0.516 * N * K, &xb_m, &xb_n);
  hipLaunchKernelGGL(k_nf4_gemm_dx<C>, dim3((unsigned)(tm * tn)), dim3(C::NT), 0, s, dY, T, N, codes, absmax_q, step,
                     K, dUp, A, r, rp, dX, lv, xb_m, xb_n);
  return hipGetLastError();
}
}  // namespace

// Tile choice for an M x N output.  Measured on MI355X (both GEMMs, seven
// workload shapes): the largest 8-wave tile that still yields at least one
// workgroup per CU (256 tiles) is fastest -- 256x256, else 256x128; below that
// the 128x128 tile, two workgroups per CU, wins.
int nf4_gemm_pick_tile(int64_t M, int64_t N) {
  auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (tiles(256, 256) >= 256) return NF4_TILE_256x256_W8;
  if (tiles(256, 128) >= 256) return NF4_TILE_256x128_W8;
  return NF4_TILE_128x128;
}

hipError_t launch_nf4_gemm_fwd(int tile, const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes,
                               const uint8_t *absmax_q, const float *step, int64_t N, const bf16_t *V,
                               const bf16_t *Bp, int64_t ldb, int64_t r, int64_t rp, bf16_t *Y, const Levels &lv,
                               hipStream_t s) {
  if (T == 0) return hipSuccess;
  switch (tile) {
    case NF4_TILE_256x256_W8: return fwd_with<T256x256w8>(X, T, K, codes, absmax_q, step, N, V, Bp, ldb, r, rp, Y, lv, s);
    case NF4_TILE_256x128_W8: return fwd_with<T256x128w8>(X, T, K, codes, absmax_q, step, N, V, Bp, ldb, r, rp, Y, lv, s);
    case NF4_TILE_128x256_W8: return fwd_with<T128x256w8>(X, T, K, codes, absmax_q, step, N, V, Bp, ldb, r, rp, Y, lv, s);
    case NF4_TILE_128x128_W8: return fwd_with<T128x128w8>(X, T, K, codes, absmax_q, step, N, V, Bp, ldb, r, rp, Y, lv, s);
    default: return fwd_with<T128x128>(X, T, K, codes, absmax_q, step, N, V, Bp, ldb, r, rp, Y, lv, s);
  }
}

hipError_t launch_nf4_gemm_dx(int tile, const bf16_t *dY, int64_t T, int64_t N, const uint8_t *codes,
                              const uint8_t *absmax_q, const float *step, int64_t K, const bf16_t *dUp, const bf16_t *A,
                              int64_t r, int64_t rp, bf16_t *dX, const Levels &lv, hipStream_t s) {
  if (T == 0) return hipSuccess;
  switch (tile) {
    case NF4_TILE_256x256_W8: return dx_with<T256x256w8>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s);
    case NF4_TILE_256x128_W8: return dx_with<T256x128w8>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s);
    case NF4_TILE_128x256_W8: return dx_with<T128x256w8>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s);
    case NF4_TILE_128x128_W8: return dx_with<T128x128w8>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s);
    default: return dx_with<T128x128>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s);
  }
}

}  // namespace qlora
