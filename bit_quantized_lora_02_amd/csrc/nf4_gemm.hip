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
// The reduction runs in steps of 64 (one NF4 block per weight row):
//  - the activation tile of step s+1 is copied global -> LDS by the load unit
//    itself (global_load_lds_dwordx4), so it never occupies registers;
//  - the codes and block constants of step s+2 are loaded into one of two
//    register slots;
//  - the MFMAs of step s are interleaved with the decode of step s+1 (level
//    lookup, one binary32 multiply per weight, bf16 pack, LDS store), so the
//    decode's VALU and LDS work runs while the matrix unit is busy;
//  - one barrier per step.
// The dequantized weight therefore exists only as one 64-deep tile in LDS.
// The LoRA term follows as a few extra reduction steps over the padded rank,
// landing in the same binary32 accumulators.  When the forward's output has too
// few tiles to occupy every CU, its reduction is split into ranges whose
// binary32 partial sums a finalize adds in order (nf4_gemm_fwd_split).
//
// LDS tiles of the A operand (and the forward B operand) are [row][64] bf16
// (128-byte rows) with the 16-byte chunk index XOR-swizzled by (row / 2) % 8:
// a 16-lane phase of ds_read_b128 then covers all 64 banks once.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int BK = 64;

template <int WAVES_M_, int WAVES_N_, int WM_, int WN_, int AHEAD_ = 1>
struct TileCfg {
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, WM = WM_, WN = WN_;
  static constexpr int AHEAD = AHEAD_;  // substeps by which the MFMA operand reads run ahead (1 or 2)
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = WAVES_M * WM * 32;
  static constexpr int BN = WAVES_N * WN * 32;
  static constexpr int A_LD = BM * 8 / NT;  // direct 16-byte loads of the A tile per thread and step
  // weights decoded per decoding thread and step (at least 16); the first DEC threads decode
  static constexpr int E = (BN * BK / NT > 16) ? BN * BK / NT : 16;
  static constexpr int DEC = BN * BK / E;
  static constexpr int NWD = E / 8;         // code words (8 nibbles each) per thread and step
  static constexpr int L_CH = BN * 8 / NT;  // 16-byte chunks of the LoRA B tile per thread (forward)
  static_assert(BM * 8 % NT == 0 && A_LD >= 1, "unsupported tile");
  static_assert((E == 16 || E == 32) && DEC % 64 == 0 && DEC <= NT, "unsupported tile");
  static_assert(WM % 2 == 0, "the MFMA rows are issued in two halves");
};

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3); }

// Keep the instruction order written in the source at this point.
__device__ __forceinline__ void fence_sched() { __builtin_amdgcn_sched_barrier(0); }

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

// Direct activation loads (global_load_lds_dwordx4: lane l's 16 bytes land
// at the wave-uniform LDS base + 16 l).  Load i of wave w fills tile rows
// 8g .. 8g+7 (g = i NW + w), one 1 KB run; lane l fills row 8g + l/8 at
// swizzled chunk slot l % 8, i.e. logical chunk (l % 8) ^ ((row / 2) % 8).
// Rows past `rows` re-read the last row (their outputs are never stored).
template <class C>
struct ALoads {
  const bf16_t *src[C::A_LD];
  int col[C::A_LD];
  int wave;
  __device__ __forceinline__ void init(const bf16_t *__restrict__ base, int64_t ld, int64_t m0, int64_t rows, int w,
                                       int lane) {
    wave = w;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      const int row = 8 * (i * C::NW + w) + (lane >> 3);
      const int64_t grow = (m0 + row < rows) ? m0 + row : rows - 1;
      src[i] = base + grow * ld;
      col[i] = 8 * ((lane & 7) ^ ((row >> 1) & 7));
    }
  }
  // Reduction columns k0 .. k0+63 into the tile at sa; a chunk starting at or
  // past kmax re-reads the last chunk (the matching weight rows decode to 0).
  __device__ __forceinline__ void issue(int64_t k0, int64_t kmax, bf16_t *sa) const {
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      int64_t c = k0 + col[i];
      c = c < kmax ? c : kmax - 8;
      __builtin_amdgcn_global_load_lds((const void *)(src[i] + c),
                                       (__attribute__((address_space(3))) void *)(sa + (i * C::NW + wave) * 512), 16,
                                       0, 0);
    }
  }
};

// Code words of one thread and step (E/2 bytes, one block constant).
template <int NWD>
__device__ __forceinline__ void load_words(const uint8_t *__restrict__ p, uint32_t (&w)[NWD]) {
  if constexpr (NWD == 4) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(p);
    w[0] = v.x, w[1] = v.y, w[2] = v.z, w[3] = v.w;
  } else {
    const u32x2_t v = *reinterpret_cast<const u32x2_t *>(p);
    w[0] = v.x, w[1] = v.y;
  }
}

// The two halves of decoding one code word: the level lookups, then the
// binary32 products with the block constant packed to bf16.
// (the lookups read the level-pair table one code byte at a time: the address
// is the byte times 8, one v_lshlrev_b32 with a byte select)
__device__ __forceinline__ void lookup8(uint32_t w, const float2 *s_lv, float (&v)[8]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float2 l = s_lv[(w >> (8 * b)) & 0xffu];
    v[2 * b] = l.x;
    v[2 * b + 1] = l.y;
  }
}
__device__ __forceinline__ u32x4_t scale_pack8(const float (&v)[8], float cq) {
  return u32x4_t{pack_bf16x2(__fmul_rn(v[0], cq), __fmul_rn(v[1], cq)),
                 pack_bf16x2(__fmul_rn(v[2], cq), __fmul_rn(v[3], cq)),
                 pack_bf16x2(__fmul_rn(v[4], cq), __fmul_rn(v[5], cq)),
                 pack_bf16x2(__fmul_rn(v[6], cq), __fmul_rn(v[7], cq))};
}

// A operand of substep kk (16 reduction columns) for this wave's row tile i, and for all WM of them.
template <class C>
__device__ __forceinline__ u32x4_t read_a_one(const bf16_t *sa, int wm, int lane, int kk, int i) {
  const int chunk = kk * 2 + (lane >> 5);
  return *reinterpret_cast<const u32x4_t *>(sa + lds_off((wm * C::WM + i) * 32 + (lane & 31), chunk));
}
template <class C>
__device__ __forceinline__ void read_a(const bf16_t *sa, int wm, int lane, int kk, u32x4_t (&a)[C::WM]) {
#pragma unroll
  for (int i = 0; i < C::WM; ++i) a[i] = read_a_one<C>(sa, wm, lane, kk, i);
}
// B operand from a [n][64] tile (forward)
template <class C>
__device__ __forceinline__ void read_b_rows(const bf16_t *sb, int wn, int lane, int kk, u32x4_t (&b)[C::WN]) {
  const int chunk = kk * 2 + (lane >> 5);
#pragma unroll
  for (int j = 0; j < C::WN; ++j)
    b[j] = *reinterpret_cast<const u32x4_t *>(sb + lds_off((wn * C::WN + j) * 32 + (lane & 31), chunk));
}
// 16-byte chunk c of row `row` of the dX weight tile sits at chunk slot c ^ 2 ((c >> 4) & 1) ^ (row & 1):
// a 16-lane phase of the decoded-tile stores (two rows, eight 32-column pieces) then covers 16 distinct
// 16-byte bank groups, and the slots only move within aligned groups of four chunks, so the transposing
// reads stay conflict-free.
__device__ __forceinline__ int dx_off(int row, int chunk, int ldb) {
  return row * ldb + ((chunk ^ (((chunk >> 4) & 1) << 1) ^ (row & 1)) << 3);
}
// B operand from a natural [k][LDB] tile with two transposing reads per tile:
// in each 16-lane group, lane i gets element (i & 3) of the 8 bytes addressed
// by lane 4m + (i >> 2), so lane a points at row base + (a >> 2), columns
// 4 (a & 3) .. +3, and reads of rows +0..3 and +4..7 give its 8 reduction values.
template <class C, int LDB>
__device__ __forceinline__ u32x4_t read_b_tr_one(const bf16_t *sb, int wn, int lane, int kk, int j) {
  typedef short s4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4_t lds_s4;
  const int grp = lane >> 4, ai = lane & 15;
  const int row = kk * 16 + 8 * (grp >> 1) + (ai >> 2);
  const int col = (wn * C::WN + j) * 32 + 16 * (grp & 1) + 4 * (ai & 3);
  const int off = dx_off(row, col >> 3, LDB) + (col & 7);
  const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(sb + off));
  const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(sb + off + 4 * LDB));
  const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{l2.x, l2.y, h2.x, h2.y};
}
template <class C, int LDB>
__device__ __forceinline__ void read_b_tr(const bf16_t *sb, int wn, int lane, int kk, u32x4_t (&b)[C::WN]) {
#pragma unroll
  for (int j = 0; j < C::WN; ++j) b[j] = read_b_tr_one<C, LDB>(sb, wn, lane, kk, j);
}

template <class C>
__device__ __forceinline__ void mma_rows(int i0, int i1, const u32x4_t (&a)[C::WM], const u32x4_t (&b)[C::WN],
                                         f32x16_t (&acc)[C::WM][C::WN]) {
#pragma unroll
  for (int i = i0; i < i1; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) acc[i][j] = mfma_32x32x16(a[i], b[j], acc[i][j]);
}

// Rows [row0, row0+BM) x columns [col0, col0+64) of a row-major bf16 matrix
// into registers and LDS (the unpipelined LoRA steps): chunk c = tid + NT*i
// covers row c>>3, 16-byte chunk c&7.  Rows >= rows (or < row_lo) or columns
// >= cols read as zero (cols % 8 == 0).
template <class C>
__device__ __forceinline__ void copy_a_tile(const bf16_t *__restrict__ src, int64_t ld, int64_t row0, int64_t rows,
                                            int64_t col0, int64_t cols, int tid, bf16_t *s, int64_t row_lo = 0) {
  u32x4_t r[C::A_LD];
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    const int c = tid + C::NT * i;
    const int64_t row = row0 + (c >> 3), col = col0 + (c & 7) * 8;
    r[i] = (row >= row_lo && row < rows && col < cols) ? *reinterpret_cast<const u32x4_t *>(src + row * ld + col)
                                                       : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    const int c = tid + C::NT * i;
    *reinterpret_cast<u32x4_t *>(s + lds_off(c >> 3, c & 7)) = r[i];
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

// The same for binary32 partial sums (split reduction): out[row ld + col] = acc.
template <class C>
__device__ __forceinline__ void store_out_f32(float *__restrict__ out, int64_t ld, int64_t m0, int64_t rows,
                                              int64_t n0, int64_t cols, int wm, int wn, int lane,
                                              const f32x16_t acc[C::WM][C::WN]) {
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      const int64_t col = n0 + (wn * C::WN + j) * 32 + (lane & 31);
      if (col >= cols) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + (wm * C::WM + i) * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (row < rows) out[row * ld + col] = acc[i][j][e];
      }
    }
}

// Wait for all but the last three vector-memory loads (the code words and the
// block constant issued after the activation tile) and for all LDS operations.
// s_waitcnt fields: vmcnt[3:0], expcnt[6:4] (7 = no wait), lgkmcnt[11:8].
__device__ __forceinline__ void wait_tile_keep3() { __builtin_amdgcn_s_waitcnt(0x0073); }

// One pipelined reduction step (see the file comment).  P = s % 2 selects the
// LDS buffers and register slots: step s is multiplied out of buffer P while
// the words in slot P^1 (step s+1) are decoded into buffer P^1, the
// activation tile of step s+1 is copied into buffer P^1 by the load unit, and
// step s+2's words are loaded into slot P.  The caller's lambdas carry the
// layout differences between the forward and dX: `load_next()` issues the
// global loads (the activation tile first, then exactly three loads for the
// words), `store_word(w, bf16x8)` writes word w of the decoded slot.  The
// LDS buffers are distinct variables, so the compiler can tell the reads of
// buffer P from the direct loads into buffer P^1.
template <class C, class ReadB, class LoadNext, class StoreWord>
__device__ __forceinline__ void pipelined_step(const bf16_t *sa, const bf16_t *sb, int wm, int wn, int lane,
                                               const uint32_t (&words)[C::NWD], const RawScale &scale,
                                               const float2 *s_lv, f32x16_t (&acc)[C::WM][C::WN], ReadB read_b,
                                               LoadNext load_next, StoreWord store_word, bool decoder) {
  load_next();  // activation tile of step s+1, then the words of step s+2
  fence_sched();
  const float cq = scale_of(scale);
  constexpr int EVERY = 4 / C::NWD;  // substeps per decoded word
  if constexpr (C::AHEAD == 1) {
    u32x4_t a[2][C::WM], b[2][C::WN];
    float v[8];
    read_a<C>(sa, wm, lane, 0, a[0]);
    read_b(sb, 0, b[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
      const bool dec = decoder && (kk % EVERY) == 0;
      if (dec) lookup8(words[kk / EVERY], s_lv, v);
      fence_sched();
      mma_rows<C>(0, C::WM / 2, a[cur], b[cur], acc);
      fence_sched();
      if (dec) store_word(kk / EVERY, scale_pack8(v, cq));
      if (kk < 3) {
        read_a<C>(sa, wm, lane, kk + 1, a[cur ^ 1]);
        read_b(sb, kk + 1, b[cur ^ 1]);
      }
      fence_sched();
      mma_rows<C>(C::WM / 2, C::WM, a[cur], b[cur], acc);
      fence_sched();
    }
  } else {
    // operand reads two substeps ahead of the MFMAs (three register sets)
    u32x4_t a[3][C::WM], b[3][C::WN];
    float v[8];
    read_a<C>(sa, wm, lane, 0, a[0]);
    read_b(sb, 0, b[0]);
    read_a<C>(sa, wm, lane, 1, a[1]);
    read_b(sb, 1, b[1]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk % 3;
      const bool dec = decoder && (kk % EVERY) == 0;
      if (dec) lookup8(words[kk / EVERY], s_lv, v);
      if (kk + 2 < 4) {
        read_a<C>(sa, wm, lane, kk + 2, a[(kk + 2) % 3]);
        read_b(sb, kk + 2, b[(kk + 2) % 3]);
      }
      fence_sched();
      mma_rows<C>(0, C::WM / 2, a[cur], b[cur], acc);
      fence_sched();
      if (dec) store_word(kk / EVERY, scale_pack8(v, cq));
      fence_sched();
      mma_rows<C>(C::WM / 2, C::WM, a[cur], b[cur], acc);
      fence_sched();
    }
  }
  wait_tile_keep3();
  __syncthreads();
}

}  // namespace

// ---------------------------------------------------------------- forward
// Y[T, N] = X[T, K] . W'[N, K]^T + V[T, rp] . B[N, :r]^T   (B row stride ldb, columns >= r read as 0)
// With psum != null the reduction is split into gridDim.y ranges of K / gridDim.y columns (a multiple
// of 64): workgroup (x, y) computes tile x over range y and stores its binary32 sums in
// psum[y][T][N]; range 0 also adds the LoRA term.  (A finalize adds the ranges in order.)
template <class C, bool MULTI>
__global__ __launch_bounds__(C::NT) void k_nf4_gemm_fwd(const bf16_t *__restrict__ X, int64_t T, int64_t K,
                                                        const uint8_t *__restrict__ codes,
                                                        const uint8_t *__restrict__ absmax_q,
                                                        const float *__restrict__ step, int64_t N,
                                                        const bf16_t *__restrict__ V, const bf16_t *__restrict__ Bp,
                                                        int64_t ldb, int64_t r, int64_t rp, bf16_t *__restrict__ Y,
                                                        Levels lv, int xb_m, int xb_n, SegTable sg,
                                                        float *__restrict__ psum) {
  __shared__ __attribute__((aligned(16))) bf16_t sA0[C::BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sA1[C::BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB0[C::BN * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB1[C::BN * BK];
  // level pairs by code byte; the alignment places the table at LDS address 0, so that a lookup address
  // is the code byte times 8 (one shift with a byte select; no base to add)
  __shared__ __attribute__((aligned(1024))) float2 s_lv[256];
  bf16_t *const sA[2] = {sA0, sA1};
  bf16_t *const sB[2] = {sB0, sB1};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const TileCoord tc = tile_of((N + C::BN - 1) / C::BN, xb_m, xb_n);
  const int64_t m0 = tc.m * C::BM, n0 = tc.n * C::BN;
  pair_levels_to_lds(lv, s_lv, tid);

  const int split = (int)blockIdx.y;
  const int64_t kc = K / gridDim.y, kbase = (int64_t)split * kc;  // this workgroup's reduction range
  const int nk = (int)(kc / BK);
  ALoads<C> al;
  al.init(X + kbase, K, m0, T, wave, lane);
  // this thread decodes weights part*E .. part*E+E-1 of tile row brow
  constexpr int PARTS = BK / C::E;
  const bool decoder = C::DEC == C::NT || tid < C::DEC;  // wave-uniform; a constant when every thread decodes
  const int brow = decoder ? tid / PARTS : 0, part = tid % PARTS;
  const int64_t wrow = (n0 + brow < N) ? n0 + brow : N - 1;  // rows past N feed columns that are never stored
  const uint8_t *crow = codes + wrow * (K / 2) + kbase / 2 + part * (C::E / 2);
  const int64_t blk0 = wrow * (K / BK) + kbase / BK;
  uint32_t rc[2][C::NWD];
  RawScale rs[2];
  auto load_words_of = [&](int s, uint32_t(&w)[C::NWD], RawScale &sc) {
    load_words<C::NWD>(crow + (int64_t)s * (BK / 2), w);
    sc = load_scale(absmax_q, step, blk0 + s);
  };
  auto read_b = [&](const bf16_t *sb, int kk, u32x4_t(&b)[C::WN]) { read_b_rows<C>(sb, wn, lane, kk, b); };

  f32x16_t acc[C::WM][C::WN];
  zero_acc<C>(acc);

  // prologue: tile 0 of A, words of steps 0 and 1, decode step 0
  al.issue(0, kc, sA[0]);
  load_words_of(0, rc[0], rs[0]);
  load_words_of(nk > 1 ? 1 : 0, rc[1], rs[1]);
  __syncthreads();  // level table visible
  {
    const float cq = scale_of(rs[0]);
    if (decoder)
      for (int w = 0; w < C::NWD; ++w) {
        float v[8];
        lookup8(rc[0][w], s_lv, v);
        *reinterpret_cast<u32x4_t *>(sB[0] + lds_off(brow, part * C::NWD + w)) = scale_pack8(v, cq);
      }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the direct loads of tile 0 have landed
  __syncthreads();

  auto step_p = [&](auto pc, int s) {
    constexpr int P = decltype(pc)::value;
    const int sa = (s + 1 < nk) ? s + 1 : nk - 1, sc = (s + 2 < nk) ? s + 2 : nk - 1;
    auto load_next = [&]() {
      al.issue((int64_t)sa * BK, kc, sA[P ^ 1]);
      fence_sched();  // activation loads first: waiting for them leaves the words in flight
      load_words_of(sc, rc[P], rs[P]);
    };
    auto store_word = [&](int w, const u32x4_t &o) {
      *reinterpret_cast<u32x4_t *>(sB[P ^ 1] + lds_off(brow, part * C::NWD + w)) = o;
    };
    pipelined_step<C>(sA[P], sB[P], wm, wn, lane, rc[P ^ 1], rs[P ^ 1], s_lv, acc, read_b, load_next,
                      store_word, decoder);
  };
  int s = 0;
  for (; s + 1 < nk; s += 2) {
    step_p(std::integral_constant<int, 0>(), s);
    step_p(std::integral_constant<int, 1>(), s + 1);
  }
  if (s < nk) step_p(std::integral_constant<int, 0>(), s);

  // LoRA up-projection: V [T, rp] . B [N, rp]^T over the rows [lo, hi), one 64-deep step at a time
  auto lora_rows = [&](const bf16_t *__restrict__ Bsrc, int64_t lo, int64_t hi) {
    for (int64_t k0 = 0; k0 < rp; k0 += BK) {
      copy_a_tile<C>(V, rp, m0, hi, k0, rp, tid, sA[0], lo);
#pragma unroll
      for (int i = 0; i < C::L_CH; ++i) {
        const int c = tid + C::NT * i;
        const int64_t brw = n0 + (c >> 3), col = k0 + (c & 7) * 8;  // r % 8 == 0 or B padded to ldb
        const u32x4_t v = (brw < N && col < r) ? *reinterpret_cast<const u32x4_t *>(Bsrc + brw * ldb + col)
                                               : u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t *>(sB[0] + lds_off(c >> 3, c & 7)) = v;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4_t a[C::WM], b[C::WN];
        read_a<C>(sA[0], wm, lane, kk, a);
        read_b_rows<C>(sB[0], wn, lane, kk, b);
        mma_rows<C>(0, C::WM, a, b, acc);
      }
      __syncthreads();
    }
  };
  if (split != 0) {
    // the LoRA term belongs to range 0 only
  } else if constexpr (!MULTI) {
    lora_rows(Bp, 0, T);
  } else {
    // many adapters: one masked up-projection per token segment that meets this tile's rows
    // (first segment ending past m0 by bisection; entries clamped to [0, T])
    auto clampT = [&](int64_t v) { return v < 0 ? (int64_t)0 : (v > T ? T : v); };
    int g0 = 0, g1 = sg.n_seg;
    while (g0 < g1) {
      const int mid = (g0 + g1) >> 1;
      if (clampT(sg.seg[mid + 1]) <= m0) g0 = mid + 1;
      else g1 = mid;
    }
    for (int g = g0; g < sg.n_seg; ++g) {
      const int64_t lo = clampT(sg.seg[g]), hi = clampT(sg.seg[g + 1]);
      if (lo >= m0 + C::BM) break;
      const int a = sg.ad[g];
      if (hi <= lo || hi <= m0 || a < 0 || a >= sg.n_pool) continue;
      lora_rows(Bp + (int64_t)a * N * r, lo, hi);
    }
  }
  if (psum) store_out_f32<C>(psum + (int64_t)split * T * N, N, m0, T, n0, N, wm, wn, lane, acc);
  else store_out<C>(Y, N, m0, T, n0, N, wm, wn, lane, acc);
}

// --------------------------------------------------------------- backward
// dX[T, K] = dY[T, N] . W'[N, K] + dUp[T, rp] . A[r, K]   (rows of A past r read as 0)
// The reduction index is the weight row n.  The B operand is decoded exactly as
// in the forward (code words of consecutive columns of one weight row, one
// block constant) and stored in its natural [n][k_out] layout, rows padded so
// that the four rows one transposing read touches cover all 64 banks; the MFMA
// operand, which needs 8 consecutive n for one k_out, is read transposed.
// Weight rows past N decode to zero, so the clamped activation columns they
// meet contribute nothing.
//
// With LoRA dropout on the layer input (DROP), the adapter term is multiplied
// elementwise by keep * q (the derivative of inverted dropout): the kernel
// then forms dUp . A first, scales each accumulator element by its keep bit
// times q, and accumulates dY . W' on top, so no second accumulator is needed.
// Keep bit (t, k) is bit k % 8 of mask[(t K + k) / 8].
// Keep bits of the output tile, staged in LDS as BM rows of BN / 8 bytes; each
// accumulator element then reads its row's 32-bit word for its 32-column tile.
template <class C>
__device__ __forceinline__ void stage_keep_bits(uint8_t *s_keep, const uint8_t *__restrict__ mask, int64_t K,
                                                int64_t m0, int64_t rows, int64_t n0, int tid) {
  constexpr int PIECES = C::BM * C::BN / 64;  // 8-byte pieces (64 columns of one row)
#pragma unroll
  for (int c = tid; c < PIECES; c += C::NT) {
    const int row = c / (C::BN / 64), part = c % (C::BN / 64);
    const int64_t col = n0 + 64 * part;  // n0 and K are multiples of 64: a piece is all in or all out
    u32x2_t v = u32x2_t{0u, 0u};
    if (m0 + row < rows && col < K) v = *reinterpret_cast<const u32x2_t *>(mask + ((m0 + row) * K + col) / 8);
    *reinterpret_cast<u32x2_t *>(s_keep + row * (C::BN / 8) + 8 * part) = v;
  }
}

template <class C, bool DROP>
__global__ __launch_bounds__(C::NT) void k_nf4_gemm_dx(const bf16_t *__restrict__ dY, int64_t T, int64_t N,
                                                       const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ absmax_q,
                                                       const float *__restrict__ step, int64_t K,
                                                       const bf16_t *__restrict__ dUp, const bf16_t *__restrict__ A,
                                                       int64_t r, int64_t rp, bf16_t *__restrict__ dX, Levels lv,
                                                       int xb_m, int xb_n, const uint8_t *__restrict__ mask, float q) {
  constexpr int LDB = C::BN + 32;  // row length (elements) of the [64][BN] B tile: 16 banks mod 64 per row
  __shared__ __attribute__((aligned(16))) bf16_t sA0[C::BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sA1[C::BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB0[BK * LDB];
  __shared__ __attribute__((aligned(16))) bf16_t sB1[BK * LDB];
  // level pairs by code byte; the alignment places the table at LDS address 0, so that a lookup address
  // is the code byte times 8 (one shift with a byte select; no base to add)
  __shared__ __attribute__((aligned(1024))) float2 s_lv[256];
  bf16_t *const sA[2] = {sA0, sA1};
  bf16_t *const sB[2] = {sB0, sB1};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const TileCoord tc = tile_of((K + C::BN - 1) / C::BN, xb_m, xb_n);
  const int64_t m0 = tc.m * C::BM, n0 = tc.n * C::BN;  // n0 indexes k_out
  pair_levels_to_lds(lv, s_lv, tid);

  const int nk = (int)((N + BK - 1) / BK);
  ALoads<C> al;
  al.init(dY, N, m0, T, wave, lane);
  // this thread decodes columns piece*E .. piece*E+E-1 of tile row bn (weight row k0 + bn)
  constexpr int PIECES = C::BN / C::E;
  const bool decoder = tid < C::DEC;  // wave-uniform (kept a run-time value here: measured faster for dX)
  const int bn = decoder ? tid / PIECES : 0, piece = tid % PIECES;
  const int64_t kc = (n0 + piece * C::E + C::E <= K) ? n0 + piece * C::E : K - C::E;  // columns past K: never stored
  uint32_t rc[2][C::NWD];
  RawScale rs[2];
  auto load_words_of = [&](int s, uint32_t(&w)[C::NWD], RawScale &sc) {
    const int64_t n = (int64_t)s * BK + bn;
    const int64_t nn = n < N ? n : N - 1;
    load_words<C::NWD>(codes + nn * (K / 2) + kc / 2, w);
    sc = load_scale(absmax_q, step, nn * (K / BK) + kc / BK);
    if (n >= N) sc.d = 0.f;  // weight rows past N decode to (signed) zero
  };
  auto read_b = [&](const bf16_t *sb, int kk, u32x4_t(&b)[C::WN]) { read_b_tr<C, LDB>(sb, wn, lane, kk, b); };

  f32x16_t acc[C::WM][C::WN];
  zero_acc<C>(acc);

  // LoRA term: dUp [T, rp] . A [r, K], reduction over the rank (rows j of A)
  auto lora_steps = [&]() {
    for (int64_t k0 = 0; k0 < rp; k0 += BK) {
      copy_a_tile<C>(dUp, rp, m0, T, k0, rp, tid, sA[0]);
      constexpr int LCH = BK * C::BN / 8 / C::NT;  // 16-byte chunks of A per thread
#pragma unroll
      for (int i = 0; i < LCH; ++i) {
        const int c = tid + C::NT * i;
        const int64_t j = k0 + c / (C::BN / 8), kcol = n0 + (c % (C::BN / 8)) * 8;
        const u32x4_t v =
            (j < r && kcol < K) ? *reinterpret_cast<const u32x4_t *>(A + j * K + kcol) : u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t *>(sB[0] + dx_off(c / (C::BN / 8), c % (C::BN / 8), LDB)) = v;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4_t a[C::WM], b[C::WN];
        read_a<C>(sA[0], wm, lane, kk, a);
        read_b_tr<C, LDB>(sB[0], wn, lane, kk, b);
        mma_rows<C>(0, C::WM, a, b, acc);
      }
      __syncthreads();
    }
  };
  al.issue(0, N, sA[0]);
  load_words_of(0, rc[0], rs[0]);
  load_words_of(nk > 1 ? 1 : 0, rc[1], rs[1]);
  __syncthreads();
  {
    const float cq = scale_of(rs[0]);
    if (decoder)
      for (int w = 0; w < C::NWD; ++w) {
        float v[8];
        lookup8(rc[0][w], s_lv, v);
        *reinterpret_cast<u32x4_t *>(sB[0] + dx_off(bn, piece * (C::E / 8) + w, LDB)) = scale_pack8(v, cq);
      }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the direct loads of tile 0 have landed
  __syncthreads();

  auto step_p = [&](auto pc, int s) {
    constexpr int P = decltype(pc)::value;
    const int sa = (s + 1 < nk) ? s + 1 : nk - 1, sc = (s + 2 < nk) ? s + 2 : nk - 1;
    auto load_next = [&]() {
      al.issue((int64_t)sa * BK, N, sA[P ^ 1]);
      fence_sched();  // activation loads first: waiting for them leaves the words in flight
      load_words_of(sc, rc[P], rs[P]);
    };
    auto store_word = [&](int w, const u32x4_t &o) {
      *reinterpret_cast<u32x4_t *>(sB[P ^ 1] + dx_off(bn, piece * (C::E / 8) + w, LDB)) = o;
    };
    pipelined_step<C>(sA[P], sB[P], wm, wn, lane, rc[P ^ 1], rs[P ^ 1], s_lv, acc, read_b, load_next,
                      store_word, decoder);
  };
  int s = 0;
  for (; s + 1 < nk; s += 2) {
    step_p(std::integral_constant<int, 0>(), s);
    step_p(std::integral_constant<int, 1>(), s + 1);
  }
  if (s < nk) step_p(std::integral_constant<int, 0>(), s);

  if constexpr (!DROP) {
    lora_steps();
  } else {
    // The adapter term times keep * q: all of dUp [BM, rp] and A [rp, BN] (rp <= 128: two 64-deep
    // chunks at most) go to LDS with the tile's keep bits; then each 32x32 tile forms its adapter
    // term in an accumulator of its own, scales it by its keep bits and q, and adds it.
    __shared__ __attribute__((aligned(16))) uint8_t s_keep[C::BM * C::BN / 8];
    stage_keep_bits<C>(s_keep, mask, K, m0, T, n0, tid);
    const int nkc = (int)(rp / BK);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (c >= nkc) break;
      copy_a_tile<C>(dUp, rp, m0, T, (int64_t)c * BK, rp, tid, sA[c]);
      constexpr int LCH = BK * C::BN / 8 / C::NT;  // 16-byte chunks of A per thread
#pragma unroll
      for (int u = 0; u < LCH; ++u) {
        const int cc = tid + C::NT * u;
        const int64_t j = (int64_t)c * BK + cc / (C::BN / 8), kcol = n0 + (cc % (C::BN / 8)) * 8;
        const u32x4_t v =
            (j < r && kcol < K) ? *reinterpret_cast<const u32x4_t *>(A + j * K + kcol) : u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t *>(sB[c] + dx_off(cc / (C::BN / 8), cc % (C::BN / 8), LDB)) = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::WM; ++i)
#pragma unroll
      for (int jt = 0; jt < C::WN; ++jt) {
        f32x16_t t;
#pragma unroll
        for (int e = 0; e < 16; ++e) t[e] = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (c >= nkc) break;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            t = mfma_32x32x16(read_a_one<C>(sA[c], wm, lane, kk, i), read_b_tr_one<C, LDB>(sB[c], wn, lane, kk, jt), t);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = (wm * C::WM + i) * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
          const uint32_t w = *reinterpret_cast<const uint32_t *>(s_keep + row * (C::BN / 8) + 4 * (wn * C::WN + jt));
          acc[i][jt][e] = __fadd_rn(acc[i][jt][e], ((w >> (lane & 31)) & 1u) ? __fmul_rn(t[e], q) : 0.f);
        }
        fence_sched();  // one tile's operands and words in flight at a time
      }
  }
  store_out<C>(dX, K, m0, T, n0, K, wm, wn, lane, acc);
}

// ---------------------------------------------------------------- dispatch
namespace {
using T128x128 = TileCfg<2, 2, 2, 2>;    // 4 waves, 64x64 per wave, two workgroups per CU
using T256x256w8 = TileCfg<2, 4, 4, 2>;  // 8 waves, 128x64 per wave, one workgroup per CU
using T256x128w8 = TileCfg<4, 2, 2, 2, 2>;  // 8 waves, 64x64 per wave, operand reads two substeps ahead
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
                    int64_t rp, bf16_t *Y, const Levels &lv, hipStream_t s, const SegTable &sg, int nsplit,
                    float *psum) {
  const int64_t tm = (T + C::BM - 1) / C::BM, tn = (N + C::BN - 1) / C::BN;
  int xb_m, xb_n;
  xcd_blocking(tm, tn, 2.0 * T * K, 0.516 * N * K, &xb_m, &xb_n);
  const dim3 grid((unsigned)(tm * tn), (unsigned)nsplit);
  if (sg.seg)
    launch(k_nf4_gemm_fwd<C, true>, grid, dim3(C::NT), 0, s, X, T, K, codes, absmax_q, step, N, V, Bp, ldb, r, rp, Y,
           lv, xb_m, xb_n, sg, psum);
  else
    launch(k_nf4_gemm_fwd<C, false>, grid, dim3(C::NT), 0, s, X, T, K, codes, absmax_q, step, N, V, Bp, ldb, r, rp, Y,
           lv, xb_m, xb_n, sg, psum);
  return hipGetLastError();
}

template <class C, bool DROP>
hipError_t dx_with(const bf16_t *dY, int64_t T, int64_t N, const uint8_t *codes, const uint8_t *absmax_q,
                   const float *step, int64_t K, const bf16_t *dUp, const bf16_t *A, int64_t r, int64_t rp,
                   bf16_t *dX, const Levels &lv, hipStream_t s, const uint8_t *mask, float q) {
  const int64_t tm = (T + C::BM - 1) / C::BM, tn = (K + C::BN - 1) / C::BN;
  int xb_m, xb_n;
  xcd_blocking(tm, tn, 2.0 * T * N, 0.516 * N * K, &xb_m, &xb_n);
  launch(k_nf4_gemm_dx<C, DROP>, dim3((unsigned)(tm * tn)), dim3(C::NT), 0, s, dY, T, N, codes, absmax_q, step, K,
         dUp, A, r, rp, dX, lv, xb_m, xb_n, mask, q);
  return hipGetLastError();
}
}  // namespace

// Split reduction of the forward GEMM: at most this many ranges, each at least this many 64-deep steps.
constexpr int kFwdMaxSplit = 16, kFwdMinSteps = 8;

// Tile choice for an M x N output.  Measured on MI355X (both GEMMs, seven
// workload shapes): the largest 8-wave tile that still yields at least one
// workgroup per CU (256 tiles) is fastest -- 256x256, else 256x128; below that
// the 8-wave 128x128 tile (two workgroups per CU) wins.
int nf4_gemm_pick_tile(int64_t M, int64_t N) {
  auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (tiles(256, 256) >= 256) return NF4_TILE_256x256_W8;
  if (tiles(256, 128) >= 256) return NF4_TILE_256x128_W8;
  // at most 128 rows over a wide output: 64x64 per wave where the 128x256 tiles still number 96 or more
  if (M <= 128 && tiles(128, 256) >= 96) return NF4_TILE_128x256_W8;
  return NF4_TILE_128x128_W8;
}

int nf4_gemm_fwd_split(int tile, int64_t T, int64_t N, int64_t K) {
  int64_t bm = 128, bn = 128;
  int per_cu = 2;  // resident workgroups per CU (the 128x128 tiles: two; the larger 8-wave tiles: one)
  if (tile == NF4_TILE_256x256_W8) bm = 256, bn = 256, per_cu = 1;
  else if (tile == NF4_TILE_256x128_W8) bm = 256, per_cu = 1;
  else if (tile == NF4_TILE_128x256_W8) bn = 256, per_cu = 1;
  const int64_t tiles = ((T + bm - 1) / bm) * ((N + bn - 1) / bn), slots = 256 * per_cu, nk = K / BK;
  int best = 1;
  for (int d = 2; d <= kFwdMaxSplit; ++d)
    if (nk % d == 0 && nk / d >= kFwdMinSteps && tiles * d <= slots) best = d;
  return best;
}

// The forward's tile: as nf4_gemm_pick_tile, except that a narrow output of a training batch (at least
// 1024 tokens; e.g. 4096 x 1024 for a grouped-query k or v projection), which would take 128x128 tiles,
// takes the 256x256 tile with its reduction split into ranges when those fill every CU.
int nf4_gemm_pick_tile_fwd(int64_t M, int64_t N, int64_t K) {
  const int t = nf4_gemm_pick_tile(M, N);
  if (t != NF4_TILE_128x128_W8 || M < 1024 || N < 256) return t;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  return tiles * nf4_gemm_fwd_split(NF4_TILE_256x256_W8, M, N, K) >= 256 ? NF4_TILE_256x256_W8 : t;
}

hipError_t launch_nf4_gemm_fwd(int tile, const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes,
                               const uint8_t *absmax_q, const float *step, int64_t N, const bf16_t *V,
                               const bf16_t *Bp, int64_t ldb, int64_t r, int64_t rp, bf16_t *Y, const Levels &lv,
                               hipStream_t s, const SegTable &sg, int nsplit, float *psum) {
  if (T == 0) return hipSuccess;
  if (nsplit < 1 || (nsplit > 1 && (!psum || K % ((int64_t)nsplit * BK) != 0))) return hipErrorInvalidValue;
  if (nsplit == 1) psum = nullptr;
#define QLORA_FWD(CFG) fwd_with<CFG>(X, T, K, codes, absmax_q, step, N, V, Bp, ldb, r, rp, Y, lv, s, sg, nsplit, psum)
  switch (tile) {
    case NF4_TILE_256x256_W8: return QLORA_FWD(T256x256w8);
    case NF4_TILE_256x128_W8: return QLORA_FWD(T256x128w8);
    case NF4_TILE_128x256_W8: return QLORA_FWD(T128x256w8);
    case NF4_TILE_128x128_W8: return QLORA_FWD(T128x128w8);
    default: return QLORA_FWD(T128x128);
  }
#undef QLORA_FWD
}

hipError_t launch_nf4_gemm_dx(int tile, const bf16_t *dY, int64_t T, int64_t N, const uint8_t *codes,
                              const uint8_t *absmax_q, const float *step, int64_t K, const bf16_t *dUp, const bf16_t *A,
                              int64_t r, int64_t rp, bf16_t *dX, const Levels &lv, hipStream_t s,
                              const uint8_t *mask, float q) {
  if (T == 0) return hipSuccess;
  if (mask) {  // dropout: the per-tile adapter epilogue needs registers that the 256x256 tile does not have
    switch (tile) {
      case NF4_TILE_256x256_W8:
      case NF4_TILE_256x128_W8:
        return dx_with<T256x128w8, true>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s, mask, q);
      case NF4_TILE_128x256_W8:
        return dx_with<T128x256w8, true>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s, mask, q);
      case NF4_TILE_128x128_W8:
        return dx_with<T128x128w8, true>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s, mask, q);
      default: return dx_with<T128x128, true>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s, mask, q);
    }
  }
  switch (tile) {
    case NF4_TILE_256x256_W8:
      return dx_with<T256x256w8, false>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s, mask, q);
    case NF4_TILE_256x128_W8:
      return dx_with<T256x128w8, false>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s, mask, q);
    case NF4_TILE_128x256_W8:
      return dx_with<T128x256w8, false>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s, mask, q);
    case NF4_TILE_128x128_W8:
      return dx_with<T128x128w8, false>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s, mask, q);
    default: return dx_with<T128x128, false>(dY, T, N, codes, absmax_q, step, K, dUp, A, r, rp, dX, lv, s, mask, q);
  }
}

}  // namespace qlora
