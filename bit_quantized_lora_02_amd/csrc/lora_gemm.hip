// lora_gemm.hip -- the skinny rank-r contractions of the LoRA branch.
//
// "QLoRA: fine-tuning a large model on one GPU" (learn.pranaymahendrakar.com),
// Researcher level, "LoRA, stated once": the adapter adds (alpha/r) B A x with
// B of shape d x r and A of shape r x k.  Its gradients (same page, "What
// QLoRA adds"; katajob.com, "What stays in full precision") are
//   U = X A^T,  dU = s dY B,  dA = dU^T X,  dB = s dY^T U.
// Every one of them has one long dimension (tokens, n_out or n_in) and a
// narrow one (the rank, r <= 128), so each is a skinny bf16 MFMA GEMM, split
// along its reduction, that writes binary32 partial sums; a finalize kernel
// then adds the splits in a fixed order (bitwise repeatable, no atomics),
// scales, and rounds to bf16 once.  U and dU of many tokens at a narrow rank
// instead reduce inside one workgroup and skip the finalize (k_lora_rows).
#include "device.h"
#include "launch.h"

namespace qlora {

// ------------------------------------------------------------- skinny GEMM
// A workgroup owns 128 rows of the long output dimension M and every rank
// column (RN = r rounded up to 16, 32, 64 or 128), and streams the large
// operand P once.  C[split][m][j] = sum over its reduction range of
// P(m, k) Q(k, j), with
//   PT = 0: P(m, k) = P[m*ldp + k]   PT = 1: P(m, k) = P[k*ldp + m]
//   QT = 0: Q(k, j) = Q[j*ldq + k]   QT = 1: Q(k, j) = Q[k*ldq + j]
// Tiles are copied global -> registers -> LDS in their natural layout
// (16-byte chunks, prefetched two 64-deep steps ahead, double-buffered LDS);
// operands whose reduction index is the row are read with ds_read_b64_tr_b16
// (lane i of a 16-lane group gets element i & 3 of the 8 bytes addressed by
// lane 4m + (i >> 2), m = 0..3).  4 waves x 32 rows, v_mfma_f32_16x16x32_bf16.
// Requirements: ldp, ldq, M (when PT = 1) and the valid Q columns Rv (when
// QT = 1) are multiples of 8; reduction extents past Kred and rows past M
// read as zero.
//
// LoRA dropout on P (DM != DROP_NONE; the adapter config of "Module 08 - QLoRA
// & Quantization" (ainiketan.in), "4. QLoRA in code", sets lora_dropout =
// 0.05).  P is then the dense layer input, and its 8-element chunk c (flat
// element index / 8 -- exactly one 16-byte load here) keeps element i iff the
// 16-bit draw i of Philox4x32-10 (Salmon et al., SC 2011) at counter
// (c, offset), key seed, is at least thr; draw i is the low (i even) or high
// half of output word i / 2.  Kept elements become bf16(fl32(x q)), dropped
// ones zero.  DROP_GENERATE draws the bits and writes them to mask[c] (every
// chunk is loaded by exactly one workgroup, once); DROP_APPLY reads them.
namespace {
typedef float f32x4s_t __attribute__((ext_vector_type(4)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4_t lds_s4_t;

__device__ __forceinline__ f32x4s_t mfma16(const u32x4_t &a, const u32x4_t &b, const f32x4s_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
// Transposing read of an 8-deep reduction run: rows row0..row0+7 of column col..
__device__ __forceinline__ u32x4_t tr_read8(const bf16_t *base, int ld, int row0, int col) {
  const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t *)(base + row0 * ld + col));
  const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t *)(base + (row0 + 4) * ld + col));
  const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{l2.x, l2.y, h2.x, h2.y};
}
constexpr int SK = 64;    // reduction step
constexpr int SBM = 128;  // rows of M per workgroup
// k-groups of four waves per workgroup, each streaming its own part of the k range (two waves per SIMD
// instead of one); rank 128 keeps one, as two would leave it 256 registers and spill
template <int RN>
constexpr int skg() {
  return RN <= 64 ? 2 : 1;
}

// Keep bits of 8-element chunk `chunk`: Philox4x32 with 10 rounds -- each round
// takes both halves of the 64-bit products of words 0 and 2 with the round
// multipliers, folds the high halves into words 1 and 3 with the key, and
// advances the key by the two Weyl increments.
__device__ __forceinline__ uint32_t keep_bits8(uint64_t chunk, const DropParams &d) {
  uint32_t x0 = (uint32_t)chunk, x1 = (uint32_t)(chunk >> 32), x2 = d.off0, x3 = d.off1;
  uint32_t k0 = d.key0, k1 = d.key1;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint32_t lo0 = 0xD2511F53u * x0, hi0 = __umulhi(0xD2511F53u, x0);
    const uint32_t lo1 = 0xCD9E8D57u * x2, hi1 = __umulhi(0xCD9E8D57u, x2);
    x0 = hi1 ^ x1 ^ k0;
    x2 = hi0 ^ x3 ^ k1;
    x1 = lo1;
    x3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  const uint32_t w[4] = {x0, x1, x2, x3};
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) bits |= (((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) >= d.thr ? 1u : 0u) << i;
  return bits;
}

// Eight bf16 values (element e in half e % 2 of word e / 2): kept ones scaled
// by q and rounded to bf16 once, dropped ones zero.
__device__ __forceinline__ u32x4_t apply_keep(const u32x4_t &v, uint32_t bits, float q) {
  u32x4_t o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float lo = ((bits >> (2 * w)) & 1u) ? __fmul_rn(bf16_lo_to_f32(v[w]), q) : 0.f;
    const float hi = ((bits >> (2 * w + 1)) & 1u) ? __fmul_rn(bf16_hi_to_f32(v[w]), q) : 0.f;
    o[w] = pack_bf16x2(lo, hi);
  }
  return o;
}
}  // namespace

// Many adapters (GR): workgroup x takes the x-th 128-row tile of the token
// segments in order (tiles never straddle a segment), with Q the segment's
// adapter Q + a q_stride (none: Rv = 0, all zero); rows past the segment read
// as zero and are not stored.
// With CT the partial sums are stored by rank column instead: C[split][j][m] (M % 4 == 0), so that a
// finalize reading them for an output [r][M] (dA) loads and stores along m.
template <bool PT, bool QT, int RN, int DM, bool GR = false, bool CT = false>
__global__ __launch_bounds__(256 * skg<RN>()) void k_skinny(const bf16_t *__restrict__ P, int64_t ldp, int64_t M,
                                                const bf16_t *__restrict__ Q, int64_t ldq, int64_t Rv, int64_t Kred,
                                                int64_t kchunk, float *__restrict__ C, DropParams dp,
                                                SegTable sg, int64_t q_stride) {
  constexpr int LDP = PT ? SBM + 16 : SK;             // LDS row length of the P tile (elements)
  constexpr int LDQ = QT ? RN + (RN >= 32 ? 16 : 0) : SK;
  constexpr int P_ROWS = PT ? SK : SBM;
  constexpr int Q_ROWS = QT ? SK : RN;
  constexpr int P_CH = SBM * SK / 8 / 256;            // 16-byte chunks of P per thread (4)
  constexpr int Q_CHUNKS = RN * SK / 8;               // 16-byte chunks of the Q tile
  constexpr int Q_CH = (Q_CHUNKS + 255) / 256;
  constexpr int NT_ = RN / 16, SKG = skg<RN>();
  // per k-group: two P and two Q buffers; after the loop group 1's region takes its accumulators
  constexpr int P_ELEMS = P_ROWS * LDP, Q_ELEMS = Q_ROWS * LDQ, G_ELEMS = 2 * (P_ELEMS + Q_ELEMS);
  static_assert(256 * 8 * NT_ * 4 <= G_ELEMS * 2, "group 1's buffers hold its accumulators");
  static_assert(P_ELEMS % 8 == 0 && Q_ELEMS % 8 == 0, "16-byte aligned buffers");
  __shared__ __attribute__((aligned(16))) bf16_t smem[SKG * G_ELEMS];
  const int kg = threadIdx.x >> 8;  // k-group
  const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6;
  bf16_t *const sPg = smem + kg * G_ELEMS, *const sQg = sPg + 2 * P_ELEMS;
  auto sP = [&](int buf) { return sPg + buf * P_ELEMS; };
  auto sQ = [&](int buf) { return sQg + buf * Q_ELEMS; };
  int64_t m0 = (int64_t)blockIdx.x * SBM, mend = M;
  if constexpr (GR) {
    int64_t b = blockIdx.x, lo = 0, hi = 0;
    int g = -1;
    for (int h = 0; h < sg.n_seg; ++h) {
      int64_t a0 = sg.seg[h], a1 = sg.seg[h + 1];
      a0 = a0 < 0 ? 0 : (a0 > M ? M : a0);
      a1 = a1 < a0 ? a0 : (a1 > M ? M : a1);
      const int64_t nt = (a1 - a0 + SBM - 1) / SBM;
      if (b < nt) {
        g = h;
        lo = a0;
        hi = a1;
        break;
      }
      b -= nt;
    }
    if (g < 0) return;  // past the last tile (the grid is an upper bound)
    m0 = lo + b * SBM;
    mend = (m0 + SBM < hi) ? m0 + SBM : hi;
    const int a = sg.ad[g];
    if (a >= 0 && a < sg.n_pool) Q += (int64_t)a * q_stride;
    else Rv = 0;
  }
  // the workgroup's k range [kb0, ke0) in steps of SK; k-group g takes steps g n .. g n + n - 1 of it
  // (n = ceil(steps / SKG)), and both groups run n iterations (a group's steps past ke0 load zeros), so that
  // they meet the same barriers
  const int64_t kb0 = (int64_t)blockIdx.y * kchunk;
  const int64_t ke0 = (kb0 + kchunk < Kred) ? kb0 + kchunk : Kred;
  const int nsteps = (int)((ke0 - kb0 + SK - 1) / SK + SKG - 1) / SKG;
  const int64_t kb = kb0 + (int64_t)kg * nsteps * SK;
  const int64_t ke = ke0;

  auto p_off = [&](int c, int &row, int &col) {  // chunk c of the P tile -> LDS (row, col)
    if (PT) { row = c >> 4; col = (c & 15) * 8; }
    else { row = c >> 3; col = (((c & 7) ^ (row & 7)) << 3); }  // swizzled 16-byte chunks
  };
  // two register slots (steps of even and odd index): the loads run two steps ahead
  u32x4_t rpA[P_CH], rqA[Q_CH], rpB[P_CH], rqB[Q_CH];
  uint32_t kmA[P_CH], kmB[P_CH];  // keep bits of the P chunks (dropout only)
  auto load = [&](int s, u32x4_t(&rp_)[P_CH], u32x4_t(&rq_)[Q_CH], uint32_t(&km_)[P_CH]) {
    const int64_t k0 = kb + (int64_t)s * SK;
#pragma unroll
    for (int i = 0; i < P_CH; ++i) {
      const int c = tid + 256 * i;
      bool ok;
      const bf16_t *src;
      if (PT) {
        const int64_t k = k0 + (c >> 4), m = m0 + (c & 15) * 8;
        ok = k < ke && m < M;
        src = P + k * ldp + m;
      } else {
        const int64_t m = m0 + (c >> 3), k = k0 + (c & 7) * 8;
        ok = m < mend && k < ke;
        src = P + m * ldp + k;
      }
      rp_[i] = ok ? *reinterpret_cast<const u32x4_t *>(src) : u32x4_t{0u, 0u, 0u, 0u};
      if constexpr (DM == DROP_APPLY) km_[i] = ok ? (uint32_t)dp.mask[(src - P) >> 3] : 0u;
      if constexpr (DM == DROP_GENERATE) {
        const int64_t chunk = (src - P) >> 3;
        km_[i] = keep_bits8((uint64_t)chunk, dp);
        if (ok) dp.mask[chunk] = (uint8_t)km_[i];
      }
    }
#pragma unroll
    for (int i = 0; i < Q_CH; ++i) {
      const int c = tid + 256 * i;
      bool ok = c < Q_CHUNKS;
      const bf16_t *src = Q;
      if (QT) {
        const int64_t k = k0 + c / (RN / 8), j = (c % (RN / 8)) * 8;
        ok = ok && k < ke && j < Rv;
        src = Q + k * ldq + j;
      } else {
        const int64_t j = c >> 3, k = k0 + (c & 7) * 8;
        ok = ok && j < Rv && k < ke;
        src = Q + j * ldq + k;
      }
      rq_[i] = ok ? *reinterpret_cast<const u32x4_t *>(src) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf, const u32x4_t(&rp_)[P_CH], const u32x4_t(&rq_)[Q_CH], const uint32_t(&km_)[P_CH]) {
#pragma unroll
    for (int i = 0; i < P_CH; ++i) {
      int row, col;
      p_off(tid + 256 * i, row, col);
      *reinterpret_cast<u32x4_t *>(&sP(buf)[row * LDP + col]) =
          (DM == DROP_NONE) ? rp_[i] : apply_keep(rp_[i], km_[i], dp.q);
    }
#pragma unroll
    for (int i = 0; i < Q_CH; ++i) {
      const int c = tid + 256 * i;
      if (c >= Q_CHUNKS) break;
      int row, col;
      if (QT) { row = c / (RN / 8); col = (c % (RN / 8)) * 8; }
      else { row = c >> 3; col = (((c & 7) ^ (row & 7)) << 3); }
      *reinterpret_cast<u32x4_t *>(&sQ(buf)[row * LDQ + col]) = rq_[i];
    }
  };

  f32x4s_t acc[2][NT_];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NT_; ++j) acc[i][j] = f32x4s_t{0.f, 0.f, 0.f, 0.f};

  const int g = lane >> 4, a = lane & 15;
  auto mma = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < SK / 32; ++kk) {
      u32x4_t pa[2], qb[NT_];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int mrow = wave * 32 + i * 16;
        if (PT) {
          pa[i] = tr_read8(sP(buf), LDP, kk * 32 + 8 * g + (a >> 2), mrow + 4 * (a & 3));
        } else {
          const int row = mrow + a, chunk = kk * 4 + g;
          pa[i] = *reinterpret_cast<const u32x4_t *>(&sP(buf)[row * LDP + ((chunk ^ (row & 7)) << 3)]);
        }
      }
#pragma unroll
      for (int j = 0; j < NT_; ++j) {
        if (QT) {
          qb[j] = tr_read8(sQ(buf), LDQ, kk * 32 + 8 * g + (a >> 2), j * 16 + 4 * (a & 3));
        } else {
          const int row = j * 16 + a, chunk = kk * 4 + g;
          qb[j] = *reinterpret_cast<const u32x4_t *>(&sQ(buf)[row * LDQ + ((chunk ^ (row & 7)) << 3)]);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT_; ++j) acc[i][j] = mfma16(pa[i], qb[j], acc[i][j]);
    }
  };

  if (nsteps > 0) {
    load(0, rpA, rqA, kmA);
    if (nsteps > 1) load(1, rpB, rqB, kmB);
    store(0, rpA, rqA, kmA);
    __syncthreads();
    for (int s = 0; s < nsteps; s += 2) {
      if (s + 2 < nsteps) load(s + 2, rpA, rqA, kmA);
      mma(0);
      if (s + 1 < nsteps) store(1, rpB, rqB, kmB);
      __syncthreads();
      if (s + 1 >= nsteps) break;
      if (s + 3 < nsteps) load(s + 3, rpB, rqB, kmB);
      mma(1);
      if (s + 2 < nsteps) store(0, rpA, rqA, kmA);
      __syncthreads();
    }
  }
  // group 1 hands its sums to group 0 through its own buffers (free after the loop's last barrier), and
  // group 0 adds them to its own: one fixed order
  if constexpr (SKG == 2) {
    f32x4s_t *xs = reinterpret_cast<f32x4s_t *>(smem + G_ELEMS);
    if (kg == 1)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT_; ++j) xs[(i * NT_ + j) * 256 + tid] = acc[i][j];
    __syncthreads();
    if (kg == 1) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NT_; ++j) {
        const f32x4s_t o = xs[(i * NT_ + j) * 256 + tid];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __fadd_rn(acc[i][j][e], o[e]);
      }
  }
  // element i of lane l of tile (mt, nt): row 16 mt + 4 (l >> 4) + i, column 16 nt + (l & 15)
  float *Cs = C + (int64_t)blockIdx.y * M * RN;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NT_; ++j) {
      const int64_t mb = m0 + wave * 32 + i * 16 + 4 * g;
      if constexpr (CT) {  // the lane's four rows are consecutive: one 16-byte store (M % 4 == 0: all or none)
        if (mb < mend) *reinterpret_cast<f32x4s_t *>(Cs + (int64_t)(j * 16 + a) * M + mb) = acc[i][j];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (mb + e < mend) Cs[(mb + e) * RN + j * 16 + a] = acc[i][j][e];
      }
    }
}

// ------------------------------------------------- whole-reduction variant
// With many rows and 16 rank columns the split reduction above spends most of
// its time in the second launch.  Here one 1024-thread workgroup owns ROWS = 8
// or 16 rows of M (8 while that still gives no more workgroups than CUs: each
// workgroup reads all of Q, so fewer rows only pay when they bring more CUs
// into play) and the whole reduction: its 16 waves take consecutive reduction ranges
// of kw columns (kw = Kred / 16 rounded up to 32), load their operands straight
// from global memory in the MFMA layout (lane (a, g) = (l & 15, l >> 4) holds
// row a, columns 8 g .. 8 g + 7 of a 32-deep step; with ROWS = 8 the lanes of
// rows 8..15 load nothing and their MFMA rows are discarded: P needs PT = 0; Q with
// QT = 0 likewise; with QT = 1 a wave copies its 32 x RN slice of Q into its own
// LDS slot and reads it back transposed), eight steps at a time, and run
// v_mfma_f32_16x16x32_bf16.  The 16 waves' binary32 results are then added in
// wave order through LDS, and the workgroup writes the finalize outputs
// itself: out1[m ld1 + n] = bf16(scale1 S) for n < n1, out2[m ld2 + n] =
// n < nvalid2 ? bf16(scale2 S) : 0 for n < n2 (S = 0 for n >= RN).  Same
// requirements as k_skinny (Kred, ldp, ldq and, for QT = 1, Rv multiples of 8).
constexpr int kRowsRN = 16, kRowsMinM = 1024;  // where it is faster (measured: 16 rank columns, >= 1024 rows)
template <bool QT, int RN, int ROWS>
__global__ __launch_bounds__(1024) void k_lora_rows(const bf16_t *__restrict__ P, int64_t ldp, int64_t M,
                                                    const bf16_t *__restrict__ Q, int64_t ldq, int64_t Rv, int64_t Kred,
                                                    bf16_t *__restrict__ out1, int64_t ld1, int64_t n1, float scale1,
                                                    bf16_t *__restrict__ out2, int64_t ld2, int64_t n2, int64_t nvalid2,
                                                    float scale2) {
  constexpr int NWV = 16, NT_ = RN / 16, D = 8;
  constexpr int LDQ = RN + (RN >= 32 ? 16 : 0);
  constexpr int QCH = QT ? RN / 16 : NT_;  // per lane and step: 16-byte chunks of the Q slice (QT) or operands
  __shared__ __attribute__((aligned(16))) float sRed[NWV][16][RN];
  __shared__ __attribute__((aligned(16))) bf16_t sQ[QT ? NWV : 1][QT ? 32 * LDQ : 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, a = lane & 15;
  const int64_t m0 = (int64_t)blockIdx.x * ROWS;
  const int64_t kw = ((Kred + NWV - 1) / NWV + 31) / 32 * 32;
  const int64_t kb = wave * kw, ke = (kb + kw < Kred) ? kb + kw : Kred;
  const int nst = ke > kb ? (int)((ke - kb + 31) / 32) : 0;
  f32x4s_t acc[NT_];
#pragma unroll
  for (int j = 0; j < NT_; ++j) acc[j] = f32x4s_t{0.f, 0.f, 0.f, 0.f};
  const bool prow = a < ROWS && m0 + a < M;
  const bf16_t *pp = P + (prow ? m0 + a : 0) * ldp + 8 * g;
  for (int s0 = 0; s0 < nst; s0 += D) {
    u32x4_t pa[D], qr[D][QCH];
#pragma unroll
    for (int d = 0; d < D; ++d) {  // every load of the D steps first (columns past ke read as zero)
      const int64_t k0 = kb + (int64_t)(s0 + d) * 32;
      pa[d] = (prow && k0 + 8 * g < ke) ? *reinterpret_cast<const u32x4_t *>(pp + k0) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < QCH; ++i) {
        bool ok;
        const bf16_t *src;
        if constexpr (QT) {
          const int c = lane + 64 * i, row = c / (RN / 8), col = (c % (RN / 8)) * 8;
          ok = k0 + row < ke && col < Rv;
          src = Q + (k0 + row) * ldq + col;
        } else {
          const int64_t col = i * 16 + a;
          ok = col < Rv && k0 + 8 * g < ke;
          src = Q + col * ldq + k0 + 8 * g;
        }
        qr[d][i] = ok ? *reinterpret_cast<const u32x4_t *>(src) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      u32x4_t qb[NT_];
      if constexpr (QT) {
        bf16_t *sq = sQ[QT ? wave : 0];  // this wave's slot: written and read by this wave only
#pragma unroll
        for (int i = 0; i < QCH; ++i) {
          const int c = lane + 64 * i, row = c / (RN / 8), col = (c % (RN / 8)) * 8;
          *reinterpret_cast<u32x4_t *>(sq + row * LDQ + col) = qr[d][i];
        }
#pragma unroll
        for (int j = 0; j < NT_; ++j) qb[j] = tr_read8(sq, LDQ, 8 * g + (a >> 2), j * 16 + 4 * (a & 3));
      } else {
#pragma unroll
        for (int j = 0; j < NT_; ++j) qb[j] = qr[d][j];
      }
#pragma unroll
      for (int j = 0; j < NT_; ++j) acc[j] = mfma16(pa[d], qb[j], acc[j]);
    }
  }
  // element e of lane l of column tile j: row 4 (l >> 4) + e, column 16 j + (l & 15)
#pragma unroll
  for (int j = 0; j < NT_; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) sRed[wave][4 * g + e][j * 16 + a] = acc[j][e];
  __syncthreads();
  const int64_t ncol = n1 > n2 ? n1 : n2;
  for (int64_t idx = tid; idx < ROWS * ncol; idx += 1024) {
    const int m = (int)(idx / ncol);
    const int64_t n = idx - m * ncol;
    if (m0 + m >= M) continue;
    float sum = 0.f;
    if (n < RN)
#pragma unroll
      for (int w = 0; w < NWV; ++w) sum += sRed[w][m][n];
    if (out1 && n < n1) out1[(m0 + m) * ld1 + n] = f32_to_bf16(scale1 * sum);
    if (out2 && n < n2) out2[(m0 + m) * ld2 + n] = (n < nvalid2) ? f32_to_bf16(scale2 * sum) : (bf16_t)0;
  }
}

// One finalize job: S = sum over splits p = 0 .. nsplit-1 (in that order) of
// part[p sstride + m N + n], then
//   out1[m*ld1 + n] = bf16(scale1 * S) for n < n1,
//   out2[m*ld2 + n] = n < nvalid2 ? bf16(scale2 * S) : 0 for n < n2.
struct FinJob {
  const float *part;
  int nsplit;
  int64_t M, N, sstride;
  bf16_t *out1;
  int64_t ld1, n1;
  float scale1, scale2;
  bf16_t *out2;
  int64_t ld2, n2, nvalid2;
  int64_t nblocks;  // 256-thread blocks of this job
  int vec;          // 1: four consecutive columns per thread (16-byte loads; see fin_job)
};

__device__ __forceinline__ void finalize_one(const FinJob &j, int64_t i) {
  const int64_t ncol = (j.n1 > j.n2) ? j.n1 : j.n2;
  if (i >= j.M * ncol) return;
  const int64_t m = i / ncol, n = i - m * ncol;
  float sum = 0.f;
  if (n < j.N) {
    // all loads first, then the additions in split order
    const float *src = j.part + m * j.N + n;
    const int64_t stride = j.sstride;
    int p = 0;
    for (; p + 8 <= j.nsplit; p += 8) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = src[(int64_t)(p + q) * stride];
#pragma unroll
      for (int q = 0; q < 8; ++q) sum += v[q];
    }
    for (; p < j.nsplit; ++p) sum += src[(int64_t)p * stride];
  }
  if (j.out1 && n < j.n1) j.out1[m * j.ld1 + n] = f32_to_bf16(j.scale1 * sum);
  if (j.out2 && n < j.n2) j.out2[m * j.ld2 + n] = (n < j.nvalid2) ? f32_to_bf16(j.scale2 * sum) : (bf16_t)0;
}

// Four consecutive columns n .. n + 3 of one row (n % 4 == 0): the same sums in the same order as
// finalize_one, with 16-byte loads of the partials and 8-byte stores.  Index math in 32 bits (the host
// takes this form only when M ncol < 2^31).
__device__ __forceinline__ void finalize_vec(const FinJob &j, int64_t i4) {
  const uint32_t ncol4 = (uint32_t)(((j.n1 > j.n2) ? j.n1 : j.n2) / 4);
  if (i4 >= (int64_t)j.M * ncol4) return;
  const uint32_t m = (uint32_t)i4 / ncol4, n = ((uint32_t)i4 - m * ncol4) * 4;
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
  if (n < j.N) {
    const float *src = j.part + (int64_t)m * j.N + n;
    const int64_t stride = j.sstride;
    int p = 0;
    for (; p + 4 <= j.nsplit; p += 4) {
      f32x4s_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4s_t *>(src + (int64_t)(p + q) * stride);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[e] += v[q][e];
    }
    for (; p < j.nsplit; ++p) {
      const f32x4s_t v = *reinterpret_cast<const f32x4s_t *>(src + (int64_t)p * stride);
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += v[e];
    }
  }
  if (j.out1 && n < j.n1) {
    bf16_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(j.scale1 * sum[e]);
    *reinterpret_cast<u32x2_t *>(j.out1 + (int64_t)m * j.ld1 + n) =
        u32x2_t{(uint32_t)o[0] | (uint32_t)o[1] << 16, (uint32_t)o[2] | (uint32_t)o[3] << 16};
  }
  if (j.out2 && n < j.n2) {
    bf16_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (n + e < j.nvalid2) ? f32_to_bf16(j.scale2 * sum[e]) : (bf16_t)0;
    *reinterpret_cast<u32x2_t *>(j.out2 + (int64_t)m * j.ld2 + n) =
        u32x2_t{(uint32_t)o[0] | (uint32_t)o[1] << 16, (uint32_t)o[2] | (uint32_t)o[3] << 16};
  }
}

// Blocks [0, a.nblocks) run job a, the rest job b (two independent outputs in one launch).
__global__ __launch_bounds__(256) void k_finalize(FinJob a, FinJob b) {
  const int64_t blk = blockIdx.x;
  const FinJob &j = blk < a.nblocks ? a : b;
  const int64_t i = (blk < a.nblocks ? blk : blk - a.nblocks) * 256 + threadIdx.x;
  if (j.vec) finalize_vec(j, i);
  else finalize_one(j, i);
}

// out[m*ldo + n] = n < ncols ? in[m*ldi + n] : 0, for n < ldo (zero-padded copy).
__global__ __launch_bounds__(256) void k_pad_copy(const bf16_t *__restrict__ in, int64_t ldi, int64_t ncols, int64_t M,
                                                  bf16_t *__restrict__ out, int64_t ldo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * ldo) return;
  const int64_t m = i / ldo, n = i - m * ldo;
  out[i] = (n < ncols) ? in[m * ldi + n] : (bf16_t)0;
}

namespace {
FinJob fin_job(const float *part, int nsplit, int64_t M, int64_t N, bf16_t *out1, int64_t ld1, int64_t n1,
               float scale1, bf16_t *out2, int64_t ld2, int64_t n2, int64_t nvalid2, float scale2, int64_t sstride) {
  FinJob j;
  j.part = part;
  j.nsplit = nsplit;
  j.M = M;
  j.N = N;
  j.sstride = sstride > 0 ? sstride : M * N;
  j.out1 = out1;
  j.ld1 = ld1;
  j.n1 = n1;
  j.scale1 = scale1;
  j.out2 = out2;
  j.ld2 = ld2;
  j.n2 = n2;
  j.nvalid2 = nvalid2;
  j.scale2 = scale2;
  const int64_t ncol = (n1 > n2) ? n1 : n2;
  // four columns per thread when every group of four lies within [0, N), [0, n1) or [0, n2) or outside
  // them, and the partials and outputs are aligned for 16- and 8-byte accesses
  auto al = [](const void *ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; };
  j.vec = ncol % 4 == 0 && N % 4 == 0 && j.sstride % 4 == 0 && n1 % 4 == 0 && n2 % 4 == 0 && al(part, 16) &&
          (!out1 || (ld1 % 4 == 0 && al(out1, 8))) && (!out2 || (ld2 % 4 == 0 && al(out2, 8))) &&
          M * ncol < ((int64_t)1 << 31);
  j.nblocks = j.vec ? (M * (ncol / 4) + 255) / 256 : (M * ncol + 255) / 256;
  return j;
}
}  // namespace

hipError_t launch_finalize(const float *part, int nsplit, int64_t M, int64_t N, bf16_t *out1, int64_t ld1, int64_t n1,
                           float scale1, bf16_t *out2, int64_t ld2, int64_t n2, int64_t nvalid2, float scale2,
                           hipStream_t s) {
  const FinJob a = fin_job(part, nsplit, M, N, out1, ld1, n1, scale1, out2, ld2, n2, nvalid2, scale2, 0);
  if (a.nblocks == 0) return hipSuccess;
  FinJob none = a;
  none.nblocks = 0;
  launch(k_finalize, dim3((unsigned)a.nblocks), dim3(256), 0, s, a, none);
  return hipGetLastError();
}

hipError_t launch_finalize_pair(const float *part_a, int nsplit_a, int64_t M_a, int64_t N_a, bf16_t *out_a,
                                int64_t ld_a, int64_t n_a, float scale_a, const float *part_b, int nsplit_b,
                                int64_t M_b, int64_t N_b, int64_t sstride_b, bf16_t *out_b, int64_t ld_b, int64_t n_b,
                                float scale_b, hipStream_t s) {
  const FinJob a = fin_job(part_a, nsplit_a, M_a, N_a, out_a, ld_a, n_a, scale_a, nullptr, 0, 0, 0, 0.f, 0);
  const FinJob b = fin_job(part_b, nsplit_b, M_b, N_b, out_b, ld_b, n_b, scale_b, nullptr, 0, 0, 0, 0.f, sstride_b);
  if (a.nblocks + b.nblocks == 0) return hipSuccess;
  launch(k_finalize, dim3((unsigned)(a.nblocks + b.nblocks)), dim3(256), 0, s, a, b);
  return hipGetLastError();
}

bool lora_rows_ok(int rn, int64_t M) { return rn == kRowsRN && M >= kRowsMinM; }

hipError_t launch_lora_rows(bool qt, int rn, const bf16_t *P, int64_t ldp, int64_t M, const bf16_t *Q, int64_t ldq,
                            int64_t Rv, int64_t Kred, bf16_t *out1, int64_t ld1, int64_t n1, float scale1,
                            bf16_t *out2, int64_t ld2, int64_t n2, int64_t nvalid2, float scale2, hipStream_t s) {
  if (rn != kRowsRN) return hipErrorInvalidValue;
  if (M == 0) return hipSuccess;
  static thread_local int cus = 0;
  if (cus <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return hipErrorInvalidDevice;
  }
  const bool r8 = (M + 7) / 8 <= cus;  // measured: 8 rows up to one workgroup per CU (T = 2048: 8.9 / 7.4 us
                                       // for U / dU against 10.7 / 9.2 with 16), 16 beyond (T = 4096)
#define QLORA_LROWS(QT_, ROWS_)                                                                                 \
  launch((k_lora_rows<QT_, kRowsRN, ROWS_>), dim3((unsigned)((M + ROWS_ - 1) / ROWS_)), dim3(1024), 0, s, P, ldp, \
         M, Q, ldq, Rv, Kred, out1, ld1, n1, scale1, out2, ld2, n2, nvalid2, scale2)
  if (qt) { if (r8) QLORA_LROWS(true, 8); else QLORA_LROWS(true, 16); }
  else { if (r8) QLORA_LROWS(false, 8); else QLORA_LROWS(false, 16); }
#undef QLORA_LROWS
  return hipGetLastError();
}

// Rank columns held by a skinny-GEMM workgroup for rank r.
int skinny_rn(int64_t r) { return r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : 128; }

// Split of the reduction for a skinny GEMM with M output rows: aim at ~256
// workgroups (one per CU) with at least two 64-deep steps each.  Every range
// writes M x RN binary32 partial sums that the finalize reads back, so fewer
// ranges cut that traffic; measured against ~1024 workgroups (70B-class layer
// at r = 64: 14.30 -> 14.14 ms per step; 8B MLP 3.300 -> 3.230 ms).
void skinny_plan(int64_t M, int64_t Kred, int *nsplit, int64_t *kchunk) {
  const int64_t tiles = (M + SBM - 1) / SBM;
  int64_t ns = (256 + tiles - 1) / tiles;
  const int64_t by_depth = Kred / 128 > 0 ? Kred / 128 : 1;
  if (ns > by_depth) ns = by_depth;
  if (ns > 32) ns = 32;  // bounds the binary32 partials (workspace) at 32 T r
  if (ns < 1) ns = 1;
  int64_t kc = (Kred + ns - 1) / ns;
  kc = (kc + SK - 1) / SK * SK;
  *kchunk = kc > 0 ? kc : SK;
  *nsplit = Kred > 0 ? (int)((Kred + *kchunk - 1) / *kchunk) : 0;
}

// Split of the grouped (many-adapter) U pass: the grid has up to tiles + n_seg
// row tiles, most of them partly filled, so the split aims at ~1024 workgroups
// over those, and never exceeds the split of the plain plan (whose partial sums
// the workspace holds).
void skinny_plan_grouped(int64_t M, int64_t n_seg, int64_t Kred, int *nsplit, int64_t *kchunk) {
  int ns_max;
  int64_t kc_max;
  skinny_plan(M, Kred, &ns_max, &kc_max);
  const int64_t tiles = (M + SBM - 1) / SBM + n_seg;
  int64_t ns = (1024 + tiles - 1) / tiles;
  if (ns > ns_max) ns = ns_max;
  if (ns < 1) ns = 1;
  int64_t kc = (Kred + ns - 1) / ns;
  kc = (kc + SK - 1) / SK * SK;
  if (kc < kc_max) kc = kc_max;  // never more ranges than the plain plan
  *kchunk = kc > 0 ? kc : SK;
  *nsplit = Kred > 0 ? (int)((Kred + *kchunk - 1) / *kchunk) : 0;
}

template <bool PT, bool QT, int DM, bool CT = false>
static hipError_t skinny_dispatch(int rn, dim3 grid, hipStream_t s, const bf16_t *P, int64_t ldp, int64_t M,
                                  const bf16_t *Q, int64_t ldq, int64_t Rv, int64_t Kred, int64_t kchunk, float *C,
                                  const DropParams &dp) {
  const SegTable none;
  switch (rn) {
    case 16: launch((k_skinny<PT, QT, 16, DM, false, CT>), grid, dim3(256 * skg<16>()), 0, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp, none, (int64_t)0); break;
    case 32: launch((k_skinny<PT, QT, 32, DM, false, CT>), grid, dim3(256 * skg<32>()), 0, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp, none, (int64_t)0); break;
    case 64: launch((k_skinny<PT, QT, 64, DM, false, CT>), grid, dim3(256 * skg<64>()), 0, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp, none, (int64_t)0); break;
    default: launch((k_skinny<PT, QT, 128, DM, false, CT>), grid, dim3(256 * skg<128>()), 0, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp, none, (int64_t)0); break;
  }
  return hipGetLastError();
}

hipError_t launch_skinny(bool pt, bool qt, int rn, const bf16_t *P, int64_t ldp, int64_t M, const bf16_t *Q,
                         int64_t ldq, int64_t Rv, int64_t Kred, int64_t kchunk, int nsplit, float *C, hipStream_t s,
                         int drop, const DropParams &dp, bool ct) {
  if (M == 0 || nsplit == 0) return hipSuccess;
  dim3 grid((unsigned)((M + SBM - 1) / SBM), (unsigned)nsplit);
  if (ct && !(pt && qt)) return hipErrorInvalidValue;  // stored by rank column only for dA^T = X^T dU
  if (ct && drop == DROP_APPLY)
    return skinny_dispatch<true, true, DROP_APPLY, true>(rn, grid, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp);
  if (ct && drop == DROP_NONE)
    return skinny_dispatch<true, true, DROP_NONE, true>(rn, grid, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp);
  // dropout applies to the layer input: U = Xd A^T (P = X by rows) and dA^T = Xd^T dU (P = X by columns)
  if (drop == DROP_GENERATE && !pt && !qt)
    return skinny_dispatch<false, false, DROP_GENERATE>(rn, grid, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp);
  if (drop == DROP_APPLY && !pt && !qt)
    return skinny_dispatch<false, false, DROP_APPLY>(rn, grid, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp);
  if (drop == DROP_APPLY && pt && qt)
    return skinny_dispatch<true, true, DROP_APPLY>(rn, grid, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp);
  if (drop != DROP_NONE) return hipErrorInvalidValue;
  if (!pt && !qt) return skinny_dispatch<false, false, DROP_NONE>(rn, grid, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp);
  if (!pt && qt) return skinny_dispatch<false, true, DROP_NONE>(rn, grid, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp);
  if (pt && !qt) return skinny_dispatch<true, false, DROP_NONE>(rn, grid, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp);
  return skinny_dispatch<true, true, DROP_NONE>(rn, grid, s, P, ldp, M, Q, ldq, Rv, Kred, kchunk, C, dp);
}

hipError_t launch_skinny_grouped(int rn, const bf16_t *P, int64_t ldp, int64_t M, const bf16_t *Q_pool, int64_t ldq,
                                 int64_t q_stride, int64_t Rv, int64_t Kred, int64_t kchunk, int nsplit,
                                 const SegTable &sg, float *C, hipStream_t s) {
  if (M == 0 || nsplit == 0 || sg.n_seg == 0) return hipSuccess;
  const dim3 grid((unsigned)((M + SBM - 1) / SBM + sg.n_seg), (unsigned)nsplit);  // tiles of all segments, at most
  const DropParams dp;
  switch (rn) {
    case 16:
      launch((k_skinny<false, false, 16, DROP_NONE, true>), grid, dim3(256 * skg<16>()), 0, s, P, ldp, M, Q_pool, ldq, Rv, Kred,
             kchunk, C, dp, sg, q_stride);
      break;
    case 32:
      launch((k_skinny<false, false, 32, DROP_NONE, true>), grid, dim3(256 * skg<32>()), 0, s, P, ldp, M, Q_pool, ldq, Rv, Kred,
             kchunk, C, dp, sg, q_stride);
      break;
    case 64:
      launch((k_skinny<false, false, 64, DROP_NONE, true>), grid, dim3(256 * skg<64>()), 0, s, P, ldp, M, Q_pool, ldq, Rv, Kred,
             kchunk, C, dp, sg, q_stride);
      break;
    default:
      launch((k_skinny<false, false, 128, DROP_NONE, true>), grid, dim3(256 * skg<128>()), 0, s, P, ldp, M, Q_pool, ldq, Rv, Kred,
             kchunk, C, dp, sg, q_stride);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_pad_copy(const bf16_t *in, int64_t ldi, int64_t ncols, int64_t M, bf16_t *out, int64_t ldo,
                           hipStream_t s) {
  const int64_t total = M * ldo;
  if (total == 0) return hipSuccess;
  launch(k_pad_copy, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, in, ldi, ncols, M, out, ldo);
  return hipGetLastError();
}

}  // namespace qlora
