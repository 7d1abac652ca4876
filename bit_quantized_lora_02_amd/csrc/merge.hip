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
// 2 or 4 B written; B is re-read from L2).  The output is cut into stripes of
// 256 columns and bands of 32 rows; each stripe gets g workgroups of four
// waves, which split its bands (g from the resident-workgroup count), and wave
// w owns columns 64 w .. 64 w + 63 of the stripe.  A wave forms the A operands
// of its 64 columns once (transposing LDS reads) and keeps them in registers;
// per band it needs only the B rows (straight from global memory into the MFMA
// operand) and the base values, both loaded one band ahead, and it never waits
// for the other waves.  The MFMA runs with the A block as its first operand,
// which leaves lane l holding P for row l % 32 at columns 8 j + 4 (l / 32) +
// 0..3, j = 0..7: the lane loads that row's 32 code bytes (two 16-byte loads;
// the two lanes of a row share them), decodes the 2 bytes of each of its runs
// through the level-pair table and adds s P.  No P goes through LDS; the bf16
// results do, once, so that a store instruction writes 128 contiguous bytes of
// each of 8 rows (8-byte runs per lane stored directly took twice as long);
// binary32 results are stored directly as 16-byte runs.  All output stores are
// nontemporal: kept out of the caches, the written stream no longer evicts the
// code lines the other waves are reading (a merge of 8192 x 28672 spent about
// as long again on reads as on writes with ordinary stores).
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {
constexpr int TM = 32;        // output rows per tile
constexpr int TK = 256;       // output columns per tile
constexpr int WK = 64;        // columns per wave
constexpr int LDA = WK + 32;  // A slot pitch (elements): a half-wave's transposing reads cover 256 distinct bytes
constexpr int LDO = WK + 8;   // bf16 output staging pitch (elements; rows 16-byte aligned)
template <int RP>
constexpr int piece_ranks() {  // the A block goes through LDS in pieces of at most 32 ranks
  return RP < 32 ? RP : 32;
}
template <int RP>
constexpr int slot_elems() {  // a wave's LDS slot: an A piece, later the bf16 outputs of a tile
  return piece_ranks<RP>() * LDA > TM * LDO ? piece_ranks<RP>() * LDA : TM * LDO;
}

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

// What a wave loads one tile ahead: the B operand of its band (rank step kk: B[n][16 kk + 8 (l / 32) ..];
// for odd ranks it is loaded element by element when used instead) and its base values: the row's 32 code bytes and raw block constant, or the lane's eight 4-element
// bf16 runs.
template <int RP, bool NF4, bool AL>
struct MergeSlot {
  u32x4_t b[AL ? RP / 16 : 1];
  u32x4_t c[NF4 ? 2 : 1];
  RawScale sc;
  u32x2_t w[NF4 ? 1 : 8];
};

// Outputs written: bf16, binary32 or both (a compile-time choice, so that no store sits in a branch).
enum { OUT_BF16 = 1, OUT_F32 = 2 };
}  // namespace

template <int RP>
constexpr int merge_minw() {  // waves per SIMD the registers must allow
  return RP <= 32 ? 4 : RP <= 64 ? 3 : 2;
}

// Every load and store of the tile loop is unconditional: a memory operation in a branch leaves the
// compiler unsure how many are in flight, and it then waits for all of them (the previous tile's stores
// included) before using the prefetched slot.  So rows past N and a wave's columns past K are clamped to
// the last row and the last 64-column block: those lanes and waves recompute, and store again, exactly
// the values the last row or block gets anyway; rank padding is loaded from a clamped index and zeroed
// by a select.  AL: r % 8 == 0, so that B rows are 16-byte aligned.
template <int RP, bool NF4, bool AL, int OUT>
__global__ __launch_bounds__(256, (merge_minw<RP>())) void k_merge(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ absmax_q, const float *__restrict__ step,
    const bf16_t *__restrict__ W_base, int64_t N, int64_t K, const bf16_t *__restrict__ A,
    const bf16_t *__restrict__ B, int r, float s, bf16_t *__restrict__ out, float *__restrict__ out_f32, int g,
    Levels lv) {
  constexpr int PR = piece_ranks<RP>();
  __shared__ __attribute__((aligned(1024))) float2 s_tab[256];
  __shared__ __attribute__((aligned(16))) bf16_t s_a[4][slot_elems<RP>()];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup x: column stripe x / g, its bands [b0, b1) (the g workgroups of a stripe share its bands)
  const int64_t nbands = (N + TM - 1) / TM, stripe = blockIdx.x / g, part = blockIdx.x % g;
  const int64_t b0 = part * nbands / g, b1 = (part + 1) * nbands / g;
  if (b0 >= b1) return;
  pair_levels_to_lds(lv, s_tab, tid);
  __syncthreads();
  bf16_t *sa = s_a[wave];  // [PR][LDA]: a piece of the A block, ranks x columns; then [TM][LDO]: outputs
  const int grp = lane >> 4, ai = lane & 15, half = lane >> 5;
  const uint32_t nl = lane & 31;  // the lane's row within the band
  // indexes in 32 bits where they fit (N, K <= 2^22, r <= 128): one 64-bit product per address
  const uint32_t Ku = (uint32_t)K, Nu = (uint32_t)N, ru = (uint32_t)r;
  const uint32_t k0 = (uint32_t)(stripe * TK + wave * WK < K ? stripe * TK + wave * WK : K - WK);  // past K: the last block
  auto clamp_row = [&](uint32_t n) { return n < Nu ? n : Nu - 1; };

  typedef MergeSlot<RP, NF4, AL> Slot;
  auto load_b_odd = [&](u32x4_t &b, uint32_t n, int kk) {  // odd ranks: B rows element by element
    const int j0 = kk * 16 + 8 * half;
    uint32_t h[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t v = B[n * ru + (j0 + q < r ? j0 + q : r - 1)];
      h[q] = j0 + q < r ? v : 0u;
    }
    b = u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
  };
  auto load_slot = [&](Slot &sl, int64_t band) {
    const uint32_t n = clamp_row((uint32_t)band * TM + nl);
    if constexpr (AL) {
#pragma unroll
      for (int kk = 0; kk < RP / 16; ++kk) {
        const int j0 = kk * 16 + 8 * half;  // rank padding (j0 >= r) is zeroed where it is used
        sl.b[kk] = *reinterpret_cast<const u32x4_t *>(B + n * ru + (j0 < r ? j0 : r - 8));
      }
    }
    const uint64_t e0 = (uint64_t)n * Ku + k0;  // the row's first column in this block (a multiple of 64)
    if constexpr (NF4) {
      sl.c[0] = *reinterpret_cast<const u32x4_t *>(codes + e0 / 2);
      sl.c[1] = *reinterpret_cast<const u32x4_t *>(codes + e0 / 2 + 16);
      sl.sc = load_scale(absmax_q, step, e0 / 64);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) sl.w[j] = *reinterpret_cast<const u32x2_t *>(W_base + e0 + 8 * j + 4 * half);
    }
  };

  // MFMA first operand (the A block): aop[kk][h] = A[16 kk + 8 (l / 32) ..][k0 + 32 h + l % 32]
  u32x4_t aop[RP / 16][2];
  auto load_aop = [&]() {
#pragma unroll
    for (int pc = 0; pc < RP / PR; ++pc) {  // ranks PR pc ..: through the wave's LDS slot
#pragma unroll
      for (int i = 0; i < PR / 8; ++i) {
        const int c = lane + 64 * i, j = pc * PR + (c >> 3), col = (c & 7) * 8;
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(A + (uint32_t)(j < r ? j : r - 1) * Ku + k0 + col);
        *reinterpret_cast<u32x4_t *>(sa + (c >> 3) * LDA + col) = j < r ? v : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int kk = 0; kk < PR / 16; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          aop[pc * (PR / 16) + kk][h] =
              read_tr8(sa, LDA, kk * 16 + 8 * (grp >> 1) + (ai >> 2), h * 32 + 16 * (grp & 1) + 4 * (ai & 3));
    }
  };

  auto do_tile = [&](Slot &cur, Slot &nxt, int64_t band) {
    load_slot(nxt, band + 1 < b1 ? band + 1 : b1 - 1);  // the last band's prefetch reloads it, unused
    // the prefetch is issued before this tile's stores: a load issued after a store completes after it,
    // so waiting for such a load would wait for the store
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t n0 = (uint32_t)band * TM;
    // the zeroing of rank padding stays here: placed next to the prefetch, it would wait for the prefetch
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t b[RP / 16];
#pragma unroll
    for (int kk = 0; kk < RP / 16; ++kk) {
      if constexpr (AL) {
        const bool pad = kk * 16 + 8 * half >= r;
        b[kk] = pad ? u32x4_t{0u, 0u, 0u, 0u} : cur.b[kk];
      } else {
        load_b_odd(b[kk], clamp_row(n0 + nl), kk);
      }
    }
    f32x16_t acc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < RP / 16; ++kk) acc[h] = mfma_32x32x16(aop[kk][h], b[kk], acc[h]);
    }
    // acc[h][4 q + i] = P[n0 + l % 32][k0 + 8 j + 4 (l / 32) + i], j = 4 h + q
    const uint32_t n = clamp_row(n0 + nl);
    const float cq = NF4 ? scale_of(cur.sc) : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t w01, w23;  // the run's base values as bf16 pairs: bf16(level * c') for the NF4 base
      if constexpr (NF4) {
        const uint32_t cw = cur.c[j >> 2][j & 3] >> (16 * half);  // its two code bytes
        const float2 l0 = s_tab[cw & 0xffu], l1 = s_tab[(cw >> 8) & 0xffu];
        w01 = pack_bf16x2(__fmul_rn(l0.x, cq), __fmul_rn(l0.y, cq));
        w23 = pack_bf16x2(__fmul_rn(l1.x, cq), __fmul_rn(l1.y, cq));
      } else {
        w01 = cur.w[j].x;
        w23 = cur.w[j].y;
      }
      const f32x16_t &a = acc[j >> 2];
      const int q = 4 * (j & 3);
      const float m0 = __fadd_rn(bf16_lo_to_f32(w01), __fmul_rn(s, a[q]));
      const float m1 = __fadd_rn(bf16_hi_to_f32(w01), __fmul_rn(s, a[q + 1]));
      const float m2 = __fadd_rn(bf16_lo_to_f32(w23), __fmul_rn(s, a[q + 2]));
      const float m3 = __fadd_rn(bf16_hi_to_f32(w23), __fmul_rn(s, a[q + 3]));
      if constexpr ((OUT & OUT_BF16) != 0)
        *reinterpret_cast<u32x2_t *>(sa + nl * LDO + 8 * j + 4 * half) = u32x2_t{pack_bf16x2(m0, m1), pack_bf16x2(m2, m3)};
      if constexpr ((OUT & OUT_F32) != 0)
        __builtin_nontemporal_store(u32x4_t{__builtin_bit_cast(uint32_t, m0), __builtin_bit_cast(uint32_t, m1),
                                            __builtin_bit_cast(uint32_t, m2), __builtin_bit_cast(uint32_t, m3)},
                                    reinterpret_cast<u32x4_t *>(out_f32 + ((uint64_t)n * Ku + k0 + 8 * j + 4 * half)));
    }
    if constexpr ((OUT & OUT_BF16) != 0) {  // back in rows of 8 lanes: 128 contiguous bytes per row and store
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (lane >> 3) + 8 * i, col = 8 * (lane & 7);
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(sa + row * LDO + col);
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(out + ((uint64_t)clamp_row(n0 + row) * Ku + k0 + col)));
      }
    }
  };

  Slot s0, s1;
  load_slot(s0, b0);
  load_aop();
  int64_t band = b0;
  for (; band + 1 < b1; band += 2) {
    do_tile(s0, s1, band);
    do_tile(s1, s0, band + 1);
  }
  if (band < b1) do_tile(s0, s1, band);
}

template <int RP, bool NF4, bool AL, int OUT>
static hipError_t merge_go(const uint8_t *codes, const uint8_t *absmax_q, const float *step, const bf16_t *W_base,
                           int64_t N, int64_t K, const bf16_t *A, const bf16_t *B, int r, float s, bf16_t *out,
                           float *out_f32, const Levels &lv, hipStream_t st) {
  static thread_local int res = 0;  // workgroups resident at once, per variant and host thread
  if (res <= 0) res = resident(k_merge<RP, NF4, AL, OUT>, 256);
  if (res <= 0) return hipErrorInvalidDeviceFunction;
  // every stripe of 256 columns gets g workgroups (at least one), which split its bands of 32 rows
  const int64_t stripes = (K + TK - 1) / TK, nbands = (N + TM - 1) / TM;
  int64_t g = res / stripes;
  g = g < 1 ? 1 : g > nbands ? nbands : g;
  const dim3 grid((unsigned)(stripes * g));
  launch(k_merge<RP, NF4, AL, OUT>, grid, dim3(256), 0, st, codes, absmax_q, step, W_base, N, K, A, B, r, s, out,
         out_f32, (int)g, lv);
  return hipGetLastError();
}

hipError_t launch_merge(const uint8_t *codes, const uint8_t *absmax_q, const float *step, const bf16_t *W_base,
                        int64_t N, int64_t K, const bf16_t *A, const bf16_t *B, int r, float s, bf16_t *out,
                        float *out_f32, const Levels &lv, hipStream_t st) {
  if (N == 0 || K == 0) return hipSuccess;
  if (K % WK != 0 || r < 1 || (!out && !out_f32)) return hipErrorInvalidValue;
  auto go = [&](auto rp, auto nf4, auto al) -> hipError_t {
    constexpr int RP = decltype(rp)::value;
    constexpr bool NF4 = decltype(nf4)::value, AL = decltype(al)::value;
    if (out && out_f32)
      return merge_go<RP, NF4, AL, OUT_BF16 | OUT_F32>(codes, absmax_q, step, W_base, N, K, A, B, r, s, out, out_f32,
                                                        lv, st);
    if (out) return merge_go<RP, NF4, AL, OUT_BF16>(codes, absmax_q, step, W_base, N, K, A, B, r, s, out, out_f32, lv, st);
    return merge_go<RP, NF4, AL, OUT_F32>(codes, absmax_q, step, W_base, N, K, A, B, r, s, out, out_f32, lv, st);
  };
  auto by_base = [&](auto rp, auto al) -> hipError_t {
    return W_base ? go(rp, std::false_type(), al) : go(rp, std::true_type(), al);
  };
  auto by_align = [&](auto rp) -> hipError_t {
    return r % 8 == 0 ? by_base(rp, std::true_type()) : by_base(rp, std::false_type());
  };
  if (r <= 16) return by_align(std::integral_constant<int, 16>());
  if (r <= 32) return by_align(std::integral_constant<int, 32>());
  if (r <= 64) return by_align(std::integral_constant<int, 64>());
  return by_align(std::integral_constant<int, 128>());
}

}  // namespace qlora
