// nf4_gemv.hip -- the forward for few tokens (T <= 64), where the layer is bound
// by streaming the 4-bit weight from HBM, not by arithmetic.
//
// Same computation as the tiled forward ("What does QLoRA change compared with
// plain LoRA when fine-tuning Llama?", katajob.com, "NF4: 4-bit NormalFloat":
// blocks expanded to bf16 inside the matmul; "QLoRA: fine-tuning a large model
// on one GPU", learn.pranaymahendrakar.com, "LoRA, stated once": the adapter
// adds (alpha/r) B A x), organised for bandwidth in two launches:
//
// 1. k_nf4_gemv: the reduction over n_in is split into K ranges.  A workgroup
//    (4 waves) owns 64 RG weight rows and one K range; each wave owns RG
//    groups of 16 rows and issues v_mfma_f32_16x16x32_bf16 with the tokens as
//    the M dimension, so one load of the activations serves RG row groups
//    (MFMA rows of tokens past T repeat token T - 1 and are never stored).
//    Each lane streams 16 bytes of codes per row group and 128-deep step (32
//    consecutive weights of one row, one block constant) and decodes them
//    straight into its four B operands, so the weight never touches LDS.  The
//    decode looks up both levels of a code byte at once in a 256-entry LDS
//    table of level pairs: per byte one shift with a byte select (the table
//    offset), one 8-byte LDS read, two binary32 multiplies by the block
//    constant and one bf16 pack.  Codes are prefetched two steps
//    ahead.  Each K range writes binary32 partial sums.  One extra workgroup
//    per K range computes the partial sums of U = X A^T over that range (one
//    per quarter range and wave).
// 2. k_gemv_finish: per token, U = the partials of U added in K-range order,
//    V = bf16(s U) (and U_out = bf16(U)); then
//    Y = bf16(sum of the weight partials in K-range order + V B^T), so the
//    result does not depend on the order in which workgroups finish.
//    (A single launch with a last-arriving-workgroup reduction needs
//    device-scope fences, which on this chip write back and invalidate the L2
//    in every workgroup and cost far more than a second launch.)
// Variants of the first launch with the same partial-sum contract, chosen by
// token count and shape: k_nf4_gemv_rows (one or two tokens, a wave per
// weight row), k_nf4_gemv_m32 (3..64 tokens, 32x32 MFMAs with the block
// constant applied per block), k_nf4_gemv_mrows (up to 64 tokens, 16x16 MFMAs
// on exactly dequantized weights).
#include <algorithm>

#include "device.h"
#include "launch.h"
#include "qlora.h"

namespace qlora {

namespace {
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// The bf16 level-pair table of the row-streaming GEMV: entry e (a code byte) is one word
// holding bf16(level[e & 15]) in its low half and bf16(level[e >> 4]) in its high half, the
// order of the two weights of the byte.  For sixteen-wave workgroups it is kept in 64
// interleaved copies (64 KB): entry e of copy c sits at byte 256 e + 4 c, i.e. in bank c of
// the 64 four-byte banks, and lane l reads copy l, so a 4-byte LDS read of the wave touches
// 64 distinct banks whatever its code bytes.  Built by 1024 threads t, each storing copies
// 4 (t & 15) .. + 3 of the entries (t >> 4) + 64 i, i < 4: the 16 lanes of each phase of a
// 16-byte store then fill the 64 banks once (with 16 entries per phase the stores were 16-way
// bank conflicts, about 1.6 us of a one-token launch at 8192 x 8192).  With fewer threads, one
// copy (entries 0..255 at bytes 0..1023).
constexpr int kTabCopies = 64;
__device__ __forceinline__ uint32_t bf16_level_pair(const Levels &lv, int e) {
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    lo = ((e & 15) == i) ? lv.v[i] : lo;
    hi = ((e >> 4) == i) ? lv.v[i] : hi;
  }
  return pack_bf16x2(lo, hi);
}
// The five levels a thread needs come from one register holding level[lane & 15] in every lane, read
// across lanes (ds_bpermute), instead of a chain of selects per level.  Every lane of the wave must
// call it (the cross-lane reads); t >= 1024 writes nothing.
__device__ __forceinline__ void bf16_pairs_rep64(const Levels &lv, uint32_t *tab, int t) {
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  float mine = 0.f;  // level[lane & 15]
#pragma unroll
  for (int v = 0; v < 16; ++v) mine = ((lane & 15) == v) ? lv.v[v] : mine;
  const int e0 = (t >> 4) & 63, c0 = 4 * (t & 15);  // entries e0 + 64 i share the low nibble e0 & 15
  const int mi = __builtin_bit_cast(int, mine);
  const float lo = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (e0 & 15), mi));
  float hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) hi[i] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * ((e0 >> 4) + 4 * i), mi));
  if (t < 1024) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t p = pack_bf16x2(lo, hi[i]);
      *reinterpret_cast<u32x4_t *>(tab + (e0 + 64 * i) * kTabCopies + c0) = u32x4_t{p, p, p, p};
    }
  }
}
__device__ __forceinline__ void bf16_pairs_one(const Levels &lv, uint32_t *tab, int tid) {
  if (tid < 256) tab[tid] = bf16_level_pair(lv, tid);
}
// bf16 levels of the two nibbles of byte b of w from the replicated table; c4 = 4 lane.  The
// byte offset 256 byte + c4 is one byte permute: [c4, byte b of w, 0, 0].
template <int B>
__device__ __forceinline__ uint32_t bf16_pair_rep64(const uint32_t *tab, uint32_t w, uint32_t c4) {
  const uint32_t off = __builtin_amdgcn_perm(w, c4, 0x0C0C0000u | ((4u + B) << 8));
  return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(tab) + off);
}

// Sum over the 64 lanes of a wave with DPP moves: pairs, quads, half rows and rows of 16
// (quad_perm, row_half_mirror, row_mirror), then row 0 into row 1 and row 2 into row 3
// (row_bcast:15), then rows 0..1 into rows 2..3 (row_bcast:31).  The total lands in lane 63.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf,
                                                                   false));
}
__device__ __forceinline__ float wave_sum_lane63(float v) {
  v = dpp_add<0xb1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4e>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x141>(v);  // row_half_mirror
  v = dpp_add<0x140>(v);  // row_mirror
  v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Partial U over a quarter of one K range: wave w of the workgroup takes
// k in [kb + w q, kb + (w+1) q), q = (ke - kb) / 4, and writes
// upart[t, j] = sum over its k of X[t, k] A[j, k] for all ranks j < r.
template <int MT>
__device__ void lora_u_partial(const bf16_t *__restrict__ X, int64_t T, int64_t K, const bf16_t *__restrict__ A,
                               int64_t r, int64_t kb, int64_t ke, float *__restrict__ upart, int wave, int lane) {
  const int g = lane >> 4;
  const int64_t q = (ke - kb) / 4, k0 = kb + wave * q, k1 = k0 + q;
  for (int jt = 0; jt * 16 < r; ++jt) {
    const int64_t j = jt * 16 + (lane & 15);
    const bool jok = j < r;
    f32x4_t acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int64_t k = k0 + 8 * g; k < k1; k += 32) {
      const u32x4_t b = jok ? *reinterpret_cast<const u32x4_t *>(A + j * K + k) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int64_t t = m * 16 + (lane & 15);
        const u32x4_t a = t < T ? *reinterpret_cast<const u32x4_t *>(X + t * K + k) : u32x4_t{0u, 0u, 0u, 0u};
        acc[m] = mfma_16x16x32(a, b, acc[m]);
      }
    }
    // element i of lane l: token 16 m + 4 (l >> 4) + i, rank 16 jt + (l & 15)
    if (jok)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t t = m * 16 + 4 * g + i;
          if (t < T) upart[t * r + j] = acc[m][i];
        }
  }
}
}  // namespace

// ------------------------------------------------------------------ the GEMV
// Work item i = (tile, split) = (i / nsplit, i % nsplit): weight rows
// 64 RG tile .. +64 RG - 1 over the K range [split kchunk, (split+1) kchunk).
// The first gmain workgroups are persistent: workgroup x takes items
// x, x + gmain, ..., and its waves stream the steps of all its items as one
// sequence, so the prefetch runs on across item boundaries.  Workgroup
// gmain + p computes the U partials of K range p (four, one per wave).
// A step is D = 128 W deep: lane group g = lane / 16 reads 16 W bytes of codes
// (32 W consecutive weights) of its row.  part: [nsplit][T][N] binary32,
// upart: [4 nsplit][T][r] binary32.  K must be a multiple of nsplit * D.
template <int MT, int RG, int W>
__global__ __launch_bounds__(256) void k_nf4_gemv(const bf16_t *__restrict__ X, int64_t T, int64_t K,
                                                  const uint8_t *__restrict__ codes,
                                                  const uint8_t *__restrict__ absmax_q,
                                                  const float *__restrict__ step, int64_t N, int nsplit,
                                                  int gmain, const bf16_t *__restrict__ A, int64_t r,
                                                  float *__restrict__ part, float *__restrict__ upart, Levels lv,
                                                  SegTable sg) {
  constexpr int D = 128 * W;              // reduction depth of one step
  constexpr int NB = W >= 2 ? W / 2 : 1;  // NF4 blocks a lane touches per step
  __shared__ __attribute__((aligned(16))) float2 s_tab[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t kchunk = K / nsplit;
  if ((int)blockIdx.x >= gmain) {
    const int64_t u = (int64_t)blockIdx.x - gmain;
    if (sg.n_seg == 0) {  // one adapter: workgroup u takes K range u for every token
      const int64_t kb = u * kchunk;
      lora_u_partial<MT>(X, T, K, A, r, kb, kb + kchunk, upart + (u * 4 + wave) * T * r, wave, lane);
      return;
    }
    // many adapters: workgroup u takes segment u / nsplit over K range u % nsplit, with its adapter
    const int g = (int)(u / nsplit);
    const int64_t p = u - (int64_t)g * nsplit, kb = p * kchunk;
    auto clampT = [&](int64_t v) { return v < 0 ? (int64_t)0 : (v > T ? T : v); };
    const int64_t lo = clampT(sg.seg[g]), hi = clampT(sg.seg[g + 1]);
    const int a = sg.ad[g];
    if (hi <= lo || a < 0 || a >= sg.n_pool) return;  // no tokens, or no adapter: U is not used
    lora_u_partial<MT>(X + lo * K, hi - lo, K, A + (int64_t)a * r * K, r, kb, kb + kchunk,
                       upart + ((p * 4 + wave) * T + lo) * r, wave, lane);
    return;
  }
  pair_levels_to_lds(lv, s_tab, tid);
  __syncthreads();
  const int g = lane >> 4;  // which 32 W-wide slice of each step
  const int nsteps = (int)(kchunk / D);
  const int64_t tiles = (N + 64 * RG - 1) / (64 * RG);
  const int64_t nitems = tiles * nsplit;
  const int64_t my_items = (nitems - blockIdx.x + gmain - 1) / gmain;
  const int64_t total = my_items * nsteps;  // steps of this workgroup
  if (total == 0) return;

  // activations: token 16 m + (lane & 15); lanes of tokens past T load token T - 1 instead (MFMA
  // output row t depends on operand row t only, and rows past T are never stored), so the loads
  // need no branch around them
  const bf16_t *xrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t t = m * 16 + (lane & 15);
    xrow[m] = X + (t < T ? t : T - 1) * K + 32 * W * g;
  }
  // row of row group q in tile `tile`: 64 RG tile + 64 q + 16 wave + (lane & 15)
  auto row_of = [&](int64_t tile, int q) { return tile * 64 * RG + 64 * q + 16 * wave + (lane & 15); };

  f32x4_t acc[RG][MT];
#pragma unroll
  for (int q = 0; q < RG; ++q)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[q][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Slot {
    u32x4_t c[RG][W];
    RawScale cq[RG][NB];
  };
  // Item i = tile * nsplit + split; a workgroup's items are gmain apart, so (tile, split) advances by
  // (gmain / nsplit, gmain % nsplit) with a carry instead of a division per step.
  const int64_t item_dt = gmain / nsplit;
  const int item_ds = gmain % nsplit;
  auto next_item = [&](int64_t &tile, int &split) {
    tile += item_dt;
    split += item_ds;
    if (split >= nsplit) {
      split -= nsplit;
      ++tile;
    }
  };
  // load stream position: item li of this workgroup (tile lt, split lsp), step ls; it stops
  // advancing at the last step, so the prefetches past the end re-read that step (unused)
  int64_t li = 0, lt = (int64_t)blockIdx.x / nsplit;
  int ls = 0, lsp = (int)((int64_t)blockIdx.x % nsplit);
  auto load_slot = [&](Slot &sl) {
    const int64_t tile = lt;
    const int64_t koff = (int64_t)lsp * kchunk + (int64_t)ls * D + 32 * W * g;
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      int64_t n = row_of(tile, q);
      n = n < N ? n : N - 1;  // rows past N re-read the last row; they are never stored
      const uint8_t *cp = codes + n * (K / 2) + koff / 2;
#pragma unroll
      for (int i = 0; i < W; ++i) sl.c[q][i] = *reinterpret_cast<const u32x4_t *>(cp + 16 * i);
#pragma unroll
      for (int b = 0; b < NB; ++b) sl.cq[q][b] = load_scale(absmax_q, step, n * (K / 64) + koff / 64 + b);
    }
    if (ls + 1 < nsteps) {
      ++ls;
    } else if (li + 1 < my_items) {
      ls = 0;
      ++li;
      next_item(lt, lsp);
    }
  };
  // compute stream position: step cs of the item at (tile ct, split csp)
  int64_t ct = (int64_t)blockIdx.x / nsplit;
  int cs = 0, csp = (int)((int64_t)blockIdx.x % nsplit);
  auto do_step = [&](Slot &cur, Slot &refill) {
    const int64_t tile = ct;
    const int64_t koff = (int64_t)csp * kchunk + (int64_t)cs * D;
    // this step's activations first, then the code prefetch: vector-memory counters complete in
    // order, so waiting for activations issued after the prefetch would wait for the prefetch too
    u32x4_t a[MT][4 * W];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4 * W; ++j)
        a[m][j] = *reinterpret_cast<const u32x4_t *>(xrow[m] + koff + 8 * j);
    load_slot(refill);
#pragma unroll
    for (int q = 0; q < RG; ++q) {
#pragma unroll
      for (int i = 0; i < W; ++i) {
        const float cq = scale_of(cur.cq[q][W >= 2 ? i / 2 : 0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4_t b = decode8_pairs(cur.c[q][i][j], cq, s_tab);
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[q][m] = mfma_16x16x32(a[m][4 * i + j], b, acc[q][m]);
        }
      }
    }
    if (++cs == nsteps) {  // item done: store its partial sums and start the next
      // accumulator element e of lane l holds token 16 m + 4 (l >> 4) + e, row n
      float *dst = part + (int64_t)csp * T * N;
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        const int64_t n = row_of(tile, q);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t t = m * 16 + 4 * g + e;
            if (n < N && t < T) dst[t * N + n] = acc[q][m][e];
          }
          acc[q][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
      cs = 0;
      next_item(ct, csp);
    }
  };
  // three fixed slots, unrolled so that no register holding a load in flight
  // is ever copied (a copy would make the wave wait for that load)
  Slot s0, s1, s2;
  load_slot(s0);
  load_slot(s1);
  for (int64_t f = 0; f < total; f += 3) {
    do_step(s0, s2);
    if (f + 1 < total) do_step(s1, s0);
    if (f + 2 < total) do_step(s2, s1);
  }
}

// ------------------------------------------------ the row-streaming GEMV
// For one or two tokens the MFMA formulation wastes most of each 16-token operand
// and its 16-row loads touch 16 weight rows per instruction.  Here a wave owns
// weight rows instead.  A work item is one segment of Ks = 2048 CH columns of
// one row (nseg = K / Ks segments per row); lane l covers columns
// 2048 c + 32 l .. 2048 c + 32 l + 31 of chunk c of the segment, so one
// 16-byte load per lane and chunk streams 1 KB of one row per wave
// instruction, like a plain copy.  Since a workgroup keeps one segment for the
// whole launch, every lane keeps its TT CH 32 activations in registers, loaded
// once: the workgroup copies the segment's activations into LDS and each wave
// takes its lanes' share from there (one global read per workgroup instead of
// one per wave; measured 2-4% faster).
//
// A lane's 32 weights of a chunk lie in one block, so the block constant
// factors out of their dot product: per chunk the lane looks up each code
// byte's two levels as a bf16 pair, accumulates v_dot2_f32_bf16 with the
// matching activation pairs, and adds c' times that sum to its binary32
// total (the block expanded to bf16 levels, scaled in binary32 after the
// block's products; the same sum reassociated, with the rounding on the
// level instead of on the product level * c').  Per code byte that is one
// byte permute (the table address), one 4-byte LDS read and one dot product.
// A wave reduction then gives the binary32 partial sum of the segment.
//
// Main workgroup g (NWV waves) owns segment g % nseg, and its wave w the rows
// NWV (g / nseg) + w + i NWV gmain / nseg (gmain % nseg == 0).  With sixteen
// waves the level pairs come from the 64-copy table (bank-conflict free,
// 64 KB, so two workgroups per CU); with four, from one copy.  A wave
// keeps SLOTS - 1 items in flight while it computes one, in fixed register
// slots (the loop is unrolled by SLOTS, so no slot is ever copied: a copy of
// a register whose load is in flight would make the wave wait for it).  The
// wave index is made wave-uniform, so the item bookkeeping and addresses stay
// in scalar registers.  The block constants of an item: lane l's block in
// chunk c is block 32 c + (l >> 1) of the segment; it is read as the aligned
// 4-byte word holding its byte (absmax_q is 16-byte aligned), and the item's
// 32 CH blocks share one binary32 step (32 CH divides 256 and the item's
// first block is a multiple of 32 CH).  part is [nseg][T][N] binary32.
// Workgroups gmain .. gmain + nsplit_u - 1 come last and form the U partials
// of K range u as in k_nf4_gemv ([4 nsplit_u][T][r]; their waves past the fourth have nothing
// to do): the main workgroups then fill every slot at once and, when the items divide evenly,
// every wave streams the same number of them (with the U workgroups first, 512 slots leave
// 496 for the main ones, and at 8192 x 8192 512 of their 7936 waves take a third item).
// Tokens T .. TT-1 are zero.
template <int TT, int CH, int SLOTS, int NWV, int MINW>
__global__ __launch_bounds__(64 * NWV, MINW) void k_nf4_gemv_rows(
    const bf16_t *__restrict__ X, int64_t T, int64_t K, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ absmax_q, const float *__restrict__ step, int64_t N, int gmain, int nseg, int nsplit_u,
    const bf16_t *__restrict__ A, int64_t r, float *__restrict__ part, float *__restrict__ upart, Levels lv) {
  constexpr bool REP = NWV == 16;  // sixteen waves share the replicated table
  constexpr int Ks = 2048 * CH;
  __shared__ __attribute__((aligned(16))) uint32_t s_tab[REP ? 256 * kTabCopies : 256];
  __shared__ __attribute__((aligned(16))) uint32_t s_x[TT][Ks / 2];  // the segment's activations
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if ((int)blockIdx.x >= gmain) {
    if (wave >= 4) return;
    const int64_t u = blockIdx.x - gmain, kchunk = K / nsplit_u, kb = u * kchunk;
    lora_u_partial<1>(X, T, K, A, r, kb, kb + kchunk, upart + (u * 4 + wave) * T * r, wave, lane);
    return;
  }
  const int g = (int)blockIdx.x, seg = g % nseg;
  const int64_t row0 = (int64_t)(g / nseg) * NWV + wave, rstride = (int64_t)(gmain / nseg) * NWV;
  const int64_t items = row0 < N ? (N - row0 + rstride - 1) / rstride : 0;

  struct Slot {
    u32x4_t c[CH];   // the lane's 16 code bytes of each chunk
    uint32_t q[CH];  // the aligned word holding the lane's block byte of each chunk
    float d;         // the item's binary32 step
  };
  // lane offsets: codes 16 lane, block-constant word (lane >> 1) & ~3; the constant's bit offset
  // 8 ((lane >> 1) & 3) equals (4 lane) & 24 and is formed from the table offset c4 = 4 lane where it is
  // used, which keeps one VGPR fewer live across the loop (64 VGPRs, eight waves per SIMD, no spill)
  const int lofs = 16 * lane, bofs = (lane >> 1) & ~3;
  int64_t li = 0;  // item of the load stream; it stops at the last item (later prefetches reload it, unused)
  auto load_slot = [&](Slot &sl) {
    const int64_t row = row0 + li * rstride;
    const uint8_t *cr = codes + row * (K / 2) + seg * (Ks / 2);
    const int64_t b0 = row * (K / 64) + seg * (Ks / 64);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      sl.c[c] = *reinterpret_cast<const u32x4_t *>(cr + 1024 * c + lofs);
      sl.q[c] = *reinterpret_cast<const uint32_t *>(absmax_q + b0 + 32 * c + bofs);
    }
    sl.d = step[b0 >> 8];
    if (li + 1 < items) ++li;
  };
  Slot sl[SLOTS];
#pragma unroll
  for (int j = 0; j + 1 < SLOTS; ++j)  // in flight while the activations and the table are loaded
    if (items > 0) load_slot(sl[j]);

  if constexpr (REP) bf16_pairs_rep64(lv, s_tab, tid);
  else bf16_pairs_one(lv, s_tab, tid);
  const uint32_t c4 = 4u * lane;
  // the workgroup reads the segment's activations once (every wave of it needs all of them), through LDS
  for (int i = tid; i < TT * Ks / 8; i += 64 * NWV) {
    const int t = i / (Ks / 8), c = i % (Ks / 8);
    *reinterpret_cast<u32x4_t *>(&s_x[t][4 * c]) =
        t < T ? *reinterpret_cast<const u32x4_t *>(X + t * K + seg * Ks + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if (items <= 0) return;
  uint32_t xr[TT][CH][16];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(&s_x[t][1024 * c + 16 * lane + 4 * h]);
#pragma unroll
        for (int e = 0; e < 4; ++e) xr[t][c][4 * h + e] = v[e];
      }

  float *pseg = part + (int64_t)seg * T * N;
  int64_t cn = row0;  // row of the item being computed
  auto do_step = [&](Slot &cur, Slot &refill) {
    load_slot(refill);
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float cq = __fmul_rn((float)__builtin_amdgcn_ubfe(cur.q[c], c4 & 24u, 8), cur.d);
      float pb[TT];  // the block's dot products
#pragma unroll
      for (int t = 0; t < TT; ++t) pb[t] = 0.f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t w = cur.c[c][wd];
        uint32_t lp[4];
        if constexpr (REP) {
          lp[0] = bf16_pair_rep64<0>(s_tab, w, c4), lp[1] = bf16_pair_rep64<1>(s_tab, w, c4);
          lp[2] = bf16_pair_rep64<2>(s_tab, w, c4), lp[3] = bf16_pair_rep64<3>(s_tab, w, c4);
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b) lp[b] = s_tab[(w >> (8 * b)) & 0xffu];
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t lb = lp[b];
          const bf16x2_t wp = __builtin_bit_cast(bf16x2_t, lb);
#pragma unroll
          for (int t = 0; t < TT; ++t) {
            const uint32_t xw = xr[t][c][4 * wd + b];
            pb[t] = __builtin_amdgcn_fdot2_f32_bf16(wp, __builtin_bit_cast(bf16x2_t, xw), pb[t], false);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[t] = fmaf(cq, pb[t], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {  // reduce over the wave, lane 63 writes the partial
      const float v = wave_sum_lane63(acc[t]);
      if (lane == 63 && t < T) pseg[t * N + cn] = v;
    }
    cn += rstride;
  };
  // step j computes slot j % SLOTS and refills slot (j + SLOTS - 1) % SLOTS; unrolled by SLOTS so that
  // every slot index is a constant, the last round cut short by wave-uniform guards (no separate tail
  // copy of the body, whose registers would have to live across the loop)
  for (int64_t f = 0; f < items; f += SLOTS) {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j)
      if (f + j < items) do_step(sl[j], sl[(j + SLOTS - 1) % SLOTS]);
  }
}

// ------------------------------------------- the row-group GEMV (3..64 tokens)
// The MFMA formulation of k_nf4_gemv with the row kernel's layout, for MT
// groups of 16 tokens (MT = 1: up to 16 tokens, MT = 2: up to 32, MT = 4: up
// to 64; with MT = 4 a lane group's 32 columns lie in one block).  A work item
// is 16 weight rows over one segment of KS = 512 / MT columns (nseg = K / KS
// segments, one per workgroup for the whole launch).  Lane (a, g) = (l & 15,
// l >> 4) keeps tokens 16 m + a's activations at segment columns CL g .. CL g +
// CL - 1 (CL = 128 / MT) in registers (64 VGPRs for either MT, loaded once;
// tokens past T are zero) and streams weight row 16 i + a's codes for the same
// columns (CL / 2 bytes: 64 / MT ... four or two 16-byte loads per item).
// MFMA step s (v_mfma_f32_16x16x32_bf16, tokens as M) takes columns CL g + 8 s
// .. + 7 of every lane group g -- the same permutation of the reduction for
// both operands, so the products are those of the layer.  The decode is
// k_nf4_gemv's: level pairs from the LDS table, fl32(level * c'), bf16 pack.
// The next item loads while the current one computes (two fixed slots, the
// loop unrolled by two).  With RED = 1, main workgroup g owns segment
// g % nseg, its wave w the row groups 4 (g / nseg) + w + i 4 gmain / nseg, and
// part is [nseg][T][N].  With RED = 4 or 8 (nseg % RED == 0) the RED waves of
// main workgroup g take the RED segments RED (g % nq) + w of one part (nq =
// nseg / RED) over the same row groups g / nq + i gmain / nq; after each item
// they exchange their sums through LDS (two buffers, one barrier per item),
// waves 0..3 add them in wave order and write one partial per part: part is
// [nq][T][N], 1 / RED of the partial bytes.  Workgroups 0 .. nsplit_u - 1
// come first and form the U partials as in k_nf4_gemv_rows (with RED = 8 their
// waves 4..7 have nothing to do).
constexpr int kMrowsMaxT = 64;
// Waves per SIMD the registers must allow: four where the kernel fits 128 VGPRs without spilling (two or
// four token groups with the workgroup sum), else three.
template <int MT, int RED>
constexpr int mrows_minw() { return (MT == 4 || (MT == 2 && RED > 1)) ? 4 : 3; }
template <int MT, int RED>
__global__ __launch_bounds__(64 * (RED == 8 ? 8 : 4), (mrows_minw<MT, RED>())) void k_nf4_gemv_mrows(
    const bf16_t *__restrict__ X, int64_t T, int64_t K, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ absmax_q, const float *__restrict__ step, int64_t N, int gmain, int nseg, int nsplit_u,
    const bf16_t *__restrict__ A, int64_t r, float *__restrict__ part, float *__restrict__ upart, Levels lv) {
  constexpr int KS = 512 / MT, CL = 128 / MT, NS = CL / 8;  // segment, lane-group columns, MFMA steps per item
  constexpr int NW = CL / 32, NB = CL >= 64 ? CL / 64 : 1;  // 16-byte code loads and blocks per lane and item
  __shared__ __attribute__((aligned(16))) float2 s_tab[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if ((int)blockIdx.x < nsplit_u) {
    if (wave >= 4) return;
    const int64_t u = blockIdx.x, kchunk = K / nsplit_u, kb = u * kchunk;
    lora_u_partial<MT>(X, T, K, A, r, kb, kb + kchunk, upart + (u * 4 + wave) * T * r, wave, lane);
    return;
  }
  static_assert(RED == 1 || RED == 4 || RED == 8, "one wave or the whole workgroup per partial");
  const int a = lane & 15, g = lane >> 4;
  const int gi = (int)blockIdx.x - nsplit_u, npart = nseg / RED, seg = RED == 1 ? gi % nseg : gi % npart * RED + wave;
  const int64_t ngroups = (N + 15) / 16;
  const int64_t rg0 = RED == 1 ? (int64_t)(gi / nseg) * 4 + wave : (int64_t)(gi / npart);
  const int64_t rgs = RED == 1 ? (int64_t)(gmain / nseg) * 4 : (int64_t)(gmain / npart);
  const int64_t items = rg0 < ngroups ? (ngroups - rg0 + rgs - 1) / rgs : 0;
  const int64_t col0 = (int64_t)seg * KS + CL * g;  // this lane group's first column
  pair_levels_to_lds(lv, s_tab, tid);
  u32x4_t xa[MT][NS];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t t = 16 * m + a;
    const bf16_t *xp = X + (t < T ? t : 0) * K + col0;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      xa[m][s] = t < T ? *reinterpret_cast<const u32x4_t *>(xp + 8 * s) : u32x4_t{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if (items <= 0) return;

  struct Slot {
    u32x4_t c[NW];    // the lane's CL / 2 code bytes (CL weights of one row)
    RawScale sc[NB];  // their blocks' constants
  };
  int64_t li = 0;  // item of the load stream; it stops at the last item (later prefetches reload it, unused)
  auto load_slot = [&](Slot &sl) {
    int64_t n = (rg0 + li * rgs) * 16 + a;
    n = n < N ? n : N - 1;  // rows past N re-read the last row; they are never stored
    const uint8_t *cp = codes + n * (K / 2) + col0 / 2;
#pragma unroll
    for (int i = 0; i < NW; ++i) sl.c[i] = *reinterpret_cast<const u32x4_t *>(cp + 16 * i);
    const int64_t b0 = n * (K / 64) + col0 / 64;
#pragma unroll
    for (int b = 0; b < NB; ++b) sl.sc[b] = load_scale(absmax_q, step, b0 + b);
    if (li + 1 < items) ++li;
  };
  float *pseg = part + (int64_t)(RED == 1 ? seg : gi % npart) * T * N;
  // RED > 1: the waves' sums of one item, [buffer][wave][token group][lane]
  __shared__ __attribute__((aligned(16))) f32x4_t s_red[RED > 1 ? 2 : 1][RED][MT][64];
  int64_t crg = rg0;  // row group of the item being computed
  auto do_step = [&](Slot &cur, Slot &refill, int buf) {
    load_slot(refill);
    f32x4_t acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float cq[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) cq[b] = scale_of(cur.sc[b]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t w = cur.c[s >> 2][s & 3];
      const u32x4_t bop = decode8_pairs(w, cq[s / 8], s_tab);
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = mfma_16x16x32(xa[m][s], bop, acc[m]);
    }
    // element e of lane l in token group m: token 16 m + 4 (l >> 4) + e, weight row 16 crg + (l & 15)
    if constexpr (RED == 1) {
      const int64_t n = crg * 16 + a;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t t = 16 * m + 4 * g + e;
          if (n < N && t < T) pseg[t * N + n] = acc[m][e];
        }
    } else {
      // wave w < 4 adds, for lanes 16 w .. 16 w + 15 of every wave, their four elements: thread l takes
      // lane 16 w + (l >> 2), element l & 3, i.e. token 16 m + 4 w + (l & 3), row 16 crg + (l >> 2); with
      // RED = 8 waves 4..7 only contribute their sums
#pragma unroll
      for (int m = 0; m < MT; ++m) s_red[buf][wave][m][lane] = acc[m];
      __syncthreads();
      if (RED == 8 && wave >= 4) {
        crg += rgs;
        return;
      }
      const int64_t n = crg * 16 + (lane >> 2);
      const float *rd = reinterpret_cast<const float *>(&s_red[buf][0][0][0]) + (16 * wave + (lane >> 2)) * 4 + (lane & 3);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float y = rd[m * 256];
#pragma unroll
        for (int v = 1; v < RED; ++v) y += rd[(v * MT + m) * 256];
        const int64_t t = 16 * m + 4 * wave + (lane & 3);
        if (n < N && t < T) pseg[t * N + n] = y;
      }
    }
    crg += rgs;
  };
  Slot s0, s1;
  load_slot(s0);
  int64_t f = 0;
  for (; f + 1 < items; f += 2) {
    do_step(s0, s1, 0);
    do_step(s1, s0, RED > 1 ? 1 : 0);
  }
  if (f < items) do_step(s0, s1, 0);
}

// ------------------------------- the 32-token row-group GEMV (3..64 tokens)
// v_mfma_f32_32x32x16_bf16 with the tokens as M (activations: operand A, MT
// groups of 32 tokens) and 32 weight rows as N (decoded codes: operand B).
// The reduction index of MFMA step (b, s) is mapped onto the columns
// 64 b + 32 h + 8 s + e of the segment (h = lane / 32 the k-half a lane
// feeds, e < 8), so that the 16 columns of one MFMA lie in block b of every
// row and lane (n, h) = (l % 32, l / 32) feeds them from one 16-byte load:
// half h of block b of weight row n, words s = 0..3.  The block constant then
// factors out as in the row kernel: the four MFMAs of a block (per token
// group) start from zero, their bf16 levels come straight from the
// level-pair table (one byte permute and one 4-byte LDS read per code byte,
// no arithmetic, shared by the token groups), and each of the lane's
// accumulators adds c' times the block's result with one fmaf (the lane's
// accumulators all belong to its row n).  Accumulator element j of lane l in
// token group m is token 32 m + 8 (j / 4) + 4 (l / 32) + j % 4, so only the
// elements that hold tokens (TG 8-token groups, T <= 8 TG) are scaled,
// exchanged and stored.  With one token group two blocks are multiplied at a
// time, with two the groups' chains alternate, so that each MFMA's successor
// does not wait for its result.
//
// A segment is KS = 256 / MT columns (4 / MT blocks); every lane keeps its
// tokens' activations of the segment in 64 VGPRs for the whole launch
// (tokens past T are zero).  One workgroup per CU (two waves per SIMD).  The eight waves of main workgroup g take the
// eight segments 8 (g % npart) + w (npart = nseg / 8) over the same item
// sequence: row group g / npart + i gmain / npart (32 rows, rows past N
// re-read the last row and are never stored), each item one KS / 64 KB stream
// per wave, SLOTS - 1 items in flight.  After an item the waves pass their
// accumulators through LDS (two buffers and one barrier per item for 256-column
// segments; one buffer and two barriers otherwise) and every thread adds the
// eight segments' values of its outputs in wave order, so each part of 8 KS
// columns writes one partial: part is [npart][T][N].  Workgroups gmain ..
// gmain + nsplit_u - 1 follow and form the U partials ([4 nsplit_u][T][r];
// waves past the fourth have nothing to do).
constexpr int kM32Red = 8;
// segment columns: 256 for one token group, 128 for two (64 VGPRs of activations either way)
constexpr int m32_seg(int64_t T) { return T > 32 ? 128 : 256; }
template <int TG>
__global__ __launch_bounds__(64 * kM32Red, 2) void k_nf4_gemv_m32(
    const bf16_t *__restrict__ X, int64_t T, int64_t K, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ absmax_q, const float *__restrict__ step, int64_t N, int gmain, int nseg, int nsplit_u,
    const bf16_t *__restrict__ A, int64_t r, float *__restrict__ part, float *__restrict__ upart, Levels lv) {
  static_assert(TG >= 1 && TG <= 8, "up to 64 tokens");
  constexpr int MT = TG > 4 ? 2 : 1;                 // 32-token groups
  constexpr int KS = m32_seg(8 * TG), NB = KS / 64;   // segment columns, blocks per item
  constexpr int NE0 = TG >= 4 ? 16 : 4 * TG;          // elements of group 0 holding tokens
  constexpr int NE = NE0 + (MT == 2 ? 4 * (TG - 4) : 0);
  constexpr int IL = MT == 1 ? 2 : 1;                 // blocks multiplied at a time
  constexpr int NBUF = KS == 256 ? 2 : 1;             // exchange buffers (one: two workgroups fit a CU)
  constexpr int SLOTS = 3;
  // the alignment places the table at LDS address 0, so that a lookup address is the byte permute alone
  __shared__ __attribute__((aligned(1024))) uint32_t s_tab[256 * kTabCopies];
  __shared__ __attribute__((aligned(16))) float s_red[NBUF][kM32Red][NE][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if ((int)blockIdx.x >= gmain) {
    if (wave >= 4) return;
    const int64_t u = blockIdx.x - gmain, kchunk = K / nsplit_u, kb = u * kchunk;
    lora_u_partial<2 * MT>(X, T, K, A, r, kb, kb + kchunk, upart + (u * 4 + wave) * T * r, wave, lane);
    return;
  }
  const int n = lane & 31, h = lane >> 5;
  const int npart = nseg / kM32Red, pi = (int)blockIdx.x % npart, seg = pi * kM32Red + wave;
  const int64_t ngroups = (N + 31) / 32;
  const int64_t rg0 = (int64_t)blockIdx.x / npart, rgs = (int64_t)gmain / npart;
  const int64_t items = rg0 < ngroups ? (ngroups - rg0 + rgs - 1) / rgs : 0;
  const int64_t col0 = (int64_t)seg * KS;  // the segment's first column

  struct Slot {
    u32x4_t c[NB];  // half h of each block of the lane's row
    uint32_t q;     // the aligned word holding the blocks' 8-bit constants
    float d;        // their binary32 step
  };
  int64_t li = 0;  // item of the load stream; it stops at the last item (later prefetches reload it, unused)
  // row addresses: a wave-uniform 64-bit base of the row group plus a 32-bit lane offset (n K / 2 < 2^27)
  const uint8_t *const cbase = codes + col0 / 2 + 16 * h;
  // the row's first block here is a multiple of NB: its constants lie in the aligned word at qofs (byte
  // qsh / 8 onwards), and its NB blocks in one group of 256
  const int64_t qofs = (col0 / 64) & ~(int64_t)3;
  const int qsh = 8 * (int)((col0 / 64) & 3);
  auto load_slot = [&](Slot &sl) {
    const int64_t r0 = (rg0 + li * rgs) * 32;          // wave-uniform
    const int nr = (int)(r0 + n < N ? n : N - 1 - r0);  // row r0 + nr, clamped to the last row
    const uint8_t *cp = cbase + r0 * (K / 2) + (uint32_t)nr * (uint32_t)(K / 2);
#pragma unroll
    for (int b = 0; b < NB; ++b) sl.c[b] = *reinterpret_cast<const u32x4_t *>(cp + 32 * b);
    const int64_t rb = r0 * (K / 64) + (int64_t)nr * (K / 64);  // the row's first block
    sl.q = *reinterpret_cast<const uint32_t *>(absmax_q + rb + qofs);
    sl.d = step[(rb + col0 / 64) >> 8];
    if (li + 1 < items) ++li;
  };
  Slot sl[SLOTS];
#pragma unroll
  for (int j = 0; j + 1 < SLOTS; ++j)  // in flight while the activations and the table are loaded
    if (items > 0) load_slot(sl[j]);

  bf16_pairs_rep64(lv, s_tab, tid);
  bf16_pairs_rep64(lv, s_tab, tid + 512);
  const uint32_t c4 = 4u * lane;
  u32x4_t xa[MT][NB][4];  // [token group][block][MFMA step]: token 32 m + n, columns 64 b + 32 h + 8 s .. + 7
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t t = 32 * m + n;
    const bf16_t *xp = X + (t < T ? t : 0) * K + col0 + 32 * h;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        xa[m][b][st] = t < T ? *reinterpret_cast<const u32x4_t *>(xp + 64 * b + 8 * st) : u32x4_t{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if (items <= 0) return;

  float *pout = part + (int64_t)pi * T * N;
  int64_t crg = rg0;  // row group of the item being computed
  int buf = 0;        // LDS exchange buffer of the item being computed
  auto do_step = [&](Slot &cur, Slot &refill) {
    load_slot(refill);
    float acc[NE];  // group 0's elements, then group 1's
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.f;
#pragma unroll
    for (int bp = 0; bp < NB; bp += IL) {
      f32x16_t t[IL][MT] = {};
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < IL; ++i) {
          const uint32_t w = cur.c[bp + i][st];
          const u32x4_t bop = {bf16_pair_rep64<0>(s_tab, w, c4), bf16_pair_rep64<1>(s_tab, w, c4),
                               bf16_pair_rep64<2>(s_tab, w, c4), bf16_pair_rep64<3>(s_tab, w, c4)};
#pragma unroll
          for (int m = 0; m < MT; ++m) t[i][m] = mfma_32x32x16(xa[m][bp + i][st], bop, t[i][m]);
        }
#pragma unroll
      for (int i = 0; i < IL; ++i) {
        const float cq = __fmul_rn((float)__builtin_amdgcn_ubfe(cur.q, qsh + 8 * (bp + i), 8), cur.d);
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] = fmaf(cq, t[i][e < NE0 ? 0 : 1][e < NE0 ? e : e - NE0], acc[e]);
      }
      __builtin_amdgcn_sched_barrier(0);  // IL blocks' lookups and MFMA results live at a time
    }
    // exchange: thread (w, l) of the workgroup adds the eight waves' flat element w + 8 k of lane l
    if constexpr (NBUF == 1) __syncthreads();  // every wave has read the previous item's sums
#pragma unroll
    for (int e = 0; e < NE; ++e) s_red[buf][wave][e][lane] = acc[e];
    __syncthreads();
#pragma unroll
    for (int e0 = 0; e0 < NE; e0 += kM32Red) {
      const int e = e0 + wave;
      if (e < NE) {
        float y = s_red[buf][0][e][lane];
#pragma unroll
        for (int v = 1; v < kM32Red; ++v) y += s_red[buf][v][e][lane];
        const int m = e < NE0 ? 0 : 1, j = e < NE0 ? e : e - NE0;
        const int64_t t = 32 * m + 8 * (j >> 2) + 4 * h + (j & 3), row = crg * 32 + n;
        if (t < T && row < N) pout[t * N + row] = y;
      }
    }
    crg += rgs;
    if constexpr (NBUF == 2) buf ^= 1;
  };
  // item j computes slot j % SLOTS and refills slot (j + SLOTS - 1) % SLOTS; unrolled by SLOTS so that
  // every slot index is a constant
  int64_t f = 0;
  for (; f + SLOTS <= items; f += SLOTS) {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) do_step(sl[j], sl[(j + SLOTS - 1) % SLOTS]);
  }
#pragma unroll
  for (int j = 0; j + 1 < SLOTS; ++j)
    if (f + j < items) do_step(sl[j], sl[(j + SLOTS - 1) % SLOTS]);
}

// Sums of the finishing kernels, in index order with every load issued first (a loop bound known only
// at run time would otherwise wait for each load before the next): the 1 <= n <= 16 weight partials
// src[0], src[stride], ..., and the U partials p = q, q + 8, ... < nup <= 64 of (t, j).  Indexes past
// the end are clamped (the load stays in bounds) and the value replaced by +0; adding +0 to a sum
// that starts at +0 changes nothing.
// kFinishMaxSplit partials by default; launches with up to kFinishMaxSplitWide use a wider variant.
constexpr int kFinishMaxSplit = 16, kFinishMaxSplitWide = 32, kFinishMaxUp = 64;
template <int PS>
__device__ __forceinline__ void load_partials(const float *__restrict__ src, int64_t stride, int n, float (&v)[PS]) {
#pragma unroll
  for (int q = 0; q < PS; ++q) v[q] = src[(int64_t)(q < n ? q : n - 1) * stride];
}
template <int PS>
__device__ __forceinline__ float add_partials(const float (&v)[PS], int n) {
  float y = 0.f;
#pragma unroll
  for (int q = 0; q < PS; ++q) y += q < n ? v[q] : 0.f;
  return y;
}
__device__ __forceinline__ float sum_partials(const float *__restrict__ src, int64_t stride, int n) {
  float v[kFinishMaxSplit];
  load_partials(src, stride, n, v);
  return add_partials(v, n);
}
__device__ __forceinline__ void load_upart(const float *__restrict__ upart, int64_t T, int64_t t, int64_t r, int j,
                                           int q, int nup, float (&v)[kFinishMaxUp / 8]) {
#pragma unroll
  for (int c = 0; c < kFinishMaxUp / 8; ++c) {
    const int p = q + 8 * c;
    v[c] = upart[((int64_t)(p < nup ? p : nup - 1) * T + t) * r + j];
  }
}
__device__ __forceinline__ float add_upart(const float (&v)[kFinishMaxUp / 8], int q, int nup) {
  float u = 0.f;
#pragma unroll
  for (int c = 0; c < kFinishMaxUp / 8; ++c) u += q + 8 * c < nup ? v[c] : 0.f;
  return u;
}
__device__ __forceinline__ float sum_upart(const float *__restrict__ upart, int64_t T, int64_t t, int64_t r, int j,
                                           int q, int nup) {
  float v[kFinishMaxUp / 8];
  load_upart(upart, T, t, r, j, q, nup, v);
  return add_upart(v, q, nup);
}

// Workgroup (x, t): U[t, :] = sum of the nup U partials upart[p][t][:] (thread
// (j, q) adds the partials p = q, q + 8, ... in order, then the eight subtotals
// are added in q order), V = bf16(s U) in LDS (U_out[t, :] = bf16(U) from
// x == 0); then for its 256 outputs n:
// Y[t, n] = bf16(sum over p (in order) of part[p][t][n] + V . B[n, :r]).
// The weight partials and, for r = 8 NBP, the row of B are loaded before the U
// sums, so that their latency overlaps that of the U partials.
template <int NBP, int PS>
__global__ __launch_bounds__(256) void k_gemv_finish(const float *__restrict__ part, const float *__restrict__ upart,
                                                     int nsplit, int nup, int64_t T, int64_t N,
                                                     const bf16_t *__restrict__ B, int64_t r, float s,
                                                     bf16_t *__restrict__ Y, bf16_t *__restrict__ U_out) {
  __shared__ float s_sub[8][QLORA_MAX_RANK];
  __shared__ float s_v[QLORA_MAX_RANK];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.y;
  const int64_t n = (int64_t)blockIdx.x * 256 + tid;
  const bool nok = n < N;
  // this thread's first U pair (j, q) = (tid % r, tid / r), its weight partials and its B row are all
  // loaded (indexes clamped into range) before the first addition
  const int iu = tid < 8 * r ? tid : 8 * (int)r - 1;
  const int64_t nn = nok ? n : N - 1;
  float uv[kFinishMaxUp / 8], pv[PS];
  u32x4_t bw[NBP > 0 ? NBP : 1];
  load_upart(upart, T, t, r, iu % r, iu / r, nup, uv);
  load_partials(part + t * N + nn, T * N, nsplit, pv);
#pragma unroll
  for (int c = 0; c < NBP; ++c) bw[c] = *reinterpret_cast<const u32x4_t *>(B + nn * r + 8 * c);
  if (tid < 8 * r) s_sub[tid / r][tid % r] = add_upart(uv, iu / r, nup);
  const float y = add_partials(pv, nsplit);
  for (int i = tid + 256; i < 8 * r; i += 256) {
    const int j = i % r, q = i / r;
    s_sub[q][j] = sum_upart(upart, T, t, r, j, q, nup);
  }
  __syncthreads();
  if (tid < r) {
    float u = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) u += s_sub[q][tid];
    s_v[tid] = bf16_lo_to_f32(f32_to_bf16(s * u));
    if (U_out && blockIdx.x == 0) U_out[t * r + tid] = f32_to_bf16(u);
  }
  __syncthreads();
  if (!nok) return;
  float l = 0.f;
  if (NBP > 0) {
#pragma unroll
    for (int c = 0; c < NBP; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        l = fmaf(s_v[8 * c + 2 * e], bf16_lo_to_f32(bw[c][e]), l);
        l = fmaf(s_v[8 * c + 2 * e + 1], bf16_hi_to_f32(bw[c][e]), l);
      }
  } else {
    const bf16_t *brow = B + n * r;
    int64_t j = 0;
    if ((r & 7) == 0)  // rows of B are 16-byte multiples: 8 ranks per load
      for (; j < r; j += 8) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t *>(brow + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          l = fmaf(s_v[j + 2 * e], bf16_lo_to_f32(w[e]), l);
          l = fmaf(s_v[j + 2 * e + 1], bf16_hi_to_f32(w[e]), l);
        }
      }
    for (; j < r; ++j) l = fmaf(s_v[j], bf16_lo_to_f32(brow[j]), l);
  }
  Y[t * N + n] = f32_to_bf16(y + l);
}

// Many adapters: workgroup (x, t) finds token t's segment by bisection (entries
// clamped to [0, T]); U[t, :] = its nup U partials added as in k_gemv_finish,
// V = bf16(s U); then for its 256 outputs n
// Y[t, n] = bf16(sum over p (in order) of part[p][t][n] + V . B_a[n, :]),
// B_a = B_pool + a N r, or the partials alone when the segment has no adapter
// (or the token no segment).
__global__ __launch_bounds__(256) void k_gemv_finish_multi(const float *__restrict__ part,
                                                           const float *__restrict__ upart, int nsplit, int nup,
                                                           int64_t T, int64_t N, const bf16_t *__restrict__ B_pool,
                                                           int64_t r, float s, SegTable sg, bf16_t *__restrict__ Y) {
  __shared__ float s_sub[8][QLORA_MAX_RANK];
  __shared__ float s_v[QLORA_MAX_RANK];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.y;
  auto clampT = [&](int64_t v) { return v < 0 ? (int64_t)0 : (v > T ? T : v); };
  int g0 = 0, g1 = sg.n_seg;  // first segment ending past t
  while (g0 < g1) {
    const int mid = (g0 + g1) >> 1;
    if (clampT(sg.seg[mid + 1]) <= t) g0 = mid + 1;
    else g1 = mid;
  }
  int a = -1;
  if (g0 < sg.n_seg && clampT(sg.seg[g0]) <= t) a = sg.ad[g0];
  const bool has = a >= 0 && a < sg.n_pool;  // uniform in the workgroup
  if (has) {
    for (int i = tid; i < 8 * r; i += 256) {
      const int j = i % r, q = i / r;
      s_sub[q][j] = sum_upart(upart, T, t, r, j, q, nup);
    }
    __syncthreads();
    if (tid < r) {
      float u = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) u += s_sub[q][tid];
      s_v[tid] = bf16_lo_to_f32(f32_to_bf16(s * u));
    }
  }
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * 256 + tid;
  if (n >= N) return;
  const float y = sum_partials(part + t * N + n, T * N, nsplit);
  float l = 0.f;
  if (has) {
    const bf16_t *brow = B_pool + ((int64_t)a * N + n) * r;  // r % 8 == 0: 16-byte rows
    for (int64_t j = 0; j < r; j += 8) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t *>(brow + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        l = fmaf(s_v[j + 2 * e], bf16_lo_to_f32(w[e]), l);
        l = fmaf(s_v[j + 2 * e + 1], bf16_hi_to_f32(w[e]), l);
      }
    }
  }
  Y[t * N + n] = f32_to_bf16(y + l);
}

hipError_t launch_gemv_finish_multi(const float *part, const float *upart, int nsplit, int64_t T, int64_t N,
                                    const bf16_t *B_pool, int64_t r, float s, const SegTable &sg, bf16_t *Y,
                                    hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((N + 255) / 256), (unsigned)T);
  if (nsplit > kFinishMaxSplit || 4 * nsplit > kFinishMaxUp) return hipErrorInvalidValue;
  launch(k_gemv_finish_multi, grid, dim3(256), 0, st, part, upart, nsplit, 4 * nsplit, T, N, B_pool, r, s, sg, Y);
  return hipGetLastError();
}

// Plan of the small-token forward: step depth (W), RG row groups per wave,
// the K split (nsplit equal ranges of whole steps) and the number of
// persistent workgroups.  Chosen from a sweep on MI355X over 8192 x 8192 and
// 28672 x 8192 weights with 1, 8 and 32 tokens, rotating through more than
// 512 MB of weight copies so that the 256 MB last-level cache cannot serve
// them: 256-deep steps up to 16 tokens; more row groups per wave for wide
// weights and more tokens (one activation load then serves several row
// groups); 512 persistent workgroups up to 16 tokens, 256 beyond; up to
// ~4096 work items of at most 16 K ranges.
void nf4_gemv_plan(int64_t T, int64_t N, int64_t K, int *rg, int *w, int *nsplit, int *gmain) {
  int ww = T <= 16 ? 2 : 1;
  while (ww > 1 && K % (128 * ww) != 0) ww /= 2;
  const bool wide = N >= 16384;
  const int rr = T <= 4 ? (wide ? 2 : 1) : (T <= 16 ? (wide ? 4 : 2) : 4);
  const int64_t steps = K / (128 * ww);
  const int64_t tiles = (N + 64 * rr - 1) / (64 * rr);
  int64_t ns = 1;
  for (int64_t d = 1; d <= steps && d <= 16; ++d)
    if (steps % d == 0 && tiles * d <= 4096) ns = d;
  const int64_t items = tiles * ns;
  const int64_t gm = T <= 16 ? 512 : 256;
  *rg = rr;
  *w = ww;
  *nsplit = (int)ns;
  *gmain = (int)(items < gm ? items : gm);
}

template <int MT, int RG, int W>
static void gemv_with(hipStream_t s, const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes,
                      const uint8_t *absmax_q, const float *step, int64_t N, int nsplit, int gmain, const bf16_t *A,
                      int64_t r, float *part, float *upart, const Levels &lv, const SegTable &sg) {
  const int64_t u_wgs = (int64_t)nsplit * (sg.n_seg > 0 ? sg.n_seg : 1);
  launch(k_nf4_gemv<MT, RG, W>, dim3((unsigned)(gmain + u_wgs)), dim3(256), 0, s, X, T, K, codes, absmax_q, step, N,
         nsplit, gmain, A, r, part, upart, lv, sg);
}

template <int MT, int W>
static void gemv_rg(int rg, hipStream_t s, const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes,
                    const uint8_t *absmax_q, const float *step, int64_t N, int nsplit, int gmain, const bf16_t *A,
                    int64_t r, float *part, float *upart, const Levels &lv, const SegTable &sg) {
  if (rg == 4) gemv_with<MT, 4, W>(s, X, T, K, codes, absmax_q, step, N, nsplit, gmain, A, r, part, upart, lv, sg);
  else if (rg == 2) gemv_with<MT, 2, W>(s, X, T, K, codes, absmax_q, step, N, nsplit, gmain, A, r, part, upart, lv, sg);
  else gemv_with<MT, 1, W>(s, X, T, K, codes, absmax_q, step, N, nsplit, gmain, A, r, part, upart, lv, sg);
}

hipError_t launch_nf4_gemv(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                           const float *step, int64_t N, int rg, int w, int nsplit, int gmain, const bf16_t *A,
                           int64_t r, float *part, float *upart, const Levels &lv, hipStream_t s, const SegTable &sg) {
  if (T == 0) return hipSuccess;
  if (T <= 16) {
    if (w == 2) gemv_rg<1, 2>(rg, s, X, T, K, codes, absmax_q, step, N, nsplit, gmain, A, r, part, upart, lv, sg);
    else gemv_rg<1, 1>(rg, s, X, T, K, codes, absmax_q, step, N, nsplit, gmain, A, r, part, upart, lv, sg);
  } else if (T <= 32) {
    gemv_rg<2, 1>(rg, s, X, T, K, codes, absmax_q, step, N, nsplit, gmain, A, r, part, upart, lv, sg);
  } else {
    gemv_rg<4, 1>(rg, s, X, T, K, codes, absmax_q, step, N, nsplit, gmain, A, r, part, upart, lv, sg);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_finish(const float *part, const float *upart, int nsplit, int64_t T, int64_t N,
                              const bf16_t *B, int64_t r, float s, bf16_t *Y, bf16_t *U_out, hipStream_t st,
                              int nsplit_u) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((N + 255) / 256), (unsigned)T);
  const int nup = 4 * (nsplit_u > 0 ? nsplit_u : nsplit);
  if (nsplit > kFinishMaxSplitWide || nup > kFinishMaxUp) return hipErrorInvalidValue;
  const int nbp = (r % 8 == 0 && r <= 32) ? (int)(r / 8) : 0;
#define QLORA_FIN(NBP_, PS_) \
  launch(k_gemv_finish<NBP_, PS_>, grid, dim3(256), 0, st, part, upart, nsplit, nup, T, N, B, r, s, Y, U_out)
#define QLORA_FIN_PS(PS_)                       \
  do {                                          \
    if (nbp == 4) QLORA_FIN(4, PS_);            \
    else if (nbp == 3) QLORA_FIN(3, PS_);       \
    else if (nbp == 2) QLORA_FIN(2, PS_);       \
    else if (nbp == 1) QLORA_FIN(1, PS_);       \
    else QLORA_FIN(0, PS_);                     \
  } while (0)
  if (nsplit <= kFinishMaxSplit) QLORA_FIN_PS(kFinishMaxSplit);
  else QLORA_FIN_PS(kFinishMaxSplitWide);
#undef QLORA_FIN_PS
#undef QLORA_FIN
  return hipGetLastError();
}

// One or two tokens (from three on the MFMA GEMV is faster): tokens held (TT), 2048-column chunks per
// item (CH), register slots (SLOTS: items in flight = SLOTS - 1 beside the one computed) and waves per
// workgroup (NWV; sixteen read the replicated level-pair table).
struct RowsPlan {
  int tt, ch, slots, nwv;
};
static RowsPlan rows_plan(int64_t T, int64_t K) {
  if (T <= 1) return RowsPlan{1, K % 4096 == 0 ? 2 : 1, 2, 16};
  return RowsPlan{2, 1, 2, 4};  // 72 VGPRs: six waves per SIMD with 4-wave workgroups, four with 16-wave ones
}
int nf4_gemv_rows_nseg(int64_t T, int64_t K) {
  if (T < 1 || T > 2 || K <= 0 || K % 2048 != 0) return 0;
  const int64_t ns = K / (2048 * rows_plan(T, K).ch);
  return ns <= kFinishMaxSplit ? (int)ns : 0;
}
bool nf4_gemv_rows_ok(int64_t T, int64_t K) { return nf4_gemv_rows_nseg(T, K) > 0; }

// 3..16 tokens: one token group, 512-column segments; 17..32: two groups, 256-column segments; 33..64:
// four groups, 128-column segments
static int mrows_mt(int64_t T) { return T <= 16 ? 1 : T <= 32 ? 2 : 4; }
// four segments per partial wherever the segments come in fours (a quarter of the partial bytes for
// one barrier per item); for two or four token groups (128 VGPRs or fewer: four waves per SIMD either
// way) eight, in workgroups of eight waves, wherever they come in eights
static int mrows_red(int mt, int64_t nseg) { return mt > 1 && nseg % 8 == 0 ? 8 : nseg % 4 == 0 ? 4 : 1; }
// at most 32 partials, which the wide finish takes: 128 segments in fours, else 32 (four token groups:
// segments in fours only)
// 3..64 tokens with n_in a multiple of eight segments (2048 columns up to 32 tokens, 1024 beyond) and at
// most 32 such parts: the 32-token kernel
static bool m32_ok(int64_t T, int64_t K) {
  const int64_t part = m32_seg(T) * kM32Red;
  return T >= 3 && T <= 64 && K > 0 && K % part == 0 && K / part <= kFinishMaxSplitWide;
}
int nf4_gemv_mrows_nseg(int64_t T, int64_t K) {
  if (m32_ok(T, K)) return (int)(K / m32_seg(T));
  if (T < 3 || T > kMrowsMaxT || K <= 0) return 0;
  const int mt = mrows_mt(T), ks = 512 / mt;
  if (K % ks != 0) return 0;
  const int64_t ns = K / ks;
  if (mt == 4 && ns % 4 != 0) return 0;  // four token groups only with the workgroup sum (registers)
  return ns / mrows_red(mt, ns) <= kFinishMaxSplitWide ? (int)ns : 0;
}
int nf4_gemv_mrows_nparts(int64_t T, int64_t K) {
  if (m32_ok(T, K)) return (int)(K / (m32_seg(T) * kM32Red));
  const int ns = nf4_gemv_mrows_nseg(T, K);
  return ns / mrows_red(mrows_mt(T), ns > 0 ? ns : 1);
}

template <int TG>
static hipError_t m32_go(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                         const float *step, int64_t N, int nseg, int nsplit_u, const bf16_t *A, int64_t r, float *part,
                         float *upart, const Levels &lv, hipStream_t s, int *nseg_out) {
  static thread_local int res = 0;  // workgroups resident at once, per variant and thread
  if (res <= 0) res = resident(k_nf4_gemv_m32<TG>, 64 * kM32Red);
  if (res <= 0) return hipErrorInvalidDeviceFunction;
  const int npart = nseg / kM32Red;
  // main workgroups: what is resident at once (the U workgroups follow them), at most one item each, a
  // multiple of npart
  int64_t g = std::min<int64_t>(res, (N + 31) / 32 * npart);
  g = std::max<int64_t>(npart, g / npart * npart);
  const int gmain = (int)g;
  launch(k_nf4_gemv_m32<TG>, dim3((unsigned)(gmain + nsplit_u)), dim3(64 * kM32Red), 0, s, X, T, K, codes, absmax_q,
         step, N, gmain, nseg, nsplit_u, A, r, part, upart, lv);
  *nseg_out = npart;
  return hipGetLastError();
}
static hipError_t launch_nf4_gemv_m32(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes,
                                      const uint8_t *absmax_q, const float *step, int64_t N, int nseg, int nsplit_u,
                                      const bf16_t *A, int64_t r, float *part, float *upart, const Levels &lv,
                                      hipStream_t s, int *nseg_out) {
#define QLORA_M32(TG_) m32_go<TG_>(X, T, K, codes, absmax_q, step, N, nseg, nsplit_u, A, r, part, upart, lv, s, nseg_out)
  switch ((T + 7) / 8) {
    case 1: return QLORA_M32(1);
    case 2: return QLORA_M32(2);
    case 3: return QLORA_M32(3);
    case 4: return QLORA_M32(4);
    case 5: return QLORA_M32(5);
    case 6: return QLORA_M32(6);
    case 7: return QLORA_M32(7);
    default: return QLORA_M32(8);
  }
#undef QLORA_M32
}

template <int MT, int RED>
static int mrows_resident() {
  static thread_local int res = 0;
  if (res <= 0) res = resident(k_nf4_gemv_mrows<MT, RED>, 64 * (RED == 8 ? 8 : 4));
  return res;
}

hipError_t launch_nf4_gemv_mrows(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                                 const float *step, int64_t N, int nsplit_u, const bf16_t *A, int64_t r, float *part,
                                 float *upart, const Levels &lv, hipStream_t s, int *nseg_out) {
  *nseg_out = 1;
  if (T == 0) return hipSuccess;
  const int nseg = nf4_gemv_mrows_nseg(T, K);
  if (nseg <= 0) return hipErrorInvalidValue;
  if (m32_ok(T, K)) return launch_nf4_gemv_m32(X, T, K, codes, absmax_q, step, N, nseg, nsplit_u, A, r, part, upart, lv,
                                               s, nseg_out);
  const int mt = mrows_mt(T), red = mrows_red(mt, nseg), npart = nseg / red;
  const int res = mt == 1   ? (red == 1 ? mrows_resident<1, 1>() : mrows_resident<1, 4>())
                  : mt == 2 ? (red == 1 ? mrows_resident<2, 1>()
                                        : red == 4 ? mrows_resident<2, 4>() : mrows_resident<2, 8>())
                            : (red == 4 ? mrows_resident<4, 4>() : mrows_resident<4, 8>());
  if (res <= 0) return hipErrorInvalidDeviceFunction;
  // main workgroups: what stays resident beside the U workgroups, at most one item per wave, a multiple
  // of the number of partials (with RED > 1 every workgroup's waves share their items)
  const int64_t per_item = red == 1 ? 4 : 1;
  int64_t g = std::min<int64_t>(std::max(1, res - nsplit_u), ((N + 15) / 16 * npart + per_item - 1) / per_item);
  g = std::max<int64_t>(npart, g / npart * npart);
  const int gmain = (int)g;
  const dim3 grid((unsigned)(gmain + nsplit_u));
  auto go = [&](auto kern) {
    launch(kern, grid, dim3(red == 8 ? 512 : 256), 0, s, X, T, K, codes, absmax_q, step, N, gmain, nseg, nsplit_u,
           A, r, part, upart, lv);
  };
  if (mt == 1)
    red == 1 ? go(k_nf4_gemv_mrows<1, 1>) : go(k_nf4_gemv_mrows<1, 4>);
  else if (mt == 2)
    red == 1 ? go(k_nf4_gemv_mrows<2, 1>) : red == 4 ? go(k_nf4_gemv_mrows<2, 4>) : go(k_nf4_gemv_mrows<2, 8>);
  else
    red == 4 ? go(k_nf4_gemv_mrows<4, 4>) : go(k_nf4_gemv_mrows<4, 8>);
  *nseg_out = npart;
  return hipGetLastError();
}

template <int TT, int CH, int SLOTS, int NWV, int MINW>
static hipError_t rows_go(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                          const float *step, int64_t N, int nseg, int nsplit_u, const bf16_t *A, int64_t r, float *part,
                          float *upart, const Levels &lv, hipStream_t s) {
  static thread_local int res = 0;  // workgroups resident at once, per variant and thread
  if (res <= 0) res = resident(k_nf4_gemv_rows<TT, CH, SLOTS, NWV, MINW>, 64 * NWV);
  if (res <= 0) return hipErrorInvalidDeviceFunction;
  // main workgroups: what is resident at once (the U workgroups follow them), at most one item per wave, a
  // multiple of nseg
  int64_t g = std::min<int64_t>(res, (N * nseg + NWV - 1) / NWV);
  g = std::max<int64_t>(nseg, g / nseg * nseg);
  const int gmain = (int)g;
  launch(k_nf4_gemv_rows<TT, CH, SLOTS, NWV, MINW>, dim3((unsigned)(gmain + nsplit_u)), dim3(64 * NWV), 0, s, X, T,
         K, codes, absmax_q, step, N, gmain, nseg, nsplit_u, A, r, part, upart, lv);
  return hipGetLastError();
}

hipError_t launch_nf4_gemv_rows(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                                const float *step, int64_t N, int nsplit_u, const bf16_t *A, int64_t r, float *part,
                                float *upart, const Levels &lv, hipStream_t s, int *nseg_out) {
  *nseg_out = 1;
  if (T == 0) return hipSuccess;
  const int nseg = nf4_gemv_rows_nseg(T, K);
  if (nseg <= 0) return hipErrorInvalidValue;
  const RowsPlan p = rows_plan(T, K);
  hipError_t e;
  if (p.tt == 1 && p.ch == 2)
    e = rows_go<1, 2, 2, 16, 8>(X, T, K, codes, absmax_q, step, N, nseg, nsplit_u, A, r, part, upart, lv, s);
  else if (p.tt == 1)
    e = rows_go<1, 1, 2, 16, 8>(X, T, K, codes, absmax_q, step, N, nseg, nsplit_u, A, r, part, upart, lv, s);
  else
    e = rows_go<2, 1, 2, 4, 6>(X, T, K, codes, absmax_q, step, N, nseg, nsplit_u, A, r, part, upart, lv, s);
  *nseg_out = nseg;
  return e;
}

}  // namespace qlora
