// launch.h -- host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

// Start/stop events of the launch being timed (set by the C ABI around a timed
// kernel, null otherwise).  hipExtLaunchKernel writes them as part of the
// kernel's own dispatch, so their difference is the kernel's execution time.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents &launch_events();  // per host thread
// Set (per host thread) when a launch was refused because a grid dimension would reach 2^32
// work-items; the C ABI reads and clears it after each launch.  The argument checks keep every
// launch below that, so this is a guard, not a path.
bool &launch_refused();

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t shm, hipStream_t s, Args... args) {
  const uint64_t lim = (uint64_t)1 << 32;
  if ((uint64_t)grid.x * block.x >= lim || (uint64_t)grid.y * block.y >= lim || (uint64_t)grid.z * block.z >= lim) {
    launch_refused() = true;
    return;
  }
  const LaunchEvents &ev = launch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, shm, s, ev.start, ev.stop, 0u, args...);
}

// Workgroups of a kernel resident on the device at once.
template <class Kern>
inline int resident(Kern kern, int threads) {
  int dev = 0, cus = 0, nb = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, 0) != hipSuccess || nb < 1 || cus < 1)
    return 0;
  return nb * cus;
}

typedef uint16_t bf16_t;
struct Levels;
struct Thresholds;

hipError_t launch_quantize_nf4(const float *W, int64_t n_out, int64_t n_in, uint8_t *codes, uint8_t *absmax_q,
                               float *absmax_step, const Thresholds &thr, hipStream_t s);
hipError_t launch_dequant(const uint8_t *codes, const uint8_t *absmax_q, const float *absmax_step, int64_t n_out,
                          int64_t n_in, bf16_t *out, const Levels &lv, hipStream_t s);

// Token segments of a batch that uses several adapters of a pool: tokens
// seg[g] .. seg[g+1]-1 use adapter ad[g] (outside [0, n_pool): none).  Device
// arrays; kernels clamp every entry, so a malformed table cannot make them
// read or write out of bounds.
struct SegTable {
  const int32_t *seg = nullptr;  // [n_seg + 1]
  const int32_t *ad = nullptr;   // [n_seg]
  int n_seg = 0;
  int n_pool = 0;
};

// Output-tile shapes of the fused NF4 GEMMs (rows x columns of the output).
enum {
  NF4_TILE_128x128 = 0,
  NF4_TILE_256x256_W8 = 3,
  NF4_TILE_256x128_W8 = 4,
  NF4_TILE_128x256_W8 = 5,
  NF4_TILE_128x128_W8 = 6
};
int nf4_gemm_pick_tile(int64_t M, int64_t N);

// Y = X W'^T + V Bp^T; with a segment table (sg.seg non-null) the rows of each
// segment use B = Bp + ad * N * r (ldb = r), and rows without an adapter none.
hipError_t launch_nf4_gemm_fwd(int tile, const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes,
                               const uint8_t *absmax_q, const float *step, int64_t N, const bf16_t *V,
                               const bf16_t *Bp, int64_t ldb, int64_t r, int64_t rp, bf16_t *Y, const Levels &lv,
                               hipStream_t s, const SegTable &sg = SegTable(), int nsplit = 1,
                               float *psum = nullptr);
// Reduction ranges for the forward GEMM with `tile` (1: none): more than one only when its tiles cannot
// occupy every CU; the binary32 sums then go to psum [nsplit][T][N] and launch_finalize adds them.
int nf4_gemm_fwd_split(int tile, int64_t T, int64_t N, int64_t K);
// The forward's tile (a narrow output of many tokens: 256x256 tiles with a split reduction).
int nf4_gemm_pick_tile_fwd(int64_t M, int64_t N, int64_t K);
// dX = dY W' + G o (dUp A); with `mask` (keep bits of X, byte (t K + k) / 8,
// bit k % 8) G = keep * q, without it G = 1.
hipError_t launch_nf4_gemm_dx(int tile, const bf16_t *dY, int64_t T, int64_t N, const uint8_t *codes,
                              const uint8_t *absmax_q, const float *step, int64_t K, const bf16_t *dUp, const bf16_t *A,
                              int64_t r, int64_t rp, bf16_t *dX, const Levels &lv, hipStream_t s,
                              const uint8_t *mask = nullptr, float q = 1.f);

// Merge for export: out = W + s B A (bf16 and/or binary32), W = W_base or the decoded NF4 weight.
hipError_t launch_merge(const uint8_t *codes, const uint8_t *absmax_q, const float *step, const bf16_t *W_base,
                        int64_t N, int64_t K, const bf16_t *A, const bf16_t *B, int r, float s, bf16_t *out,
                        float *out_f32, const Levels &lv, hipStream_t st);

// Small-token forward (T <= 64, n_in % 128 == 0): the split-K GEMV over the
// weight (binary32 partials per K range, plus the partials of U = X A^T from
// one extra workgroup per range), then one finishing launch that adds the
// partials in range order, forms V = bf16(s U), adds V B^T and rounds Y.
constexpr int64_t kGemvMaxT = 64;
void nf4_gemv_plan(int64_t T, int64_t N, int64_t K, int *rg, int *w, int *nsplit, int *gmain);
// With a segment table (sg.n_seg > 0) the U partials come per segment and K range, with each
// segment's adapter A + a r K (segments without an adapter leave their rows unwritten).
hipError_t launch_nf4_gemv(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                           const float *step, int64_t N, int rg, int w, int nsplit, int gmain, const bf16_t *A,
                           int64_t r, float *part, float *upart, const Levels &lv, hipStream_t s,
                           const SegTable &sg = SegTable());
hipError_t launch_gemv_finish(const float *part, const float *upart, int nsplit, int64_t T, int64_t N,
                              const bf16_t *B, int64_t r, float s, bf16_t *Y, bf16_t *U_out, hipStream_t st,
                              int nsplit_u = 0);
// Row-streaming GEMV for one or two tokens (K % 2048 == 0, at most 16 row segments): binary32
// partials of nseg row segments (part [nseg][T][N], nseg = nf4_gemv_rows_nseg(T, K), also returned in
// *nseg_out) plus the U partials of nsplit_u K ranges (upart [4 nsplit_u][T][r]).
int nf4_gemv_rows_nseg(int64_t T, int64_t K);  // 0: the kernel does not take (T, K)
// Row-group GEMV for 3..64 tokens.  With 3..32 tokens and K % 2048 == 0 (at most 32 partials) the 32-token
// kernel: 256-column segments, one partial per eight (part [K / 2048][T][N]).  Otherwise segments of 512
// columns up to 16 tokens, 256 up to 32, 128 beyond (at most 32 partials): binary32 partials of the
// nseg = nf4_gemv_mrows_nseg(T, K) segments (part [nseg][T][N]), or of their fours or eights.  Plus the U
// partials as above; *nseg_out is the number of partials written.
int nf4_gemv_mrows_nseg(int64_t T, int64_t K);    // 0: the kernel does not take (T, K)
int nf4_gemv_mrows_nparts(int64_t T, int64_t K);  // partials it writes (0 as above)
hipError_t launch_nf4_gemv_mrows(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                                 const float *step, int64_t N, int nsplit_u, const bf16_t *A, int64_t r, float *part,
                                 float *upart, const Levels &lv, hipStream_t s, int *nseg_out);
bool nf4_gemv_rows_ok(int64_t T, int64_t K);
hipError_t launch_nf4_gemv_rows(const bf16_t *X, int64_t T, int64_t K, const uint8_t *codes, const uint8_t *absmax_q,
                                const float *step, int64_t N, int nsplit_u, const bf16_t *A, int64_t r, float *part,
                                float *upart, const Levels &lv, hipStream_t s, int *nseg_out);
// Many adapters: Y = bf16(sum of the weight partials + bf16(s U[t]) B_a^T) with B_a = B_pool + a N r
// for the adapter a of token t's segment (none: the partials alone).
hipError_t launch_gemv_finish_multi(const float *part, const float *upart, int nsplit, int64_t T, int64_t N,
                                    const bf16_t *B_pool, int64_t r, float s, const SegTable &sg, bf16_t *Y,
                                    hipStream_t st);

// Dropout on the adapter input P (a dense row-major [rows, ld] activation):
// 8-element chunk c of P (flat element index / 8) has its keep bits in byte c
// of `mask`; kept elements become bf16(fl32(x q)), dropped ones 0.
enum { DROP_NONE = 0, DROP_GENERATE = 1, DROP_APPLY = 2 };
struct DropParams {
  uint8_t *mask = nullptr;  // DROP_GENERATE writes it, DROP_APPLY reads it
  uint32_t thr = 0;         // a 16-bit draw below thr drops its element
  float q = 1.f;            // fl32(1 / (1 - p))
  uint32_t key0 = 0, key1 = 0, off0 = 0, off1 = 0;  // generator key and counter words 2, 3
};

// Skinny GEMM of the LoRA branch: C[split][m][j] (j < rn) over one reduction
// chunk; pt / qt select the storage of the long operand P and the rank-wide
// operand Q (see lora_gemm.hip); `drop` (DROP_*) applies dropout to P.
int skinny_rn(int64_t r);
void skinny_plan(int64_t M, int64_t Kred, int *nsplit, int64_t *kchunk);
void skinny_plan_grouped(int64_t M, int64_t n_seg, int64_t Kred, int *nsplit, int64_t *kchunk);
hipError_t launch_skinny(bool pt, bool qt, int rn, const bf16_t *P, int64_t ldp, int64_t M, const bf16_t *Q,
                         int64_t ldq, int64_t Rv, int64_t Kred, int64_t kchunk, int nsplit, float *C, hipStream_t s,
                         int drop = DROP_NONE, const DropParams &dp = DropParams(), bool ct = false);
// U of a batch with many adapters: C[split][t][j] = sum over the range of P[t, k] Q_a[j, k] with
// Q_a = Q_pool + a q_stride for token t's adapter a (rows P [M, ldp], Q_a [r, ldq]; none: zero).
hipError_t launch_skinny_grouped(int rn, const bf16_t *P, int64_t ldp, int64_t M, const bf16_t *Q_pool, int64_t ldq,
                                 int64_t q_stride, int64_t Rv, int64_t Kred, int64_t kchunk, int nsplit,
                                 const SegTable &sg, float *C, hipStream_t s);
hipError_t launch_finalize(const float *part, int nsplit, int64_t M, int64_t N, bf16_t *out1, int64_t ld1, int64_t n1,
                           float scale1, bf16_t *out2, int64_t ld2, int64_t n2, int64_t nvalid2, float scale2,
                           hipStream_t s);
// Two finalize jobs with one output each, in one launch; job b's splits are sstride_b apart (0: M_b N_b).
hipError_t launch_finalize_pair(const float *part_a, int nsplit_a, int64_t M_a, int64_t N_a, bf16_t *out_a,
                                int64_t ld_a, int64_t n_a, float scale_a, const float *part_b, int nsplit_b,
                                int64_t M_b, int64_t N_b, int64_t sstride_b, bf16_t *out_b, int64_t ld_b, int64_t n_b,
                                float scale_b, hipStream_t s);
// The same contraction (pt = 0) with the whole reduction in each workgroup, writing the finalize
// outputs directly (no partial sums, no second launch); lora_rows_ok(rn, M) says where it is used.
bool lora_rows_ok(int rn, int64_t M);
hipError_t launch_lora_rows(bool qt, int rn, const bf16_t *P, int64_t ldp, int64_t M, const bf16_t *Q, int64_t ldq,
                            int64_t Rv, int64_t Kred, bf16_t *out1, int64_t ld1, int64_t n1, float scale1,
                            bf16_t *out2, int64_t ld2, int64_t n2, int64_t nvalid2, float scale2, hipStream_t s);
hipError_t launch_pad_copy(const bf16_t *in, int64_t ldi, int64_t ncols, int64_t M, bf16_t *out, int64_t ldo,
                           hipStream_t s);

}  // namespace qlora
