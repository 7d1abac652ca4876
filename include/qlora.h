/*
 * qlora.h -- C ABI of the MI355X (gfx950) NF4-quantized linear with a LoRA branch.
 *
 * The layer:  Y = X . deq(W)^T + s . (X . A^T) . B^T,   s = fl32(alpha / r),  no bias.
 *
 * Sources (page title, section):
 *  - "What does QLoRA change compared with plain LoRA when fine-tuning Llama?"
 *    (katajob.com), "NF4: 4-bit NormalFloat": 16 levels for a zero-centred
 *    normal, per-block scaling over 64 contiguous weights, blocks expanded to
 *    bf16 inside the matmul and discarded.  "Double quantization": the block
 *    constants are stored in 8 bits with a second-level scale per group.
 *    "What stays in full precision": A and B are bf16, gradients flow through
 *    the dequantized weight, W is never written.
 *  - "QLoRA: fine-tuning a large model on one GPU" (learn.pranaymahendrakar.com),
 *    Researcher level, "LoRA, stated once": h = W0 x + (alpha/r) B A x, with
 *    B of shape d x r and A of shape r x k; Developer level, the printed
 *    adapter shapes lora_A (r, in) and lora_B (out, r).
 *  - "qlora" (chipfoundryservices.com glossary), table "How QLoRA Works": quantize
 *    at load, forward dequantizes then computes, backward in bf16, only the
 *    adapter is trained.
 *
 * Conventions shared by every entry point
 *  - Plain C types only.  bf16 tensors are passed as uint16_t bit patterns.
 *  - Device pointers point to memory of the current HIP device; host pointers
 *    are marked "host".  All tensors are dense and row-major.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued asynchronously on it; no entry point synchronizes the
 *    host, allocates device memory or keeps a pointer after it returns.  The
 *    caller keeps every buffer alive until the stream work is done.
 *  - Argument checks run before any HIP call.  Failures return a negative
 *    QLORA_E* code and leave a message for qlora_last_error(); nothing aborts
 *    and no C++ exception crosses the ABI.  A device fault inside a kernel
 *    surfaces at the caller's next synchronization, as usual for HIP.
 *  - Inputs must be finite (a precondition, not checked).
 *  - Device pointers must be 16-byte aligned.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t qlora_bf16; /* bf16 bit pattern */

#define QLORA_OK 0
#define QLORA_EINVAL (-1)     /* bad pointer, shape, rank, alignment or op          */
#define QLORA_EWORKSPACE (-2) /* workspace smaller than qlora_workspace_bytes says  */
#define QLORA_ENODEV (-3)     /* no HIP device, or the current device is not gfx950 */
#define QLORA_EHIP (-4)       /* a HIP launch or runtime call failed                */

#define QLORA_OP_FWD 0
#define QLORA_OP_BWD 1
#define QLORA_OP_FWD_DROPOUT 2 /* qlora_linear_fwd_dropout; its backward uses QLORA_OP_BWD */
#define QLORA_OP_FWD_MULTI 3   /* qlora_linear_fwd_multi */

#define QLORA_MAX_RANK 128

/*
 * An NF4 weight of logical shape [n_out, n_in] (katajob, "NF4" and "Double
 * quantization").  Layout in device memory:
 *   codes       [n_out * n_in / 2]  byte j holds element 2j (low nibble) and
 *                                   element 2j+1 (high nibble) of the row-major
 *                                   flattened weight; code i = i-th smallest level
 *   absmax_q    [n_out * n_in / 64] 8-bit constant of each 64-element block
 *   absmax_step [ceil(n_out * n_in / 16384)] binary32 step of each group of
 *                                   256 consecutive block constants
 * Decoding: w' = bf16_rne(fl32(level[code] * fl32(absmax_q[b] * absmax_step[b / 256]))).
 * Requirements: n_in % 64 == 0 (a block never straddles a row) and n_out >= 1;
 * qlora_linear_fwd/bwd also need n_out % 8 == 0 (16-byte rows of dY and Y).
 * Both sizes are at most 2^22 and n_out * n_in at most 2^34; the layer calls
 * also need T <= 2^22 and T * n_out, T * n_in below 2^32 (so that no launch
 * reaches 2^32 work-items in a grid dimension; larger sizes give QLORA_EINVAL).
 * The struct itself is host memory; the three arrays are device memory owned
 * by the caller.  qlora_linear_fwd/bwd never write them.
 */
typedef struct qlora_nf4 {
  int64_t n_out;
  int64_t n_in;
  uint8_t *codes;
  uint8_t *absmax_q;
  float *absmax_step;
} qlora_nf4;

/* Byte sizes of the three NF4 arrays for [n_out, n_in] (host only, no HIP call).
 * 4 + 8/64 + 32/16384 = 4.127 bits per weight (katajob, "Double quantization":
 * 0.5 bit/weight of binary32 constants, of which double quantization saves
 * roughly 0.37).  Returns QLORA_EINVAL on a shape the layout does not allow. */
int qlora_nf4_storage(int64_t n_out, int64_t n_in, size_t *codes_bytes, size_t *absmax_q_bytes,
                      size_t *absmax_step_bytes);

/* The 16 NF4 levels, ascending, binary32, into host memory `levels` (no HIP
 * call).  Construction: standard-normal quantiles at probabilities equally
 * spaced between 1/2 and 1 - (1/30 + 1/32)/2, seven below zero and eight above,
 * plus an exact zero, divided by the largest so the extremes are -1 and +1
 * (katajob, "NF4": levels placed for a zero-centred normal). */
int qlora_nf4_codebook(float levels[16]);

/* Workspace bytes needed by `op` (a QLORA_OP_* value) for these
 * sizes, into host *bytes (no HIP call).  The forward workspace is
 * O(T*r + n_out*r + T*n_out) -- the last term only when few tokens or few output
 * tiles make it split the reduction over n_in into at most 16 ranges, each
 * writing binary32 partial sums of Y -- and never O(n_out*n_in): the dequantized
 * weight is never stored. */
int qlora_workspace_bytes(int op, int64_t T, int64_t n_out, int64_t n_in, int32_t r, size_t *bytes);

/* Quantize a binary32 weight W [n_out, n_in] (device) into q's arrays (device,
 * caller-allocated with qlora_nf4_storage sizes).  Block absmax c_b over 64
 * contiguous elements; code = nearest level to fl32(w / c_b), ties to the lower
 * code, c_b = 0 gives code 7; per group of 256 constants, step d = fl32(max/255)
 * and absmax_q = clamp(round_half_even(fl32(c_b / d)), 0, 255).  Codes use the
 * exact binary32 c_b (katajob, "NF4" and "Double quantization"). */
int qlora_quantize_nf4(const float *W, const qlora_nf4 *q, void *stream);

/* Expand q to bf16 W_out [n_out, n_in] (device): w' = bf16_rne(fl32(level[code]
 * * c'_b)) for every weight, the expansion of each block to the compute dtype
 * that the method performs inside the matmul (katajob, "NF4: 4-bit NormalFloat";
 * ainiketan, Module 08, section 3: dequantized on the fly).  W_out is caller-
 * owned, 16-byte aligned, n_out * n_in bf16.  For tests and export only: the
 * forward and backward never materialize the dequantized weight.  Errors:
 * QLORA_EINVAL (NULL or misaligned pointer, shape), QLORA_ENODEV, QLORA_EHIP. */
int qlora_dequant(const qlora_nf4 *q, qlora_bf16 *W_out, void *stream);

/*
 * Forward (pranaymahendrakar, "LoRA, stated once"; glossary, step 3):
 *   U = X . A^T                               [T, r]
 *   Y = X . deq(W)^T + s . U . B^T            [T, n_out],  s = fl32(alpha / r)
 * X [T, n_in], A [r, n_in], B [n_out, r], Y [T, n_out] bf16, device.
 * U_out [T, r] bf16 (device) receives U for the backward, or NULL.
 * T >= 0 (T = 0 does nothing), 1 <= r <= QLORA_MAX_RANK.
 * ws: device workspace of at least qlora_workspace_bytes(QLORA_OP_FWD, ...).
 * Accumulation is binary32; Y is rounded to bf16 once.  For 1 to 32 tokens
 * with n_in % 2048 == 0, and 33 to 64 with n_in % 1024 == 0, the block
 * constant multiplies each block's binary32 dot product with the bf16-rounded
 * levels instead of each weight (the same sum reassociated; the result is
 * within the stated tolerance of the dequantized product, not bit-identical to
 * the tiled path's).
 */
int qlora_linear_fwd(const qlora_bf16 *X, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A, const qlora_bf16 *B,
                     int32_t r, float alpha, qlora_bf16 *Y, qlora_bf16 *U_out, void *ws, size_t ws_bytes,
                     void *stream);

/*
 * The same forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * identical arguments and results, without ws / ws_bytes.  Its workspace is a
 * static device array of 128 MiB per GPU, reserved when the library's code is
 * loaded on that GPU and held until the process ends; the call itself makes no
 * allocation.  Every forward of this build's workloads fits (the largest, 4096
 * tokens against a 1024 x 8192 weight with its reduction split in four ranges,
 * needs 65 MiB; 64 tokens against 28672 x 8192 need 61 MiB); a shape whose forward
 * needs more returns QLORA_EWORKSPACE before any HIP call.  All calls on one
 * GPU share the array: calls that overlap in time on that GPU (other streams,
 * other host threads) race and must be ordered by the caller.  Nothing in the
 * array needs to start at zero.  Errors as for qlora_linear_fwd, plus QLORA_EHIP
 * if the array's device address cannot be obtained.
 */
int qlora_linear_fwd_noalloc(const qlora_bf16 *X, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A,
                             const qlora_bf16 *B, int32_t r, float alpha, qlora_bf16 *Y, qlora_bf16 *U_out,
                             void *stream);

/*
 * Backward of the forward above with respect to X, A and B; W gets no gradient
 * (katajob, "What stays in full precision"; glossary, step 4):
 *   dU = s . dY . B                 [T, r]
 *   dA = dU^T . X                   [r, n_in]
 *   dB = s . dY^T . U               [n_out, r]
 *   dX = dY . deq(W) + dU . A       [T, n_in]
 * dY [T, n_out] bf16 device.  U [T, r] as saved by the forward, or NULL to
 * recompute it from X and A.  dX may be NULL to skip it.  dA, dB, dX are
 * overwritten (never accumulated); with T = 0, dA and dB are set to zero.
 * ws: at least qlora_workspace_bytes(QLORA_OP_BWD, ...).  The reductions over
 * T and n_out run in a fixed order, so results are bitwise repeatable.
 */
int qlora_linear_bwd(const qlora_bf16 *X, const qlora_bf16 *dY, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A,
                     const qlora_bf16 *B, int32_t r, float alpha, const qlora_bf16 *U, qlora_bf16 *dX,
                     qlora_bf16 *dA, qlora_bf16 *dB, void *ws, size_t ws_bytes, void *stream);

/*
 * LoRA dropout on the adapter input ("Module 08 - QLoRA & Quantization",
 * ainiketan.in, "4. QLoRA in code", and the Developer level of the
 * pranaymahendrakar page configure lora_dropout = 0.05).  Inverted dropout on
 * the adapter branch only; the base product reads X itself:
 *   Xd = keep o bf16(fl32(X q)),  q = fl32(1 / (1 - p))
 *   U  = Xd . A^T
 *   Y  = X . deq(W)^T + s . U . B^T
 * Keep bits: X is viewed as a flat row-major array of T * n_in bf16 values;
 * its 8-element chunk c (elements 8c .. 8c+7) is one Philox4x32-10 block
 * (Salmon, Moraes, Dror, Shaw, SC 2011) with counter words
 * (c mod 2^32, c div 2^32, offset mod 2^32, offset div 2^32) and key words
 * (seed mod 2^32, seed div 2^32).  Element 8c+i takes the 16-bit draw formed by
 * bits 16(i mod 2) .. 16(i mod 2)+15 of output word i div 2 and is kept iff the
 * draw is >= D = round_half_even(p * 65536).  Bit i of byte c of mask_out is
 * its keep flag.
 * mask_out: device, [T * n_in / 8] bytes, 16-byte aligned, written completely
 * (it is the backward's input).  0 <= p < 1 (p = 0 keeps everything).  Use
 * `offset` to draw a fresh mask per step with one seed.  The workspace is
 * qlora_workspace_bytes(QLORA_OP_FWD_DROPOUT, ...).  Other arguments and
 * conventions as for qlora_linear_fwd.
 */
int qlora_linear_fwd_dropout(const qlora_bf16 *X, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A,
                             const qlora_bf16 *B, int32_t r, float alpha, float p, uint64_t seed, uint64_t offset,
                             uint8_t *mask_out, qlora_bf16 *Y, qlora_bf16 *U_out, void *ws, size_t ws_bytes,
                             void *stream);

/*
 * Backward of qlora_linear_fwd_dropout (same p, the mask it wrote, and the U
 * it saved or NULL to recompute U = Xd . A^T).  The derivative of the dropout
 * is keep * q (straight through the rounding to bf16):
 *   dU = s . dY . B
 *   dA = dU^T . Xd
 *   dB = s . dY^T . U
 *   dX = dY . deq(W) + (keep q) o (dU . A)
 * Workspace: qlora_workspace_bytes(QLORA_OP_BWD, ...).  Other arguments and
 * conventions as for qlora_linear_bwd.
 */
int qlora_linear_bwd_dropout(const qlora_bf16 *X, const qlora_bf16 *dY, int64_t T, const qlora_nf4 *q,
                             const qlora_bf16 *A, const qlora_bf16 *B, int32_t r, float alpha, float p,
                             const uint8_t *mask, const qlora_bf16 *U, qlora_bf16 *dX, qlora_bf16 *dA,
                             qlora_bf16 *dB, void *ws, size_t ws_bytes, void *stream);

/*
 * Forward of a batch whose tokens use different adapters over one NF4 base
 * (pranaymahendrakar, Researcher level, "The variants worth knowing": one base
 * model in memory, many adapters, requests for different adapters batched
 * together).  The pool holds n_pool adapters of one rank r:
 *   A_pool [n_pool, r, n_in], B_pool [n_pool, n_out, r]   bf16, device
 * (pad an adapter of smaller rank with zero rows of A and zero columns of B).
 * Tokens seg_offsets[g] .. seg_offsets[g+1]-1 use adapter seg_adapter[g]; an
 * index outside [0, n_pool) means none (the base product alone).  For token t
 * with adapter a:  Y[t] = X[t] . deq(W)^T + s . (X[t] . A_a^T) . B_a^T.
 * seg_offsets [n_seg + 1] and seg_adapter [n_seg]: device int32 arrays, read by
 * the kernels (no host copy); they must describe a partition of [0, T):
 * seg_offsets[0] = 0, non-decreasing, seg_offsets[n_seg] = T.  The kernels clamp
 * every entry, so a malformed table gives wrong rows but no access out of
 * bounds.  r % 8 == 0, 1 <= n_seg.  Workspace: QLORA_OP_FWD_MULTI.  Cost: the
 * base product once; U per 128-token tile of each segment; each output tile
 * adds one rank-deep up-projection per segment that meets its rows (few
 * tokens, at most 64: per token in the finishing kernel).
 */
int qlora_linear_fwd_multi(const qlora_bf16 *X, int64_t T, const qlora_nf4 *q, const qlora_bf16 *A_pool,
                           const qlora_bf16 *B_pool, int32_t n_pool, int32_t r, float alpha, const int32_t *seg_offsets,
                           const int32_t *seg_adapter, int32_t n_seg, qlora_bf16 *Y, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * Merge a trained adapter into a 16-bit base for export ("Module 08 - QLoRA &
 * Quantization", ainiketan.in, "7. A subtle but important deployment note";
 * katajob, "What it costs", 3. Merging):
 *   Wm = W + s . B . A        [n_out, n_in],  s = fl32(alpha / r)
 * W is either the reloaded bf16 base W_base [n_out, n_in] (device; q NULL) or
 * the dequantized NF4 weight deq(q) (q non-NULL; W_base NULL; its shape must
 * equal n_out x n_in).  Exactly one of them.  A [r, n_in], B [n_out, r] bf16.
 * Arithmetic: P = B . A in binary32 (MFMA), m = fl32(w + fl32(s P)).
 * Outputs (device, either may be NULL but not both): W_out bf16 = bf16_rne(m);
 * W_out_f32 binary32 = m, the input qlora_quantize_nf4 takes to quantize the
 * merged weight again.  n_in % 64 == 0, 1 <= r <= QLORA_MAX_RANK.
 */
int qlora_merge(const qlora_nf4 *q, const qlora_bf16 *W_base, int64_t n_out, int64_t n_in, const qlora_bf16 *A,
                const qlora_bf16 *B, int32_t r, float alpha, qlora_bf16 *W_out, float *W_out_f32, void *stream);

/*
 * One AdamW step of the adapter matrices ("What stays in full precision",
 * katajob: A and B are bf16 with ordinary AdamW state; pranaymahendrakar,
 * Developer level, "The walkthrough": about 8 bytes of state per trainable
 * parameter).  Decoupled weight decay (Loshchilov and Hutter, ICLR 2019) with a
 * constant schedule multiplier; step t >= 1:
 *   m     = b1 m + (1 - b1) g
 *   v     = b2 v + (1 - b2) g^2
 *   theta = theta - lr (wd theta + (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps))
 * in binary32 (each operation rounded once).  The hyperparameters are binary64;
 * the host forms b1, 1 - b1, b2, 1 - b2, eps, 1 - lr wd, lr / (1 - b1^t) and
 * sqrt(1 - b2^t) in binary64 and rounds each to binary32 once.
 * theta is `master` when given (updated in place), else the bf16 `param`
 * widened; `param` receives bf16_rne(theta).
 * Every array of a tensor is device memory of n elements, 16-byte aligned, and
 * updated in place except `grad`; tensors must not overlap.  `tensors` is a
 * host array of `count` descriptors (any count; the library launches one kernel
 * per 32 of them; no elements at all means no HIP call).  0 <= beta1, beta2 < 1,
 * eps > 0, lr >= 0, weight_decay >= 0, all finite.
 */
typedef struct qlora_adamw_tensor {
  qlora_bf16 *param;      /* [n] bf16 parameter                       */
  const qlora_bf16 *grad; /* [n] bf16 gradient (e.g. dA or dB)        */
  float *exp_avg;         /* [n] binary32 first moment m              */
  float *exp_avg_sq;      /* [n] binary32 second moment v             */
  float *master;          /* [n] binary32 master copy of param, or NULL */
  int64_t n;
} qlora_adamw_tensor;

int qlora_adamw_step(const qlora_adamw_tensor *tensors, int32_t count, double lr, double beta1, double beta2,
                     double eps, double weight_decay, int64_t step, void *stream);

/*
 * The same AdamW step with block-wise 8-bit moments ("Module 08 - QLoRA &
 * Quantization", ainiketan.in, "4. QLoRA in code" and "5. Other memory-saving
 * levers": paged_adamw_8bit; block-wise state quantization after Dettmers et
 * al., "8-bit Optimizers via Block-wise Quantization", ICLR 2022; paging to host
 * memory is not done).  Each moment of a tensor of n elements is stored as n
 * 8-bit codes plus one binary32 absmax per block of 2048 consecutive elements
 * (ceil(n / 2048) of them).  A code is a byte of a dynamic book: for the first
 * moment bit 7 is the sign and, among the other 7 bits, E = the number of
 * leading zeros, then a set indicator bit, then F = 6 - E fraction bits f, the
 * magnitude being fl32((0.1 + 0.9 ((f + 1) / 2^F)) / 10^E) (binary64 in that
 * order; all-zero bits: 0); for the second moment all 8 bits are used the same
 * way (F = 7 - E).  A stored moment is fl32(book[code] * absmax).  Each step:
 * decode, the binary32 update of qlora_adamw_step, new absmax = the block's
 * largest magnitude, code = the nearest book magnitude to fl32(value / absmax)
 * (ties to the smaller; 0 when the absmax is 0).  Zeroed codes and absmax are
 * the zero state.  Codes 16-byte aligned; absmax 4-byte aligned; the rest as
 * for qlora_adamw_step.
 */
typedef struct qlora_adamw8_tensor {
  qlora_bf16 *param;
  const qlora_bf16 *grad;
  uint8_t *exp_avg_code;     /* [n]               */
  float *exp_avg_absmax;     /* [ceil(n / 2048)]  */
  uint8_t *exp_avg_sq_code;  /* [n]               */
  float *exp_avg_sq_absmax;  /* [ceil(n / 2048)]  */
  float *master;             /* [n] or NULL       */
  int64_t n;
} qlora_adamw8_tensor;

int qlora_adamw8_step(const qlora_adamw8_tensor *tensors, int32_t count, double lr, double beta1, double beta2,
                      double eps, double weight_decay, int64_t step, void *stream);

/* Static text for a QLORA_E* code. */
const char *qlora_strerror(int code);

/* Detail of the last failing call on this host thread ("" if none). */
const char *qlora_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
