/*
 * qlora_oracle.c -- plain, slow CPU oracle for the NF4-quantized linear with a
 * LoRA branch.  TEST INFRASTRUCTURE ONLY: the product path never links, loads
 * or calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no fused multiply-add contraction, no flush-to-zero: every float operation
 * below is one IEEE-754 binary32 or binary64 operation rounded to nearest-even).
 *
 * Sources, cited by page title and section:
 *  [NF4]  "What does QLoRA change compared with plain LoRA when fine-tuning
 *         Llama?" (katajob), section "NF4: 4-bit NormalFloat": sixteen levels
 *         tuned to a zero-centred normal; per-block scaling over contiguous
 *         groups of (commonly) 64 weights, one constant per block; at run time
 *         a block is expanded to the compute dtype (bfloat16) for the matmul.
 *  [DQ]   same page, section "Double quantization": the per-block constants are
 *         themselves quantized to 8 bits with a second-level scale per group.
 *  [LORA] "QLoRA: fine-tuning a large model on one GPU" (pranaymahendrakar),
 *         Researcher level, "LoRA, stated once": h = W0 x + (alpha/r) B A x with
 *         B in R^{d x r}, A in R^{r x k}.
 *  [BWD]  same page, "What QLoRA adds", and the katajob page, "What stays in
 *         full precision": gradients reach A and B through the dequantized
 *         base weight; the base weight gets no gradient and no update.
 *  [STEPS] "qlora" glossary (chipfoundryservices), table "How QLoRA Works":
 *         quantize at load (4-bit), forward dequantizes then computes, backward
 *         in bfloat16, only the adapter is updated.
 *  [OPT8] "Module 08 - QLoRA & Quantization" (ainiketan), "4. QLoRA in code" and
 *         "5. Other memory-saving levers": paged 8-bit AdamW state.
 *  [OPT]  katajob, "What stays in full precision" (A and B keep ordinary AdamW
 *         state) and pranaymahendrakar, Developer level, "The walkthrough" (about
 *         8 bytes of Adam state per trainable parameter).
 *  [MULTI] pranaymahendrakar, Researcher level, "The variants worth knowing":
 *         one base model in memory, many adapters, requests for different
 *         adapters batched together.
 *  [MERGE] "Module 08 - QLoRA & Quantization" (ainiketan), "7. A subtle but
 *         important deployment note"; katajob, "What it costs" (3. Merging).
 *  [DROP] "Module 08 - QLoRA & Quantization" (ainiketan), "4. QLoRA in code":
 *         the adapter config sets lora_dropout = 0.05 (so does the Developer
 *         level of the pranaymahendrakar page).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - level construction: normal quantiles at equally spaced probabilities
 *    between 1/2 and p_hi = 1 - (1/30 + 1/32)/2, eight on the positive side and
 *    seven on the negative side, plus an exact zero, all divided by the largest
 *    quantile so that the extremes are exactly -1 and +1; rounded to binary32
 *    once.  (The value of p_hi is not on the pages; it is a declared choice.)
 *  - code i is the i-th smallest level; element 2j of the row-major weight goes
 *    into the low nibble of byte j, element 2j+1 into the high nibble;
 *  - encode: x = fl32(w / c_b); nearest level, ties to the lower code; c_b = 0
 *    gives code 7 (the zero level) for the whole block;
 *  - double quantization: unsigned 8-bit linear codes over groups of 256
 *    consecutive block constants, step d = fl32(max / 255), q = round-half-even
 *    of fl32(c / d) clamped to [0, 255]; decoding uses c' = fl32(q * d);
 *  - dequant: w' = bf16_rne(fl32(level[code] * c'));
 *  - scale s = fl32(alpha / r); no bias; dropout on the adapter input only
 *    where a caller asks for it (the [DROP] functions at the end).
 *
 * The forward and backward contractions are written out in binary64 from their
 * definitions; inputs arrive as binary64 arrays (the bf16 activations and
 * adapters widen exactly), the dequantized weight as bf16 bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------- codebook */

/* Standard normal CDF written with the complementary error function. */
static double std_normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Standard normal quantile by bisection on the CDF, run until the bracket
 * cannot shrink any further in binary64. */
static double std_normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (;;) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (std_normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  /* pick whichever end of the final bracket has the closer CDF value */
  return (fabs(std_normal_cdf(lo) - p) <= fabs(std_normal_cdf(hi) - p)) ? lo : hi;
}

/* The 16 NF4 levels, ascending, in binary64 before rounding (see the reading
 * above).  Exposed so the tests can check the unrounded values too. */
void oracle_nf4_levels_f64(double out[16]) {
  const double p_hi = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
  const double qmax = std_normal_quantile(p_hi);
  double v[16];
  int n = 0;
  /* seven negative levels: -Phi^-1(1/2 + j (p_hi - 1/2) / 7), j = 7..1 */
  for (int j = 7; j >= 1; --j) v[n++] = -std_normal_quantile(0.5 + j * (p_hi - 0.5) / 7.0) / qmax;
  v[n++] = 0.0;
  /* eight positive levels: Phi^-1(1/2 + i (p_hi - 1/2) / 8), i = 1..8 */
  for (int i = 1; i <= 8; ++i) v[n++] = std_normal_quantile(0.5 + i * (p_hi - 0.5) / 8.0) / qmax;
  /* already ascending by construction; keep an explicit sort for clarity */
  for (int i = 1; i < 16; ++i)
    for (int j = i; j > 0 && v[j - 1] > v[j]; --j) { double t = v[j]; v[j] = v[j - 1]; v[j - 1] = t; }
  memcpy(out, v, sizeof v);
}

void oracle_nf4_levels(float out[16]) {
  double v[16];
  oracle_nf4_levels_f64(v);
  for (int i = 0; i < 16; ++i) out[i] = (float)v[i]; /* one rounding to binary32 */
}

/* ------------------------------------------------------------- bf16 helper */

/* binary32 -> bfloat16 bit pattern, round to nearest, ties to even. */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40); /* NaN stays NaN */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* --------------------------------------------------------------- quantize */

/* Nearest level to x, ties to the lower code.  Distances are taken in binary64:
 * for |x| >= 2^-29 both operands are binary32 values in [-1, 1] whose ulps are
 * at least 2^-52, so every difference is exact; for smaller |x| the zero level
 * is nearer than any other by a wide margin.  Hence this is the exact argmin. */
static int nearest_code(float x, const float lv[16]) {
  int best = 0;
  double bd = fabs((double)x - (double)lv[0]);
  for (int i = 1; i < 16; ++i) {
    double d = fabs((double)x - (double)lv[i]);
    if (d < bd) { bd = d; best = i; } /* strict: an equal distance keeps the lower code */
  }
  return best;
}

/*
 * Block-wise NF4 quantization with double quantization of the constants.
 *   W          [n_out * n_in] binary32, row-major; n_in % 64 == 0
 *   codes      [n_out * n_in / 2]
 *   absmax_q   [n_out * n_in / 64]          8-bit block constants
 *   absmax_step[ceil(n_out * n_in / 64 / 256)] binary32 second-level steps
 *   absmax_f32 [n_out * n_in / 64] or NULL: the un-quantized block absmax
 * Returns 0, or -1 when n_in is not a multiple of 64.
 */
int oracle_quantize_nf4(const float *W, int64_t n_out, int64_t n_in, uint8_t *codes, uint8_t *absmax_q,
                        float *absmax_step, float *absmax_f32) {
  if (n_in % 64 != 0 || n_out < 0) return -1;
  float lv[16];
  oracle_nf4_levels(lv);
  const int64_t nblk = n_out * n_in / 64;
  float *c = (float *)malloc(sizeof(float) * (size_t)(nblk > 0 ? nblk : 1));
  /* [NF4] one absmax per 64 contiguous weights; encode with the exact binary32 constant */
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nblk; ++b) {
    const float *w = W + b * 64;
    float m = 0.0f;
    for (int e = 0; e < 64; ++e) { float a = fabsf(w[e]); if (a > m) m = a; }
    c[b] = m;
    int q[64];
    for (int e = 0; e < 64; ++e) q[e] = (m == 0.0f) ? 7 : nearest_code(w[e] / m, lv);
    for (int j = 0; j < 32; ++j) codes[b * 32 + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
  }
  /* [DQ] groups of 256 consecutive constants, unsigned 8-bit, step = group max / 255 */
  const int64_t ngrp = (nblk + 255) / 256;
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < ngrp; ++g) {
    const int64_t b0 = g * 256, b1 = (b0 + 256 < nblk) ? b0 + 256 : nblk;
    float s = 0.0f;
    for (int64_t b = b0; b < b1; ++b) if (c[b] > s) s = c[b];
    const float d = s / 255.0f;
    absmax_step[g] = (s == 0.0f) ? 0.0f : d;
    for (int64_t b = b0; b < b1; ++b) {
      int qb = 0;
      if (s != 0.0f) {
        float t = c[b] / d;
        float r = rintf(t); /* default rounding mode: nearest, ties to even */
        qb = (r < 0.0f) ? 0 : (r > 255.0f) ? 255 : (int)r;
      }
      absmax_q[b] = (uint8_t)qb;
    }
  }
  if (absmax_f32) memcpy(absmax_f32, c, sizeof(float) * (size_t)nblk);
  free(c);
  return 0;
}

/* Dequantize to bf16 bit patterns: w' = bf16_rne(fl32(level[code] * fl32(q * d))). */
int oracle_dequant(const uint8_t *codes, const uint8_t *absmax_q, const float *absmax_step, int64_t n_out,
                   int64_t n_in, uint16_t *W_out) {
  if (n_in % 64 != 0 || n_out < 0) return -1;
  float lv[16];
  oracle_nf4_levels(lv);
  const int64_t n = n_out * n_in;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int64_t b = i / 64, g = b / 256;
    const float cq = (float)absmax_q[b] * absmax_step[g];
    const int code = (i & 1) ? (codes[i >> 1] >> 4) : (codes[i >> 1] & 15);
    W_out[i] = f32_to_bf16_rne(lv[code] * cq);
  }
  return 0;
}

static inline double bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ---------------------------------------------------------------- forward */

/*
 * [LORA] forward for selected token rows, with the adapter reading Xa (the
 * layer input itself, or its dropped-out copy, see [DROP] below):
 *   U[t, j] = sum_k Xa[t, k] A[j, k]
 *   Y[t, n] = sum_k X[t, k] W'[n, k] + s * sum_j U[t, j] B[n, j],   s = fl32(alpha / r)
 * X, Xa [T, K], A [r, K], B [N, r] binary64; Wdq [N, K] bf16 bits.
 * rows: n_rows indices into [0, T) (or NULL for all rows, then n_rows = T).
 * Y [n_rows, N], U [n_rows, r] binary64 (U may be NULL).
 */
void oracle_linear_fwd_xa(const double *X, const double *Xa, int64_t T, const uint16_t *Wdq, int64_t N, int64_t K,
                          const double *A, const double *B, int32_t r, float alpha, const int64_t *rows,
                          int64_t n_rows, double *Y, double *U) {
  const double s = (double)(alpha / (float)r);
  if (!rows) n_rows = T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    const int64_t t = rows ? rows[i] : i;
    const double *x = X + t * K, *xa = Xa + t * K;
    double *u = (double *)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
    for (int32_t j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += xa[k] * A[(int64_t)j * K + k];
      u[j] = acc;
      if (U) U[i * r + j] = acc;
    }
    for (int64_t n = 0; n < N; ++n) {
      const uint16_t *w = Wdq + n * K;
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += x[k] * bf16_to_f64(w[k]);
      double lora = 0.0;
      for (int32_t j = 0; j < r; ++j) lora += u[j] * B[n * r + j];
      Y[i * N + n] = acc + s * lora;
    }
    free(u);
  }
}

/* The layer without dropout: the adapter reads X itself. */
void oracle_linear_fwd(const double *X, int64_t T, const uint16_t *Wdq, int64_t N, int64_t K, const double *A,
                       const double *B, int32_t r, float alpha, const int64_t *rows, int64_t n_rows, double *Y,
                       double *U) {
  oracle_linear_fwd_xa(X, X, T, Wdq, N, K, A, B, r, alpha, rows, n_rows, Y, U);
}

/* --------------------------------------------------------------- backward */

/*
 * [BWD] backward of the layer above with respect to X, A and B (W gets none):
 *   U  = Xa A^T                     [T, r]
 *   dU = s * dY B                   [T, r]
 *   dA = dU^T Xa                    [r, K]
 *   dB = s * dY^T U                 [N, r]
 *   dX = dY W' + G o (dU A)         [T, K]   (only for the selected rows)
 * G [T, K] is the elementwise derivative of Xa with respect to X (NULL: Xa = X,
 * G = 1); "o" is the elementwise product.
 * dX [n_rows, K] (may be NULL), dA [r, K], dB [N, r] binary64.
 */
void oracle_linear_bwd_xa(const double *X, const double *Xa, const double *G, const double *dY, int64_t T,
                          const uint16_t *Wdq, int64_t N, int64_t K, const double *A, const double *B, int32_t r,
                          float alpha, const int64_t *rows, int64_t n_rows, double *dX, double *dA, double *dB) {
  const double s = (double)(alpha / (float)r);
  double *U = (double *)calloc((size_t)(T * r > 0 ? T * r : 1), sizeof(double));
  double *dU = (double *)calloc((size_t)(T * r > 0 ? T * r : 1), sizeof(double));
  /* U[t, j] = sum_k Xa[t, k] A[j, k];  dU[t, j] = s * sum_n dY[t, n] B[n, j] */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < r; ++j) {
      double a = 0.0;
      for (int64_t k = 0; k < K; ++k) a += Xa[t * K + k] * A[(int64_t)j * K + k];
      U[t * r + j] = a;
    }
    double *g = dU + t * r;
    for (int64_t n = 0; n < N; ++n) {
      const double y = dY[t * N + n];
      for (int32_t j = 0; j < r; ++j) g[j] += y * B[n * r + j];
    }
    for (int32_t j = 0; j < r; ++j) g[j] *= s;
  }
  /* dA[j, :] = sum_t dU[t, j] Xa[t, :] */
#pragma omp parallel for schedule(static)
  for (int32_t j = 0; j < r; ++j) {
    double *out = dA + (int64_t)j * K;
    for (int64_t k = 0; k < K; ++k) out[k] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const double a = dU[t * r + j];
      for (int64_t k = 0; k < K; ++k) out[k] += a * Xa[t * K + k];
    }
  }
  /* dB[n, :] = s * sum_t dY[t, n] U[t, :]   (each thread owns a range of rows n) */
#pragma omp parallel
  {
#ifdef _OPENMP
    const int64_t nth = omp_get_num_threads(), me = omp_get_thread_num();
#else
    const int64_t nth = 1, me = 0;
#endif
    const int64_t n0 = N * me / nth, n1 = N * (me + 1) / nth;
    for (int64_t n = n0; n < n1; ++n)
      for (int32_t j = 0; j < r; ++j) dB[n * r + j] = 0.0;
    for (int64_t t = 0; t < T; ++t)
      for (int64_t n = n0; n < n1; ++n) {
        const double y = dY[t * N + n];
        for (int32_t j = 0; j < r; ++j) dB[n * r + j] += y * U[t * r + j];
      }
    for (int64_t n = n0; n < n1; ++n)
      for (int32_t j = 0; j < r; ++j) dB[n * r + j] *= s;
  }
  /* dX[t, k] = sum_n dY[t, n] W'[n, k] + G[t, k] * sum_j dU[t, j] A[j, k] */
  if (dX) {
    if (!rows) n_rows = T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      const int64_t t = rows ? rows[i] : i;
      double *out = dX + i * K;
      for (int64_t k = 0; k < K; ++k) out[k] = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double g = dY[t * N + n];
        const uint16_t *w = Wdq + n * K;
        for (int64_t k = 0; k < K; ++k) out[k] += g * bf16_to_f64(w[k]);
      }
      if (!G) {
        for (int32_t j = 0; j < r; ++j) {
          const double g = dU[t * r + j];
          for (int64_t k = 0; k < K; ++k) out[k] += g * A[(int64_t)j * K + k];
        }
      } else {
        for (int64_t k = 0; k < K; ++k) {
          double lora = 0.0;
          for (int32_t j = 0; j < r; ++j) lora += dU[t * r + j] * A[(int64_t)j * K + k];
          out[k] += G[t * K + k] * lora;
        }
      }
    }
  }
  free(U);
  free(dU);
}

/* The layer without dropout. */
void oracle_linear_bwd(const double *X, const double *dY, int64_t T, const uint16_t *Wdq, int64_t N, int64_t K,
                       const double *A, const double *B, int32_t r, float alpha, const int64_t *rows,
                       int64_t n_rows, double *dX, double *dA, double *dB) {
  oracle_linear_bwd_xa(X, X, NULL, dY, T, Wdq, N, K, A, B, r, alpha, rows, n_rows, dX, dA, dB);
}

/* ------------------------------------------------------------ LoRA dropout */

/*
 * [DROP] "Module 08 - QLoRA & Quantization" (ainiketan.in), section "4. QLoRA in
 * code", and the Developer level of the pranaymahendrakar page: the adapter is
 * configured with lora_dropout = 0.05.  The pages give only the probability;
 * the readings taken here (each listed in the design notes):
 *  - inverted dropout on the adapter's input only: Xa = keep ? bf16_rne(fl32(x q)) : 0,
 *    q = fl32(1 / (1 - p)) (one binary64 division, rounded once); the base
 *    product reads the undropped X;
 *  - its derivative is the straight-through keep * q (the rounding to bf16 is
 *    not differentiated), so dX gets G = keep * q on the adapter term;
 *  - keep decisions come from the counter-based generator Philox4x32-10
 *    (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
 *    numbers: as easy as 1, 2, 3", SC 2011).  X is viewed as a flat row-major
 *    array; its 8-element chunk c = (t K + k) / 8 is one generator call with
 *    counter (c mod 2^32, c div 2^32, offset mod 2^32, offset div 2^32) and key
 *    (seed mod 2^32, seed div 2^32).  Element i of the chunk takes the 16-bit
 *    draw h_i = bits 16 (i mod 2) .. +15 of output word i div 2 and is kept
 *    iff h_i >= D, D = round_half_even(p 65536);
 *  - the keep flags are stored as bits: bit i of byte c.
 */

/* Philox4x32 with 10 rounds: each round multiplies words 0 and 2 by the two
 * round constants, keeping both halves of the 64-bit products, mixes the high
 * halves with words 1 and 3 and the key by exclusive or, and swaps the
 * pairs; the key is advanced by the two Weyl constants between rounds. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t y0 = hi1 ^ x1 ^ k0, y1 = lo1, y2 = hi0 ^ x3 ^ k1, y3 = lo0;
    x0 = y0;
    x1 = y1;
    x2 = y2;
    x3 = y3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

/* Drop threshold D for probability p (0 <= p < 1). */
uint32_t oracle_dropout_threshold(double p) { return (uint32_t)nearbyint(p * 65536.0); }

/* Keep bits of n_chunks 8-element chunks (n_chunks = T K / 8). */
void oracle_dropout_mask(int64_t n_chunks, double p, uint64_t seed, uint64_t offset, uint8_t *mask) {
  const uint32_t D = oracle_dropout_threshold(p);
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < n_chunks; ++c) {
    const uint32_t ctr[4] = {(uint32_t)c, (uint32_t)((uint64_t)c >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
    uint32_t o[4];
    oracle_philox4x32_10(ctr, key, o);
    uint8_t byte = 0;
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = (o[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      if (h >= D) byte |= (uint8_t)(1u << i);
    }
    mask[c] = byte;
  }
}

/* Xa as bf16 bits and G = keep * q in binary64, from X (bf16 bits) and the keep bits. */
void oracle_dropout_apply(const uint16_t *X, int64_t n, const uint8_t *mask, double p, uint16_t *Xa, double *G) {
  const float q = (float)(1.0 / (1.0 - p));
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int keep = (mask[i >> 3] >> (i & 7)) & 1;
    uint32_t u = (uint32_t)X[i] << 16;
    float x;
    memcpy(&x, &u, 4);
    if (Xa) Xa[i] = keep ? f32_to_bf16_rne(x * q) : 0;
    if (G) G[i] = keep ? (double)q : 0.0;
  }
}

/* ------------------------------------------------------------------ AdamW */

/*
 * [OPT] katajob, "What stays in full precision": A and B are bf16 tensors with
 * ordinary AdamW state; pranaymahendrakar, Developer level, "The walkthrough":
 * Adam keeps about 8 bytes per trainable parameter (two binary32 moments).
 * AdamW is Adam with weight decay decoupled from the gradient (I. Loshchilov,
 * F. Hutter, "Decoupled Weight Decay Regularization", ICLR 2019), here with a
 * constant schedule multiplier.  One step t >= 1 over n parameters, all in
 * binary64:
 *   m     <- b1 m + (1 - b1) g
 *   v     <- b2 v + (1 - b2) g^2
 *   theta <- theta - lr (wd theta + (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps))
 * (the decay term uses the parameter before the step).  theta, m, v in place.
 */
void oracle_adamw_step(double *theta, const double *g, double *m, double *v, int64_t n, double lr, double b1,
                       double b2, double eps, double wd, int64_t t) {
  const double bc1 = 1.0 - pow(b1, (double)t), bc2 = 1.0 - pow(b2, (double)t);
  for (int64_t i = 0; i < n; ++i) {
    m[i] = b1 * m[i] + (1.0 - b1) * g[i];
    v[i] = b2 * v[i] + (1.0 - b2) * g[i] * g[i];
    const double mhat = m[i] / bc1, vhat = v[i] / bc2;
    theta[i] = theta[i] - lr * (wd * theta[i] + mhat / (sqrt(vhat) + eps));
  }
}

/* ------------------------------------------------------------------ merge */

/*
 * [MERGE] "Module 08 - QLoRA & Quantization" (ainiketan), "7. A subtle but
 * important deployment note", and katajob, "What it costs" (3. Merging): for
 * serving, the trained adapter is folded into a 16-bit base (the reloaded
 * original, or here also the dequantized NF4 base it was trained against),
 * and the merged model may then be quantized again.  With [LORA]'s layer
 * h = W0 x + s B A x the merged weight is
 *   Wm[n, k] = W[n, k] + s * sum_j B[n, j] A[j, k]         (binary64)
 * W [N, K], A [r, K], B [N, r], Wm [N, K]; s = fl32(alpha / r).
 */
void oracle_merge(const double *W, int64_t N, int64_t K, const double *A, const double *B, int32_t r, float alpha,
                  double *Wm) {
  const double s = (double)(alpha / (float)r);
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0.0;
      for (int32_t j = 0; j < r; ++j) acc += B[n * r + j] * A[(int64_t)j * K + k];
      Wm[n * K + k] = W[n * K + k] + s * acc;
    }
}

/* ------------------------------------------------------- many adapters */

/*
 * [MULTI] pranaymahendrakar, Researcher level, "The variants worth knowing":
 * since the update is separable, one server holds one base model and many
 * adapters and batches requests for different adapters together.  Tokens
 * come in segments: tokens seg[s] .. seg[s+1]-1 use adapter ad[s] of a pool
 * (A_pool [n_pool][r][K], B_pool [n_pool][N][r]); an adapter index outside
 * [0, n_pool) means no adapter (the base product alone).  Per token t with
 * adapter a, [LORA]'s layer:
 *   U[t, j] = sum_k X[t, k] A_a[j, k]
 *   Y[t, n] = sum_k X[t, k] W'[n, k] + s * sum_j U[t, j] B_a[n, j]
 * Y [T, N] binary64.  Tokens outside every segment also get the base alone.
 */
void oracle_linear_fwd_multi(const double *X, int64_t T, const uint16_t *Wdq, int64_t N, int64_t K,
                             const double *A_pool, const double *B_pool, int32_t n_pool, int32_t r, float alpha,
                             const int32_t *seg, const int32_t *ad, int32_t n_seg, double *Y) {
  const double s = (double)(alpha / (float)r);
  int32_t *tok_ad = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  for (int64_t t = 0; t < T; ++t) tok_ad[t] = -1;
  for (int32_t g = 0; g < n_seg; ++g)
    for (int64_t t = seg[g]; t < seg[g + 1] && t < T; ++t)
      if (t >= 0) tok_ad[t] = (ad[g] >= 0 && ad[g] < n_pool) ? ad[g] : -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < T; ++t) {
    const double *x = X + t * K;
    const int32_t a = tok_ad[t];
    double *u = (double *)calloc((size_t)(r > 0 ? r : 1), sizeof(double));
    if (a >= 0)
      for (int32_t j = 0; j < r; ++j) {
        const double *arow = A_pool + ((int64_t)a * r + j) * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += x[k] * arow[k];
        u[j] = acc;
      }
    for (int64_t n = 0; n < N; ++n) {
      const uint16_t *w = Wdq + n * K;
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += x[k] * bf16_to_f64(w[k]);
      double lora = 0.0;
      if (a >= 0)
        for (int32_t j = 0; j < r; ++j) lora += u[j] * B_pool[((int64_t)a * N + n) * r + j];
      Y[t * N + n] = acc + s * lora;
    }
    free(u);
  }
  free(tok_ad);
}

/* ------------------------------------------------- AdamW with 8-bit state */

/*
 * [OPT8] "Module 08 - QLoRA & Quantization" (ainiketan), "4. QLoRA in code"
 * and "5. Other memory-saving levers": a paged 8-bit AdamW (paged_adamw_8bit)
 * keeps the optimizer state smaller.  The 8-bit state follows the block-wise
 * quantization of optimizer states of Dettmers, Lewis, Shleifer and
 * Zettlemoyer ("8-bit Optimizers via Block-wise Quantization", ICLR 2022):
 * each moment is stored as 8-bit codes plus one binary32 absmax per block of
 * 2048 consecutive elements, the codes indexing a dynamic (exponent + linear
 * fraction) code book.  Paging to host memory is not part of this.
 * Readings (listed in the design notes):
 *  - code book: in a signed byte (first moment) bit 7 is the sign; among the
 *    other 7 bits, E = the number of leading zeros, then a set indicator bit,
 *    then F = 6 - E fraction bits f; the magnitude is
 *    fl32((0.1 + 0.9 ((f + 1) / 2^F)) / 10^E) (binary64, in that order), and
 *    all-zero bits mean 0.  An unsigned byte (second moment) has no sign bit:
 *    E counts leading zeros among 8 bits and F = 7 - E.  Magnitudes grow with
 *    the unsigned value of the bits, so the code is the count of thresholds
 *    below the value;
 *  - encode: x = fl32(value / absmax) with absmax the block's largest
 *    magnitude (all codes 0 when it is 0); nearest magnitude, ties to the
 *    smaller (thresholds: the largest binary32 value not above each exact
 *    midpoint); the sign bit is set for x < 0 unless the magnitude is 0;
 *  - decode: fl32(table[code] * absmax);
 *  - the step is the binary32 AdamW of the fused kernel, every operation
 *    rounded once, in this order.  This function fixes that declared order
 *    (a regression pin: the kernel must keep it bit for bit); the reference
 *    that judges a step's values is the binary64 [OPT8-64] below:
 *      m = fl(fl(b1 m) + fl(c1 g)),  v = fl(fl(b2 v) + fl(fl(c2 g) g)),
 *      d = fl(fl(sqrt(v) / sb) + eps),  theta = fl(fl(theta dk) - fl(ss fl(m / d)))
 *    with b1 = fl32(beta1), c1 = fl32(1 - beta1), b2 = fl32(beta2),
 *    c2 = fl32(1 - beta2), eps = fl32(eps), dk = fl32(1 - lr wd),
 *    ss = fl32(lr / (1 - beta1^t)), sb = fl32(sqrt(1 - beta2^t)), each formed
 *    in binary64 and rounded once.
 */
static float dyn_magnitude(int E, int F, int f) {
  double p10 = 1.0;
  for (int i = 0; i < E; ++i) p10 *= 10.0; /* exact: 10^E < 2^53 */
  const double frac = (double)(f + 1) / (double)(1 << F);
  return (float)((0.1 + 0.9 * frac) / p10);
}

/* Value of every byte: signed (first moment) or unsigned (second moment) book. */
void oracle_dyn_codebook(int is_signed, float out[256]) {
  const int bits = is_signed ? 7 : 8;
  for (int b = 0; b < 256; ++b) {
    const int p = is_signed ? (b & 127) : b;
    float mag = 0.0f;
    if (p != 0) {
      int top = bits - 1;
      while (!((p >> top) & 1)) --top; /* position of the indicator bit */
      const int E = bits - 1 - top, F = top;
      mag = dyn_magnitude(E, F, p - (1 << F));
    }
    out[b] = (is_signed && (b & 128)) ? -mag : mag;
  }
}

/* Nearest code of a normalized value (|x| <= 1), ties to the smaller magnitude. */
static int dyn_encode(float x, int is_signed, const float book[256]) {
  const int n = is_signed ? 128 : 256;
  const float a = fabsf(x);
  int p = 0;
  for (int i = 1; i < n; ++i) {
    const double mid = ((double)book[i - 1] + (double)book[i]) * 0.5; /* exact */
    if ((double)a > mid) p = i;
  }
  if (is_signed && x < 0.0f && p != 0) p |= 128;
  return p;
}

int oracle_dyn_encode(float x, int is_signed) {
  float book[256];
  oracle_dyn_codebook(is_signed, book);
  return dyn_encode(x, is_signed, book);
}

/*
 * One step over n parameters: param bf16 bits (and master binary32 or NULL),
 * grad bf16 bits, m_code/v_code [n] bytes, m_absmax/v_absmax [ceil(n / 2048)]
 * binary32, all updated in place.
 */
void oracle_adamw8_step(uint16_t *param, float *master, const uint16_t *grad, uint8_t *m_code, float *m_absmax,
                        uint8_t *v_code, float *v_absmax, int64_t n, double lr, double beta1, double beta2,
                        double eps, double wd, int64_t t) {
  float sbook[256], ubook[256];
  oracle_dyn_codebook(1, sbook);
  oracle_dyn_codebook(0, ubook);
  const float b1 = (float)beta1, c1 = (float)(1.0 - beta1), b2 = (float)beta2, c2 = (float)(1.0 - beta2);
  const float ef = (float)eps, dk = (float)(1.0 - lr * wd);
  const float ss = (float)(lr / (1.0 - pow(beta1, (double)t))), sb = (float)sqrt(1.0 - pow(beta2, (double)t));
  const int64_t nblk = (n + 2047) / 2048;
  float *m = (float *)malloc(sizeof(float) * 2048), *v = (float *)malloc(sizeof(float) * 2048);
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int64_t e0 = blk * 2048, e1 = (e0 + 2048 < n) ? e0 + 2048 : n;
    float am = 0.0f, av = 0.0f;
    for (int64_t e = e0; e < e1; ++e) {
      uint32_t u = (uint32_t)grad[e] << 16;
      float g;
      memcpy(&g, &u, 4);
      float th;
      if (master) th = master[e];
      else {
        u = (uint32_t)param[e] << 16;
        memcpy(&th, &u, 4);
      }
      float mo = sbook[m_code[e]] * m_absmax[blk];
      float vo = ubook[v_code[e]] * v_absmax[blk];
      float mm = b1 * mo;
      mm = mm + c1 * g;
      float cg = c2 * g;
      float vv = b2 * vo;
      vv = vv + cg * g;
      float d = sqrtf(vv) / sb;
      d = d + ef;
      const float q = mm / d;
      float tn = th * dk;
      tn = tn - ss * q;
      if (master) master[e] = tn;
      param[e] = f32_to_bf16_rne(tn);
      m[e - e0] = mm;
      v[e - e0] = vv;
      if (fabsf(mm) > am) am = fabsf(mm);
      if (vv > av) av = vv;
    }
    m_absmax[blk] = am;
    v_absmax[blk] = av;
    for (int64_t e = e0; e < e1; ++e) {
      m_code[e] = (uint8_t)(am > 0.0f ? dyn_encode(m[e - e0] / am, 1, sbook) : 0);
      v_code[e] = (uint8_t)(av > 0.0f ? dyn_encode(v[e - e0] / av, 0, ubook) : 0);
    }
  }
  free(m);
  free(v);
}

/*
 * [OPT8-64] The same 8-bit step judged without the kernel's binary32 order:
 * every operation is exact or binary64, so no rounding of binary32 arithmetic
 * is shared with a GPU step.
 *  - decode: a book magnitude (binary32) times a block absmax (binary32) is
 *    exact in binary64 (48 significant bits);
 *  - step: the binary64 AdamW of oracle_adamw_step on the decoded moments;
 *  - encode: per block of 2048, absmax = max |m| (max v), x = m / absmax in
 *    binary64, and the code is the number of exact midpoints of adjacent book
 *    magnitudes strictly below |x| (ties to the smaller magnitude), with the
 *    sign bit for x < 0 unless the magnitude is 0 (first moment only).
 * Inputs: theta (binary64: the master copy or the bf16 parameter), grad bf16
 * bits, the state before the step.  Outputs: theta_out, the moments before
 * encoding (m_out, v_out), their codes and the binary64 block absmax.
 */
static int dyn_encode_f64(double x, int is_signed, const float book[256]) {
  const int n = is_signed ? 128 : 256;
  const double a = fabs(x);
  int p = 0;
  for (int i = 1; i < n; ++i)
    if (a > ((double)book[i - 1] + (double)book[i]) * 0.5) p = i; /* midpoints are exact in binary64 */
  if (is_signed && x < 0.0 && p != 0) p |= 128;
  return p;
}

void oracle_adamw8_step_f64(const double *theta, const uint16_t *grad, const uint8_t *m_code,
                            const float *m_absmax, const uint8_t *v_code, const float *v_absmax, int64_t n, double lr,
                            double beta1, double beta2, double eps, double wd, int64_t t, double *theta_out,
                            double *m_out, double *v_out, uint8_t *m_code_out, double *m_absmax_out,
                            uint8_t *v_code_out, double *v_absmax_out) {
  float sbook[256], ubook[256];
  oracle_dyn_codebook(1, sbook);
  oracle_dyn_codebook(0, ubook);
  double *g = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
  for (int64_t e = 0; e < n; ++e) {
    const uint32_t u = (uint32_t)grad[e] << 16;
    float gf;
    memcpy(&gf, &u, 4);
    g[e] = (double)gf;
    theta_out[e] = theta[e];
    m_out[e] = (double)sbook[m_code[e]] * (double)m_absmax[e / 2048];
    v_out[e] = (double)ubook[v_code[e]] * (double)v_absmax[e / 2048];
  }
  oracle_adamw_step(theta_out, g, m_out, v_out, n, lr, beta1, beta2, eps, wd, t);
  free(g);
  for (int64_t e0 = 0; e0 < n; e0 += 2048) {
    const int64_t e1 = (e0 + 2048 < n) ? e0 + 2048 : n;
    double am = 0.0, av = 0.0;
    for (int64_t e = e0; e < e1; ++e) {
      if (fabs(m_out[e]) > am) am = fabs(m_out[e]);
      if (v_out[e] > av) av = v_out[e];
    }
    m_absmax_out[e0 / 2048] = am;
    v_absmax_out[e0 / 2048] = av;
    for (int64_t e = e0; e < e1; ++e) {
      m_code_out[e] = (uint8_t)(am > 0.0 ? dyn_encode_f64(m_out[e] / am, 1, sbook) : 0);
      v_code_out[e] = (uint8_t)(av > 0.0 ? dyn_encode_f64(v_out[e] / av, 0, ubook) : 0);
    }
  }
}
