/*
 * Host AddressSanitizer driver for the CPU oracle (test infrastructure).  Every oracle entry point runs on
 * small inputs held in heap buffers of exactly the documented sizes, so that any read or write past them,
 * any use after free and any leak is reported by ASan.  Built and run by tests/test_asan_cpu.py with
 *   gcc -O1 -g -fsanitize=address -fno-omit-frame-pointer -fopenmp oracle/qlora_oracle.c tests/asan/oracle_asan.c -lm
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_quantize_nf4(const float *W, int64_t n_out, int64_t n_in, uint8_t *codes, uint8_t *absmax_q,
                        float *absmax_step, float *absmax_f32);
int oracle_dequant(const uint8_t *codes, const uint8_t *absmax_q, const float *absmax_step, int64_t n_out,
                   int64_t n_in, uint16_t *W_out);
void oracle_linear_fwd(const double *X, int64_t T, const uint16_t *Wdq, int64_t N, int64_t K, const double *A,
                       const double *B, int32_t r, float alpha, const int64_t *rows, int64_t n_rows, double *Y,
                       double *U);
void oracle_linear_bwd(const double *X, const double *dY, int64_t T, const uint16_t *Wdq, int64_t N, int64_t K,
                       const double *A, const double *B, int32_t r, float alpha, const int64_t *rows,
                       int64_t n_rows, double *dX, double *dA, double *dB);
void oracle_dropout_mask(int64_t n_chunks, double p, uint64_t seed, uint64_t offset, uint8_t *mask);
void oracle_dropout_apply(const uint16_t *X, int64_t n, const uint8_t *mask, double p, uint16_t *Xa, double *G);
void oracle_adamw_step(double *theta, const double *g, double *m, double *v, int64_t n, double lr, double b1,
                       double b2, double eps, double wd, int64_t t);
void oracle_merge(const double *W, int64_t N, int64_t K, const double *A, const double *B, int32_t r, float alpha,
                  double *Wm);
void oracle_linear_fwd_multi(const double *X, int64_t T, const uint16_t *Wdq, int64_t N, int64_t K,
                             const double *A_pool, const double *B_pool, int32_t n_pool, int32_t r, float alpha,
                             const int32_t *seg, const int32_t *ad, int32_t n_seg, double *Y);
void oracle_adamw8_step(uint16_t *param, float *master, const uint16_t *grad, uint8_t *m_code, float *m_absmax,
                        uint8_t *v_code, float *v_absmax, int64_t n, double lr, double beta1, double beta2,
                        double eps, double wd, int64_t t);
void oracle_adamw8_step_f64(const double *theta, const uint16_t *grad, const uint8_t *m_code, const float *m_absmax,
                            const uint8_t *v_code, const float *v_absmax, int64_t n, double lr, double beta1,
                            double beta2, double eps, double wd, int64_t t, double *theta_out, double *m_out,
                            double *v_out, uint8_t *m_code_out, double *m_absmax_out, uint8_t *v_code_out,
                            double *v_absmax_out);

static uint32_t rng = 12345u;
static double uni(void) {
  rng = rng * 1664525u + 1013904223u;
  return ((rng >> 8) + 0.5) / 16777216.0 - 0.5;
}
static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) exit(3);
  return p;
}
static uint16_t bf16_of(double x) { /* truncation is enough for test inputs */
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

int main(void) {
  /* a weight with a partial double-quantization group: 5 x 4160 = 325 blocks */
  const int64_t N = 5, K = 4160, T = 3, r = 3;
  const int64_t nw = N * K, nblk = nw / 64, ngrp = (nblk + 255) / 256;
  float *W = xmalloc(sizeof(float) * nw);
  for (int64_t i = 0; i < nw; ++i) W[i] = (float)(0.02 * uni());
  uint8_t *codes = xmalloc(nw / 2), *aq = xmalloc(nblk);
  float *step = xmalloc(sizeof(float) * ngrp), *af = xmalloc(sizeof(float) * nblk);
  if (oracle_quantize_nf4(W, N, K, codes, aq, step, af) != 0) return 1;
  if (oracle_quantize_nf4(W, N, K, codes, aq, step, NULL) != 0) return 1;
  uint16_t *Wd = xmalloc(sizeof(uint16_t) * nw);
  if (oracle_dequant(codes, aq, step, N, K, Wd) != 0) return 1;

  double *X = xmalloc(sizeof(double) * T * K), *dY = xmalloc(sizeof(double) * T * N);
  double *A = xmalloc(sizeof(double) * r * K), *B = xmalloc(sizeof(double) * N * r);
  for (int64_t i = 0; i < T * K; ++i) X[i] = uni();
  for (int64_t i = 0; i < T * N; ++i) dY[i] = uni();
  for (int64_t i = 0; i < r * K; ++i) A[i] = 0.01 * uni();
  for (int64_t i = 0; i < N * r; ++i) B[i] = 0.01 * uni();
  double *Y = xmalloc(sizeof(double) * T * N), *U = xmalloc(sizeof(double) * T * r);
  double *dX = xmalloc(sizeof(double) * T * K), *dA = xmalloc(sizeof(double) * r * K);
  double *dB = xmalloc(sizeof(double) * N * r);
  oracle_linear_fwd(X, T, Wd, N, K, A, B, (int32_t)r, 6.0f, NULL, 0, Y, U);
  oracle_linear_bwd(X, dY, T, Wd, N, K, A, B, (int32_t)r, 6.0f, NULL, 0, dX, dA, dB);
  const int64_t rows[2] = {0, T - 1};
  double *Y2 = xmalloc(sizeof(double) * 2 * N), *U2 = xmalloc(sizeof(double) * 2 * r);
  double *dX2 = xmalloc(sizeof(double) * 2 * K);
  oracle_linear_fwd(X, T, Wd, N, K, A, B, (int32_t)r, 6.0f, rows, 2, Y2, U2);
  oracle_linear_bwd(X, dY, T, Wd, N, K, A, B, (int32_t)r, 6.0f, rows, 2, dX2, dA, dB);

  /* dropout on the adapter input: T * K / 8 chunks */
  uint8_t *mask = xmalloc(T * K / 8);
  oracle_dropout_mask(T * K / 8, 0.05, 7, 3, mask);
  uint16_t *Xb = xmalloc(sizeof(uint16_t) * T * K), *Xa = xmalloc(sizeof(uint16_t) * T * K);
  double *G = xmalloc(sizeof(double) * T * K);
  for (int64_t i = 0; i < T * K; ++i) Xb[i] = bf16_of(X[i]);
  oracle_dropout_apply(Xb, T * K, mask, 0.05, Xa, G);

  /* AdamW, merge, many adapters */
  const int64_t n = 2049 + 2048; /* two full 8-bit blocks and a ragged one */
  double *th = xmalloc(sizeof(double) * n), *g = xmalloc(sizeof(double) * n);
  double *m = calloc(n, sizeof(double)), *v = calloc(n, sizeof(double));
  for (int64_t i = 0; i < n; ++i) th[i] = uni(), g[i] = 1e-3 * uni();
  oracle_adamw_step(th, g, m, v, n, 1e-3, 0.9, 0.999, 1e-8, 0.01, 1);
  double *Wm = xmalloc(sizeof(double) * nw), *Wf = xmalloc(sizeof(double) * nw);
  for (int64_t i = 0; i < nw; ++i) Wf[i] = W[i];
  oracle_merge(Wf, N, K, A, B, (int32_t)r, 6.0f, Wm);
  const int32_t n_pool = 2, seg[3] = {0, 1, 3}, ad[2] = {1, 5};
  double *Ap = xmalloc(sizeof(double) * n_pool * r * K), *Bpl = xmalloc(sizeof(double) * n_pool * N * r);
  for (int64_t i = 0; i < n_pool * r * K; ++i) Ap[i] = 0.01 * uni();
  for (int64_t i = 0; i < n_pool * N * r; ++i) Bpl[i] = 0.01 * uni();
  oracle_linear_fwd_multi(X, T, Wd, N, K, Ap, Bpl, n_pool, (int32_t)r, 6.0f, seg, ad, 2, Y);

  const int64_t nb8 = (n + 2047) / 2048;
  uint16_t *p16 = xmalloc(sizeof(uint16_t) * n), *g16 = xmalloc(sizeof(uint16_t) * n);
  float *master = xmalloc(sizeof(float) * n);
  uint8_t *mc = calloc(n, 1), *vc = calloc(n, 1);
  float *ma = calloc(nb8, sizeof(float)), *va = calloc(nb8, sizeof(float));
  for (int64_t i = 0; i < n; ++i) p16[i] = bf16_of(0.02 * uni()), g16[i] = bf16_of(1e-3 * uni()), master[i] = 0.f;
  for (int t = 1; t <= 3; ++t) oracle_adamw8_step(p16, master, g16, mc, ma, vc, va, n, 1e-3, 0.9, 0.999, 1e-8, 0.01, t);
  oracle_adamw8_step(p16, NULL, g16, mc, ma, vc, va, n, 1e-3, 0.9, 0.999, 1e-8, 0.01, 4);
  double *to = xmalloc(sizeof(double) * n), *mo = xmalloc(sizeof(double) * n), *vo = xmalloc(sizeof(double) * n);
  double *mao = xmalloc(sizeof(double) * nb8), *vao = xmalloc(sizeof(double) * nb8);
  uint8_t *mco = xmalloc(n), *vco = xmalloc(n);
  oracle_adamw8_step_f64(th, g16, mc, ma, vc, va, n, 1e-3, 0.9, 0.999, 1e-8, 0.01, 5, to, mo, vo, mco, mao, vco, vao);

  free(W), free(codes), free(aq), free(step), free(af), free(Wd), free(X), free(dY), free(A), free(B);
  free(Y), free(U), free(dX), free(dA), free(dB), free(Y2), free(U2), free(dX2), free(mask), free(Xb), free(Xa);
  free(G), free(th), free(g), free(m), free(v), free(Wm), free(Wf), free(Ap), free(Bpl), free(p16), free(g16);
  free(master), free(mc), free(vc), free(ma), free(va), free(to), free(mo), free(vo), free(mao), free(vao);
  free(mco), free(vco);
  printf("oracle asan driver ok\n");
  return 0;
}
