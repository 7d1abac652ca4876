// Host AddressSanitizer driver for the C ABI (test infrastructure).  It is linked with the library's
// sources compiled for the host only (no device code), and drives every argument-error path and every
// host-only call; all of them return before the library's first kernel launch, so no GPU is needed.
// ASan reports any out-of-bounds access, use after free or leak in the validation, planning, error-text
// and timing code.  Built and run by tests/test_asan_cpu.py.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qlora.h"
#include "qlora_timing.h"

static int g_fail = 0;
#define EXPECT(call, want)                                                                               \
  do {                                                                                                   \
    const int rc_ = (call);                                                                              \
    if (rc_ != (want)) {                                                                                 \
      printf("line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, rc_, (want), qlora_last_error()); \
      g_fail = 1;                                                                                        \
    }                                                                                                    \
  } while (0)

int main() {
  void *F = (void *)0x10000;  // aligned, never dereferenced: each call below fails before using it
  void *M = (void *)0x10008;  // misaligned
  qlora_bf16 *Fb = (qlora_bf16 *)F, *Mb = (qlora_bf16 *)M;
  size_t a = 0, b = 0, c = 0;
  EXPECT(qlora_nf4_storage(4096, 4096, &a, &b, &c), QLORA_OK);
  EXPECT(qlora_nf4_storage(4, 100, &a, &b, &c), QLORA_EINVAL);
  EXPECT(qlora_nf4_storage(1 << 22, 1 << 22, &a, &b, &c), QLORA_EINVAL);
  EXPECT(qlora_nf4_storage(4, 64, nullptr, &b, &c), QLORA_EINVAL);
  float lv[16];
  EXPECT(qlora_nf4_codebook(lv), QLORA_OK);
  EXPECT(qlora_nf4_codebook(nullptr), QLORA_EINVAL);
  const int64_t shapes[][4] = {{16, 256, 256, 8},    {2048, 4096, 4096, 16}, {1, 8192, 8192, 16},
                               {40, 28672, 8192, 16}, {128, 8192, 8192, 16},  {4096, 28672, 8192, 64},
                               {0, 64, 64, 1},        {64, 8, 65536, 128}};
  for (auto &s : shapes)
    for (int op = 0; op < 4; ++op) EXPECT(qlora_workspace_bytes(op, s[0], s[1], s[2], (int32_t)s[3], &a), QLORA_OK);
  EXPECT(qlora_workspace_bytes(7, 1, 64, 64, 8, &a), QLORA_EINVAL);
  EXPECT(qlora_workspace_bytes(0, 1, 64, 64, 129, &a), QLORA_EINVAL);
  EXPECT(qlora_workspace_bytes(0, 1 << 11, 1 << 21, 64, 8, &a), QLORA_EINVAL);
  EXPECT(qlora_workspace_bytes(0, 1, 64, 64, 8, nullptr), QLORA_EINVAL);

  qlora_nf4 q = {256, 256, (uint8_t *)F, (uint8_t *)F, (float *)F};
  qlora_nf4 qbad = {256, 100, (uint8_t *)F, (uint8_t *)F, (float *)F};
  qlora_nf4 qmis = {256, 256, (uint8_t *)M, (uint8_t *)F, (float *)F};
  EXPECT(qlora_quantize_nf4(nullptr, &q, nullptr), QLORA_EINVAL);
  EXPECT(qlora_quantize_nf4((const float *)F, &qbad, nullptr), QLORA_EINVAL);
  EXPECT(qlora_quantize_nf4((const float *)F, &qmis, nullptr), QLORA_EINVAL);
  EXPECT(qlora_dequant(nullptr, Fb, nullptr), QLORA_EINVAL);
  EXPECT(qlora_dequant(&q, nullptr, nullptr), QLORA_EINVAL);

  size_t ws = 0;
  EXPECT(qlora_workspace_bytes(QLORA_OP_FWD, 16, 256, 256, 8, &ws), QLORA_OK);
  EXPECT(qlora_linear_fwd(Fb, 16, &q, Fb, Fb, 8, 16.f, Fb, Fb, F, ws - 1, nullptr), QLORA_EWORKSPACE);
  EXPECT(qlora_linear_fwd(Fb, 16, &q, Fb, Fb, 0, 16.f, Fb, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_linear_fwd(Fb, 16, &q, Fb, Fb, 129, 16.f, Fb, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_linear_fwd(Mb, 16, &q, Fb, Fb, 8, 16.f, Fb, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_linear_fwd(Fb, -1, &q, Fb, Fb, 8, 16.f, Fb, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_linear_fwd(Fb, 16, nullptr, Fb, Fb, 8, 16.f, Fb, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_linear_fwd(Fb, 16, &q, Fb, Fb, 8, 1.f / 0.f, Fb, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_linear_fwd_noalloc(Fb, 16, &qbad, Fb, Fb, 8, 16.f, Fb, Fb, nullptr), QLORA_EINVAL);
  qlora_nf4 qhuge = {1 << 17, 8192, (uint8_t *)F, (uint8_t *)F, (float *)F};
  EXPECT(qlora_linear_fwd_noalloc(Fb, 64, &qhuge, Fb, Fb, 16, 32.f, Fb, nullptr, nullptr), QLORA_EWORKSPACE);
  EXPECT(qlora_workspace_bytes(QLORA_OP_BWD, 16, 256, 256, 8, &ws), QLORA_OK);
  EXPECT(qlora_linear_bwd(Fb, Fb, 16, &q, Fb, Fb, 8, 16.f, nullptr, Fb, nullptr, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_linear_bwd(Fb, Fb, 16, &q, Fb, Fb, 8, 16.f, nullptr, Fb, Fb, Fb, F, ws - 1, nullptr),
         QLORA_EWORKSPACE);
  EXPECT(qlora_linear_bwd(Fb, Mb, 16, &q, Fb, Fb, 8, 16.f, nullptr, Fb, Fb, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_workspace_bytes(QLORA_OP_FWD_DROPOUT, 16, 256, 256, 8, &ws), QLORA_OK);
  EXPECT(qlora_linear_fwd_dropout(Fb, 16, &q, Fb, Fb, 8, 16.f, 1.0f, 1, 0, (uint8_t *)F, Fb, Fb, F, ws, nullptr),
         QLORA_EINVAL);
  EXPECT(qlora_linear_fwd_dropout(Fb, 16, &q, Fb, Fb, 8, 16.f, 0.1f, 1, 0, nullptr, Fb, Fb, F, ws, nullptr),
         QLORA_EINVAL);
  EXPECT(qlora_linear_bwd_dropout(Fb, Fb, 16, &q, Fb, Fb, 8, 16.f, -0.5f, (const uint8_t *)F, nullptr, Fb, Fb, Fb,
                                  F, ws, nullptr),
         QLORA_EINVAL);
  const int32_t *Fi = (const int32_t *)F;
  EXPECT(qlora_workspace_bytes(QLORA_OP_FWD_MULTI, 16, 256, 256, 8, &ws), QLORA_OK);
  EXPECT(qlora_linear_fwd_multi(Fb, 16, &q, Fb, Fb, 2, 12, 16.f, Fi, Fi, 1, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_linear_fwd_multi(Fb, 16, &q, Fb, Fb, 0, 8, 16.f, Fi, Fi, 1, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_linear_fwd_multi(Fb, 16, &q, Fb, Fb, 2, 8, 16.f, nullptr, Fi, 1, Fb, F, ws, nullptr), QLORA_EINVAL);
  EXPECT(qlora_merge(&q, Fb, 256, 256, Fb, Fb, 8, 16.f, Fb, nullptr, nullptr), QLORA_EINVAL);
  EXPECT(qlora_merge(&q, nullptr, 256, 256, Fb, Fb, 8, 16.f, nullptr, nullptr, nullptr), QLORA_EINVAL);
  EXPECT(qlora_merge(&q, nullptr, 128, 256, Fb, Fb, 8, 16.f, Fb, nullptr, nullptr), QLORA_EINVAL);

  qlora_adamw_tensor t1 = {Fb, Fb, (float *)F, (float *)F, nullptr, 100};
  qlora_adamw_tensor tbad = {Fb, nullptr, (float *)F, (float *)F, nullptr, 100};
  EXPECT(qlora_adamw_step(nullptr, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, nullptr), QLORA_EINVAL);
  EXPECT(qlora_adamw_step(&tbad, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, nullptr), QLORA_EINVAL);
  EXPECT(qlora_adamw_step(&t1, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0, nullptr), QLORA_EINVAL);
  EXPECT(qlora_adamw_step(&t1, 1, 1e-3, 1.5, 0.999, 1e-8, 0.0, 1, nullptr), QLORA_EINVAL);
  qlora_adamw8_tensor e1 = {Fb, Fb, (uint8_t *)F, (float *)F, (uint8_t *)F, (float *)F, nullptr, 100};
  qlora_adamw8_tensor e2 = {Fb, Fb, (uint8_t *)F, (float *)((char *)F + 2), (uint8_t *)F, (float *)F, nullptr, 100};
  EXPECT(qlora_adamw8_step(&e1, -1, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, nullptr), QLORA_EINVAL);
  EXPECT(qlora_adamw8_step(&e2, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, nullptr), QLORA_EINVAL);
  EXPECT(qlora_adamw8_step(&e1, 1, 1e-3, 0.9, 0.999, -1.0, 0.0, 1, nullptr), QLORA_EINVAL);

  for (int code = -6; code <= 1; ++code)
    if (!qlora_strerror(code) || !strlen(qlora_strerror(code))) g_fail = 1;
  if (!qlora_last_error()) g_fail = 1;

  double ms[4];
  int64_t n = -1;
  double tot = -1.0;
  EXPECT(qlora_timing_enable("nf4_gemm_fwd", 1), QLORA_OK);
  EXPECT(qlora_timing_enable("*", 1), QLORA_OK);
  EXPECT(qlora_timing_enable("*", 0), QLORA_OK);
  EXPECT(qlora_timing_enable(nullptr, 1), QLORA_EINVAL);
  EXPECT(qlora_timing_read("nf4_gemm_fwd", &n, &tot), QLORA_OK);
  EXPECT(qlora_timing_read_each("nf4_gemm_fwd", ms, 4, &n), QLORA_OK);
  EXPECT(qlora_timing_read_each("nf4_gemm_fwd", nullptr, 4, &n), QLORA_EINVAL);
  EXPECT(qlora_timing_read_each("nf4_gemm_fwd", nullptr, 0, nullptr), QLORA_EINVAL);
  if (n != 0) g_fail = 1;
  printf(g_fail ? "abi asan driver FAILED\n" : "abi asan driver ok\n");
  return g_fail;
}
