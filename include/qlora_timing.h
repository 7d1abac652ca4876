/*
 * qlora_timing.h -- measurement hooks of libqlora.so (host only).
 *
 * These are not part of the layer's interface (quantize, dequantize, forward,
 * backward and the optimizer, merge and many-adapter calls in qlora.h): they
 * let a benchmark time one named kernel on the stream it is launched on, with
 * no extra packets between kernels.  While a name is enabled, every launch of
 * that kernel passes a start and a stop event that the kernel's own dispatch
 * packet stamps (hipExtLaunchKernel), so their difference is the kernel's
 * execution time.  With no name enabled a launch takes no lock and records
 * nothing.  Events are created on need and kept for reuse (per device) once
 * read back; the pool lives until the process ends.  A timed launch costs the
 * host about 25 us more than an untimed one (measured on MI355X), so time
 * wall-clock steps with timing off.
 *
 * Kernel names: "nf4_gemm_fwd", "nf4_gemm_dx", "nf4_gemv", "adamw", "adamw8",
 * "merge", "lora_u_multi", ... (the launch labels of the library), or "*" for
 * every launch.  Errors: QLORA_EINVAL for a NULL name or output pointer;
 * QLORA_EHIP if waiting for or reading an event fails (the record is cleared
 * anyway).
 */
#ifndef QLORA_TIMING_H
#define QLORA_TIMING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enable (1) or disable (0) timing of `kernel`; several names can be enabled
 * at once, and disabling "*" disables every name. */
int qlora_timing_enable(const char *kernel, int enable);

/* Wait for the recorded launches of `kernel`, return their number and summed
 * milliseconds, and clear the record. */
int qlora_timing_read(const char *kernel, int64_t *launches, double *total_ms);

/* The same with each launch's milliseconds, in launch order, written to
 * ms[0 .. min(cap, *launches)); `ms` is caller-owned host memory (may be NULL
 * when cap is 0).  *launches is the number recorded, which may exceed cap. */
int qlora_timing_read_each(const char *kernel, double *ms, int64_t cap, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_TIMING_H */
