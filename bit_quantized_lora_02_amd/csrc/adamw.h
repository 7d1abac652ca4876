// adamw.h -- kernel-argument layout of the fused AdamW step (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

constexpr int kAdamMaxTensors = 32;  // tensors per launch (descriptors ride in the kernel arguments)
constexpr int kAdamChunk = 2048;     // elements per 256-thread workgroup

struct AdamTensor {
  uint16_t *p;        // bf16 parameter
  const uint16_t *g;  // bf16 gradient
  float *m, *v;       // binary32 moments
  float *master;      // binary32 master copy or null
  int64_t n;          // elements
  int64_t block0;     // first workgroup of this tensor
};

struct AdamParams {
  AdamTensor t[kAdamMaxTensors];
  int count;
  float b1, omb1, b2, omb2, eps, decay, step_size, sqrt_bc2;
};

hipError_t launch_adamw(const AdamParams &a, int64_t blocks, hipStream_t s);

}  // namespace qlora
