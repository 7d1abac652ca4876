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
  float rbc2;     // RN(1 / sqrt_bc2), for recip_div
  int fast_bc2;   // sqrt_bc2 lies where recip_div is exact (always, for beta2 in [0, 1))
};

hipError_t launch_adamw(const AdamParams &a, int64_t blocks, hipStream_t s);

// 8-bit state: one workgroup per block of 2048 elements of one tensor.
constexpr int kAdam8Block = 2048;
struct Adam8Tensor {
  uint16_t *p;
  const uint16_t *g;
  uint8_t *mq;  // first-moment codes (signed book)
  float *ma;    // first-moment absmax per block
  uint8_t *vq;  // second-moment codes (unsigned book)
  float *va;    // second-moment absmax per block
  float *master;
  int64_t n;
  int64_t block0;
};
struct Adam8Params {
  Adam8Tensor t[kAdamMaxTensors];
  int count;
  float b1, omb1, b2, omb2, eps, decay, step_size, sqrt_bc2;
  float rbc2;
  int fast_bc2;
};
hipError_t launch_adamw8(const Adam8Params &a, int64_t blocks, hipStream_t s);

}  // namespace qlora
