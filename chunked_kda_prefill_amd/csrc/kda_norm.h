// Arguments and launcher of the gated-RMSNorm kernel (kda_norm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct NormArgs {
  const uint16_t *x;          // bf16 bits, row (t, h) at t * x_stride + h * 128
  const uint16_t *z;          // bf16 bits, row (t, h) at t * z_stride + h * 128
  const float *w;             // [128]
  uint16_t *y;                // bf16 bits [T, H, 128]
  int64_t x_stride, z_stride; // elements per token
  int64_t T;
  int32_t H;
  float eps;
  int32_t act;                // 0 sigmoid, 1 SiLU
};
hipError_t launch_gated_rmsnorm(const NormArgs &a, hipStream_t stream);

}  // namespace kda
