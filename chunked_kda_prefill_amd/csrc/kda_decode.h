// Arguments and launcher of the token-serial decode kernel (kda_decode.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
  const uint16_t *q, *k, *v;  // bf16 bits [T, H, 128]
  const float *g;             // [T, H, 128]
  const float *beta;          // [T, H]
  const int32_t *cu;          // cu_seqlens [N + 1]
  const float *h0;            // [N, H, 128, 128] or null
  float *hT;                  // [N, H, 128, 128] or null
  uint16_t *o;                // bf16 bits [T, H, 128]
  int64_t T;
  int32_t N, H;
  float scale;
  const uint16_t *b;  // fused prologue, as in IntraArgs
  int64_t b_stride;
  float qk_eps;
  // fused gated-RMSNorm epilogue when y is set: y[t, h, :] from o's fp32
  // row, the gate row at z + t * z_stride + h * 128 and the weight nw [128]
  uint16_t *y;
  const uint16_t *z;
  int64_t z_stride;
  const float *nw;
  float neps;
  int32_t act;  // 0 sigmoid, 1 SiLU
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace kda
