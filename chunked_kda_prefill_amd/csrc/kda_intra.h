// Arguments and launcher of the intra-chunk kernel (kda_intra.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct IntraArgs {
  const uint16_t *q, *k, *v;  // bf16 bits [T, H, 128]
  const float *g;             // [T, H, 128]
  const float *beta;          // [T, H]
  const int32_t *cu;          // cu_seqlens [N + 1]
  int32_t *chunk_first;       // [N + 1]   (written by the kernel when inline_table)
  int4 *chunk_info;           // [nc_max]  (same)
  int32_t *flags;             // [1]       (same)
  uint8_t *blocks;            // H * nc_max intermediate blocks
  int64_t nc_max, T;
  int32_t N, H;
  float scale;
  // N <= INLINE_SEQS: every workgroup builds the chunk offsets in LDS and
  // workgroup 0 writes the workspace table; else chunk_table_kernel has
  // written it before this launch
  int32_t inline_table;
  // fused prologue: beta = sigmoid(b[t * b_stride + h]) when b is set (bf16
  // logits, beta unused); q and k L2-normalised per (token, head) as
  // x / sqrt(sum x^2 + qk_eps) when qk_eps >= 0
  const uint16_t *b;
  int64_t b_stride;
  float qk_eps;
};
hipError_t launch_intra(const IntraArgs &a, hipStream_t stream);

}  // namespace kda
