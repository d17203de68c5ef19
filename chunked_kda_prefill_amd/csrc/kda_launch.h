// Host-side launchers, one per kernel; each lives in its kernel's source
// file and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

hipError_t launch_chunk_table(const int32_t *cu, int64_t T, int32_t N, int64_t nc_max,
                              int32_t *chunk_first, int4 *chunk_info, int32_t *flags,
                              hipStream_t stream);

hipError_t launch_gate_cumsum(const float *g, const int32_t *chunk_first, const int4 *chunk_info,
                              int64_t nc_max, int32_t N, int32_t H, float *G, hipStream_t stream);

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

struct RecurArgs {
  const uint8_t *blocks;
  const int32_t *chunk_first;
  const int4 *chunk_info;
  const float *h0;      // [N, H, 128, 128] or null
  float *hT;            // [N, H, 128, 128] or null
  uint16_t *o;          // bf16 bits [T, H, 128]
  int64_t nc_max, T;
  int32_t N, H;
};
hipError_t launch_recurrence(const RecurArgs &a, hipStream_t stream);

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
