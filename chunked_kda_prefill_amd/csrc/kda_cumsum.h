// Chunk-local inclusive gate cumsum (KDA TPU report, section 6.1: the
// cumsum runs inside the kernel that already holds the chunk's gate block,
// restarting at every chunk).  Shared by the intra-chunk kernel and the
// standalone cumsum kernel, so both sum in the same order.
//
// Chunk layout used by both: four waves per chunk; wave a holds the rows of
// subblock a (rows 16a .. 16a+15), lane (n, grp) = (lane & 15, lane >> 4)
// holds row 16a + n and, for j = 0..7, the four channels slot_ch(j, grp) ..
// slot_ch(j, grp) + 3.  Those channel slots are the permuted MFMA k order of
// kda_internal.h (k-step s = j / 2, element e = 4 (j % 2) + 0..3), so values
// computed per element drop straight into MFMA operand registers.
//
// The scan runs down the 16 rows of a subblock with DPP row shifts (a DPP
// row is the 16 lanes that share one grp), four steps per value; subblocks
// are then joined by adding the totals of the subblocks before them.
#pragma once

#include "kda_internal.h"

namespace kda {

constexpr int CHUNK_WAVES = BT / SB;          // 4
constexpr int CHUNK_THREADS = 64 * CHUNK_WAVES;  // 256

__device__ __forceinline__ int slot_ch(int j, int grp) {
  return 32 * (j >> 1) + 16 * (j & 1) + 4 * grp;
}

// Lane l - K of the same 16-lane row, or 0 for the first K lanes of a row.
template <int K>
__device__ __forceinline__ float dpp_row_shr(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + K, 0xF, 0xF, true));
}

// Inclusive sum over rows 0..n of the lane's subblock (Hillis-Steele).
__device__ __forceinline__ float subblock_scan(float x) {
  x += dpp_row_shr<1>(x);
  x += dpp_row_shr<2>(x);
  x += dpp_row_shr<4>(x);
  x += dpp_row_shr<8>(x);
  return x;
}

__device__ __forceinline__ float4 subblock_scan(float4 v) {
  return make_float4(subblock_scan(v.x), subblock_scan(v.y), subblock_scan(v.z),
                     subblock_scan(v.w));
}

// Gate rows of one lane: row `row` (< n, else zeros: padding with g = 0
// keeps the cumsum at its value at row n - 1 past a partial chunk's end).
__device__ __forceinline__ void gate_slots_load(const float *__restrict__ g, int64_t t0, int n,
                                                int H, int h, int row, int grp, float4 (&x)[8]) {
  const bool ok = row < n;
  const float *p = g + ((t0 + (ok ? row : 0)) * (int64_t)H + h) * DK;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    x[j] = ok ? *reinterpret_cast<const float4 *>(p + slot_ch(j, grp)) : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Chunk-level G at channel slots: carry of subblock a = sum of the totals of
// subblocks 0..a-1, accumulated in that order starting from zero.
__device__ __forceinline__ float subblock_carry(const float *tot, int a, int ch) {
  float acc = 0.f;
  for (int b = 0; b < a; ++b) acc += tot[b * DK + ch];
  return acc;
}

}  // namespace kda
