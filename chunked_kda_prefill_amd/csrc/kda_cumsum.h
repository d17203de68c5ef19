// Chunk-local inclusive gate cumsum (KDA TPU report, section 6.1: the
// cumsum runs inside the kernel that already holds the chunk's gate block,
// restarting at every chunk).  Shared by the standalone cumsum kernel and the
// intra-chunk kernel's prologue.
#pragma once

#include "kda_internal.h"

namespace kda {

// Reads g rows t0 .. t0+n-1 of head h (zero for rows >= n, i.e. padding with
// g = 0 so that G stays at G[n-1] past the end of a partial chunk) and
// writes G[64][gld] (fp32, natural-log units) into LDS.  Called by all 256
// threads of the workgroup; `tot` is an LDS scratch of 8 x 128 floats.
//
// Thread layout: channel group cg = tid & 31 owns channels 4cg..4cg+3 (one
// 16-byte load per row, so 32 lanes read a row's 512 bytes), row group
// rg = tid >> 5 owns rows 8rg..8rg+7.  Each thread scans its 8 rows in
// registers; the 8 row-group totals are then combined through LDS.
template <int GLD>
__device__ __forceinline__ void chunk_gate_cumsum(const float *__restrict__ g, int64_t t0, int n,
                                                  int H, int h, float (*G)[GLD], float (*tot)[DK]) {
  const int tid = threadIdx.x;
  const int cg = tid & 31;
  const int rg = tid >> 5;
  float4 x[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int i = rg * 8 + r;
    if (i < n) {
      x[r] = *reinterpret_cast<const float4 *>(g + ((t0 + i) * (int64_t)H + h) * DK + cg * 4);
    } else {
      x[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int r = 1; r < 8; ++r) {
    x[r].x += x[r - 1].x;
    x[r].y += x[r - 1].y;
    x[r].z += x[r - 1].z;
    x[r].w += x[r - 1].w;
  }
  *reinterpret_cast<float4 *>(&tot[rg][cg * 4]) = x[7];
  __syncthreads();
  float4 off = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q = 0; q < rg; ++q) {
    const float4 t = *reinterpret_cast<const float4 *>(&tot[q][cg * 4]);
    off.x += t.x;
    off.y += t.y;
    off.z += t.z;
    off.w += t.w;
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float4 y = x[r];
    y.x += off.x;
    y.y += off.y;
    y.z += off.z;
    y.w += off.w;
    *reinterpret_cast<float4 *>(&G[rg * 8 + r][cg * 4]) = y;
  }
}

}  // namespace kda
