// Chunk-local inclusive gate cumsum (KDA TPU report, section 6.1: the
// cumsum runs inside the kernel that already holds the chunk's gate block,
// restarting at every chunk).  Shared by the standalone cumsum kernel and the
// intra-chunk kernel's prologue.
#pragma once

#include "kda_internal.h"

namespace kda {

// Reads g rows t0 .. t0+n-1 of head h (zero for rows >= n, i.e. padding with
// g = 0 so that G stays at G[n-1] past the end of a partial chunk) and
// writes G (fp32, natural-log units) into LDS at element gidx(row, channel),
// which must keep each aligned group of 4 channels contiguous.  Called by all
// NT threads of the workgroup; `tot` is an LDS scratch of (NT/32) x 128
// floats.
//
// Thread layout: channel group cg = tid & 31 owns channels 4cg..4cg+3 (one
// 16-byte load per row, so 32 lanes read a row's 512 bytes), row group
// rg = tid >> 5 owns RPT = 64 / (NT / 32) consecutive rows.  Each thread
// scans its rows in registers; the row-group totals are combined through
// LDS.
template <int NT, typename GIdx>
__device__ __forceinline__ void chunk_gate_cumsum(const float *__restrict__ g, int64_t t0, int n,
                                                  int H, int h, float *G, GIdx gidx, float *tot) {
  constexpr int NRG = NT / 32;
  constexpr int RPT = BT / NRG;
  const int tid = threadIdx.x;
  const int cg = tid & 31;
  const int rg = tid >> 5;
  float4 x[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = rg * RPT + r;
    if (i < n) {
      x[r] = *reinterpret_cast<const float4 *>(g + ((t0 + i) * (int64_t)H + h) * DK + cg * 4);
    } else {
      x[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int r = 1; r < RPT; ++r) {
    x[r].x += x[r - 1].x;
    x[r].y += x[r - 1].y;
    x[r].z += x[r - 1].z;
    x[r].w += x[r - 1].w;
  }
  *reinterpret_cast<float4 *>(&tot[rg * DK + cg * 4]) = x[RPT - 1];
  __syncthreads();
  float4 off = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q = 0; q < rg; ++q) {
    const float4 t = *reinterpret_cast<const float4 *>(&tot[q * DK + cg * 4]);
    off.x += t.x;
    off.y += t.y;
    off.z += t.z;
    off.w += t.w;
  }
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    float4 y = x[r];
    y.x += off.x;
    y.y += off.y;
    y.z += off.z;
    y.w += off.w;
    *reinterpret_cast<float4 *>(&G[gidx(rg * RPT + r, cg * 4)]) = y;
  }
}

}  // namespace kda
