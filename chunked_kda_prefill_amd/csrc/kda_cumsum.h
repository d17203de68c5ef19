// Chunk-local inclusive gate cumsum (KDA TPU report, section 6.1: the
// cumsum runs inside the kernel that already holds the chunk's gate block,
// restarting at every chunk).  Shared by the standalone cumsum kernel and the
// intra-chunk kernel's prologue.
#pragma once

#include "kda_internal.h"

namespace kda {

// Chunk-local cumsum in two halves so that a caller can issue the loads
// early (e.g. for the next chunk while the current one computes) and scan
// later.  Thread layout for NT threads: channel group cg = tid & 31 owns
// channels 4cg..4cg+3 (one 16-byte load per row, so 32 lanes read a row's
// 512 bytes); row group rg = tid >> 5 owns RPT = 64 / (NT / 32) consecutive
// rows.
template <int NT>
struct GateRows {
  static constexpr int NRG = NT / 32;
  static constexpr int RPT = BT / NRG;
  float4 x[RPT];
};

// Loads g rows t0 .. t0+n-1 of head h; rows >= n read as zero (padding with
// g = 0 keeps G at G[n-1] past the end of a partial chunk).
template <int NT>
__device__ __forceinline__ void gate_rows_load(const float *__restrict__ g, int64_t t0, int n, int H,
                                               int h, GateRows<NT> &gr) {
  const int tid = threadIdx.x;
  const int cg = tid & 31;
  const int rg = tid >> 5;
#pragma unroll
  for (int r = 0; r < GateRows<NT>::RPT; ++r) {
    const int i = rg * GateRows<NT>::RPT + r;
    gr.x[r] = i < n ? *reinterpret_cast<const float4 *>(g + ((t0 + i) * (int64_t)H + h) * DK + cg * 4)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Inclusive scan over the chunk's rows: each thread scans its rows in
// registers, the row-group totals are combined through LDS (`tot`, at least
// (NT/32) x 128 floats), and G (fp32, natural-log units) is written at
// element gidx(row, channel), which must keep aligned groups of 4 channels
// contiguous.  Called by all NT threads; contains one barrier.
template <int NT, typename GIdx>
__device__ __forceinline__ void gate_rows_scan(GateRows<NT> gr, float *G, GIdx gidx, float *tot) {
  constexpr int RPT = GateRows<NT>::RPT;
  const int tid = threadIdx.x;
  const int cg = tid & 31;
  const int rg = tid >> 5;
#pragma unroll
  for (int r = 1; r < RPT; ++r) {
    gr.x[r].x += gr.x[r - 1].x;
    gr.x[r].y += gr.x[r - 1].y;
    gr.x[r].z += gr.x[r - 1].z;
    gr.x[r].w += gr.x[r - 1].w;
  }
  *reinterpret_cast<float4 *>(&tot[rg * DK + cg * 4]) = gr.x[RPT - 1];
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
    float4 y = gr.x[r];
    y.x += off.x;
    y.y += off.y;
    y.z += off.z;
    y.w += off.w;
    *reinterpret_cast<float4 *>(&G[gidx(rg * RPT + r, cg * 4)]) = y;
  }
}

// Both halves back to back.
template <int NT, typename GIdx>
__device__ __forceinline__ void chunk_gate_cumsum(const float *__restrict__ g, int64_t t0, int n,
                                                  int H, int h, float *G, GIdx gidx, float *tot) {
  GateRows<NT> gr;
  gate_rows_load<NT>(g, t0, n, H, h, gr);
  gate_rows_scan<NT>(gr, G, gidx, tot);
}

}  // namespace kda
