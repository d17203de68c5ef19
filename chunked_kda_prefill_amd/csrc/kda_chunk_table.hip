// Chunk table and standalone gate cumsum.  The table itself is built by
// chunk_table_build (kda_chunk_table.h); it is built on the device so that a
// call never synchronises with the host.
#include "kda_chunk_table.h"
#include "kda_cumsum.h"
#include "kda_internal.h"
#include "kda_launch.h"

namespace kda {

// One workgroup of 256 threads.
__global__ __launch_bounds__(TABLE_THREADS) void chunk_table_kernel(
    const int32_t *__restrict__ cu, int64_t T, int32_t N, int64_t nc_max,
    int32_t *__restrict__ chunk_first, int4 *__restrict__ chunk_info, int32_t *__restrict__ flags) {
  __shared__ TableScratch sc;
  chunk_table_build(cu, T, N, nc_max, true, chunk_first, chunk_info, flags, nullptr, sc);
}

// Standalone chunk-local cumsum: one workgroup per (chunk slot, head), with
// the intra-chunk kernel's chunk layout and summation order (kda_cumsum.h):
// a DPP scan down each 16-row subblock, plus the running total of the
// subblocks before it.
__global__ __launch_bounds__(CHUNK_THREADS) void gate_cumsum_kernel(const float *__restrict__ g,
                                                                    const int32_t *__restrict__ chunk_first,
                                                                    const int4 *__restrict__ chunk_info,
                                                                    int32_t N, int32_t H,
                                                                    float *__restrict__ Gout) {
  __shared__ __align__(16) float tot[CHUNK_WAVES * DK];
  const int64_t c = blockIdx.x / H;
  const int h = blockIdx.x % H;
  if (c >= chunk_first[N]) return;
  const int4 info = chunk_info[c];
  const int64_t t0 = info.x;
  const int n = info.y;
  const int tid = threadIdx.x;
  const int w = tid >> 6, nn = tid & 15, grp = (tid >> 4) & 3;
  const int row = SB * w + nn;
  float4 x[8];
  gate_slots_load(g, t0, n, H, h, row, grp, x);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = subblock_scan(x[j]);
  if (nn == SB - 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<float4 *>(&tot[w * DK + slot_ch(j, grp)]) = x[j];
  }
  __syncthreads();
  if (row < n) {
    float *out = Gout + ((t0 + row) * (int64_t)H + h) * DK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ch = slot_ch(j, grp);
      const float4 y = make_float4(subblock_carry(tot, w, ch) + x[j].x,
                                   subblock_carry(tot, w, ch + 1) + x[j].y,
                                   subblock_carry(tot, w, ch + 2) + x[j].z,
                                   subblock_carry(tot, w, ch + 3) + x[j].w);
      *reinterpret_cast<float4 *>(out + ch) = y;
    }
  }
}

hipError_t launch_chunk_table(const int32_t *cu, int64_t T, int32_t N, int64_t nc_max,
                              int32_t *chunk_first, int4 *chunk_info, int32_t *flags,
                              hipStream_t stream) {
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(TABLE_THREADS), 0, stream, cu, T, N, nc_max,
                     chunk_first, chunk_info, flags);
  return hipGetLastError();
}

hipError_t launch_gate_cumsum(const float *g, const int32_t *chunk_first, const int4 *chunk_info,
                              int64_t nc_max, int32_t N, int32_t H, float *G, hipStream_t stream) {
  if (nc_max <= 0) return hipSuccess;
  hipLaunchKernelGGL(gate_cumsum_kernel, dim3((unsigned)(nc_max * H)), dim3(CHUNK_THREADS), 0,
                     stream, g,
                     chunk_first, chunk_info, N, H, G);
  return hipGetLastError();
}

}  // namespace kda
