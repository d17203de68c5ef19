// Chunk table and standalone gate cumsum.
//
// The chunk table is the device-side bookkeeping of the flat packed-chunk
// grid (KDA TPU report, section 6.5): chunks are taken relative to each
// sequence's start (so a sequence's results do not depend on where it is
// packed), a sequence of length L owns ceil(L/64) chunks, and each chunk
// records its sequence id and local index.  It is built on the device so
// that a call never synchronises with the host.
#include "kda_cumsum.h"
#include "kda_internal.h"
#include "kda_launch.h"

namespace kda {

// One workgroup of 256 threads.  cu_seqlens is clamped into [0, T] first so
// that malformed device input can never send a later kernel out of bounds.
__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t *__restrict__ cu, int64_t T,
                                                          int32_t N, int64_t nc_max,
                                                          int32_t *__restrict__ chunk_first,
                                                          int4 *__restrict__ chunk_info,
                                                          int32_t *__restrict__ flags) {
  __shared__ int64_t scan[256];
  __shared__ int64_t carry_s;
  __shared__ int32_t bad_s;
  const int tid = threadIdx.x;
  if (tid == 0) {
    carry_s = 0;
    bad_s = 0;
  }
  __syncthreads();

  auto clampi = [&](int64_t x) -> int64_t { return x < 0 ? 0 : (x > T ? T : x); };

  // Per block of 256 sequences: chunk counts, their exclusive scan (with the
  // running carry of earlier blocks), then one chunk_info row per chunk.
  for (int64_t base = 0; base < N; base += 256) {
    const int64_t s = base + tid;
    int64_t cnt = 0, a = 0, L = 0;
    if (s < N) {
      const int64_t a_raw = cu[s], b_raw = cu[s + 1];
      a = clampi(a_raw);
      const int64_t b = clampi(b_raw);
      L = b > a ? b - a : 0;
      cnt = (L + BT - 1) / BT;
      bool bad = (a != a_raw) || (b != b_raw) || (b_raw < a_raw);
      if (s == 0 && a_raw != 0) bad = true;
      if (s == N - 1 && b_raw != T) bad = true;
      if (bad) atomicOr(&bad_s, 1);
    }
    scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int64_t add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int64_t first = carry_s + scan[tid] - cnt;
    if (s < N) {
      chunk_first[s] = (int32_t)(first < nc_max ? first : nc_max);
      for (int64_t j = 0; j < cnt; ++j) {
        const int64_t c = first + j;
        if (c >= nc_max) {
          atomicOr(&bad_s, 1);
          break;
        }
        const int64_t len = L - j * BT < BT ? L - j * BT : BT;
        chunk_info[c] = make_int4((int)(a + j * BT), (int)len, (int)s, (int)j);
      }
    }
    __syncthreads();
    if (tid == 255) carry_s += scan[255];
    __syncthreads();
  }
  const int64_t total = carry_s;
  const int64_t nc = total < nc_max ? total : nc_max;
  if (tid == 0) chunk_first[N] = (int32_t)nc;

  // Rows past the real chunk count are inert.
  for (int64_t c = nc + tid; c < nc_max; c += 256) chunk_info[c] = make_int4(0, 0, -1, -1);
  __syncthreads();
  if (tid == 0) flags[0] = bad_s;
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
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, stream, cu, T, N, nc_max,
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
