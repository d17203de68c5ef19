// Chunk table and standalone gate cumsum.  The table itself is built by
// chunk_table_build (kda_chunk_table.h); it is built on the device so that a
// call never synchronises with the host.
#include "kda_chunk_table.h"
#include "kda_cumsum.h"
#include "kda_internal.h"
#include "kda_launch.h"
#include "kda_plan.h"

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

// ---------------------------------------------------------------------------
// Plan of the single-launch path (what it writes: kda_plan.h).  One
// workgroup of 256 threads: the chunk table (chunk_table_build, with the
// per-sequence chunk offsets also kept in LDS), a bitonic sort of the
// sequences by chunk count, the per-XCD unit lists, and zeroed counters and
// ready flags.  Up to PLAN_MAX_SEQS sequences.
// ---------------------------------------------------------------------------
constexpr int PLAN_THREADS = 256;

struct __align__(16) PlanSmem {
  TableScratch sc;
  int32_t first[PLAN_MAX_SEQS + 1];
  int64_t key[PLAN_MAX_SEQS];
  int32_t nsorted[PLAN_MAX_SEQS];
  int64_t red[PLAN_THREADS];
  int64_t xunits[XCDS];
};

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(PlanArgs a) {
  __shared__ PlanSmem sm;
  const int tid = threadIdx.x;
  const int N = a.N, H = a.H;
  chunk_table_build(a.cu, a.T, N, a.nc_max, true, a.chunk_first, a.chunk_info, a.flags, sm.first,
                    sm.sc);
  __syncthreads();

  // zeroed ready flags (one per block) and counters
  const int64_t nunits = (int64_t)H * a.nc_max;
  for (int64_t i = tid; i < nunits; i += PLAN_THREADS) a.ready[i] = 0;
  if (tid < XCDS) {
    a.sync[SYNC_TICKET + SYNC_STRIDE * tid] = 0;
    a.sync[SYNC_UNIT + SYNC_STRIDE * tid] = 0;
  }
  if (tid < 3) a.sync[SYNC_DIAG + tid] = tid == 0 ? -1 : 0;

  // sequences sorted by chunk count, longest first, ties by index: ascending
  // order of ((2^31 - 1 - n) << 32) | s, padded to a power of two
  int P2 = 1;
  while (P2 < N) P2 <<= 1;
  for (int i = tid; i < P2; i += PLAN_THREADS) {
    int64_t k = INT64_MAX;
    if (i < N) {
      const int n = sm.first[i + 1] - sm.first[i];
      k = ((int64_t)(0x7FFFFFFF - n) << 32) | (uint32_t)i;
    }
    sm.key[i] = k;
  }
  __syncthreads();
  for (int k = 2; k <= P2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P2; i += PLAN_THREADS) {
        const int l = i ^ j;
        if (l > i) {
          const int64_t x0 = sm.key[i], x1 = sm.key[l];
          const bool up = (i & k) == 0;
          if ((x0 > x1) == up) {
            sm.key[i] = x1;
            sm.key[l] = x0;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < N; i += PLAN_THREADS) {
    const int sq = (int)(sm.key[i] & 0xFFFFFFFF);
    a.order[i] = sq;
    sm.nsorted[i] = sm.first[sq + 1] - sm.first[sq];
  }
  __syncthreads();
  const int jmax = N > 0 ? sm.nsorted[0] : 0;
  // S_j = number of sequences with more than j chunks (nsorted does not
  // increase); C_j = H S_j chains; XCD x holds ceil((C_j - x) / 8) of them
  auto seqs_longer = [&](int j) {
    int lo = 0, hi = N;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sm.nsorted[mid] > j) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  auto row_count = [](int64_t C, int x) -> int64_t { return C > x ? (C - x + 7) >> 3 : 0; };

  // units per XCD
  int64_t part[XCDS];
#pragma unroll
  for (int x = 0; x < XCDS; ++x) part[x] = 0;
  for (int j = tid; j < jmax; j += PLAN_THREADS) {
    const int64_t C = (int64_t)H * seqs_longer(j);
#pragma unroll
    for (int x = 0; x < XCDS; ++x) part[x] += row_count(C, x);
  }
  for (int x = 0; x < XCDS; ++x) {
    sm.red[tid] = part[x];
    __syncthreads();
    for (int off = PLAN_THREADS / 2; off > 0; off >>= 1) {
      if (tid < off) sm.red[tid] += sm.red[tid + off];
      __syncthreads();
    }
    if (tid == 0) sm.xunits[x] = sm.red[0];
    __syncthreads();
  }
  if (tid == 0) {
    int64_t acc = 0;
    for (int x = 0; x < XCDS; ++x) {
      a.sync[SYNC_XOFF + x] = (int32_t)acc;
      acc += sm.xunits[x];
    }
    a.sync[SYNC_XOFF + XCDS] = (int32_t)acc;
  }

  // unit lists: XCD by XCD, rows j in blocks of PLAN_THREADS, each row's
  // entries at its exclusive prefix of row counts
  int64_t base = 0;
  for (int x = 0; x < XCDS; ++x) {
    int64_t carry = 0;
    for (int jb = 0; jb < jmax; jb += PLAN_THREADS) {
      const int j = jb + tid;
      const int64_t cnt = j < jmax ? row_count((int64_t)H * seqs_longer(j), x) : 0;
      sm.red[tid] = cnt;
      __syncthreads();
      for (int off = 1; off < PLAN_THREADS; off <<= 1) {
        const int64_t add = tid >= off ? sm.red[tid - off] : 0;
        __syncthreads();
        sm.red[tid] += add;
        __syncthreads();
      }
      const int64_t pos = base + carry + sm.red[tid] - cnt;
      for (int64_t r = 0; r < cnt; ++r) {
        const int64_t rho = 8 * r + x;
        const int i = (int)(rho / H), h = (int)(rho % H);
        const int sq = (int)(sm.key[i] & 0xFFFFFFFF);
        const int64_t c = (int64_t)sm.first[sq] + j;
        a.units[pos + r] = (int32_t)(c * H + h);
      }
      carry += sm.red[PLAN_THREADS - 1];
      __syncthreads();
    }
    base += sm.xunits[x];
  }
}

hipError_t launch_plan(const PlanArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, a);
  return hipGetLastError();
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
