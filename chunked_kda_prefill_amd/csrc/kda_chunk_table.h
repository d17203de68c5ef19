// Chunk table of the flat packed-chunk grid (KDA TPU report, section 6.5):
// chunks are taken relative to each sequence's start (so a sequence's results
// do not depend on where it is packed), a sequence of length L owns
// ceil(L/64) chunks, and each chunk records (token start, length, sequence,
// local index).  cu_seqlens is clamped into [0, T] first so that malformed
// device input can never send a later kernel out of bounds; a flag word
// records that it was malformed.
//
// chunk_table_build() is run by one 256-thread workgroup: the standalone
// chunk-table kernel, or every workgroup of the intra-chunk kernel when the
// batch is small enough to keep the per-sequence chunk offsets in LDS.  Up to
// 64 sequences, one wave builds it with a shuffle scan and no barriers but
// the last (every workgroup of the intra kernel pays this prologue).
#pragma once

#include "kda_internal.h"

namespace kda {

constexpr int TABLE_THREADS = 256;
constexpr int INLINE_SEQS = 1024;  // batches up to this size keep first[] in LDS

// Scratch in LDS for one build.
struct TableScratch {
  int64_t scan[TABLE_THREADS];
  int64_t carry;
  int32_t bad;
};

__device__ __forceinline__ int64_t table_clamp(int64_t x, int64_t T) {
  return x < 0 ? 0 : (x > T ? T : x);
}

// Builds the chunk offsets of sequences 0..N-1 (clamped to nc_max) into
// first_lds[0..N] when first_lds is given (N <= INLINE_SEQS), and writes the
// workspace table (chunk_first, chunk_info with inert rows past the real
// chunk count, flags) when `write` is set.  Called by all 256 threads.
__device__ __forceinline__ void chunk_table_build(const int32_t *__restrict__ cu, int64_t T,
                                                  int32_t N, int64_t nc_max, bool write,
                                                  int32_t *__restrict__ chunk_first,
                                                  int4 *__restrict__ chunk_info,
                                                  int32_t *__restrict__ flags, int32_t *first_lds,
                                                  TableScratch &sc) {
  const int tid = threadIdx.x;
  if (N <= 64) {
    // Up to 64 sequences: one wave, one sequence per lane, the scan across
    // lanes by shuffles; the other waves only meet the closing barrier.
    if (tid < 64) {
      const int s = tid;
      int64_t cnt = 0, a = 0, L = 0;
      bool bad = false;
      if (s < N) {
        const int64_t a_raw = cu[s], b_raw = cu[s + 1];
        a = table_clamp(a_raw, T);
        const int64_t b = table_clamp(b_raw, T);
        L = b > a ? b - a : 0;
        cnt = (L + BT - 1) / BT;
        bad = (a != a_raw) || (b != b_raw) || (b_raw < a_raw);
        if (s == 0 && a_raw != 0) bad = true;
        if (s == N - 1 && b_raw != T) bad = true;
      }
      int64_t incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t up = __shfl_up(incl, off, 64);
        if (s >= off) incl += up;
      }
      const int64_t first = incl - cnt;
      const int64_t total = __shfl(incl, 63, 64);
      const int64_t nc = total < nc_max ? total : nc_max;
      if (s < N) {
        const int32_t f = (int32_t)(first < nc_max ? first : nc_max);
        if (first_lds) first_lds[s] = f;
        if (write) {
          chunk_first[s] = f;
          for (int64_t j = 0; j < cnt; ++j) {
            const int64_t c = first + j;
            if (c >= nc_max) {
              bad = true;
              break;
            }
            const int64_t len = L - j * BT < BT ? L - j * BT : BT;
            chunk_info[c] = make_int4((int)(a + j * BT), (int)len, (int)s, (int)j);
          }
        }
      }
      if (s == 0) {
        if (first_lds) first_lds[N] = (int32_t)nc;
        if (write) chunk_first[N] = (int32_t)nc;
      }
      if (write) {
        for (int64_t c = nc + s; c < nc_max; c += 64) chunk_info[c] = make_int4(0, 0, -1, -1);
        const bool any_bad = __any(bad);
        if (s == 0) flags[0] = any_bad ? 1 : 0;
      }
    }
    __syncthreads();
    return;
  }
  if (tid == 0) {
    sc.carry = 0;
    sc.bad = 0;
  }
  __syncthreads();

  // Per block of 256 sequences: chunk counts, their exclusive scan (with the
  // running carry of earlier blocks), then one chunk_info row per chunk.
  for (int64_t base = 0; base < N; base += TABLE_THREADS) {
    const int64_t s = base + tid;
    int64_t cnt = 0, a = 0, L = 0;
    if (s < N) {
      const int64_t a_raw = cu[s], b_raw = cu[s + 1];
      a = table_clamp(a_raw, T);
      const int64_t b = table_clamp(b_raw, T);
      L = b > a ? b - a : 0;
      cnt = (L + BT - 1) / BT;
      bool bad = (a != a_raw) || (b != b_raw) || (b_raw < a_raw);
      if (s == 0 && a_raw != 0) bad = true;
      if (s == N - 1 && b_raw != T) bad = true;
      if (bad) atomicOr(&sc.bad, 1);
    }
    sc.scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < TABLE_THREADS; off <<= 1) {
      const int64_t add = tid >= off ? sc.scan[tid - off] : 0;
      __syncthreads();
      sc.scan[tid] += add;
      __syncthreads();
    }
    const int64_t first = sc.carry + sc.scan[tid] - cnt;
    if (s < N) {
      const int32_t f = (int32_t)(first < nc_max ? first : nc_max);
      if (first_lds) first_lds[s] = f;
      if (write) {
        chunk_first[s] = f;
        for (int64_t j = 0; j < cnt; ++j) {
          const int64_t c = first + j;
          if (c >= nc_max) {
            atomicOr(&sc.bad, 1);
            break;
          }
          const int64_t len = L - j * BT < BT ? L - j * BT : BT;
          chunk_info[c] = make_int4((int)(a + j * BT), (int)len, (int)s, (int)j);
        }
      }
    }
    __syncthreads();
    if (tid == TABLE_THREADS - 1) sc.carry += sc.scan[TABLE_THREADS - 1];
    __syncthreads();
  }
  const int64_t total = sc.carry;
  const int32_t bad = sc.bad;  // read before the last barrier: the caller may reuse sc after it
  const int64_t nc = total < nc_max ? total : nc_max;
  if (tid == 0) {
    if (first_lds) first_lds[N] = (int32_t)nc;
    if (write) chunk_first[N] = (int32_t)nc;
  }
  if (write) {
    // Rows past the real chunk count are inert.
    for (int64_t c = nc + tid; c < nc_max; c += TABLE_THREADS) chunk_info[c] = make_int4(0, 0, -1, -1);
  }
  __syncthreads();
  if (write && tid == 0) flags[0] = bad;
}

// The record chunk_table_build writes for chunk c of sequence s (first[] its
// chunk offsets): the same arithmetic, so both paths agree bit for bit.
__device__ __forceinline__ int4 chunk_record_of(const int32_t *__restrict__ cu, int64_t T,
                                                const int32_t *first, int s, int64_t c) {
  const int64_t a = table_clamp(cu[s], T);
  const int64_t b = table_clamp(cu[s + 1], T);
  const int64_t L = b > a ? b - a : 0;
  const int64_t j = c - first[s];
  const int64_t len = L - j * BT < BT ? L - j * BT : BT;
  return make_int4((int)(a + j * BT), (int)len, s, (int)j);
}

}  // namespace kda
