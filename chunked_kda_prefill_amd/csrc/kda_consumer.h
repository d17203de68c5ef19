// Chain consumer of the single-launch path: the chunk recurrence and output
// (KDA TPU report, section 6.2; MI355X serving post, section 1.1) of whole
// (sequence, head) chains, one workgroup per chain at a time, reading each
// intermediate block as soon as its producer has flagged it ready.
//
// Per chunk, with h the entry state:
//     v_new = U - W h;   o = qg h + Aqk v_new;   h <- Diag(gamma) h + kg^T v_new
// Wave w keeps value tiles 2w and 2w + 1 (32 value columns) of the fp32
// state in MFMA C tiles for the whole chain; the state and v_new feed the
// MFMAs as bf16 B operands straight from their C tiles, in the permuted k
// order the intra-chunk kernel wrote its A fragments in (kda_internal.h).
//
// One LDS copy of the block (the workspace of the producers' LDS is not
// needed here, so the two share the space).  It is split in two regions:
//   A = -W, qg (the first phase's A fragments), the wave's own U tiles and
//       gamma;
//   B = kg^T and Aqk (the second phase).
// Region A of chunk c + 1 is copied while phase B of chunk c runs, and
// region B of chunk c + 1 while phase A of chunk c + 1 runs; two barriers
// per chunk separate the copies from the reads.
//
// Visibility.  Producer and consumer of a block run on the same XCD and
// share its L2: the producer's plain stores are complete in L2 once its
// waves have waited for them (s_waitcnt vmcnt(0)) before the barrier that
// precedes its ready-flag store.  The flag itself is stored and polled as a
// relaxed device-scope atomic (coherent device-wide, never a stale L1
// copy).  The consumer issues the block's copy only after it has seen the
// flag; the copy reads L2 (no line of a block can be in the consumer's L1:
// L1 starts each kernel empty, blocks are written once per call, and each
// is read once, after its flag).  Every wait for a flag is bounded in time; a wait that gives up sets
// FLAG_TIMEOUT in the workspace flags word and the chain goes on (its
// results are then invalid, never out of bounds).
#pragma once

#include "kda_internal.h"

namespace kda {

struct ConsumerArgs {
  const uint8_t *blocks;       // H * nc_max intermediate blocks
  const int32_t *chunk_first;  // [N + 1]
  const int4 *chunk_info;      // [nc_max]
  const int32_t *order;        // [N] sequences, longest first
  const int32_t *ready;        // [H * nc_max] block ready flags
  int32_t *flags;              // workspace flags word
  int32_t *diag;               // [3]: last block a wait gave up on, its flag, waits given up
  const float *h0;             // [N, H, 128, 128] or null
  float *hT;                   // [N, H, 128, 128] or null
  uint16_t *o;                 // bf16 bits [T, H, 128]
  int64_t nc_max, T;
  int32_t N, H;
};

namespace cons {

constexpr int ROUND = 1024;  // one wave's copy: 64 lanes x 16 bytes
// region A: -W and qg, 32 rounds, eight per wave; then each wave's own U
// tiles (4 rounds) and a quarter of gamma (8 lanes x 16 bytes)
constexpr int A_SHARED_PER_WAVE = (OFF_KGT - OFF_WN) / ROUND / 4;  // 8
constexpr int A_ROUNDS = A_SHARED_PER_WAVE + 4 + 1;                 // per wave
// region B: kg^T and Aqk, 22 rounds over four waves (6, 6, 5, 5)
constexpr int B_TOTAL = (OFF_U - OFF_KGT) / ROUND;  // 22
static_assert((OFF_KGT - OFF_WN) % (4 * ROUND) == 0, "region A splits over four waves");
static_assert((OFF_U - OFF_KGT) % ROUND == 0, "region B is whole rounds");
// o of a chunk: one 16-byte store per token tile per lane
constexpr int O_STORES = 4;
// bounded wait for a ready flag, in ticks of the 100 MHz real-time counter:
// a block that is not ready within 100 ms is given up on
constexpr uint64_t WAIT_TICKS = 10000000ull;

// s_waitcnt immediate for "at most n vector memory operations outstanding"
// (lgkmcnt and expcnt at their maxima)
__host__ __device__ constexpr int vm_wait(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// One buffer_load_dwordx4 ... lds round, bypassing the CU's L1 (sc0): 16
// bytes per lane from byte soff + voff of the resource into LDS at
// m0v + 16 lane.  M0 is the compiler's: it is saved and restored around the
// load (its value is taken when the load issues).
__device__ __forceinline__ void dma_sc0(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                        uint32_t m0v) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(m0v);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %4 offen sc0 lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(m), "s"(so)
      : "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t *blk) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(blk), 0, BLOCK_BYTES, BUF_DWORD3);
}

// Region A rounds of wave w: its eighth of -W and qg, its U tiles (value
// tiles 2w and 2w+1 are the 4 KB at OFF_U + 4096 w), its quarter of gamma.
// The copy keeps the block's byte offsets in LDS.
__device__ __forceinline__ void copy_region_a(const uint8_t *blk, uint32_t lbase, int w, int l) {
  const __amdgpu_buffer_rsrc_t r = block_rsrc(blk);
#pragma unroll
  for (int k = 0; k < A_SHARED_PER_WAVE; ++k) {
    const uint32_t off = OFF_WN + (w * A_SHARED_PER_WAVE + k) * ROUND;
    dma_sc0(r, 16 * l, off, lbase + off);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t off = OFF_U + (4 * w + k) * ROUND;
    dma_sc0(r, 16 * l, off, lbase + off);
  }
  // gamma: 512 bytes, 128 per wave, copied by lanes 0..7 only (the other
  // lanes are switched off: an LDS-DMA lane writes LDS even when its source
  // is out of range)
  const uint32_t off = OFF_GAM + 128 * w;
  if (l < 8) dma_sc0(r, 16 * l, off, lbase + off);
}

// Region B rounds of wave w: rounds w, w + 4, ... of kg^T and Aqk.
__device__ __forceinline__ void copy_region_b(const uint8_t *blk, uint32_t lbase, int w, int l) {
  const __amdgpu_buffer_rsrc_t r = block_rsrc(blk);
#pragma unroll
  for (int k = 0; k < (B_TOTAL + 3) / 4; ++k) {
    const int rr = w + 4 * k;
    if (rr < B_TOTAL) {
      const uint32_t off = OFF_KGT + rr * ROUND;
      dma_sc0(r, 16 * l, off, lbase + off);
    }
  }
}

// A ready flag is read and written as a relaxed device-scope atomic (a load
// or store with cache policy sc1): that access is coherent across the whole
// device, so a poll can never keep returning a stale copy from the CU's L1.
// (A workgroup-scope load, sc0, may be served by L1, where one stale line
// holds the flags of 32 chunks of a chain.)
__device__ __forceinline__ int32_t load_flag(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits (bounded) until block `blk_idx` is flagged ready.  Every lane of the
// wave polls the same word; the loop branch is wave-uniform.  After one wait
// has timed out (`gave_up`, per wave) the wave waits no more: the call's
// results are invalid by then, and FLAG_TIMEOUT says so.
__device__ __forceinline__ void wait_ready(const ConsumerArgs &a, int64_t blk_idx, bool &gave_up) {
  if (gave_up) return;
  const int32_t *p = a.ready + blk_idx;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const int32_t v = __builtin_amdgcn_readfirstlane(load_flag(p));
    if (v != 0) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 > WAIT_TICKS) {
      gave_up = true;
      if ((threadIdx.x & 63) == 0) {
        atomicOr(a.flags, FLAG_TIMEOUT);
        // what the wait was for: the block and how many waves gave up
        a.diag[0] = (int32_t)blk_idx;
        a.diag[1] = v;
        atomicAdd(a.diag + 2, 1);
      }
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

constexpr int lt_mt(int x) { return x < 2 ? x : (x < 4 ? 2 : 3); }
constexpr int lt_s(int x) { return (x == 3 || x == 5) ? 1 : 0; }

__device__ __forceinline__ int4 chunk_record(const int4 *info, int64_t c) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 v = ((const __attribute__((address_space(4))) i32x4 *)(uintptr_t)info)[c];
  return make_int4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x8 frag(const uint8_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

}  // namespace cons

// One chain: sequence s, head h.  `lds` is a BLOCK_BYTES buffer; all four
// waves of the workgroup call this together.  w is the wave index (scalar).
__device__ __forceinline__ void consume_chain(const ConsumerArgs &a, uint8_t *lds, int s, int h,
                                              int w, int l, bool &gave_up) {
  using namespace cons;
  const int nn = l & 15, grp = l >> 4;
  const int nt0 = 2 * w;  // the wave's value tiles: nt0, nt0 + 1
  const int64_t nc_max = a.nc_max;
  int64_t c_beg = ((const __attribute__((address_space(4))) int32_t *)(uintptr_t)a.chunk_first)[s];
  int64_t c_end = ((const __attribute__((address_space(4))) int32_t *)(uintptr_t)a.chunk_first)[s + 1];
  c_beg = c_beg < 0 ? 0 : (c_beg > nc_max ? nc_max : c_beg);
  c_end = c_end < c_beg ? c_beg : (c_end > nc_max ? nc_max : c_end);
  const int64_t st_base = ((int64_t)s * a.H + h) * DK * DV;
  const uint8_t *chain_blocks = a.blocks + (int64_t)h * nc_max * BLOCK_BYTES;
  const int64_t flag_base = (int64_t)h * nc_max;
  const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(lds));

  // state slice: key tiles t = 0..7, value tiles nt0 + q
  f32x4 S[8][2];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * t + 4 * grp + r;
        const int col = VCOL(nt0 + q, nn);
        S[t][q][r] = a.h0 ? a.h0[st_base + row * DV + col] : 0.f;
      }

  // the LDS buffer may still be read by another wave for the previous chain
  __syncthreads();
  if (c_beg < c_end) {
    wait_ready(a, flag_base + c_beg, gave_up);
    copy_region_a(chain_blocks + c_beg * BLOCK_BYTES, lbase, w, l);
    copy_region_b(chain_blocks + c_beg * BLOCK_BYTES, lbase, w, l);
    __builtin_amdgcn_s_waitcnt(vm_wait(0));
  }
  __syncthreads();

  for (int64_t c = c_beg; c < c_end; ++c) {
    const int4 info = chunk_record(a.chunk_info, c);
    const int64_t t0 = info.x < 0 ? 0 : (info.x > a.T ? a.T : info.x);
    const int n = (int)(info.y < 0 ? 0 : (info.y > a.T - t0 ? a.T - t0 : (info.y > BT ? BT : info.y)));

    // ---- phase A: v_new = U - W h and o^T = h^T qg^T (region A) ----
    bf16x8 fw[4], fq[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      fw[mt] = frag(lds + OFF_WN + ((mt * 4 + 0) * 64 + l) * 16);
      fq[mt] = frag(lds + OFF_QG + ((mt * 4 + 0) * 64 + l) * 16);
    }
    bf16x8 hb[4][2];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) hb[s4][q][e] = (bf16_t)S[2 * s4 + (e >> 2)][q][e & 3];
    f32x4 vn[4][2], ot[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const bf16x4 u = *reinterpret_cast<const bf16x4 *>(lds + U_OFFSET(nt0 + q, mt, l));
#pragma unroll
        for (int r = 0; r < 4; ++r) vn[mt][q][r] = (float)u[r];
        ot[mt][q] = zero4();
      }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 gm = *reinterpret_cast<const float4 *>(lds + OFF_GAM + (16 * t + 4 * grp) * 4);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        S[t][q][0] *= gm.x;
        S[t][q][1] *= gm.y;
        S[t][q][2] *= gm.z;
        S[t][q][3] *= gm.w;
      }
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      bf16x8 nw[4], nq[4];
      if (s4 < 3) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          nw[mt] = frag(lds + OFF_WN + ((mt * 4 + s4 + 1) * 64 + l) * 16);
          nq[mt] = frag(lds + OFF_QG + ((mt * 4 + s4 + 1) * 64 + l) * 16);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          vn[mt][q] = mfma_bf16(fw[mt], hb[s4][q], vn[mt][q]);
          ot[mt][q] = mfma_bf16(hb[s4][q], fq[mt], ot[mt][q]);
        }
      if (s4 < 3) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          fw[mt] = nw[mt];
          fq[mt] = nq[mt];
        }
      }
    }
    bf16x8 vb[2][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) vb[s2][q][e] = (bf16_t)vn[2 * s2 + (e >> 2)][q][e & 3];

    // region A is consumed by every wave, region B of this chunk has landed
    __builtin_amdgcn_s_waitcnt(vm_wait(0));
    __syncthreads();
    const bool more = c + 1 < c_end;
    if (more) {
      wait_ready(a, flag_base + c + 1, gave_up);
      copy_region_a(chain_blocks + (c + 1) * BLOCK_BYTES, lbase, w, l);
    }

    // ---- phase B: h <- Diag(gamma) h + kg^T v_new; o^T += v_new^T Aqk^T ----
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 fk[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) fk[t] = frag(lds + OFF_KGT + ((t * 2 + s2) * 64 + l) * 16);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int q = 0; q < 2; ++q) S[t][q] = mfma_bf16(fk[t], vb[s2][q], S[t][q]);
    }
#pragma unroll
    for (int x = 0; x < AQK_FRAGS; ++x) {
      const bf16x8 fa = frag(lds + OFF_AQK + (x * 64 + l) * 16);
#pragma unroll
      for (int q = 0; q < 2; ++q) ot[lt_mt(x)][q] = mfma_bf16(vb[lt_s(x)][q], fa, ot[lt_mt(x)][q]);
    }

    // o rows of this chunk: lane (nn, grp) holds 8 consecutive value columns
    // VCOL(nt0, 4 grp) .. + 7 of token 16 mt + nn; the resource ends after
    // the chunk's last valid row, so rows past n are dropped and every store
    // instruction issues (the copy above is waited for by count)
    {
      const int row_bytes = a.H * DV * 2;
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<bf16_t *>(a.o) + (t0 * a.H + h) * DV, 0, n * row_bytes, BUF_DWORD3);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 v = {(bf16_t)ot[mt][0][0], (bf16_t)ot[mt][0][1], (bf16_t)ot[mt][0][2],
                          (bf16_t)ot[mt][0][3], (bf16_t)ot[mt][1][0], (bf16_t)ot[mt][1][1],
                          (bf16_t)ot[mt][1][2], (bf16_t)ot[mt][1][3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro,
                                               (16 * mt + nn) * row_bytes + 2 * VCOL(nt0, 4 * grp),
                                               0, CPOL_NT);
      }
    }
    static_assert(O_STORES == 4, "four o stores per wave and chunk");

    // region B is consumed; region A of the next chunk has landed (the o
    // stores issued after it may still be in flight)
    if (more)
      __builtin_amdgcn_s_waitcnt(vm_wait(O_STORES));
    else
      __builtin_amdgcn_s_waitcnt(vm_wait(0));
    __syncthreads();
    if (more) copy_region_b(chain_blocks + (c + 1) * BLOCK_BYTES, lbase, w, l);
  }

  if (a.hT) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * t + 4 * grp + r;
          const int col = VCOL(nt0 + q, nn);
          a.hT[st_base + row * DV + col] = S[t][q][r];
        }
  }
}

}  // namespace kda
