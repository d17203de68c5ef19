// Chunk recurrence fused with the output (KDA TPU report, section 6.2; MI355X
// serving post, section 1.1: the state stays on chip across chunks and the
// output is formed in the same pass, with no per-chunk state checkpoint).
//
// Per (sequence, head) chain and chunk, with h the entry state [128, 128]:
//     v_new = U - W h
//     o     = qg h + Aqk v_new              (reads the entry state h)
//     h     = Diag(gamma) h + kg^T v_new
// The 128 value columns of the state are independent, so each of the 4 waves
// of a chain's workgroup keeps a [128, 32] fp32 slice of the state in 16 MFMA
// C tiles for the whole sequence; the state and v_new are fed back to the
// MFMAs as B operands straight from their C tiles (bf16), in the permuted k
// order the intra-chunk kernel wrote its A fragments in.
#include "kda_internal.h"
#include "kda_launch.h"

namespace kda {

namespace {

__device__ constexpr int LT_MT[6] = {0, 1, 2, 2, 3, 3};
__device__ constexpr int LT_S[6] = {0, 0, 0, 1, 0, 1};

// The chunk table is read-only while this kernel runs: reading it through
// the constant address space gives scalar loads.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4 chunk_record(const int4 *info, int64_t c) {
  const i32x4 v = ((const __attribute__((address_space(4))) i32x4 *)(uintptr_t)info)[c];
  return make_int4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x8 load_frag(const uint8_t *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// o rows of token tile mt of one chunk: the transposed output tiles of value
// tiles 2w and 2w+1 give lane (nn, grp) token 16 mt + nn and the value
// columns VCOL(2w + q2, 4 grp + r) = 32 w + 8 grp + 4 q2 + r, i.e. 8
// consecutive columns: one 16-byte store.
__device__ __forceinline__ void store_o_tile(const RecurArgs &a, int h, int w, int nn, int grp,
                                             int64_t t0, int n, int mt, const bf16x8 &ov) {
  const int row = 16 * mt + nn;
  if (row < n)
    *reinterpret_cast<bf16x8 *>(a.o + ((t0 + row) * a.H + h) * DV + 32 * w + 8 * grp) = ov;
}

}  // namespace

// One workgroup of 4 waves per (sequence, head) chain; wave w owns value
// tiles 2w and 2w+1 (32 columns) of the state.  The chain's intermediate
// blocks stream through two LDS buffers: while the waves compute chunk c from
// one buffer, chunk c+1's block is copied global -> LDS into the other by
// global_load_lds_dwordx4 (no register staging), so the four waves share one
// copy of the fragments and the copy latency hides behind the MFMAs.
constexpr int REC_THREADS = 256;
constexpr int DMA_ROUND = REC_THREADS * 16;               // bytes per copy round
constexpr int DMA_FULL = BLOCK_BYTES / DMA_ROUND;          // 19 full rounds
constexpr int DMA_TAIL = BLOCK_BYTES - DMA_FULL * DMA_ROUND;  // 512 bytes
static_assert(DMA_TAIL % 16 == 0 && DMA_TAIL <= 64 * 16, "tail fits one wave");

// One global_load_lds_dwordx4: 16 bytes per lane from src into LDS at
// lds_wave_base + 16 * lane.  Written as inline assembly so that the
// compiler does not treat it as an LDS store it must wait for before every
// later LDS read (it cannot tell the two block buffers apart); the kernel
// waits for these copies itself, at the top of each chunk.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void dma16(const uint8_t *src, uint8_t *lds_wave_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t *src, uint8_t *lds_wave_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(base)
               : "memory", "m0");
}

// Copy one intermediate block into an LDS buffer: lane l of wave w copies
// the 16 bytes at round * 4096 + w * 1024 + l * 16.  The copy is issued in
// four parts spread over a chunk's MFMA work, so that the wave never stalls
// on a burst of memory instructions.
constexpr int DMA_PART = (DMA_FULL + 3) / 4;
__device__ __forceinline__ void copy_block_part(const uint8_t *src, uint8_t *dst, int w, int l,
                                                int part) {
#pragma unroll
  for (int r = part * DMA_PART; r < (part + 1) * DMA_PART && r < DMA_FULL; ++r)
    dma16(src + r * DMA_ROUND + w * 1024 + l * 16, dst + r * DMA_ROUND + w * 1024);
  if (part == 3 && w == 0 && l < DMA_TAIL / 16)
    dma16(src + DMA_FULL * DMA_ROUND + l * 16, dst + DMA_FULL * DMA_ROUND);
}
// Touch the block two chunks ahead, one dword per 128-byte line, so that its
// copy a chunk later hits L2 instead of HBM.  The loaded dwords land in a
// junk LDS word per lane (global_load_lds: no registers, so nothing waits on
// them until the explicit wait at the next chunk, which leaves exactly these
// TOUCH_LOADS instructions in flight).
constexpr int LINE_BYTES = 128;
constexpr int TOUCH_LINES = (BLOCK_BYTES + LINE_BYTES - 1) / LINE_BYTES;  // 612
constexpr int TOUCH_LOADS = (TOUCH_LINES + REC_THREADS - 1) / REC_THREADS;  // 3
__device__ __forceinline__ void touch_block(const uint8_t *src, uint8_t *junk_wave, int tid) {
#pragma unroll
  for (int k = 0; k < TOUCH_LOADS; ++k) {
    int line = tid + REC_THREADS * k;
    line = line < TOUCH_LINES ? line : 0;
    dma4(src + line * LINE_BYTES, junk_wave);
  }
}
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8]):
// all LDS/scalar work done and all vector memory done except the last
// TOUCH_LOADS (or none) issued
constexpr int WAIT_ALL_BUT_TOUCH = TOUCH_LOADS | (7 << 4);
constexpr int WAIT_ALL = 0 | (7 << 4);
static_assert(TOUCH_LOADS < 16, "fits the low vmcnt field");

__device__ __forceinline__ void copy_block(const uint8_t *src, uint8_t *dst, int w, int l) {
#pragma unroll
  for (int part = 0; part < 4; ++part) copy_block_part(src, dst, w, l, part);
}

__global__ __launch_bounds__(REC_THREADS) void recurrence_kernel(RecurArgs a) {
  __shared__ __align__(16) uint8_t lds[2][BLOCK_BYTES];
  __shared__ __align__(16) uint8_t junk[REC_THREADS / 64][64 * 4];
  const int64_t chain = blockIdx.x;
  if (chain >= (int64_t)a.N * a.H) return;
  const int s = (int)(chain / a.H), h = (int)(chain % a.H);
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, nn = l & 15, grp = l >> 4;
  // chunk range and token ranges are clamped so that a workspace that does
  // not hold a valid chunk table can never send this kernel out of bounds
  const int64_t nc_max = a.nc_max;
  int64_t c_beg = a.chunk_first[s], c_end = a.chunk_first[s + 1];
  c_beg = c_beg < 0 ? 0 : (c_beg > nc_max ? nc_max : c_beg);
  c_end = c_end < c_beg ? c_beg : (c_end > nc_max ? nc_max : c_end);
  const int64_t st_base = ((int64_t)s * a.H + h) * DK * DV;
  const uint8_t *chain_blocks = a.blocks + (int64_t)h * nc_max * BLOCK_BYTES;

  // state slice: key tiles t = 0..7, value tiles 2w + q2
  f32x4 S[8][2];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * t + 4 * grp + r;
        const int col = VCOL(2 * w + q2, nn);
        S[t][q2][r] = a.h0 ? a.h0[st_base + row * DV + col] : 0.f;
      }

  if (c_beg < c_end) copy_block(chain_blocks + c_beg * BLOCK_BYTES, lds[0], w, l);

  // o of chunk c is stored at the start of chunk c+1, right after the next
  // copy is issued, so that the store latency overlaps a whole chunk of work
  // instead of the wait for that copy
  bf16x8 o_pend[4];
  int64_t o_t0 = 0;
  int o_n = 0;

  bool touched = false;  // loads of touch_block still in flight
  for (int64_t c = c_beg; c < c_end; ++c) {
    const int cur = (int)((c - c_beg) & 1);
    // this thread's copies (and earlier stores) are done; after the barrier
    // every thread's are, and nobody still reads the other buffer
    if (touched)
      __builtin_amdgcn_s_waitcnt(WAIT_ALL_BUT_TOUCH);
    else
      __builtin_amdgcn_s_waitcnt(WAIT_ALL);
    __syncthreads();
    const bool more = c + 1 < c_end;
    const uint8_t *next_src = chain_blocks + (c + 1) * BLOCK_BYTES;
    uint8_t *next_dst = lds[cur ^ 1];
    const uint8_t *blk = lds[cur];
    const int4 info = chunk_record(a.chunk_info, c);
    const int64_t t0 = info.x < 0 ? 0 : (info.x > a.T ? a.T : info.x);
    const int n = (int)(info.y < 0 ? 0 : (info.y > a.T - t0 ? a.T - t0 : info.y));

    // fragments of -W and qg for key slab 0 (the rest are prefetched one
    // slab ahead inside the loop below)
    bf16x8 fw[4], fq[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      fw[mt] = load_frag(blk + OFF_WN + ((mt * 4 + 0) * 64 + l) * 16);
      fq[mt] = load_frag(blk + OFF_QG + ((mt * 4 + 0) * 64 + l) * 16);
    }

    // entry state as bf16 MFMA operands (k slabs of 32 key rows)
    bf16x8 hb[4][2];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int e = 0; e < 8; ++e) hb[s4][q2][e] = (bf16_t)S[2 * s4 + (e >> 2)][q2][e & 3];

    // v_new starts from U (C layout: [token][value]); o^T from zero
    f32x4 vn[4][2], ot[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const bf16x4 u = *reinterpret_cast<const bf16x4 *>(
            blk + OFF_U + (((2 * w + q2) * 4 + mt) * 64 + l) * 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) vn[mt][q2][r] = (float)u[r];
        ot[mt][q2] = zero4();
      }

    // the state is no longer needed unscaled: apply Diag(gamma) now, while
    // the MFMAs below run
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 gm = *reinterpret_cast<const float4 *>(blk + OFF_GAM + (16 * t + 4 * grp) * 4);
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        S[t][q2][0] *= gm.x;
        S[t][q2][1] *= gm.y;
        S[t][q2][2] *= gm.z;
        S[t][q2][3] *= gm.w;
      }
    }

    // v_new += (-W) h   and   o^T += h^T qg^T   (o is formed transposed so
    // that each lane ends up with 4 consecutive value columns of one token)
    bf16x8 fk[2][8];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      // one quarter of the next chunk's copy (and, first, last chunk's o)
      if (c > c_beg) store_o_tile(a, h, w, nn, grp, o_t0, o_n, s4, o_pend[s4]);
      if (more) copy_block_part(next_src, next_dst, w, l, s4);
      if (s4 == 3) {
        touched = c + 2 < c_end;
        if (touched) touch_block(chain_blocks + (c + 2) * BLOCK_BYTES, junk[w], tid);
      }
      bf16x8 nw[4], nq[4];
      if (s4 < 3) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          nw[mt] = load_frag(blk + OFF_WN + ((mt * 4 + s4 + 1) * 64 + l) * 16);
          nq[mt] = load_frag(blk + OFF_QG + ((mt * 4 + s4 + 1) * 64 + l) * 16);
        }
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int t = 0; t < 8; ++t)
            fk[s2][t] = load_frag(blk + OFF_KGT + ((t * 2 + s2) * 64 + l) * 16);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          vn[mt][q2] = mfma_bf16(fw[mt], hb[s4][q2], vn[mt][q2]);
          ot[mt][q2] = mfma_bf16(hb[s4][q2], fq[mt], ot[mt][q2]);
        }
      if (s4 < 3) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          fw[mt] = nw[mt];
          fq[mt] = nq[mt];
        }
      }
    }

    // v_new as bf16 operands (k slabs of 32 tokens)
    bf16x8 vb[2][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int e = 0; e < 8; ++e) vb[s2][q2][e] = (bf16_t)vn[2 * s2 + (e >> 2)][q2][e & 3];

    // h <- Diag(gamma) h + kg^T v_new   (the serial dependency: first)
    bf16x8 fah[AQK_FRAGS], fal[AQK_FRAGS];
#pragma unroll
    for (int x = 0; x < AQK_FRAGS; ++x) {
      fah[x] = load_frag(blk + OFF_AQK + (x * 64 + l) * 16);
      fal[x] = load_frag(blk + OFF_AQK + ((AQK_FRAGS + x) * 64 + l) * 16);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) S[t][q2] = mfma_bf16(fk[s2][t], vb[s2][q2], S[t][q2]);

    // o^T += v_new^T Aqk^T   (Aqk in hi + lo bf16)
#pragma unroll
    for (int x = 0; x < AQK_FRAGS; ++x)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        ot[LT_MT[x]][q2] = mfma_bf16(vb[LT_S[x]][q2], fah[x], ot[LT_MT[x]][q2]);
        ot[LT_MT[x]][q2] = mfma_bf16(vb[LT_S[x]][q2], fal[x], ot[LT_MT[x]][q2]);
      }

    // o^T of this chunk as bf16 (nearest even), stored at the next chunk
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int r = 0; r < 4; ++r) o_pend[mt][4 * q2 + r] = (bf16_t)ot[mt][q2][r];
    o_t0 = t0;
    o_n = n;
  }
  if (c_end > c_beg) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) store_o_tile(a, h, w, nn, grp, o_t0, o_n, mt, o_pend[mt]);
  }
  // no load may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(WAIT_ALL);

  if (a.hT) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * t + 4 * grp + r;
          const int col = VCOL(2 * w + q2, nn);
          a.hT[st_base + row * DV + col] = S[t][q2][r];
        }
  }
}

hipError_t launch_recurrence(const RecurArgs &a, hipStream_t stream) {
  const int64_t chains = (int64_t)a.N * a.H;
  hipLaunchKernelGGL(recurrence_kernel, dim3((unsigned)chains), dim3(REC_THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
