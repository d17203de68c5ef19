// Chunk recurrence fused with the output (KDA TPU report, section 6.2; MI355X
// serving post, section 1.1: the state stays on chip across chunks and the
// output is formed in the same pass, with no per-chunk state checkpoint).
//
// Per (sequence, head) chain and chunk, with h the entry state [128, 128]:
//     v_new = U - W h
//     o     = qg h + Aqk v_new              (reads the entry state h)
//     h     = Diag(gamma) h + kg^T v_new
// The 128 value columns of the state are independent, so each chain is
// split over 4 single-wave workgroups of 32 columns each.  A wave keeps its
// [128, 32] fp32 slice of the state in 16 MFMA C tiles for the whole
// sequence; the state and v_new are fed back to the MFMAs as B operands
// straight from their C tiles (bf16), in the permuted k order the
// intra-chunk kernel wrote its A fragments in.
#include "kda_internal.h"
#include "kda_launch.h"

namespace kda {

namespace {

__device__ constexpr int LT_MT[6] = {0, 1, 2, 2, 3, 3};
__device__ constexpr int LT_S[6] = {0, 0, 0, 1, 0, 1};

__device__ __forceinline__ bf16x8 load_frag(const uint8_t *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

}  // namespace

// blockIdx -> (chain, quarter): the 4 quarters of a chain get block ids that
// are equal mod 8, so the dispatcher puts them on the same XCD and they
// share its L2 for the chain's intermediate blocks.
__global__ __launch_bounds__(64) void recurrence_kernel(RecurArgs a) {
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int quarter = slot & 3;
  const int64_t chain = (int64_t)(slot >> 2) * 8 + xcd;
  if (chain >= (int64_t)a.N * a.H) return;
  const int s = (int)(chain / a.H), h = (int)(chain % a.H);
  const int l = threadIdx.x, nn = l & 15, grp = l >> 4;
  // chunk range and token ranges are clamped so that a workspace that does
  // not hold a valid chunk table can never send this kernel out of bounds
  const int64_t nc_max = a.nc_max;
  int64_t c_beg = a.chunk_first[s], c_end = a.chunk_first[s + 1];
  c_beg = c_beg < 0 ? 0 : (c_beg > nc_max ? nc_max : c_beg);
  c_end = c_end < c_beg ? c_beg : (c_end > nc_max ? nc_max : c_end);
  const int64_t st_base = ((int64_t)s * a.H + h) * DK * DV;

  // state slice: key tiles t = 0..7, value tiles 2*quarter + q2
  f32x4 S[8][2];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * t + 4 * grp + r;
        const int col = 16 * (2 * quarter + q2) + nn;
        S[t][q2][r] = a.h0 ? a.h0[st_base + row * DV + col] : 0.f;
      }

  for (int64_t c = c_beg; c < c_end; ++c) {
    const int4 info = a.chunk_info[c];
    const int64_t t0 = info.x < 0 ? 0 : (info.x > a.T ? a.T : info.x);
    const int n = (int)(info.y < 0 ? 0 : (info.y > a.T - t0 ? a.T - t0 : info.y));
    const uint8_t *blk = a.blocks + ((int64_t)h * a.nc_max + c) * BLOCK_BYTES;

    // entry state as bf16 B operands (k slabs of 32 key rows)
    bf16x8 hb[4][2];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int e = 0; e < 8; ++e) hb[s4][q2][e] = (bf16_t)S[2 * s4 + (e >> 2)][q2][e & 3];

    // v_new starts from U; o from zero
    f32x4 vn[4][2], oc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const bf16x4 u = *reinterpret_cast<const bf16x4 *>(
            blk + OFF_U + (((2 * quarter + q2) * 4 + mt) * 64 + l) * 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) vn[mt][q2][r] = (float)u[r];
        oc[mt][q2] = zero4();
      }

    // v_new += (-W) h ;  o += qg h
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const bf16x8 wn = load_frag(blk + OFF_WN + ((mt * 4 + s4) * 64 + l) * 16);
        const bf16x8 qg = load_frag(blk + OFF_QG + ((mt * 4 + s4) * 64 + l) * 16);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          vn[mt][q2] = mfma_bf16(wn, hb[s4][q2], vn[mt][q2]);
          oc[mt][q2] = mfma_bf16(qg, hb[s4][q2], oc[mt][q2]);
        }
      }

    // v_new as bf16 B operands (k slabs of 32 tokens)
    bf16x8 vb[2][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int e = 0; e < 8; ++e) vb[s2][q2][e] = (bf16_t)vn[2 * s2 + (e >> 2)][q2][e & 3];

    // o += Aqk v_new  (Aqk in hi + lo bf16)
#pragma unroll
    for (int x = 0; x < AQK_FRAGS; ++x) {
      const bf16x8 ah = load_frag(blk + OFF_AQK + (x * 64 + l) * 16);
      const bf16x8 al = load_frag(blk + OFF_AQK + ((AQK_FRAGS + x) * 64 + l) * 16);
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        oc[LT_MT[x]][q2] = mfma_bf16(ah, vb[LT_S[x]][q2], oc[LT_MT[x]][q2]);
        oc[LT_MT[x]][q2] = mfma_bf16(al, vb[LT_S[x]][q2], oc[LT_MT[x]][q2]);
      }
    }

    // h <- Diag(gamma) h + kg^T v_new
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
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 kg = load_frag(blk + OFF_KGT + ((t * 2 + s2) * 64 + l) * 16);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) S[t][q2] = mfma_bf16(kg, vb[s2][q2], S[t][q2]);
      }

    // o rows of this chunk (bf16, round to nearest even)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * grp + r;
          if (row < n) {
            const bf16_t ov = (bf16_t)oc[mt][q2][r];
            a.o[((t0 + row) * a.H + h) * DV + 16 * (2 * quarter + q2) + nn] =
                __builtin_bit_cast(uint16_t, ov);
          }
        }
  }

  if (a.hT) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * t + 4 * grp + r;
          const int col = 16 * (2 * quarter + q2) + nn;
          a.hT[st_base + row * DV + col] = S[t][q2][r];
        }
  }
}

hipError_t launch_recurrence(const RecurArgs &a, hipStream_t stream) {
  const int64_t chains = (int64_t)a.N * a.H;
  const int64_t blocks = (chains + 7) / 8 * 32;
  hipLaunchKernelGGL(recurrence_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
