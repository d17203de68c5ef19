// Internal definitions shared by the KDA HIP kernels (gfx950 / CDNA4 only).
//
// Geometry: K = V = 128 head dims, BT = 64-token chunks, SB = 16-token
// subblocks (KDA TPU report, sections 1 and 4).  Every matrix product runs on
// v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulate) except the
// 16x16 triangular inverses, which use v_mfma_f32_16x16x16_bf16 on hi + lo
// operand splits.
//
// MFMA lane layout used throughout (wave64, lane l, n = l & 15, grp = l >> 4):
//   A fragment  (16 x 32, bf16x8):  A[row = n][k = 8*grp + e],   e = 0..7
//   B fragment  (32 x 16, bf16x8):  B[k = 8*grp + e][col = n]
//   C/D tile    (16 x 16, f32x4):   C[row = 4*grp + r][col = n], r = 0..3
// A contraction only needs A and B to agree on which physical k index each
// (grp, e) slot holds.  When a B operand is made from two C tiles that are
// stacked along k (rows 32s..32s+15 and 32s+16..32s+31), slot (grp, e) holds
// physical row  P(s, grp, e) = 32 s + 16 (e >> 2) + 4 grp + (e & 3).
// The recurrence keeps its state and v_new in C tiles and feeds them straight
// back as B operands in that permuted order, so the intra-chunk kernel writes
// every A operand of the recurrence (W, q*Gamma, kg^T, Aqk) pre-permuted.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int DK = 128;
constexpr int DV = 128;
constexpr int BT = 64;
constexpr int SB = 16;
constexpr int SB_REF = 7;  // subblock reference row (its midpoint)

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer resource on gfx950 (32-bit data format, no
// swizzle).  With stride 0 the hardware range check compares each lane's
// byte offset with the record count, and out-of-range lanes read zero and
// write nothing.
constexpr int BUF_DWORD3 = 0x00020000;
// Cache-policy operand of buffer loads and stores: non-temporal.
constexpr int CPOL_NT = 2;

// ---------------------------------------------------------------------------
// Per-(head, chunk) intermediate block written by the intra-chunk kernel and
// read by the recurrence kernel.  Each "fragment" is 64 lanes x 16 bytes, in
// the exact register order the consumer's MFMA expects, so the consumer does
// one coalesced 16-byte load per lane per fragment.
//   WN   : -W as A operand of v_new = U - W h.  [token tile mt 0..3]
//          [key slab s 0..3] fragments; lane (n, grp) slot e holds
//          -W[16 mt + n][P(s, grp, e)].
//   QG   : scale * q * Gamma, same shape and order as WN.
//   KGT  : kg^T as A operand of S += kg^T v_new.  [key tile 0..7][token slab
//          s 0..1]; lane slot e holds kg[P(s, grp, e)][16 mt + n].
//   AQK  : Aqk as A operand of o += Aqk v_new (bf16).  Only the six
//          (mt, s) fragments with any j <= i are stored, indexed by AQK_IDX.
//   U    : U as the C-tile initialiser of v_new: [value tile nt 0..7][token
//          tile pair 0..1] entries of 64 lanes x 16 bytes; bytes 8 m .. 8 m + 7
//          of lane (n, grp) hold the C tile of token tile mt = 2 pair + m,
//          element r = U[16 mt + 4 grp + r][VCOL(nt, n)] (bf16).  VCOL permutes
//          the value columns inside each 32-column slice so that the
//          recurrence's transposed output tiles give every lane 8
//          consecutive columns of a token (one 16-byte store).
//   GAM  : gamma = exp(G_last) per key channel, fp32 [128].
// ---------------------------------------------------------------------------
constexpr int FRAG_BYTES = 64 * 16;
constexpr int OFF_WN = 0;
constexpr int OFF_QG = OFF_WN + 16 * FRAG_BYTES;
constexpr int OFF_KGT = OFF_QG + 16 * FRAG_BYTES;
constexpr int OFF_AQK = OFF_KGT + 16 * FRAG_BYTES;
constexpr int AQK_FRAGS = 6;
constexpr int OFF_U = OFF_AQK + AQK_FRAGS * FRAG_BYTES;
constexpr int UTILE_BYTES = 64 * 8;  // one value tile x token tile C tile (bf16)
// byte offset of U's C tile (value tile nt, token tile mt) for lane l
__host__ __device__ constexpr int U_OFFSET(int nt, int mt, int l) {
  return OFF_U + ((nt * 2 + (mt >> 1)) * 64 + l) * 16 + (mt & 1) * 8;
}
constexpr int OFF_GAM = OFF_U + 32 * UTILE_BYTES;
constexpr int BLOCK_BYTES = OFF_GAM + DK * 4;
static_assert(BLOCK_BYTES % 256 == 0, "intermediate blocks stay 256-byte aligned");

// Value column held by lane n of value tile nt in the recurrence's state,
// v_new and U tiles: column x = n of the tile maps to
// 32 (nt / 2) + 8 (x / 4) + 4 (nt % 2) + x % 4.
__host__ __device__ constexpr int VCOL(int nt, int n) {
  return 32 * (nt >> 1) + 8 * (n >> 2) + 4 * (nt & 1) + (n & 3);
}

// Aqk fragment (token tile mt, token slab s) -> storage index; valid for
// s <= mt / 2, i.e. (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
__host__ __device__ constexpr int AQK_IDX(int mt, int s) {
  return (mt == 0 ? 0 : mt == 1 ? 1 : mt == 2 ? 2 : 4) + s;
}

// Workspace header: flags word, chunk_first[N+1], chunk_info[NCmax][4].
struct WsLayout {
  int64_t off_flags, off_chunk_first, off_chunk_info, off_blocks;
  int64_t nc_max, total;
};

__host__ __device__ inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

__host__ __device__ inline int64_t nc_max_of(int64_t T, int64_t N) {
  return (T + (int64_t)(BT - 1) * N) / BT;
}

__host__ __device__ inline WsLayout ws_layout(int64_t T, int64_t N, int64_t H) {
  WsLayout L;
  L.nc_max = nc_max_of(T, N);
  L.off_flags = 0;
  L.off_chunk_first = 256;
  L.off_chunk_info = align256(L.off_chunk_first + 4 * (N + 1));
  L.off_blocks = align256(L.off_chunk_info + 16 * (L.nc_max > 0 ? L.nc_max : 1));
  L.total = L.off_blocks + H * L.nc_max * (int64_t)BLOCK_BYTES;
  return L;
}

// ---------------------------------------------------------------------------
// Device helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


// exp(x) for natural-log x: one multiply and the hardware base-2 exponential.
__device__ __forceinline__ float exp_nat(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float x) { return (bf16_t)x; }

__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return (float)x; }

// hi = bf16(x), lo = bf16(x - hi): hi + lo carries ~16 mantissa bits.
// Writes element e of the two bf16 vectors.
template <typename V>
__device__ __forceinline__ void split_bf16(float x, V &hi, V &lo, int e) {
  const bf16_t h = (bf16_t)x;
  hi[e] = h;
  lo[e] = (bf16_t)(x - (float)h);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace kda
