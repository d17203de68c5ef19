// Chunk recurrence fused with the output (KDA TPU report, section 6.2; MI355X
// serving post, section 1.1: the state stays on chip across chunks and the
// output is formed in the same pass, with no per-chunk state checkpoint).
//
// Per (sequence, head) chain and chunk, with h the entry state [128, 128]:
//     v_new = U - W h
//     o     = qg h + Aqk v_new              (reads the entry state h)
//     h     = Diag(gamma) h + kg^T v_new
// The 128 value columns of the state are independent.  A chain is split
// over PARTS workgroups, each owning TILES value tiles of 16 columns (wave w
// owns TPW of them) and keeping its [128, 16 TPW] fp32 slice of the state in
// MFMA C tiles for the whole sequence; the state and v_new are fed back to
// the MFMAs as B operands straight from their C tiles (bf16), in the
// permuted k order the intra-chunk kernel wrote its A fragments in.  Fewer
// columns per wave shorten the serial per-chunk work of every wave, which
// is what bounds a chain; the split is picked at launch so that the
// workgroups still fit the device once each.
#include "kda_internal.h"
#include "kda_recurrence.h"

namespace kda {

namespace {

// The six (token tile, token slab) fragments of a 64 x 64 lower-triangular
// operand: index x -> (mt, s) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
constexpr int lt_mt(int x) { return x < 2 ? x : (x < 4 ? 2 : 3); }
constexpr int lt_s(int x) { return (x == 3 || x == 5) ? 1 : 0; }

// The chunk table is read-only while this kernel runs: reading it through
// the constant address space gives scalar loads.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4 chunk_record(const int4 *info, int64_t c) {
  const i32x4 v = ((const __attribute__((address_space(4))) i32x4 *)(uintptr_t)info)[c];
  return make_int4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ int32_t chunk_first_of(const int32_t *chunk_first, int64_t s) {
  return ((const __attribute__((address_space(4))) int32_t *)(uintptr_t)chunk_first)[s];
}

__device__ __forceinline__ bf16x8 load_frag(const uint8_t *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// One buffer_load_dwordx4 ... lds: 16 bytes per lane from byte off + 16 lane
// of a block (buffer resource r, voff = 16 lane) into LDS at lds_base + off +
// 16 lane.  The block offset travels in a scalar register and the LDS
// address in M0, so a round costs three instructions.  Written as inline
// assembly so that the compiler does not treat it as an LDS store it must
// wait for before every later LDS read (it cannot tell the two block buffers
// apart); the kernel waits for these copies itself, once per chunk.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void dma_round(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t off,
                                          uint32_t lds_base) {
  // both scalars are wave-uniform; readfirstlane keeps them in SGPRs where
  // the compiler cannot prove it
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base + off);
  const uint32_t soff = __builtin_amdgcn_readfirstlane(off);
  // M0 belongs to the compiler: its value is saved in a scratch SGPR and put
  // back after the load has issued (the LDS address is taken from M0 at
  // issue), so the asm hands every register back as it found it
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %4 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(m0v), "s"(soff)
      : "memory");
}
// Buffer resource over one intermediate block, and the wave-uniform LDS
// address of a block buffer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t *blk) {
  // the block address is wave-uniform: keep it in scalar registers even where
  // the compiler computed it with vector instructions
  const uint64_t a = (uint64_t)(uintptr_t)blk;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  uint8_t *u = reinterpret_cast<uint8_t *>((uintptr_t)(((uint64_t)hi << 32) | lo));
  return __builtin_amdgcn_make_buffer_rsrc(u, 0, BLOCK_BYTES, BUF_DWORD3);
}
__device__ __forceinline__ uint32_t lds_base_of(const uint8_t *buf) {
  return __builtin_amdgcn_readfirstlane(lds_addr(buf));
}

// s_waitcnt immediate that waits for LDS (and scalar) accesses only:
// vmcnt and expcnt at their maxima, lgkmcnt 0
constexpr int LGKM_ONLY = 0xF | (0x7 << 4) | (0x3 << 14);

constexpr int ROUND = 1024;                  // one wave's copy: 64 lanes x 16 bytes
constexpr int SHARED_ROUNDS = OFF_U / ROUND;  // -W, qg, kg^T, Aqk: every part needs them
static_assert(OFF_U % ROUND == 0, "shared fragments are whole rounds");
static_assert(OFF_GAM + DK * 4 == BLOCK_BYTES, "gamma ends the block");

// NC compute waves (TPW value tiles each) and NCP copy waves per workgroup.
template <int NC, int NCP, int TPW>
struct RecCfg {
  static constexpr int THREADS = 64 * (NC + NCP);
  static constexpr int NCW = NC;              // compute waves
  static constexpr int TILES = NC * TPW;      // value tiles per workgroup
  static constexpr int PARTS = 8 / TILES;     // workgroups per chain
  static constexpr int U_ROUNDS = TILES * 4 * UTILE_BYTES / ROUND;
  // shared fragments, this part's U tiles, and gamma (half a round)
  static constexpr int ROUNDS = SHARED_ROUNDS + U_ROUNDS + 1;
  static_assert(TILES * PARTS == 8, "parts cover the 128 value columns");
  // o of a chunk (64 tokens x 16 TILES columns, bf16) is staged in LDS for
  // the copy waves to store, in another part's U tiles of the block buffer
  // (never copied by this workgroup)
  static constexpr int O_ROW = 32 * TILES;  // bytes per token row
  static constexpr int O_BYTES = BT * O_ROW;
  // The staged row is stored in pieces of consecutive output columns: the
  // part's 16 TILES columns are one contiguous range for an even number of
  // tiles (VCOL interleaves the two tiles of a 32-column slice), but a
  // single tile holds four runs of 4 columns, 8 columns apart.
  static constexpr int PIECE = TILES == 1 ? 8 : 16;  // bytes
  static_assert(NCP == 0 || 2 * O_BYTES <= 32 * UTILE_BYTES, "o fits in the U tiles of the other parts");
};

// Copy round k of part p's share of a block (same offsets in LDS as in the
// block): shared rounds, then the part's U tiles, then gamma (lanes < 32).
template <class C>
__device__ __forceinline__ void copy_round(__amdgpu_buffer_rsrc_t r, uint32_t lbase, int k, int p,
                                           int l) {
  int off;
  if (k < SHARED_ROUNDS)
    off = k * ROUND;
  else if (k < SHARED_ROUNDS + C::U_ROUNDS)
    off = OFF_U + (p * C::U_ROUNDS + (k - SHARED_ROUNDS)) * ROUND;
  else
    off = OFF_GAM;
  if (k < C::ROUNDS - 1 || l < DK * 4 / 16) dma_round(r, 16 * l, off, lbase);
}

// Without copy waves: compute wave w copies rounds w, w + NC, ..., a
// quarter of them at each key slab of the chunk before.
template <class C>
__device__ __forceinline__ void copy_step(const uint8_t *src, uint8_t *dst, int w, int p, int l,
                                          int step) {
  constexpr int per_wave = (C::ROUNDS + C::NCW - 1) / C::NCW;
  constexpr int per_step = (per_wave + 3) / 4;
  const __amdgpu_buffer_rsrc_t r = block_rsrc(src);
  const uint32_t lbase = lds_base_of(dst);
#pragma unroll
  for (int j = step * per_step; j < (step + 1) * per_step && j < per_wave; ++j) {
    const int k = w + C::NCW * j;
    if (k < C::ROUNDS) copy_round<C>(r, lbase, k, p, l);
  }
}

typedef unsigned u32x2v __attribute__((ext_vector_type(2)));

// Where the o of a chunk is staged: the U tiles of part p + 1.
template <class C>
__device__ __forceinline__ int o_stage_off(int p) {
  return OFF_U + ((p + 1) % C::PARTS) * C::TILES * 2 * ROUND;
}

// Byte offset, within a staged o row, of the 4 columns VCOL(nt, 4 grp) ..
// + 3 (value tile nt of part p), and the output column of staged piece k.
// The staged pieces of a row are XOR-permuted by the row: the 16 rows one
// lane group writes (one piece each) are O_ROW bytes apart, so without it
// every 256 / O_ROW-th row would hit the same LDS banks.
template <class C>
__device__ __forceinline__ int o_stage_swz(int row) {
  constexpr int PER_ROW = C::O_ROW / C::PIECE;
  return (row / (256 / C::O_ROW)) % PER_ROW;
}
template <class C>
__device__ __forceinline__ int o_stage_col(int nt, int grp, int p, int row) {
  const int off = C::TILES == 1 ? 8 * grp : 2 * (VCOL(nt, 4 * grp) - 16 * C::TILES * p);
  const int piece = off / C::PIECE;
  return ((piece ^ o_stage_swz<C>(row)) * C::PIECE) | (off % C::PIECE);
}
template <class C>
__device__ __forceinline__ int o_piece_col(int k, int p) {
  return C::TILES == 1 ? VCOL(p, 4 * k) : 16 * C::TILES * p + 8 * k;
}

// Copy wave cw stores o of chunk c (staged in LDS buffer `buf` by the
// compute waves) to its rows of o: 16 bytes per lane, through a buffer
// resource that ends after the chunk's last valid row, so that the lanes of
// rows past n are dropped by the range check and every store instruction is
// issued (the copy waves count their outstanding stores exactly).
template <class C, int NCP>
struct OStore {
  static constexpr int STORES = NCP > 0 ? C::O_BYTES / C::PIECE / (64 * NCP) : 1;  // per copy wave and chunk
  static_assert(STORES >= 1 && STORES < 16, "fits the low vmcnt field");
};
template <class C, int NCP>
__device__ __forceinline__ void store_o_staged(const RecurArgs &a, const uint8_t *buf, int64_t c,
                                               int h, int p, int cw, int l) {
  const int4 info = chunk_record(a.chunk_info, c);
  const int64_t t0 = info.x < 0 ? 0 : (info.x > a.T ? a.T : info.x);
  const int n = (int)(info.y < 0 ? 0 : (info.y > a.T - t0 ? a.T - t0 : (info.y > BT ? BT : info.y)));
  constexpr int PER_ROW = C::O_ROW / C::PIECE;  // pieces per token row
  const uint8_t *src = buf + o_stage_off<C>(p);
  const int row_bytes = a.H * DV * 2;  // < 2^25: H <= 65535
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<bf16_t *>(a.o) + (t0 * a.H + h) * DV, 0, n * row_bytes, BUF_DWORD3);
#pragma unroll
  for (int k = 0; k < OStore<C, NCP>::STORES; ++k) {
    const int i = (k * NCP + cw) * 64 + l;
    const int row = i / PER_ROW, piece = (i % PER_ROW) ^ o_stage_swz<C>(row);
    const int off = row * row_bytes + 2 * o_piece_col<C>(piece, p);
    if (C::PIECE == 16) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(src + i * 16);
      __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, off, 0, CPOL_NT);
    } else {
      const u32x2v v = *reinterpret_cast<const u32x2v *>(src + i * 8);
      __builtin_amdgcn_raw_buffer_store_b64(v, rsrc, off, 0, CPOL_NT);
    }
  }
}

// Rounds [K0, K1) of part p's share, with compile-time offsets.
template <class C, int K0, int K1>
__device__ __forceinline__ void copy_range(__amdgpu_buffer_rsrc_t r, uint32_t lbase, int p, int l) {
#pragma unroll
  for (int k = K0; k < K1; ++k) copy_round<C>(r, lbase, k, p, l);
}

// Copy wave cw's share of part p's block: the first or the second half of
// the rounds (two copy waves per workgroup).
template <class C, int NCP>
__device__ __forceinline__ void copy_share(const uint8_t *src, uint8_t *dst, int cw, int p, int l) {
  static_assert(NCP == 0 || NCP == 2, "the copy is split between two copy waves");
  constexpr int HALF = (C::ROUNDS + 1) / 2;
  const __amdgpu_buffer_rsrc_t r = block_rsrc(src);
  const uint32_t lbase = lds_base_of(dst);
  if (cw == 0)
    copy_range<C, 0, HALF>(r, lbase, p, l);
  else
    copy_range<C, HALF, C::ROUNDS>(r, lbase, p, l);
}

// Touch of a block two chunks ahead: one dword of every PARTS-th 128-byte
// line of the block (offset by the part), loaded by LDS DMA into a 256-byte
// sink that nobody reads.  The lines land in the XCD's L2, which the parts
// of a chain share, so that the block's copy one chunk later hits there
// instead of waiting on HBM.  Lanes past the block fail the buffer
// resource's range check.  Copy wave CW issues touches [K0, K1).
template <class C, int CW>
struct Touch {
  static constexpr int LINES = (BLOCK_BYTES / 128 + C::PARTS - 1) / C::PARTS;  // per part
  static constexpr int TOTAL = (LINES + 63) / 64;  // one line per lane
  static constexpr int K0 = CW == 0 ? 0 : (TOTAL + 1) / 2;
  static constexpr int K1 = CW == 0 ? (TOTAL + 1) / 2 : TOTAL;
  static constexpr int N = K1 - K0;  // touch instructions of this wave per block
};
template <class C, int CW>
__device__ __forceinline__ void touch_share(const uint8_t *src, uint32_t sink, int p, int l) {
  const __amdgpu_buffer_rsrc_t r = block_rsrc(src);
#pragma unroll
  for (int k = Touch<C, CW>::K0; k < Touch<C, CW>::K1; ++k) {
    const uint32_t voff = ((k * 64 + l) * C::PARTS + p) * 128;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(r), "s"(sink)
        : "memory");
  }
}
__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4);  // vmcnt n, expcnt any, lgkmcnt 0
}
// Copy wave CW before chunk c's barrier: chunk c's copy is complete.  Issued
// after it, in order, and free to stay outstanding: the touch of chunk c + 1
// (`touch`) and the o stores of chunk c - 2 (`stores`).
template <class C, int NCP, int CW>
__device__ __forceinline__ void wait_copy(bool touch, bool stores) {
  constexpr int N = Touch<C, CW>::N, S = OStore<C, NCP>::STORES;
  static_assert(N + S < 64, "fits the vmcnt field");
  if (touch && stores)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(N + S));
  else if (touch)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
  else if (stores)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(S));
  else
    __builtin_amdgcn_s_waitcnt(0);
}
template <class C, int NCP>
__device__ __forceinline__ void touch_block(const uint8_t *src, uint32_t sink, int cw, int p, int l) {
  if (cw == 0)
    touch_share<C, 0>(src, sink, p, l);
  else
    touch_share<C, 1>(src, sink, p, l);
}

// What one workgroup group computes: a whole chain (segments == 1), or one
// run of a segment of a chain (the two phases of chunk-parallel state
// passing, kda_recurrence.h).
enum { INIT_H0 = 0, INIT_IDENTITY = 1, INIT_ZERO = 2, INIT_XSTATE = 3 };
enum { EXIT_NONE = 0, EXIT_FINAL = 1, EXIT_XSTATE = 2, EXIT_MAP = 3 };
struct RunDesc {
  int64_t chain;  // -1: no run
  int seg, init, exit, map, prefix;
  bool use_u, write_o;
};
template <bool SEG>
__device__ __forceinline__ RunDesc describe_run(const RecurArgs &a, int64_t run) {
  const int64_t chains = (int64_t)a.N * a.H;
  const int P = SEG ? a.segments : 1;
  RunDesc d;
  d.chain = -1;
  d.seg = 0;
  d.init = INIT_H0;
  d.exit = EXIT_FINAL;
  d.map = 0;
  d.prefix = 0;
  d.use_u = true;
  d.write_o = true;
  if (P <= 1) {
    if (run < chains) d.chain = run;
    return d;
  }
  if (a.phase == 1) {
    // per chain: segment 0, then (M, b) of segments 1 .. P-2
    const int64_t per = 1 + 2 * (int64_t)(P - 2);
    if (run >= chains * per) return d;
    d.chain = run / per;
    const int r = (int)(run % per);
    if (r == 0) {
      d.exit = P == 1 ? EXIT_FINAL : EXIT_XSTATE;
      return d;
    }
    d.seg = 1 + (r - 1) / 2;
    d.map = (r - 1) % 2;  // 0: M (from the identity, U = 0); 1: b (from zero, U)
    d.init = d.map == 0 ? INIT_IDENTITY : INIT_ZERO;
    d.use_u = d.map == 1;
    d.write_o = false;
    d.exit = EXIT_MAP;
    return d;
  }
  // phase 2: segments 1 .. P-1 from h_1 and the maps before them
  const int64_t per = P - 1;
  if (run >= chains * per) return d;
  d.chain = run / per;
  d.seg = 1 + (int)(run % per);
  d.init = INIT_XSTATE;
  d.prefix = d.seg;
  d.exit = d.seg == P - 1 ? EXIT_FINAL : EXIT_NONE;
  return d;
}

// S <- M S + b for a compute wave's state slice (value tiles nt0 .. nt0 +
// TPW - 1, MFMA C layout).  M and b are fp32 [128][128] (key x key, key x
// value) in global memory.  The product runs on bf16 MFMAs with both
// operands split into hi + lo parts (hi.hi + hi.lo + lo.hi, ~16 mantissa
// bits), A = M in the permuted k order of the state's B operands.
template <int TPW>
__device__ __forceinline__ void prefix_step(f32x4 (&S)[8][TPW], const float *M, const float *bv,
                                            int nt0, int nn, int grp) {
  bf16x8 bh[4][TPW], bl[4][TPW];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
    for (int q = 0; q < TPW; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = S[2 * s4 + (e >> 2)][q][e & 3];
        split_bf16(x, bh[s4][q], bl[s4][q], e);
      }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    f32x4 acc[TPW];
#pragma unroll
    for (int q = 0; q < TPW; ++q) acc[q] = zero4();
    const float *row = M + (16 * t + nn) * DK;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const float4 lo4 = *reinterpret_cast<const float4 *>(row + 32 * s4 + 4 * grp);
      const float4 hi4 = *reinterpret_cast<const float4 *>(row + 32 * s4 + 16 + 4 * grp);
      const float av[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
      bf16x8 ah, al;
#pragma unroll
      for (int e = 0; e < 8; ++e) split_bf16(av[e], ah, al, e);
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        acc[q] = mfma_bf16(ah, bh[s4][q], acc[q]);
        acc[q] = mfma_bf16(ah, bl[s4][q], acc[q]);
        acc[q] = mfma_bf16(al, bh[s4][q], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < TPW; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[t][q][r] = acc[q][r] + bv[(16 * t + 4 * grp + r) * DV + VCOL(nt0 + q, nn)];
  }
}

}  // namespace

// Kernel: PARTS workgroups per chain, NC + NCP waves each.  The NC compute
// waves never issue a copy: the NCP copy waves (on otherwise idle SIMDs)
// stream chunk c+1's block into the other LDS buffer while the compute
// waves work on chunk c, and both meet at one barrier per chunk.  Workgroups of one chain
// get block indices congruent mod 8, so that (with the round-robin
// workgroup-to-XCD dispatch) they run on one XCD and share its L2: a block is
// read from HBM once and hit in L2 by the other parts.  The chain's
// intermediate blocks stream through two LDS buffers: while the waves compute
// chunk c from one buffer, chunk c+1's block is copied global -> LDS into
// the other by buffer_load_dwordx4 ... lds (no register staging).
template <int NC, int NCP, int TPW, bool SEG>
__global__ __launch_bounds__(64 * (NC + NCP)) void recurrence_kernel(RecurArgs a) {
  using C = RecCfg<NC, NCP, TPW>;
  __shared__ __align__(16) uint8_t lds[2][BLOCK_BYTES];
  __shared__ __align__(16) uint8_t touch_sink[256];  // written by the touches, never read
  const int b = blockIdx.x;
  const int xcd = b & 7, i = b >> 3;
  // run index: a chain, or (segments > 1) one run of a chain's segment
  const int64_t run = (int64_t)(i / C::PARTS) * 8 + xcd;
  const int p = i % C::PARTS;
  const int64_t chains = (int64_t)a.N * a.H;
  const RunDesc rd = describe_run<SEG>(a, run);
  if (rd.chain < 0) return;
  const int64_t chain = rd.chain;
  const int s = __builtin_amdgcn_readfirstlane((int)(chain / a.H));
  const int h = __builtin_amdgcn_readfirstlane((int)(chain % a.H));
  const int tid = threadIdx.x;
  // The wave index lives in a scalar register, so that every branch on a
  // wave's role is a scalar jump.  MFMAs do not honour EXEC: under an
  // exec-masked branch, a skipped path's MFMAs would still accumulate.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, nn = l & 15, grp = l >> 4;
  const int nt0 = p * C::TILES + w * TPW;  // a compute wave's first value tile
  // chunk range and token ranges are clamped so that a workspace that does
  // not hold a valid chunk table can never send this kernel out of bounds
  const int64_t nc_max = a.nc_max;
  int64_t c_beg = chunk_first_of(a.chunk_first, s), c_end = chunk_first_of(a.chunk_first, s + 1);
  c_beg = c_beg < 0 ? 0 : (c_beg > nc_max ? nc_max : c_beg);
  c_end = c_end < c_beg ? c_beg : (c_end > nc_max ? nc_max : c_end);
  if (SEG) {
    // segment rd.seg of the chain: chunks [c_beg + seg m, c_beg + (seg + 1) m)
    // (chunk indices < 2^31: nc_max H fits int32); wave-uniform scalars
    const int n = (int)(c_end - c_beg);
    const int m = (n + a.segments - 1) / a.segments;
    const int s0 = (int)c_beg + rd.seg * m;
    const int e0 = (int)c_end;
    c_beg = __builtin_amdgcn_readfirstlane(s0 < e0 ? s0 : e0);
    c_end = __builtin_amdgcn_readfirstlane(s0 + m < e0 ? s0 + m : e0);
  }
  const int64_t st_base = ((int64_t)s * a.H + h) * DK * DV;
  (void)chains;
  const uint8_t *chain_blocks = a.blocks + (int64_t)h * nc_max * BLOCK_BYTES;

  if (NCP > 0 && w >= NC) {
    // ---- copy waves: chunk c+1's block while chunk c is computed, the
    // touch of chunk c+2's, and the o of chunk c-1 (staged in LDS by the
    // compute waves) to memory ----
    // Each iteration issues the copy, the touch, then the stores; the wait
    // at the top of the next one covers the copy but not what was issued
    // after it (vector memory operations complete in order).
    const int cw = w - NC;
    const uint32_t sink = lds_base_of(touch_sink);
    if (c_beg < c_end) copy_share<C, NCP>(chain_blocks + c_beg * BLOCK_BYTES, lds[0], cw, p, l);
    if (c_beg + 1 < c_end) touch_block<C, NCP>(chain_blocks + (c_beg + 1) * BLOCK_BYTES, sink, cw, p, l);
    for (int64_t c = c_beg; c < c_end; ++c) {
      const bool touch = c + 1 < c_end, stores = c > c_beg + 1 && rd.write_o;
      if (cw == 0)
        wait_copy<C, NCP, 0>(touch, stores);
      else
        wait_copy<C, NCP, 1>(touch, stores);
      __syncthreads();
      const int cur = (int)((c - c_beg) & 1);
      if (c + 1 < c_end)
        copy_share<C, NCP>(chain_blocks + (c + 1) * BLOCK_BYTES, lds[cur ^ 1], cw, p, l);
      if (c + 2 < c_end) touch_block<C, NCP>(chain_blocks + (c + 2) * BLOCK_BYTES, sink, cw, p, l);
      if (c > c_beg && rd.write_o) store_o_staged<C, NCP>(a, lds[cur ^ 1], c - 1, h, p, cw, l);
    }
    __syncthreads();  // the compute waves have staged the last chunk's o
    if (c_end > c_beg && rd.write_o)
      store_o_staged<C, NCP>(a, lds[(int)((c_end - 1 - c_beg) & 1)], c_end - 1, h, p, cw, l);
    // no copy may still be writing LDS when the workgroup ends
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  // ---- compute waves ----
  // state slice: key tiles t = 0..7, value tiles nt0 + q
  f32x4 S[8][TPW];
  const float *init = rd.init == INIT_H0 ? (a.h0 ? a.h0 + st_base : nullptr)
                      : rd.init == INIT_XSTATE ? a.xstate + chain * DK * DV : nullptr;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int q = 0; q < TPW; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * t + 4 * grp + r;
        const int col = VCOL(nt0 + q, nn);
        S[t][q][r] = init ? init[row * DV + col] : (rd.init == INIT_IDENTITY && row == col ? 1.f : 0.f);
      }
  // phase 2: the entry state of segment seg from h_1 through the maps of
  // segments 1 .. seg - 1
  for (int q2 = 1; SEG && q2 < rd.prefix; ++q2) {
    const float *M = a.maps + ((chain * (a.segments - 2) + (q2 - 1)) * 2) * DK * DV;
    prefix_step<TPW>(S, M, M + DK * DV, nt0, nn, grp);
  }

  if (NCP == 0 && c_beg < c_end) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
      copy_step<C>(chain_blocks + c_beg * BLOCK_BYTES, lds[0], w, p, l, st);
  }

  // o of chunk c is stored during chunk c+1, one token tile per key slab,
  // so that the stores overlap a whole chunk of work.  With two value tiles
  // per wave the lane holds 8 consecutive columns of a token (VCOL), else 4.
  bf16x4 o_pend[4][TPW];
  int64_t o_t0 = 0;
  int o_n = 0;
  auto store_o_tile = [&](int mt) {
    const int row = 16 * mt + nn;
    if (row < o_n) {
      bf16_t *dst = reinterpret_cast<bf16_t *>(a.o) + ((o_t0 + row) * a.H + h) * DV +
                    VCOL(nt0, 4 * grp);
      if (TPW == 2) {
        const bf16x8 v = {o_pend[mt][0][0], o_pend[mt][0][1], o_pend[mt][0][2], o_pend[mt][0][3],
                          o_pend[mt][TPW - 1][0], o_pend[mt][TPW - 1][1], o_pend[mt][TPW - 1][2],
                          o_pend[mt][TPW - 1][3]};
        *reinterpret_cast<bf16x8 *>(dst) = v;
      } else {
        *reinterpret_cast<bf16x4 *>(dst) = o_pend[mt][0];
      }
    }
  };

  for (int64_t c = c_beg; c < c_end; ++c) {
    const int cur = (int)((c - c_beg) & 1);
    // after the barrier the copy waves' copies of this chunk are done, and
    // nobody still reads the other buffer (with copy waves, the compute
    // waves' only memory accesses are LDS ones)
    if (NCP > 0)
      __builtin_amdgcn_s_waitcnt(LGKM_ONLY);
    else
      __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
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
    bf16x8 hb[4][TPW];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int q = 0; q < TPW; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) hb[s4][q][e] = (bf16_t)S[2 * s4 + (e >> 2)][q][e & 3];

    // v_new starts from U (C layout: [token][value]); o^T from zero
    f32x4 vn[4][TPW], ot[4][TPW];
    // one 16-byte read per token tile pair (both C tiles of the pair, in
    // the lane's own 16 bytes: contiguous across lanes, no bank conflicts)
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const bf16x8 u = *reinterpret_cast<const bf16x8 *>(blk + U_OFFSET(nt0 + q, 2 * mp, l));
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int r = 0; r < 4; ++r) vn[2 * mp + m][q][r] = rd.use_u ? (float)u[4 * m + r] : 0.f;
          ot[2 * mp + m][q] = zero4();
        }
      }

    // the state is no longer needed unscaled: apply Diag(gamma) now, while
    // the MFMAs below run
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 gm = *reinterpret_cast<const float4 *>(blk + OFF_GAM + (16 * t + 4 * grp) * 4);
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        S[t][q][0] *= gm.x;
        S[t][q][1] *= gm.y;
        S[t][q][2] *= gm.z;
        S[t][q][3] *= gm.w;
      }
    }

    // v_new += (-W) h   and   o^T += h^T qg^T   (o is formed transposed so
    // that each lane ends up with consecutive value columns of one token)
    bf16x8 fk[2][8];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      // one token tile of last chunk's o (and, without copy waves, a quarter
      // of the next chunk's copy)
      if (NCP == 0 && c > c_beg && rd.write_o) store_o_tile(s4);
      if (NCP == 0 && c + 1 < c_end)
        copy_step<C>(chain_blocks + (c + 1) * BLOCK_BYTES, lds[cur ^ 1], w, p, l, s4);
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
        for (int q = 0; q < TPW; ++q) vn[mt][q] = mfma_bf16(fw[mt], hb[s4][q], vn[mt][q]);
      if (rd.write_o) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q < TPW; ++q) ot[mt][q] = mfma_bf16(hb[s4][q], fq[mt], ot[mt][q]);
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
    bf16x8 vb[2][TPW];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int q = 0; q < TPW; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) vb[s2][q][e] = (bf16_t)vn[2 * s2 + (e >> 2)][q][e & 3];

    // h <- Diag(gamma) h + kg^T v_new   (the serial dependency: first)
    bf16x8 fa[AQK_FRAGS];
#pragma unroll
    for (int x = 0; x < AQK_FRAGS; ++x) {
      fa[x] = load_frag(blk + OFF_AQK + (x * 64 + l) * 16);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int q = 0; q < TPW; ++q) S[t][q] = mfma_bf16(fk[s2][t], vb[s2][q], S[t][q]);

    // o^T += v_new^T Aqk^T
    if (rd.write_o) {
#pragma unroll
      for (int x = 0; x < AQK_FRAGS; ++x)
#pragma unroll
        for (int q = 0; q < TPW; ++q) {
          ot[lt_mt(x)][q] = mfma_bf16(vb[lt_s(x)][q], fa[x], ot[lt_mt(x)][q]);
        }
    }

    // o^T of this chunk as bf16 (nearest even), stored during the next one:
    // by the copy waves from LDS, or (without them) by this wave
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q = 0; q < TPW; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) o_pend[mt][q][r] = (bf16_t)ot[mt][q][r];
    if (NCP > 0 && rd.write_o) {
      uint8_t *ost = lds[cur] + o_stage_off<C>(p);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int q = 0; q < TPW; ++q)
          *reinterpret_cast<bf16x4 *>(ost + (16 * mt + nn) * C::O_ROW +
                                      o_stage_col<C>(nt0 + q, grp, p, 16 * mt + nn)) =
              o_pend[mt][q];
    }
    o_t0 = t0;
    o_n = n;
  }
  if (NCP > 0) {
    __builtin_amdgcn_s_waitcnt(LGKM_ONLY);
    __syncthreads();  // the copy waves store the last chunk's o
  } else if (c_end > c_beg && rd.write_o) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) store_o_tile(mt);
  }

  float *exit_state = rd.exit == EXIT_FINAL ? (a.hT ? a.hT + st_base : nullptr)
                      : rd.exit == EXIT_XSTATE ? a.xstate + chain * DK * DV
                      : rd.exit == EXIT_MAP
                          ? a.maps + ((chain * (a.segments - 2) + (rd.seg - 1)) * 2 + rd.map) * DK * DV
                          : nullptr;
  if (exit_state) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int q = 0; q < TPW; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * t + 4 * grp + r;
          const int col = VCOL(nt0 + q, nn);
          exit_state[row * DV + col] = S[t][q][r];
        }
  }
  // no copy may still be writing LDS when the workgroup ends
  if (NCP == 0) __builtin_amdgcn_s_waitcnt(0);
}

template <int NC, int NCP, int TPW>
static hipError_t launch_rec(const RecurArgs &a, int64_t runs, hipStream_t stream) {
  using C = RecCfg<NC, NCP, TPW>;
  const int64_t groups = (runs + 7) / 8;  // runs per XCD slot, rounded up
  const int64_t grid = groups * 8 * C::PARTS;
  if (a.segments > 1)
    hipLaunchKernelGGL((recurrence_kernel<NC, NCP, TPW, true>), dim3((unsigned)grid),
                       dim3(C::THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((recurrence_kernel<NC, NCP, TPW, false>), dim3((unsigned)grid),
                       dim3(C::THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_recurrence(const RecurArgs &a, hipStream_t stream) {
  const int64_t chains = (int64_t)a.N * a.H;
  if (chains <= 0) return hipSuccess;
  // runs of this launch (describe_run): chains, or the runs of a phase
  int64_t runs = chains;
  if (a.segments > 1)
    runs = a.phase == 1 ? chains * (1 + 2 * (int64_t)(a.segments - 2)) : chains * (a.segments - 1);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // split each run over as many workgroups as still fit the device once
  // (one compute wave per workgroup when eight per chain fit: measured
  // ~8% faster than two at 16 and 32 chains)
  if (runs * 8 <= cus) return launch_rec<1, 2, 1>(a, runs, stream);
  if (runs * 4 <= cus) return launch_rec<2, 2, 1>(a, runs, stream);
  if (runs * 2 <= cus) return launch_rec<4, 2, 1>(a, runs, stream);
  return launch_rec<4, 0, 2>(a, runs, stream);
}

}  // namespace kda
