// Intra-chunk kernel: gate cumsum + strip-GEMMs + (I+L)^-1 + WY factors.
//
// Each (chunk, head) unit is handled by one 8-wave workgroup (persistent: a
// workgroup walks several units, see intra_kernel).  With G the chunk-local
// inclusive cumsum of g, Gamma = exp(G), rows i, j of the chunk, and the
// padding convention q = k = v = 0, g = 0, beta = 0 past a partial chunk's
// end (so every quantity below is exactly zero or exactly carried there):
//
//   Aqk = scale * lower-incl-diag( (Q*Gamma)(K/Gamma)^T )           [64, 64]
//   L   = strictly-lower( diag(beta) (K*Gamma)(K/Gamma)^T )           [64, 64]
//   T   = (I + L)^-1,   T' = T diag(beta)
//   U   = T' V,   W = T' (K*Gamma),   qg = scale Q*Gamma,
//   kg  = K * exp(G_last - G),   gamma = exp(G_last)
//
// KDA TPU report: section 4 (subblock-midpoint strip-GEMMs with bf16 inputs
// and fp32 accumulation; the fused right-hand side [beta v | beta k 2^G];
// no row-serial elimination), section 6.1 (cumsum fused in), section 6.2
// (what the recurrence consumes), section 6.3 (no backward-only columns).
//
// Strip factors.  Subblock a (rows 16a..16a+15) is referenced at its
// midpoint r_a = 16a + 7.  Per element, E1 = exp(G_i - G_{r(i)}) and
// E2 = 1/E1 = exp(G_{r(i)} - G_i) stay within 8 * 5 = 40 nats (57.7 bits)
// because g >= -5, and
//   exp(G_i - G_j) = E1_i * exp(G_{r_a} - G_{r_b}) * E2_j    (i in a, j in b),
// where the middle factor C_ab <= 1 is one value per channel.  So with
// q^ = q*E1, k^ = k*E1 and k~ = k*E2 computed once per element,
//   Aqk block (a,b) = q^_a (k~_b * C_ab)^T,   L block (a,b) = k^_a (k~_b * C_ab)^T.
// The Aqk strips use hi + lo bf16 on both operands (hi*hi + hi*lo + lo*hi);
// the L strips feed an fp32 inverse whose result is rounded again, so plain
// bf16 operands are enough there.  Gamma = E1 * exp(G_{r_a}) and
// exp(G_last - G_j) = E2_j * exp(G_last - G_{r_b}) likewise need no further
// per-element exponentials.
//
// Inverse.  The four diagonal 16x16 blocks use the finite Neumann product
// (I + X)(I + X^2)(I + X^4)(I + X^8) with X = -L_aa, exact because X is
// strictly lower (X^16 = 0); the off-diagonal blocks are merged as
// T_ab = -T_aa sum_{c=b}^{a-1} L_ac T_cb, one block diagonal at a time.  All
// of it runs in fp32 on v_mfma_f32_16x16x4_f32.  While waves 0-3 invert the
// diagonal blocks, waves 4-7 write the q*Gamma and kg fragments, which do
// not depend on T.
#include "kda_cumsum.h"
#include "kda_internal.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int NT = INTRA_THREADS;  // 8 waves

// Row-major [64][128] tiles with their 16-byte chunks XOR-swizzled by the row
// (chunk' = chunk ^ (row & 7)), so that the 16-byte fragment reads of 8
// consecutive rows hit different LDS banks.
__device__ __forceinline__ int sw_bf16(int row, int ch) {  // bf16 element index
  return row * DK + ((((ch >> 3) ^ (row & 7)) << 3) | (ch & 7));
}
__device__ __forceinline__ int sw_f32(int row, int ch) {  // fp32 element index
  return row * DK + ((((ch >> 2) ^ (row & 7)) << 2) | (ch & 3));
}
// The 64 x 64 fp32 L and T: 16-byte chunks swizzled by (row & 15), so the
// 16 rows an MFMA operand read touches land in different banks.
__device__ __forceinline__ int sw_lt(int row, int col) {
  return row * BT + ((((col >> 2) ^ (row & 15)) << 2) | (col & 3));
}

// Per-channel tables: R[a] = exp(G_{r_a}), Q[b] = exp(G_last - G_{r_b}),
// C[p] = exp(G_{r_a} - G_{r_b}) for the six off-diagonal pairs, and gamma.
constexpr int TAB_R = 0, TAB_Q = 4, TAB_C = 8, TAB_GAM = 14, TAB_ROWS = 15;
__device__ constexpr int OFF_A[6] = {1, 2, 2, 3, 3, 3};
__device__ constexpr int OFF_B[6] = {0, 0, 1, 0, 1, 2};

struct __align__(16) IntraSmem {
  bf16_t qh[BT * DK];   // q^ hi
  bf16_t ql[BT * DK];   // q^ lo
  bf16_t kh[BT * DK];   // k^ (bf16)
  bf16_t v[BT * DK];    // v
  float kt[BT * DK];    // k~ (fp32); holds the cumsum scratch before that
  float G[BT * DK];     // G; then L (first 64 x 64) and T (next 64 x 64)
  float tab[TAB_ROWS][DK];
  float beta[BT];
};
static_assert(2 * BT * BT <= BT * DK, "L and T fit where G was");
static_assert(sizeof(IntraSmem) <= 160 * 1024, "fits the CU's LDS");

// The six (token tile, token slab) pairs of a 64 x 64 lower-triangular
// operand that hold any j <= i; index = AQK_IDX(mt, s).
__device__ constexpr int LT_MT[6] = {0, 1, 2, 2, 3, 3};
__device__ constexpr int LT_S[6] = {0, 0, 0, 1, 0, 1};

__device__ __forceinline__ void store_bf16x4(uint8_t *p, const bf16x4 &x) {
  *reinterpret_cast<bf16x4 *>(p) = x;
}
__device__ __forceinline__ void store_bf16x8(uint8_t *p, const bf16x8 &x) {
  *reinterpret_cast<bf16x8 *>(p) = x;
}

__device__ __forceinline__ float bf(uint16_t b) { return bf16_bits_to_f32(b); }

// 16 x 16 x 16 fp32 product from C-layout registers: At holds A^T and B holds
// B (lane (nn, grp), element r = row 4grp + r, column nn); k runs over
// 4 grp + s.  Returns acc + A B in the same layout.
__device__ __forceinline__ f32x4 mm16(const f32x4 &At, const f32x4 &B, f32x4 acc) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma_f32(At[s], B[s], acc);
  return acc;
}

}  // namespace

// Inputs of one (chunk, head) unit, loaded into registers ahead of use.
struct UnitInputs {
  int64_t t0;
  int n;
  uint2 q4[4], k4[4], v4[4];  // row er, 4-channel chunks (ec + 8 kk)
  float beta;                 // threads < 64: row tid
  GateRows<NT> g;
};

__device__ __forceinline__ void load_unit(const IntraArgs &a, const int4 info, int h, int er, int ec,
                                          UnitInputs &in) {
  // the chunk table is written by the same call; clamping keeps even a
  // corrupted one in bounds
  in.t0 = info.x < 0 ? 0 : (info.x > a.T ? a.T : info.x);
  in.n = (int)(info.y < 0 ? 0 : (info.y > a.T - in.t0 ? a.T - in.t0 : (info.y > BT ? BT : info.y)));
  const bool ok = er < in.n;
  const int64_t off = ((in.t0 + er) * a.H + h) * DK;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int ch = 4 * (ec + 8 * kk);
    in.q4[kk] = ok ? *reinterpret_cast<const uint2 *>(a.q + off + ch) : make_uint2(0, 0);
    in.k4[kk] = ok ? *reinterpret_cast<const uint2 *>(a.k + off + ch) : make_uint2(0, 0);
    in.v4[kk] = ok ? *reinterpret_cast<const uint2 *>(a.v + off + ch) : make_uint2(0, 0);
  }
  const int tid = threadIdx.x;
  in.beta = (tid < BT && tid < in.n) ? a.beta[(in.t0 + tid) * a.H + h] : 0.f;
  gate_rows_load<NT>(a.g, in.t0, in.n, a.H, h, in.g);
}

// One (chunk, head) unit.  `nxt` receives the next unit's inputs, loaded
// once this unit's own inputs are consumed.
__device__ __forceinline__ void intra_unit(const IntraArgs &a, IntraSmem &sm, int64_t u,
                                           int64_t units, UnitInputs &nxt) {
  // threadIdx.x through an opaque move, so that address arithmetic derived
  // from it stays inside the unit loop instead of being hoisted out of it
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
  const int w = tid >> 6, l = tid & 63, nn = l & 15, grp = l >> 4;
  const int er = tid >> 3;  // element-phase row
  const int ec = tid & 7;   // element-phase chunk lane: chunks ec + 8 kk
  float *Ls = sm.G;         // after the factors are built
  float *Ts = sm.G + BT * BT;
  const int64_t c = u / a.H;
  const int h = (int)(u % a.H);
  // the next unit's chunk record, fetched now so that its data loads can be
  // issued later without waiting on it
  const int64_t un = u + gridDim.x;
  const int4 info_next = un < units ? a.chunk_info[un / a.H] : make_int4(0, 0, 0, 0);
  UnitInputs in = nxt;
  const int n = in.n;
  uint8_t *blk = a.blocks + ((int64_t)h * a.nc_max + c) * BLOCK_BYTES;
  // every wave is done with the previous unit's LDS
  __syncthreads();

  // ---- stage v and beta, scan g into G; then start the next unit's loads
  // thread t owns row er = t / 8 and the 4-channel chunks c = (t % 8) + 8 kk,
  // kk = 0..3 (8 lanes cover 8 consecutive chunks, which keeps the LDS
  // accesses below free of bank conflicts) ----
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    *reinterpret_cast<uint2 *>(&sm.v[sw_bf16(er, 4 * (ec + 8 * kk))]) = in.v4[kk];
  if (tid < BT) sm.beta[tid] = in.beta;
  gate_rows_scan<NT>(in.g, sm.G, sw_f32, sm.kt);
  __syncthreads();

  // ---- per-channel tables and per-element factors ----
  for (int idx = tid; idx < TAB_ROWS * DK; idx += NT) {
    const int tb = idx / DK, ch = idx % DK;
    float val;
    if (tb < TAB_Q) {
      val = exp_nat(sm.G[sw_f32(SB * tb + SB_REF, ch)]);
    } else if (tb < TAB_C) {
      val = exp_nat(sm.G[sw_f32(BT - 1, ch)] - sm.G[sw_f32(SB * (tb - TAB_Q) + SB_REF, ch)]);
    } else if (tb < TAB_GAM) {
      const int p = tb - TAB_C;
      val = exp_nat(sm.G[sw_f32(SB * OFF_A[p] + SB_REF, ch)] -
                    sm.G[sw_f32(SB * OFF_B[p] + SB_REF, ch)]);
    } else {
      val = exp_nat(sm.G[sw_f32(BT - 1, ch)]);
    }
    sm.tab[tb][ch] = val;
  }
  {
    const int rr = SB * (er / SB) + SB_REF;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = 4 * (ec + 8 * kk);
      const float4 gi = *reinterpret_cast<const float4 *>(&sm.G[sw_f32(er, ch)]);
      const float4 gr = *reinterpret_cast<const float4 *>(&sm.G[sw_f32(rr, ch)]);
      const float d[4] = {gi.x - gr.x, gi.y - gr.y, gi.z - gr.z, gi.w - gr.w};
      const uint16_t *qb = reinterpret_cast<const uint16_t *>(&in.q4[kk]);
      const uint16_t *kb = reinterpret_cast<const uint16_t *>(&in.k4[kk]);
      bf16x4 qhv, qlv, khv;
      float ktv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float e1 = exp_nat(d[e]), e2 = exp_nat(-d[e]);
        split_bf16(bf(qb[e]) * e1, qhv, qlv, e);
        khv[e] = (bf16_t)(bf(kb[e]) * e1);
        ktv[e] = bf(kb[e]) * e2;
      }
      *reinterpret_cast<bf16x4 *>(&sm.qh[sw_bf16(er, ch)]) = qhv;
      *reinterpret_cast<bf16x4 *>(&sm.ql[sw_bf16(er, ch)]) = qlv;
      *reinterpret_cast<bf16x4 *>(&sm.kh[sw_bf16(er, ch)]) = khv;
      *reinterpret_cast<float4 *>(&sm.kt[sw_f32(er, ch)]) = make_float4(ktv[0], ktv[1], ktv[2], ktv[3]);
    }
  }
  __syncthreads();

  // ---- the current unit's inputs are consumed: start the next unit's loads
  if (un < units) load_unit(a, info_next, (int)(un % a.H), er, ec, nxt);

  // ---- Aqk^T and L blocks: waves 0-5 one off-diagonal pair each, waves 6
  // and 7 two diagonal pairs each ----
  {
    const int npairs = w < 6 ? 1 : 2;
    for (int pi = 0; pi < npairs; ++pi) {
      const int ba = w < 6 ? OFF_A[w] : (w - 6) * 2 + pi;
      const int bb = w < 6 ? OFF_B[w] : ba;
      const float *cab = w < 6 ? sm.tab[TAB_C + w] : nullptr;
      const int j = SB * bb + nn;  // column-side rows (k~ C_ab)
      const int i = SB * ba + nn;  // row-side rows (q^, k^)
      f32x4 accA = zero4(), accL = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch0 = 32 * s + 8 * grp;
        const float4 k0 = *reinterpret_cast<const float4 *>(&sm.kt[sw_f32(j, ch0)]);
        const float4 k1 = *reinterpret_cast<const float4 *>(&sm.kt[sw_f32(j, ch0 + 4)]);
        float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        if (cab) {
          const float4 c0 = *reinterpret_cast<const float4 *>(&cab[ch0]);
          const float4 c1 = *reinterpret_cast<const float4 *>(&cab[ch0 + 4]);
          const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) kv[e] *= cv[e];
        }
        bf16x8 kth, ktl;
#pragma unroll
        for (int e = 0; e < 8; ++e) split_bf16(kv[e], kth, ktl, e);
        const bf16x8 qhv = *reinterpret_cast<const bf16x8 *>(&sm.qh[sw_bf16(i, ch0)]);
        const bf16x8 qlv = *reinterpret_cast<const bf16x8 *>(&sm.ql[sw_bf16(i, ch0)]);
        const bf16x8 khv = *reinterpret_cast<const bf16x8 *>(&sm.kh[sw_bf16(i, ch0)]);
        // Aqk^T block: rows j (A = k~), columns i (B = q^), hi/lo
        accA = mfma_bf16(kth, qhv, accA);
        accA = mfma_bf16(kth, qlv, accA);
        accA = mfma_bf16(ktl, qhv, accA);
        // L block: rows i (A = k^), columns j (B = k~), bf16
        accL = mfma_bf16(khv, kth, accL);
      }
      // Aqk^T: lane holds [j = 16bb + 4grp + r][i = 16ba + nn]; it becomes half
      // (bb & 1) of the recurrence's Aqk fragment (mt = ba, s = bb >> 1).
      bf16x4 ah, al;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool keep = (ba > bb) || (4 * grp + r <= nn);
        split_bf16(keep ? accA[r] * a.scale : 0.f, ah, al, r);
      }
      const int idx = AQK_IDX(ba, bb >> 1), half = bb & 1;
      store_bf16x4(blk + OFF_AQK + (idx * 64 + l) * 16 + half * 8, ah);
      store_bf16x4(blk + OFF_AQK + ((AQK_FRAGS + idx) * 64 + l) * 16 + half * 8, al);
      if (ba == bb && (ba & 1) == 0) {
        // blocks (0,1) and (2,3) lie above the diagonal: zero half 1
        const bf16x4 z = {(bf16_t)0.f, (bf16_t)0.f, (bf16_t)0.f, (bf16_t)0.f};
        store_bf16x4(blk + OFF_AQK + (idx * 64 + l) * 16 + 8, z);
        store_bf16x4(blk + OFF_AQK + ((AQK_FRAGS + idx) * 64 + l) * 16 + 8, z);
      }
      // L: lane holds [i = 16ba + 4grp + r][j = 16bb + nn], row-scaled by beta_i
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int il = 4 * grp + r;
        const bool keep = (ba > bb) || (nn < il);
        Ls[sw_lt(SB * ba + il, SB * bb + nn)] = keep ? accL[r] * sm.beta[SB * ba + il] : 0.f;
      }
    }
  }
  __syncthreads();

  if (w < 4) {
    // ---- diagonal block w of T: Neumann product in registers ----
    // Every 16 x 16 matrix M lives in MFMA C layout (lane (nn, grp) holds
    // M[4grp + r][nn], r = 0..3), next to its transpose.  With the k order
    // k = 4 grp + s, a product A B is  sum_s mfma(At[s], B[s])  for A^T and B
    // in that layout, so the chain needs no LDS round trips.
    const int d0 = SB * w;
    f32x4 YC, YtC, PC, PtC;  // X = -L_ww and X^T; P = I + X and P^T
    {
      const float4 row = *reinterpret_cast<const float4 *>(&Ls[sw_lt(d0 + nn, d0 + 4 * grp)]);
      const float rv[4] = {row.x, row.y, row.z, row.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * grp + r;
        YC[r] = (nn < m) ? -Ls[sw_lt(d0 + m, d0 + nn)] : 0.f;
        YtC[r] = (m < nn) ? -rv[r] : 0.f;
        PC[r] = (m == nn) ? 1.f : YC[r];
        PtC[r] = (m == nn) ? 1.f : YtC[r];
      }
    }
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const f32x4 Y2C = mm16(YtC, YC, zero4());    // Y Y
      const f32x4 PnC = mm16(PtC, Y2C, PC);        // P + P Y^2
      if (it < 2) {
        const f32x4 Y2tC = mm16(YC, YtC, zero4());  // Y^T Y^T
        PtC = mm16(Y2C, PtC, PtC);                  // P^T + (Y^2)^T P^T
        YC = Y2C;
        YtC = Y2tC;
      }
      PC = PnC;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) Ts[sw_lt(d0 + 4 * grp + r, d0 + nn)] = PC[r];
  } else {
    // ---- waves 4-7: qg fragments (token tile u) and kg^T fragments (key
    // tiles 2u, 2u+1), which do not depend on T ----
    const int u = w - 4;
    {
      const int i = SB * u + nn;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int ch = 32 * s + 16 * hh + 4 * grp;
          const bf16x4 qhv = *reinterpret_cast<const bf16x4 *>(&sm.qh[sw_bf16(i, ch)]);
          const bf16x4 qlv = *reinterpret_cast<const bf16x4 *>(&sm.ql[sw_bf16(i, ch)]);
          const float4 rv = *reinterpret_cast<const float4 *>(&sm.tab[TAB_R + u][ch]);
          const float rr[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            f[4 * hh + e] = (bf16_t)(a.scale * ((float)qhv[e] + (float)qlv[e]) * rr[e]);
        }
        store_bf16x8(blk + OFF_QG + ((u * 4 + s) * 64 + l) * 16, f);
      }
    }
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int mtc = 2 * u + q2;
      const int ch = 16 * mtc + nn;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jj = 32 * s + 16 * (e >> 2) + 4 * grp + (e & 3);
          f[e] = (bf16_t)(sm.kt[sw_f32(jj, ch)] * sm.tab[TAB_Q + (jj >> 4)][ch]);
        }
        store_bf16x8(blk + OFF_KGT + ((mtc * 2 + s) * 64 + l) * 16, f);
      }
    }
    if (u == 0) {
      const float2 gv = *reinterpret_cast<const float2 *>(&sm.tab[TAB_GAM][2 * l]);
      *reinterpret_cast<float2 *>(blk + OFF_GAM + 8 * l) = gv;
    }
  }
  __syncthreads();

  // ---- off-diagonal blocks: T_ab = -T_aa sum_{c=b}^{a-1} L_ac T_cb, one
  // block diagonal d = a - b at a time (wave b computes block (b+d, b)) ----
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int ba = w + d, bb = w;
      f32x4 MC = zero4();
      for (int cb = bb; cb < ba; ++cb) {
        // A = L_ac: its transpose in C layout is row nn, 4 consecutive columns
        const float4 lr = *reinterpret_cast<const float4 *>(&Ls[sw_lt(SB * ba + nn, SB * cb + 4 * grp)]);
        const f32x4 LtC = {lr.x, lr.y, lr.z, lr.w};
        f32x4 TC;
#pragma unroll
        for (int r = 0; r < 4; ++r) TC[r] = Ts[sw_lt(SB * cb + 4 * grp + r, SB * bb + nn)];
        MC = mm16(LtC, TC, MC);
      }
      const float4 tr = *reinterpret_cast<const float4 *>(&Ts[sw_lt(SB * ba + nn, SB * ba + 4 * grp)]);
      const f32x4 TaatC = {tr.x, tr.y, tr.z, tr.w};
      const f32x4 TabC = mm16(TaatC, MC, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) Ts[sw_lt(SB * ba + 4 * grp + r, SB * bb + nn)] = -TabC[r];
    }
    __syncthreads();
  }

  // ---- T' = T diag(beta) as hi/lo A fragments (rows i, 8 columns j),
  // built once into LDS where q^ was: waves 0-5 one fragment each ----
  bf16_t *tfr = sm.qh;  // [hi: 6 x 64 lanes x 8][lo: 6 x 64 x 8]
  if (w < 6) {
    const int x = w;
    const int i = SB * LT_MT[x] + nn;
    const int j0 = 32 * LT_S[x] + 8 * grp;
    const float4 t0v = *reinterpret_cast<const float4 *>(&Ts[sw_lt(i, j0)]);
    const float4 t1v = *reinterpret_cast<const float4 *>(&Ts[sw_lt(i, j0 + 4)]);
    const float4 b0v = *reinterpret_cast<const float4 *>(&sm.beta[j0]);
    const float4 b1v = *reinterpret_cast<const float4 *>(&sm.beta[j0 + 4]);
    const float tv[8] = {t0v.x, t0v.y, t0v.z, t0v.w, t1v.x, t1v.y, t1v.z, t1v.w};
    const float bv[8] = {b0v.x, b0v.y, b0v.z, b0v.w, b1v.x, b1v.y, b1v.z, b1v.w};
    bf16x8 fh, fl;
#pragma unroll
    for (int e = 0; e < 8; ++e) split_bf16((j0 + e <= i) ? tv[e] * bv[e] : 0.f, fh, fl, e);
    *reinterpret_cast<bf16x8 *>(&tfr[(x * 64 + l) * 8]) = fh;
    *reinterpret_cast<bf16x8 *>(&tfr[((6 + x) * 64 + l) * 8]) = fl;
  }
  __syncthreads();
  bf16x8 th[6], tl[6];
#pragma unroll
  for (int x = 0; x < 6; ++x) {
    th[x] = *reinterpret_cast<const bf16x8 *>(&tfr[(x * 64 + l) * 8]);
    tl[x] = *reinterpret_cast<const bf16x8 *>(&tfr[((6 + x) * 64 + l) * 8]);
  }

  // Transposed LDS read of a row-major bf16 tile (ds_read_b64_tr_b16): within
  // each group of 16 lanes, lane j addresses row r0 + j/4, columns
  // c0 + 4 (j%4) .. +3, and lane i receives tile[r0 + 0..3][c0 + i].  Two
  // such reads give a B fragment's 8 consecutive k rows for column c0 + nn.
  auto tr4 = [&](const bf16_t *tile, int r0, int c0) -> bf16x4 {
    const bf16_t *p = &tile[sw_bf16(r0 + (nn >> 2), c0 + 4 * (nn & 3))];
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4 *)(p));
  };

  // ---- U = T' V: wave w writes value tile nt = w (C layout) ----
  {
    const int nt = w;
    bf16x8 vb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x4 lo4 = tr4(sm.v, 32 * s + 8 * grp, 16 * nt);
      const bf16x4 hi4 = tr4(sm.v, 32 * s + 8 * grp + 4, 16 * nt);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vb[s][e] = lo4[e];
        vb[s][4 + e] = hi4[e];
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s) {
        const int x = AQK_IDX(mt, s);
        acc = mfma_bf16(th[x], vb[s], acc);
        acc = mfma_bf16(tl[x], vb[s], acc);
      }
      bf16x4 uv;
#pragma unroll
      for (int r = 0; r < 4; ++r) uv[r] = (bf16_t)acc[r];
      store_bf16x4(blk + OFF_U + ((nt * 4 + mt) * 64 + l) * 8, uv);
    }
  }

  // ---- W^T = (K*Gamma)^T T'^T: wave w owns key tile w ----
  {
    const int mtc = w;
    const int ch = 16 * mtc + nn;
    bf16x8 kgm[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // rows 32s + 8grp .. +7 all lie in subblock 2s + grp/2
      const float rv = sm.tab[TAB_R + 2 * s + (grp >> 1)][ch];
      const bf16x4 lo4 = tr4(sm.kh, 32 * s + 8 * grp, 16 * mtc);
      const bf16x4 hi4 = tr4(sm.kh, 32 * s + 8 * grp + 4, 16 * mtc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kgm[s][e] = (bf16_t)((float)lo4[e] * rv);
        kgm[s][4 + e] = (bf16_t)((float)hi4[e] * rv);
      }
    }
#pragma unroll
    for (int nti = 0; nti < 4; ++nti) {
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s <= (nti >> 1); ++s) {
        const int x = AQK_IDX(nti, s);
        acc = mfma_bf16(kgm[s], th[x], acc);
        acc = mfma_bf16(kgm[s], tl[x], acc);
      }
      // lane holds W^T[16 mtc + 4grp + r][16 nti + nn] -> -W, half (mtc & 1)
      // of the fragment (token tile nti, key slab mtc >> 1)
      bf16x4 wv;
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[r] = (bf16_t)(-acc[r]);
      store_bf16x4(blk + OFF_WN + ((nti * 4 + (mtc >> 1)) * 64 + l) * 16 + (mtc & 1) * 8, wv);
    }
  }
}

// Persistent: one workgroup per CU walks the (chunk, head) units with a
// stride of the grid size; the next unit's inputs are loaded into registers
// while the current one computes, so HBM reads overlap the LDS/MFMA work.
__global__ __launch_bounds__(NT) void intra_kernel(IntraArgs a) {
  __shared__ IntraSmem sm;
  int64_t nc = a.chunk_first[a.N];
  nc = nc < 0 ? 0 : (nc > a.nc_max ? a.nc_max : nc);
  const int64_t units = nc * a.H;
  int64_t u = blockIdx.x;
  if (u >= units) return;
  UnitInputs nxt;
  load_unit(a, a.chunk_info[u / a.H], (int)(u % a.H), threadIdx.x >> 3, threadIdx.x & 7, nxt);
  for (; u < units; u += gridDim.x) intra_unit(a, sm, u, units, nxt);
}

hipError_t launch_intra(const IntraArgs &a, hipStream_t stream) {
  if (a.nc_max <= 0) return hipSuccess;
  // one workgroup per compute unit (the LDS footprint allows no more)
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t units = a.nc_max * a.H;
  const int64_t grid = units < cus ? units : cus;
  hipLaunchKernelGGL(intra_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
