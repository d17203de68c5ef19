// Token-serial KDA step for decode and speculative verification (MI355X
// Kimi K3 post, section 1.2: one fused kernel per decode step that keeps the
// recurrent state on chip while it applies a sequence's new tokens; section
// 1.3: 16 users, 1 token each or a 4-token verification window).
//
// Per (sequence, head), for each of the sequence's tokens t in order, with
// S the fp32 state [128 keys][128 values]:
//     S   <- Diag(exp g_t) S
//     S   <- S + beta_t k_t (v_t - S^T k_t)^T
//     o_t  = scale S^T q_t                     (reads the updated state)
// which is the gated delta rule the chunked prefill computes in chunk form.
// With few tokens per sequence the work is the state's read and write (128
// KiB per (sequence, head)), so the kernel streams the state once and keeps
// it in registers across the tokens.
//
// Work split.  The 128 value columns evolve independently, so a workgroup
// owns 64 of them for one (sequence, head): lane l of wave w holds column
// v0 + l and key rows 32 w .. 32 w + 31 (32 registers).  Both reductions over
// the keys (S^T k and S^T q) are a per-lane sum over its 32 rows, then the
// four waves' partial sums added in LDS in a fixed order, so results are
// deterministic.  State loads and stores are 256-byte row segments per wave.
#include "kda_internal.h"
#include "kda_decode.h"

namespace kda {

namespace {

constexpr int DEC_COLS = 64;               // value columns per workgroup
constexpr int DEC_WAVES = 4;               // key rows split over the waves
constexpr int DEC_ROWS = DK / DEC_WAVES;   // key rows per wave

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Sum over the 64 lanes of a wave, in VALU cross-lane steps only: DPP
// within each 16-lane row (xor 1, xor 2 by quad permutes, then the half-row
// and row mirrors), then the permlane swaps between rows 0-1 / 2-3 and
// between the two halves.  With both operands x, v_permlane16_swap returns
// the even rows' partners in .second and the odd rows' in .first, and
// v_permlane32_swap the low half's in .second and the high half's in .first.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float x, int lane) {
  x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_add<0x141>(x);  // row_half_mirror
  x = dpp_add<0x140>(x);  // row_mirror
  const uint32_t u = __float_as_uint(x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x += __uint_as_float(((lane >> 4) & 1) ? p16[0] : p16[1]);
  const uint32_t v = __float_as_uint(x);
  const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  x += __uint_as_float(lane >= 32 ? p32[0] : p32[1]);
  return x;
}

}  // namespace

// COLS value columns per workgroup: 64 (two workgroups per (sequence,
// head), lane l holding column l of its half), or 128 with the gated-RMSNorm
// epilogue fused in (one workgroup per (sequence, head), lane l holding
// columns l and l + 64, so wave 0 ends up with the whole output row).
template <int COLS>
__global__ __launch_bounds__(64 * DEC_WAVES) void decode_kernel(DecodeArgs a) {
  constexpr int NC = COLS / 64;  // columns per lane
  constexpr bool EPI = COLS == DV;
  __shared__ float ks[DK], qs[DK], eg[DK];
  __shared__ float red[DEC_WAVES][COLS];
  __shared__ float nrm[DEC_WAVES];
  const int64_t wg = blockIdx.x;
  const int part = (int)(wg % (DV / COLS));
  const int64_t sh = wg / (DV / COLS);
  const int h = (int)(sh % a.H);
  const int s = (int)(sh / a.H);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  int col[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) col[j] = part * COLS + j * 64 + l;
  const int r0 = w * DEC_ROWS;
  const int64_t st_base = ((int64_t)s * a.H + h) * DK * DV;

  // the sequence's tokens, with cu_seqlens clamped into [0, T] (malformed
  // offsets never send the kernel out of bounds)
  int64_t t_beg = a.cu[s], t_end = a.cu[s + 1];
  t_beg = t_beg < 0 ? 0 : (t_beg > a.T ? a.T : t_beg);
  t_end = t_end < t_beg ? t_beg : (t_end > a.T ? a.T : t_end);

  float S[NC][DEC_ROWS];
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int r = 0; r < DEC_ROWS; ++r)
      S[j][r] = a.h0 ? a.h0[st_base + (int64_t)(r0 + r) * DV + col[j]] : 0.f;
  float nw[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) nw[j] = EPI && a.y ? a.nw[col[j]] : 0.f;

  // a token's inputs, per thread: its k (threads 0-127, with g) or q
  // element, its value columns (and gate elements), and beta (or its logit)
  struct Tok {
    uint16_t x, v[NC], z[NC];  // raw bits: nothing waits on a load before its use
    uint32_t b;                // the beta logit's bf16 bits, or fp32 beta's bits
    float g;
  };
  auto load_tok = [&](int64_t t) {
    const int64_t tok = (t * a.H + h) * DK;
    Tok r;
    if (tid < DK) {
      r.x = a.k[tok + tid];
      r.g = a.g[tok + tid];
    } else {
      r.x = a.q[tok + tid - DK];
      r.g = 0.f;
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      r.v[j] = a.v[tok + col[j]];
      r.z[j] = EPI && a.y ? a.z[t * a.z_stride + (int64_t)h * DK + col[j]] : 0;
    }
    r.b = a.b ? (uint32_t)a.b[t * a.b_stride + h] : __float_as_uint(a.beta[t * a.H + h]);
    return r;
  };
  Tok cur = {};
  if (t_beg < t_end) cur = load_tok(t_beg);

  for (int64_t t = t_beg; t < t_end; ++t) {
    const int64_t tok = (t * a.H + h) * DK;
    // the next token's loads are in flight while this token is applied
    Tok nxt = cur;
    if (t + 1 < t_end) nxt = load_tok(t + 1);
    const float x = bf16_to_f32(cur.x);
    if (tid < DK) {
      ks[tid] = x;
      eg[tid] = expf(cur.g);
    } else {
      qs[tid - DK] = x;
    }
    if (a.qk_eps >= 0.f) {
      // fused prologue: the squared norms of k (waves 0, 1) and q (waves 2,
      // 3), a cross-lane sum within each wave, then two partial sums in LDS
      const float sq = wave_sum(x * x, l);
      if (l == 0) nrm[w] = sq;
    }
    const float beta = a.b ? 1.f / (1.f + expf(-bf16_to_f32((uint16_t)cur.b)))
                           : __uint_as_float(cur.b);
    __syncthreads();
    float rk = 1.f, rq = 1.f;
    if (a.qk_eps >= 0.f) {
      const float sk = (nrm[0] + nrm[1]) + a.qk_eps, sq = (nrm[2] + nrm[3]) + a.qk_eps;
      rk = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;  // a zero row stays zero (qk_eps = 0)
      rq = sq > 0.f ? 1.f / sqrtf(sq) : 0.f;
    }

    // decay, then this wave's part of (S^T k)[col]
    float pu[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) pu[j] = 0.f;
#pragma unroll
    for (int r = 0; r < DEC_ROWS; ++r) {
      const float e = eg[r0 + r], kr = ks[r0 + r] * rk;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        S[j][r] *= e;
        pu[j] = fmaf(S[j][r], kr, pu[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) red[w][j * 64 + l] = pu[j];
    __syncthreads();
    float dd[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = j * 64 + l;
      const float u = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
      dd[j] = beta * (bf16_to_f32(cur.v[j]) - u);
    }

    // rank-one write, then this wave's part of (S^T q)[col]
    float po[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) po[j] = 0.f;
#pragma unroll
    for (int r = 0; r < DEC_ROWS; ++r) {
      const float kr = ks[r0 + r] * rk, qr = qs[r0 + r] * rq;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        S[j][r] = fmaf(kr, dd[j], S[j][r]);
        po[j] = fmaf(S[j][r], qr, po[j]);
      }
    }
    __syncthreads();  // every wave has read red (u) and ks, qs, eg
#pragma unroll
    for (int j = 0; j < NC; ++j) red[w][j * 64 + l] = po[j];
    __syncthreads();
    if (w == 0) {
      float o[NC];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int c = j * 64 + l;
        o[j] = a.scale * (((red[0][c] + red[1][c]) + red[2][c]) + red[3][c]);
        a.o[tok + col[j]] = __builtin_bit_cast(uint16_t, (__bf16)o[j]);  // nearest even
      }
      if constexpr (EPI) {
        if (a.y) {
          // fused epilogue on the fp32 row: y = w * o / sqrt(mean o^2 + eps) * act(z)
          float ss = 0.f;
#pragma unroll
          for (int j = 0; j < NC; ++j) ss = fmaf(o[j], o[j], ss);
          ss = wave_sum(ss, l);
          const float dn = ss * (1.f / DV) + a.neps;
          const float rs = dn > 0.f ? 1.f / sqrtf(dn) : 0.f;
#pragma unroll
          for (int j = 0; j < NC; ++j) {
            const float z = bf16_to_f32(cur.z[j]);
            const float sg = 1.f / (1.f + expf(-z));
            const float act = a.act == 0 ? sg : z * sg;
            a.y[tok + col[j]] = __builtin_bit_cast(uint16_t, (__bf16)(nw[j] * (o[j] * rs) * act));
          }
        }
      }
    }
    // the next token's staging writes come after wave 0 has read red: it
    // reaches the next barrier only after that read
    cur = nxt;
  }

  if (a.hT) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int r = 0; r < DEC_ROWS; ++r) a.hT[st_base + (int64_t)(r0 + r) * DV + col[j]] = S[j][r];
  }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if (a.y) {
    const int64_t wgs = (int64_t)a.N * a.H;
    if (wgs <= 0) return hipSuccess;
    hipLaunchKernelGGL(decode_kernel<DV>, dim3((unsigned)wgs), dim3(64 * DEC_WAVES), 0, stream, a);
  } else {
    const int64_t wgs = (int64_t)a.N * a.H * (DV / DEC_COLS);
    if (wgs <= 0) return hipSuccess;
    hipLaunchKernelGGL(decode_kernel<DEC_COLS>, dim3((unsigned)wgs), dim3(64 * DEC_WAVES), 0, stream,
                       a);
  }
  return hipGetLastError();
}

}  // namespace kda
