// Gated RMSNorm on the operation's output ("Kimi K3 Prefill PP16" notes,
// third throughput section, KDA switch table: the KDA output tail runs the
// gated RMSNorm straight from a strided input, where a reshape used to force
// a non-contiguous copy first; RMSNorm after Zhang and Sennrich).
//
// Per (token t, head h) row x of 128 channels, gate row z and weight w:
//     y = w * x / sqrt(mean(x^2) + eps) * act(z)
// with act = sigmoid or SiLU (z * sigmoid(z)).  An all-zero row with eps = 0
// stays zero.
//
// The work is one read of x and z and one write of y (768 B per row at
// 2 bytes per element), so the kernel is a streaming one: 16 lanes own a row
// and load 16 bytes each (8 channels), a wave covers 4 rows, a workgroup 16.
// (A resident grid that loads the next row group before finishing the
// current one, and 4 row groups per workgroup with every load issued first,
// both measured slower: 30 µs against 27.6 µs at 8192 x 16 rows.)
// The row's sum of squares is a 4-step xor butterfly inside its 16 lanes.
// x rows, z rows and y rows are 256 contiguous bytes each, so every access
// is a full 256-byte segment.
#include "kda_internal.h"
#include "kda_norm.h"

namespace kda {

namespace {

constexpr int NORM_LANES = 16;                     // lanes per row
constexpr int NORM_ROWS = 256 / NORM_LANES;        // rows per workgroup
constexpr int64_t NORM_MAX_WGS = 1 << 20;          // grid-stride beyond this

__device__ __forceinline__ void unpack8(const uint4 &u, float f[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)a);  // nearest even
  const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)b);
  return lo | (hi << 16);
}

}  // namespace

__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(NormArgs a) {
  const int lane = threadIdx.x & (NORM_LANES - 1);
  const int c0 = lane * 8;
  float w[8];
  {
    const float4 w0 = *reinterpret_cast<const float4 *>(a.w + c0);
    const float4 w1 = *reinterpret_cast<const float4 *>(a.w + c0 + 4);
    w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
    w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
  }
  const int64_t rows = a.T * a.H;
  for (int64_t base = (int64_t)blockIdx.x * NORM_ROWS; base < rows;
       base += (int64_t)gridDim.x * NORM_ROWS) {
    const int64_t r = base + threadIdx.x / NORM_LANES;
    // rows past the end take part in no load or store; the butterfly below
    // stays within each row's own 16 lanes
    const bool live = r < rows;
    uint4 xr = make_uint4(0u, 0u, 0u, 0u), zr = xr;
    if (live) {
      const int64_t t = r / a.H;
      const int64_t h = r - t * a.H;
      xr = *reinterpret_cast<const uint4 *>(a.x + t * a.x_stride + h * DK + c0);
      zr = *reinterpret_cast<const uint4 *>(a.z + t * a.z_stride + h * DK + c0);
    }
    float x[8], z[8];
    unpack8(xr, x);
    unpack8(zr, z);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
#pragma unroll
    for (int m = NORM_LANES / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    const float d = ss * (1.f / DK) + a.eps;
    const float rs = d > 0.f ? 1.f / sqrtf(d) : 0.f;
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sg = 1.f / (1.f + expf(-z[i]));
      const float act = a.act == 0 ? sg : z[i] * sg;
      y[i] = w[i] * (x[i] * rs) * act;
    }
    if (live) {
      const uint4 out = make_uint4(pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]),
                                   pack2(y[6], y[7]));
      *reinterpret_cast<uint4 *>(a.y + r * DK + c0) = out;
    }
  }
}

hipError_t launch_gated_rmsnorm(const NormArgs &a, hipStream_t stream) {
  const int64_t rows = a.T * a.H;
  if (rows <= 0) return hipSuccess;
  int64_t wgs = (rows + NORM_ROWS - 1) / NORM_ROWS;
  if (wgs > NORM_MAX_WGS) wgs = NORM_MAX_WGS;
  hipLaunchKernelGGL(gated_rmsnorm_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
