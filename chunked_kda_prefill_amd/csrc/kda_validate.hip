// Opt-in check of the device-content contracts that the forward kernels
// trust without reading them twice: g inside [-5, 0] (the KDA TPU report's
// lower bound, section 4), beta inside [0, 1] (a sigmoid's range), and
// cu_seqlens monotone from 0 to T.  The forward kernels stay in bounds on
// any input (they clamp cu_seqlens); this only reports, as bits of one
// int32 word.  Not part of the forward: it reads g once more (512 B per
// (token, head)).
//
// Two launches: a one-thread kernel clears the word (a kernel, not a memset,
// so that the pair can sit in a captured graph), then a grid-stride scan in
// which each wave ORs its lanes' verdicts together and one lane, only if
// something was found, ORs them into the word with a global atomic.
#include "kda_internal.h"
#include "kda_validate.h"

namespace kda {

namespace {

constexpr int VAL_THREADS = 256;
constexpr int64_t VAL_MAX_WGS = 2048;

__device__ __forceinline__ bool g_ok(float x) { return x >= -5.f && x <= 0.f; }  // NaN fails

}  // namespace

__global__ void validate_clear_kernel(int32_t *flags) { flags[0] = 0; }

__global__ __launch_bounds__(VAL_THREADS) void validate_kernel(ValidateArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * VAL_THREADS + threadIdx.x;
  const int64_t nth = (int64_t)gridDim.x * VAL_THREADS;
  int32_t bad = 0;
  // g as float4: T * H * 128 is a multiple of 4, and g is 16-byte aligned
  const int64_t n4 = a.T * a.H * (DK / 4);
  const float4 *g4 = reinterpret_cast<const float4 *>(a.g);
  for (int64_t i = tid; i < n4; i += nth) {
    const float4 v = g4[i];
    if (!(g_ok(v.x) && g_ok(v.y) && g_ok(v.z) && g_ok(v.w))) bad |= VALID_BAD_G;
  }
  if (a.beta) {
    for (int64_t i = tid; i < a.T * a.H; i += nth) {
      const float b = a.beta[i];
      if (!(b >= 0.f && b <= 1.f)) bad |= VALID_BAD_BETA;
    }
  }
  for (int64_t i = tid; i < a.N; i += nth) {
    const int32_t lo = a.cu[i], hi = a.cu[i + 1];
    if (hi < lo || (i == 0 && lo != 0) || (i == a.N - 1 && (int64_t)hi != a.T)) bad |= VALID_BAD_CU;
  }
  // one OR per wave that found anything
  int32_t w = bad;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) w |= __shfl_xor(w, m);
  if ((threadIdx.x & 63) == 0 && w) atomicOr(a.flags, w);
}

hipError_t launch_validate(const ValidateArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(validate_clear_kernel, dim3(1), dim3(1), 0, stream, a.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t work = a.T * a.H * (DK / 4);
  if (a.N > work) work = a.N;
  int64_t wgs = (work + VAL_THREADS - 1) / VAL_THREADS;
  if (wgs < 1) wgs = 1;
  if (wgs > VAL_MAX_WGS) wgs = VAL_MAX_WGS;
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)wgs), dim3(VAL_THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
