// Arguments and launcher of the input validator (kda_validate.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// error bits of the validator's flag word
constexpr int32_t VALID_BAD_CU = 1;    // cu_seqlens not monotone from 0 to T
constexpr int32_t VALID_BAD_G = 2;     // some g outside [-5, 0], or NaN
constexpr int32_t VALID_BAD_BETA = 4;  // some beta outside [0, 1], or NaN

struct ValidateArgs {
  const float *g;     // [T, H, 128]
  const float *beta;  // [T, H] or null (not checked)
  const int32_t *cu;  // [N + 1]
  int32_t *flags;     // [1], cleared by the launch, then OR-ed
  int64_t T;
  int32_t N, H;
};
hipError_t launch_validate(const ValidateArgs &a, hipStream_t stream);

}  // namespace kda
