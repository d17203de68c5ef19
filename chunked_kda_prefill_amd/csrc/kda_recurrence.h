// Arguments and launcher of the chunk recurrence kernel (kda_recurrence.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct RecurArgs {
  const uint8_t *blocks;
  const int32_t *chunk_first;
  const int4 *chunk_info;
  const float *h0;      // [N, H, 128, 128] or null
  float *hT;            // [N, H, 128, 128] or null
  uint16_t *o;          // bf16 bits [T, H, 128]
  int64_t nc_max, T;
  int32_t N, H;
};
hipError_t launch_recurrence(const RecurArgs &a, hipStream_t stream);

}  // namespace kda
