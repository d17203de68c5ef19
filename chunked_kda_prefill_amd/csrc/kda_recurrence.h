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
  // Chunk-parallel state passing (segments > 1).  Each chain of n chunks is
  // cut into `segments` runs of m = ceil(n / segments) chunks; chunk c of
  // the chain maps the state affinely, h' = A_c h + B_c, so a segment's runs
  // compose into h' = M h + b.
  //   phase 1: segment 0 from the chain's initial state (o written; its exit
  //            state to xstate); segments 1 .. segments-2 twice, from the
  //            identity with U = 0 (M) and from zero with U (b), no o, both
  //            to maps;
  //   phase 2: segment p >= 1 from h_p = M_{p-1}(... (M_1 h_1 + b_1) ...) +
  //            b_{p-1}, h_1 = xstate (o written; the last segment writes
  //            the final state).
  int32_t segments = 1, phase = 0;
  float *maps = nullptr;    // [N * H][segments - 2][2][128][128]: M, then b
  float *xstate = nullptr;  // [N * H][128][128]
};
hipError_t launch_recurrence(const RecurArgs &a, hipStream_t stream);

}  // namespace kda
