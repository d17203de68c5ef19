// Host-side launchers, one per kernel; each lives in its kernel's source
// file and returns the launch status.  Each kernel's arguments sit in a
// header of its own, so that a kernel's sources are exactly its .hip file
// and the headers it includes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_decode.h"
#include "kda_intra.h"
#include "kda_norm.h"
#include "kda_recurrence.h"
#include "kda_validate.h"

namespace kda {

hipError_t launch_chunk_table(const int32_t *cu, int64_t T, int32_t N, int64_t nc_max,
                              int32_t *chunk_first, int4 *chunk_info, int32_t *flags,
                              hipStream_t stream);

hipError_t launch_gate_cumsum(const float *g, const int32_t *chunk_first, const int4 *chunk_info,
                              int64_t nc_max, int32_t N, int32_t H, float *G, hipStream_t stream);

}  // namespace kda
