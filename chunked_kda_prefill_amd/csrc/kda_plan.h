// Arguments and launcher of the plan kernel (kda_chunk_table.hip), which
// prepares the single-launch path of kda_chunk_fwd.
//
// The single launch runs the intra-chunk units and the chunk recurrence in
// one persistent grid.  Every workgroup reads the XCD it runs on and draws a
// ticket there: the first few become chain consumers (the recurrence and
// output of whole chains), the others producers (intra-chunk units).  A
// chain's units are produced and consumed on one XCD, so that its
// intermediate blocks pass through that XCD's L2.  The plan kernel writes
// what they need, all inside the workspace:
//   - the chunk table (chunk_first, chunk_info, flags), as chunk_table_kernel;
//   - order[N]: the sequences sorted by chunk count, longest first (ties by
//     index).  Chain rank rho = i * H + h is (sequence order[i], head h);
//     rank rho belongs to XCD rho % 8;
//   - units: for each XCD x, its units in chunk-major order: for local chunk
//     j = 0, 1, ..., the chains of XCD x that have more than j chunks, by
//     rank.  Entry = c * H + h (global chunk c, head h).  Because the
//     sequences are sorted, the chains with more than j chunks are the first
//     C_j = H * #{sequences with more than j chunks} ranks, so row j of XCD x
//     holds ceil((C_j - x) / 8) entries;
//   - sync: per XCD a role ticket and a unit counter (zeroed), and the
//     offsets of the per-XCD unit lists;
//   - ready[H * nc_max]: one flag per intermediate block (zeroed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {

constexpr int XCDS = 8;            // XCDs of an MI355X
constexpr int PLAN_MAX_SEQS = 1024;  // the plan sorts up to this many sequences in LDS
constexpr int MAX_CONSUMERS = 8;   // consumer workgroups per XCD

// int32 offsets inside the sync region: each XCD's ticket and unit counter
// share a 128-byte line of their own (at SYNC_STRIDE x), then the offsets
constexpr int SYNC_STRIDE = 32;
constexpr int SYNC_TICKET = 0;   // + SYNC_STRIDE x: role ticket of XCD x
constexpr int SYNC_UNIT = 1;     // + SYNC_STRIDE x: unit counter of XCD x
constexpr int SYNC_XOFF = SYNC_STRIDE * XCDS;  // [XCDS + 1] start of each XCD's list; [XCDS] = total
constexpr int SYNC_DIAG = SYNC_XOFF + 16;  // [3] diagnostics of a wait that gave up
constexpr int SYNC_WORDS = SYNC_XOFF + 32;
static_assert(4 * SYNC_WORDS <= SYNC_BYTES, "the sync words fit their workspace region");

struct PlanArgs {
  const int32_t *cu;
  int64_t T, nc_max;
  int32_t N, H;
  int32_t *chunk_first;
  int4 *chunk_info;
  int32_t *flags;
  int32_t *sync;   // [SYNC_WORDS]
  int32_t *order;  // [N]
  int32_t *units;  // [H * nc_max]
  int32_t *ready;  // [H * nc_max]
};
hipError_t launch_plan(const PlanArgs &a, hipStream_t stream);

}  // namespace kda
