// C ABI of libkda: argument validation on the host, then kernel launches on
// the caller's stream.  Nothing here reads device memory, allocates, or
// synchronises.
#include "kda.h"
#include "kda_chunk_table.h"
#include "kda_internal.h"
#include "kda_launch.h"

#include <mutex>
#include <stdint.h>

using namespace kda;

// ---------------------------------------------------------------------------
// Workspace of kda_chunk_fwd_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device memory: its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only
// that address is handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::once_flag scratch_once[MAX_DEVICES];
void *scratch_ptr[MAX_DEVICES];
hipError_t scratch_err[MAX_DEVICES];

// The calling thread's current device's copy of `scratch`, or null (with
// the lookup's error in *err).
void *device_scratch(hipError_t *err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(scratch_once[dev], [dev]() {
    void *p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = scratch_err[dev];
  return scratch_ptr[dev];
}

}  // namespace

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [p, p + bytes) and [q, q + qbytes) overlap?
bool overlap(const void *p, int64_t bytes, const void *q, int64_t qbytes) {
  if (!p || !q || bytes <= 0 || qbytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + (uintptr_t)bytes;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + (uintptr_t)qbytes;
  return a0 < b1 && b0 < a1;
}

kda_status check_sizes(int64_t T, int32_t N, int32_t H) {
  if (T < 0 || N < 1 || H < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (T > INT32_MAX || H > 65535) return KDA_ERR_UNSUPPORTED;
  const int64_t nc_max = nc_max_of(T, N);
  // grids are 1-D: (chunk slots x heads) and (sequences x heads) workgroups
  if (nc_max * (int64_t)H > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)N * H > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

struct Ws {
  WsLayout L;
  int32_t *flags;
  int32_t *chunk_first;
  int4 *chunk_info;
  uint8_t *blocks;
};

kda_status carve(void *workspace, size_t workspace_bytes, int64_t T, int32_t N, int32_t H,
                 Ws &ws) {
  if (!workspace) return KDA_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 256)) return KDA_ERR_INVALID_ARGUMENT;
  ws.L = ws_layout(T, N, H);
  if ((int64_t)workspace_bytes < ws.L.total) return KDA_ERR_WORKSPACE_TOO_SMALL;
  uint8_t *base = static_cast<uint8_t *>(workspace);
  ws.flags = reinterpret_cast<int32_t *>(base + ws.L.off_flags);
  ws.chunk_first = reinterpret_cast<int32_t *>(base + ws.L.off_chunk_first);
  ws.chunk_info = reinterpret_cast<int4 *>(base + ws.L.off_chunk_info);
  ws.blocks = base + ws.L.off_blocks;
  return KDA_OK;
}

kda_status check_inputs(const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const int32_t *cu, int64_t T,
                        const void *b = nullptr, int64_t b_stride = 0, int32_t H = 0) {
  if (!cu || !aligned(cu, 4)) return KDA_ERR_INVALID_ARGUMENT;
  if (T > 0) {
    if (!q || !k || !v || !g) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16))
      return KDA_ERR_INVALID_ARGUMENT;
    if (b) {  // beta logits of a strided slice
      if (!aligned(b, 2) || b_stride < H || b_stride > (int64_t(1) << 24))
        return KDA_ERR_INVALID_ARGUMENT;
    } else if (!beta || !aligned(beta, 4)) {
      return KDA_ERR_INVALID_ARGUMENT;
    }
  }
  return KDA_OK;
}

kda_status hip_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// The device regions a forward call reads: q, k, v, g, beta (or the beta
// logits b of a strided slice), cu_seqlens and the initial state.
struct Inputs {
  const void *p[8];
  int64_t bytes[8];
  int n = 0;
  void add(const void *ptr, int64_t b) {
    p[n] = ptr;
    bytes[n] = b;
    ++n;
  }
  // does [w, w + wbytes) overlap any of them?
  bool hit(const void *w, int64_t wbytes) const {
    for (int i = 0; i < n; ++i)
      if (overlap(w, wbytes, p[i], bytes[i])) return true;
    return false;
  }
};

Inputs forward_inputs(const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const float *initial_state, const int32_t *cu,
                      int64_t T, int32_t N, int32_t H, const uint16_t *b, int64_t b_stride) {
  const int64_t tok = T * H * DK;
  Inputs in;
  in.add(q, tok * 2);
  in.add(k, tok * 2);
  in.add(v, tok * 2);
  in.add(g, tok * 4);
  in.add(beta, T * H * 4);
  if (b && T > 0) in.add(b, ((T - 1) * b_stride + H) * 2);
  in.add(cu, ((int64_t)N + 1) * 4);
  in.add(initial_state, (int64_t)N * H * DK * DV * 4);
  return in;
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
  }
  return "KDA_ERR_UNKNOWN";
}

size_t kda_chunk_fwd_workspace_size(int64_t T, int32_t N, int32_t H) {
  if (check_sizes(T, N, H) != KDA_OK) return 0;
  return (size_t)ws_layout(T, N, H).total;
}

kda_status kda_workspace_layout(int64_t T, int32_t N, int32_t H, int64_t out[5]) {
  if (!out) return KDA_ERR_INVALID_ARGUMENT;
  const kda_status st = check_sizes(T, N, H);
  if (st != KDA_OK) return st;
  const WsLayout L = ws_layout(T, N, H);
  out[0] = L.off_flags;
  out[1] = L.off_chunk_first;
  out[2] = L.off_chunk_info;
  out[3] = L.off_blocks;
  out[4] = BLOCK_BYTES;
  return KDA_OK;
}

kda_status kda_chunk_table(const int32_t *cu_seqlens, int64_t T, int32_t N, int32_t *chunk_first,
                           int32_t *chunk_info, int32_t *flags, hipStream_t stream) {
  kda_status st = check_sizes(T, N, 1);
  if (st != KDA_OK) return st;
  if (!cu_seqlens || !chunk_first || !chunk_info || !flags) return KDA_ERR_INVALID_ARGUMENT;
  if (!aligned(cu_seqlens, 4) || !aligned(chunk_first, 4) || !aligned(chunk_info, 16) ||
      !aligned(flags, 4))
    return KDA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_chunk_table(cu_seqlens, T, N, nc_max_of(T, N), chunk_first,
                                       reinterpret_cast<int4 *>(chunk_info), flags, stream));
}

kda_status kda_gate_cumsum(const float *g, const int32_t *cu_seqlens, int64_t T, int32_t N,
                           int32_t H, float *G, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  kda_status st = check_sizes(T, N, H);
  if (st != KDA_OK) return st;
  if (!cu_seqlens || !aligned(cu_seqlens, 4)) return KDA_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!g || !G || !aligned(g, 16) || !aligned(G, 16))) return KDA_ERR_INVALID_ARGUMENT;
  if (overlap(G, T * H * DK * 4, g, T * H * DK * 4)) return KDA_ERR_INVALID_ARGUMENT;
  Ws ws;
  if ((st = carve(workspace, workspace_bytes, T, N, H, ws)) != KDA_OK) return st;
  if (overlap(workspace, ws.L.total, g, T * H * DK * 4) ||
      overlap(workspace, ws.L.total, G, T * H * DK * 4) ||
      overlap(workspace, ws.L.total, cu_seqlens, ((int64_t)N + 1) * 4) ||
      overlap(G, T * H * DK * 4, cu_seqlens, ((int64_t)N + 1) * 4))
    return KDA_ERR_INVALID_ARGUMENT;
  hipError_t e = launch_chunk_table(cu_seqlens, T, N, ws.L.nc_max, ws.chunk_first, ws.chunk_info,
                                    ws.flags, stream);
  if (e != hipSuccess) return KDA_ERR_HIP;
  return hip_status(
      launch_gate_cumsum(g, ws.chunk_first, ws.chunk_info, ws.L.nc_max, N, H, G, stream));
}

static kda_status check_outputs(const float *initial_state, int64_t T, int32_t N, int32_t H,
                                const void *o, const float *final_state) {
  if (T > 0 && (!o || !aligned(o, 16))) return KDA_ERR_INVALID_ARGUMENT;
  if ((initial_state && !aligned(initial_state, 16)) || (final_state && !aligned(final_state, 16)))
    return KDA_ERR_INVALID_ARGUMENT;
  const int64_t st_bytes = (int64_t)N * H * DK * DV * 4;
  if (overlap(o, T * H * DK * 2, final_state, st_bytes) ||
      overlap(o, T * H * DK * 2, initial_state, st_bytes))
    return KDA_ERR_INVALID_ARGUMENT;
  // final_state may alias initial_state exactly, but not partially
  if (final_state && initial_state && final_state != initial_state &&
      overlap(final_state, st_bytes, initial_state, st_bytes))
    return KDA_ERR_INVALID_ARGUMENT;
  return KDA_OK;
}

static kda_status run_recurrence(const float *initial_state, int64_t T, int32_t N, int32_t H,
                                 void *o, float *final_state, const Ws &ws, hipStream_t stream) {
  RecurArgs ra;
  ra.blocks = ws.blocks;
  ra.chunk_first = ws.chunk_first;
  ra.chunk_info = ws.chunk_info;
  ra.h0 = initial_state;
  ra.hT = final_state;
  ra.o = static_cast<uint16_t *>(o);
  ra.nc_max = ws.L.nc_max;
  ra.T = T;
  ra.N = N;
  ra.H = H;
  return hip_status(launch_recurrence(ra, stream));
}

// Fused prologue options of an entry point: beta from bf16 logits b with
// row stride b_stride (b null: beta as given), and q, k L2-normalised with
// qk_eps when qk_eps >= 0.
struct Prologue {
  const uint16_t *b = nullptr;
  int64_t b_stride = 0;
  float qk_eps = -1.f;
};

static kda_status run_intra(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const int32_t *cu_seqlens, int64_t T, int32_t N,
                            int32_t H, float scale, const Ws &ws, hipStream_t stream,
                            const Prologue &pro = Prologue()) {
  // small batches: the intra-chunk kernel builds the chunk table itself (one
  // launch less); larger ones get the standalone table kernel first
  const bool inline_table = N <= INLINE_SEQS && ws.L.nc_max > 0;
  if (!inline_table) {
    hipError_t e = launch_chunk_table(cu_seqlens, T, N, ws.L.nc_max, ws.chunk_first,
                                      ws.chunk_info, ws.flags, stream);
    if (e != hipSuccess) return KDA_ERR_HIP;
  }
  IntraArgs ia;
  ia.q = static_cast<const uint16_t *>(q);
  ia.k = static_cast<const uint16_t *>(k);
  ia.v = static_cast<const uint16_t *>(v);
  ia.g = g;
  ia.beta = beta;
  ia.cu = cu_seqlens;
  ia.chunk_first = ws.chunk_first;
  ia.chunk_info = ws.chunk_info;
  ia.flags = ws.flags;
  ia.blocks = ws.blocks;
  ia.nc_max = ws.L.nc_max;
  ia.T = T;
  ia.N = N;
  ia.H = H;
  ia.scale = scale;
  ia.inline_table = inline_table ? 1 : 0;
  ia.b = pro.b;
  ia.b_stride = pro.b_stride;
  ia.qk_eps = pro.qk_eps;
  return hip_status(launch_intra(ia, stream));
}

kda_status kda_chunk_intra(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const int32_t *cu_seqlens, int64_t T, int32_t N,
                           int32_t H, float scale, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  kda_status st = check_sizes(T, N, H);
  if (st != KDA_OK) return st;
  if ((st = check_inputs(q, k, v, g, beta, cu_seqlens, T)) != KDA_OK) return st;
  Ws ws;
  if ((st = carve(workspace, workspace_bytes, T, N, H, ws)) != KDA_OK) return st;
  if (forward_inputs(q, k, v, g, beta, nullptr, cu_seqlens, T, N, H, nullptr, 0)
          .hit(workspace, ws.L.total))
    return KDA_ERR_INVALID_ARGUMENT;
  return run_intra(q, k, v, g, beta, cu_seqlens, T, N, H, scale, ws, stream);
}

// Host-side checks of a forward call's arguments (sizes, pointers, alignment,
// overlaps): o must not overlap any input; final_state may alias only the
// initial state, exactly.
static kda_status check_forward_args(const void *q, const void *k, const void *v, const float *g,
                                     const float *beta, const float *initial_state,
                                     const int32_t *cu_seqlens, int64_t T, int32_t N, int32_t H,
                                     const void *o, const float *final_state,
                                     const Prologue &pro) {
  kda_status st = check_sizes(T, N, H);
  if (st != KDA_OK) return st;
  if ((st = check_inputs(q, k, v, g, beta, cu_seqlens, T, pro.b, pro.b_stride, H)) != KDA_OK)
    return st;
  if ((st = check_outputs(initial_state, T, N, H, o, final_state)) != KDA_OK) return st;
  const int64_t tok = T * H * DK;
  const int64_t st_bytes = (int64_t)N * H * DK * DV * 4;
  const Inputs in = forward_inputs(q, k, v, g, beta, initial_state, cu_seqlens, T, N, H, pro.b,
                                   pro.b_stride);
  const Inputs in_no_h0 = forward_inputs(q, k, v, g, beta, nullptr, cu_seqlens, T, N, H, pro.b,
                                         pro.b_stride);
  if (in.hit(o, tok * 2) || in_no_h0.hit(final_state, st_bytes)) return KDA_ERR_INVALID_ARGUMENT;
  return KDA_OK;
}

static kda_status chunk_fwd_impl(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *initial_state,
                                 const int32_t *cu_seqlens, int64_t T, int32_t N, int32_t H,
                                 float scale, void *o, float *final_state, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream, const Prologue &pro) {
  kda_status st = check_forward_args(q, k, v, g, beta, initial_state, cu_seqlens, T, N, H, o,
                                     final_state, pro);
  if (st != KDA_OK) return st;
  const int64_t tok = T * H * DK;
  const int64_t st_bytes = (int64_t)N * H * DK * DV * 4;
  const Inputs in = forward_inputs(q, k, v, g, beta, initial_state, cu_seqlens, T, N, H, pro.b,
                                   pro.b_stride);
  Ws ws;
  if ((st = carve(workspace, workspace_bytes, T, N, H, ws)) != KDA_OK) return st;
  // the workspace is written while inputs are still being read
  if (in.hit(workspace, ws.L.total) || overlap(workspace, ws.L.total, o, tok * 2) ||
      overlap(workspace, ws.L.total, final_state, st_bytes))
    return KDA_ERR_INVALID_ARGUMENT;

  if ((st = run_intra(q, k, v, g, beta, cu_seqlens, T, N, H, scale, ws, stream, pro)) != KDA_OK)
    return st;
  return run_recurrence(initial_state, T, N, H, o, final_state, ws, stream);
}

// The gated-RMSNorm epilogue fused into the decode kernel (y set).
struct Epilogue {
  void *y = nullptr;
  const void *z = nullptr;
  int64_t z_stride = 0;
  const float *nw = nullptr;
  float eps = 0.f;
  int32_t act = KDA_ACT_SIGMOID;
};

static kda_status decode_fwd_impl(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *initial_state,
                                  const int32_t *cu_seqlens, int64_t T, int32_t N, int32_t H,
                                  float scale, void *o, float *final_state, hipStream_t stream,
                                  const Prologue &pro, const Epilogue &epi = Epilogue()) {
  kda_status st = check_sizes(T, N, H);
  if (st != KDA_OK) return st;
  if ((int64_t)N * H * 2 > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if ((st = check_inputs(q, k, v, g, beta, cu_seqlens, T, pro.b, pro.b_stride, H)) != KDA_OK)
    return st;
  if ((st = check_outputs(initial_state, T, N, H, o, final_state)) != KDA_OK) return st;
  const int64_t tok = T * H * DK;
  const int64_t st_bytes_all = (int64_t)N * H * DK * DV * 4;
  const Inputs in = forward_inputs(q, k, v, g, beta, initial_state, cu_seqlens, T, N, H, pro.b,
                                   pro.b_stride);
  const Inputs in_no_h0 = forward_inputs(q, k, v, g, beta, nullptr, cu_seqlens, T, N, H, pro.b,
                                         pro.b_stride);
  // every workgroup reads cu_seqlens while others write o and the state
  if (in.hit(o, tok * 2) || in_no_h0.hit(final_state, st_bytes_all))
    return KDA_ERR_INVALID_ARGUMENT;
  if (epi.y && T > 0 && (epi.z && overlap(final_state, st_bytes_all, epi.z,
                                          ((T - 1) * epi.z_stride + (int64_t)H * DK) * 2)))
    return KDA_ERR_INVALID_ARGUMENT;
  if (epi.y && T > 0) {
    if (!epi.z || !epi.nw || !aligned(epi.y, 2) || !aligned(epi.z, 2) || !aligned(epi.nw, 4))
      return KDA_ERR_INVALID_ARGUMENT;
    if (!(epi.eps >= 0.f) || epi.eps == INFINITY) return KDA_ERR_INVALID_ARGUMENT;
    if (epi.act != KDA_ACT_SIGMOID && epi.act != KDA_ACT_SILU) return KDA_ERR_INVALID_ARGUMENT;
    const int64_t row = (int64_t)H * DK;
    // up to 2^31 elements: (T - 1) * z_stride (T < 2^31) stays inside int64
    if (epi.z_stride < row || epi.z_stride > ((int64_t)1 << 31)) return KDA_ERR_INVALID_ARGUMENT;
    const int64_t zbytes = ((T - 1) * epi.z_stride + row) * 2;
    const int64_t st_bytes = (int64_t)N * H * DK * DV * 4;
    // y is written: it overlaps nothing else the call reads or writes
    const void *others[] = {q, k, v, g, o, epi.z};
    const int64_t sizes[] = {tok * 2, tok * 2, tok * 2, tok * 4, tok * 2, zbytes};
    for (int i = 0; i < 6; ++i)
      if (overlap(epi.y, tok * 2, others[i], sizes[i])) return KDA_ERR_INVALID_ARGUMENT;
    if (overlap(epi.y, tok * 2, beta, T * H * 4) || overlap(epi.y, tok * 2, epi.nw, DV * 4) ||
        overlap(epi.y, tok * 2, initial_state, st_bytes) ||
        overlap(epi.y, tok * 2, final_state, st_bytes) ||
        (pro.b && overlap(epi.y, tok * 2, pro.b, ((T - 1) * pro.b_stride + H) * 2)))
      return KDA_ERR_INVALID_ARGUMENT;
  }
  DecodeArgs da;
  da.q = static_cast<const uint16_t *>(q);
  da.k = static_cast<const uint16_t *>(k);
  da.v = static_cast<const uint16_t *>(v);
  da.g = g;
  da.beta = beta;
  da.cu = cu_seqlens;
  da.h0 = initial_state;
  da.hT = final_state;
  da.o = static_cast<uint16_t *>(o);
  da.T = T;
  da.N = N;
  da.H = H;
  da.scale = scale;
  da.b = pro.b;
  da.b_stride = pro.b_stride;
  da.qk_eps = pro.qk_eps;
  da.y = static_cast<uint16_t *>(epi.y);
  da.z = static_cast<const uint16_t *>(epi.z);
  da.z_stride = epi.z_stride;
  da.nw = epi.nw;
  da.neps = epi.eps;
  da.act = epi.act;
  return hip_status(launch_decode(da, stream));
}

kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                         int64_t T, int32_t N, int32_t H, float scale, void *o,
                         float *final_state, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  return chunk_fwd_impl(q, k, v, g, beta, initial_state, cu_seqlens, T, N, H, scale, o,
                        final_state, workspace, workspace_bytes, stream, Prologue());
}

kda_status kda_chunk_fwd_fused(const void *q, const void *k, const void *v, const float *g,
                               const void *b, int64_t b_stride, float qk_eps,
                               const float *initial_state, const int32_t *cu_seqlens, int64_t T,
                               int32_t N, int32_t H, float scale, void *o, float *final_state,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T > 0 && !b) return KDA_ERR_INVALID_ARGUMENT;
  if (qk_eps != qk_eps) return KDA_ERR_INVALID_ARGUMENT;  // NaN
  Prologue pro;
  pro.b = static_cast<const uint16_t *>(b);
  pro.b_stride = b_stride;
  pro.qk_eps = qk_eps >= 0.f ? qk_eps : -1.f;
  return chunk_fwd_impl(q, k, v, g, nullptr, initial_state, cu_seqlens, T, N, H, scale, o,
                        final_state, workspace, workspace_bytes, stream, pro);
}

// Workspace of the segmented forward: the plain workspace, then per chain
// the exit state of segment 0 and the maps (M, b) of segments 1 .. P-2.
static int64_t segmented_extra(int32_t N, int32_t H, int32_t segments) {
  const int64_t per_chain = 1 + 2 * (int64_t)(segments > 2 ? segments - 2 : 0);
  return (int64_t)N * H * per_chain * DK * DV * 4;
}

size_t kda_chunk_fwd_segmented_workspace_size(int64_t T, int32_t N, int32_t H, int32_t segments) {
  if (check_sizes(T, N, H) != KDA_OK || segments < 1 || segments > KDA_MAX_SEGMENTS) return 0;
  return (size_t)(align256(ws_layout(T, N, H).total) + segmented_extra(N, H, segments));
}

kda_status kda_chunk_fwd_segmented(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *initial_state,
                                   const int32_t *cu_seqlens, int64_t T, int32_t N, int32_t H,
                                   float scale, int32_t segments, void *o, float *final_state,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (segments < 1 || segments > KDA_MAX_SEGMENTS) return KDA_ERR_INVALID_ARGUMENT;
  kda_status st = check_forward_args(q, k, v, g, beta, initial_state, cu_seqlens, T, N, H, o,
                                     final_state, Prologue());
  if (st != KDA_OK) return st;
  Ws ws;
  if ((st = carve(workspace, workspace_bytes, T, N, H, ws)) != KDA_OK) return st;
  const int64_t base = align256(ws.L.total);
  const int64_t total = base + segmented_extra(N, H, segments);
  if ((int64_t)workspace_bytes < total) return KDA_ERR_WORKSPACE_TOO_SMALL;
  const int64_t tok = T * H * DK;
  const int64_t st_bytes = (int64_t)N * H * DK * DV * 4;
  if (forward_inputs(q, k, v, g, beta, initial_state, cu_seqlens, T, N, H, nullptr, 0)
          .hit(workspace, total) ||
      overlap(workspace, total, o, tok * 2) || overlap(workspace, total, final_state, st_bytes))
    return KDA_ERR_INVALID_ARGUMENT;
  if ((st = run_intra(q, k, v, g, beta, cu_seqlens, T, N, H, scale, ws, stream)) != KDA_OK)
    return st;
  if (segments == 1) return run_recurrence(initial_state, T, N, H, o, final_state, ws, stream);
  RecurArgs ra;
  ra.blocks = ws.blocks;
  ra.chunk_first = ws.chunk_first;
  ra.chunk_info = ws.chunk_info;
  ra.h0 = initial_state;
  ra.hT = final_state;
  ra.o = static_cast<uint16_t *>(o);
  ra.nc_max = ws.L.nc_max;
  ra.T = T;
  ra.N = N;
  ra.H = H;
  ra.segments = segments;
  float *extra = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + base);
  ra.xstate = extra;
  ra.maps = extra + (int64_t)N * H * DK * DV;
  ra.phase = 1;
  if (launch_recurrence(ra, stream) != hipSuccess) return KDA_ERR_HIP;
  ra.phase = 2;
  return hip_status(launch_recurrence(ra, stream));
}

kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *initial_state,
                                 const int32_t *cu_seqlens, int64_t T, int32_t N, int32_t H,
                                 float scale, void *o, float *final_state, hipStream_t stream) {
  kda_status st = check_sizes(T, N, H);
  if (st != KDA_OK) return st;
  const int64_t need = ws_layout(T, N, H).total;
  if (need > (int64_t)KDA_NOALLOC_WORKSPACE_BYTES) return KDA_ERR_WORKSPACE_TOO_SMALL;
  // host-side argument checks first: nothing touches the device before them
  if ((st = check_forward_args(q, k, v, g, beta, initial_state, cu_seqlens, T, N, H, o,
                               final_state, Prologue())) != KDA_OK)
    return st;
  hipError_t e = hipSuccess;
  void *ws = device_scratch(&e);
  if (!ws) return KDA_ERR_HIP;
  return chunk_fwd_impl(q, k, v, g, beta, initial_state, cu_seqlens, T, N, H, scale, o,
                        final_state, ws, KDA_NOALLOC_WORKSPACE_BYTES, stream, Prologue());
}

kda_status kda_decode_fwd(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                          int64_t T, int32_t N, int32_t H, float scale, void *o,
                          float *final_state, hipStream_t stream) {
  return decode_fwd_impl(q, k, v, g, beta, initial_state, cu_seqlens, T, N, H, scale, o,
                         final_state, stream, Prologue());
}

kda_status kda_decode_fwd_fused(const void *q, const void *k, const void *v, const float *g,
                                const void *b, int64_t b_stride, float qk_eps,
                                const float *initial_state, const int32_t *cu_seqlens, int64_t T,
                                int32_t N, int32_t H, float scale, void *o, float *final_state,
                                hipStream_t stream) {
  if (T > 0 && !b) return KDA_ERR_INVALID_ARGUMENT;
  if (qk_eps != qk_eps) return KDA_ERR_INVALID_ARGUMENT;  // NaN
  Prologue pro;
  pro.b = static_cast<const uint16_t *>(b);
  pro.b_stride = b_stride;
  pro.qk_eps = qk_eps >= 0.f ? qk_eps : -1.f;
  return decode_fwd_impl(q, k, v, g, nullptr, initial_state, cu_seqlens, T, N, H, scale, o,
                         final_state, stream, pro);
}

kda_status kda_decode_step_fused(const void *q, const void *k, const void *v, const float *g,
                                 const void *b, int64_t b_stride, float qk_eps,
                                 const float *initial_state, const int32_t *cu_seqlens, int64_t T,
                                 int32_t N, int32_t H, float scale, const void *gate,
                                 int64_t gate_stride, const float *norm_weight, float norm_eps,
                                 int32_t activation, void *o, void *y, float *final_state,
                                 hipStream_t stream) {
  if (T > 0 && (!b || !y)) return KDA_ERR_INVALID_ARGUMENT;
  if (qk_eps != qk_eps) return KDA_ERR_INVALID_ARGUMENT;  // NaN
  Prologue pro;
  pro.b = static_cast<const uint16_t *>(b);
  pro.b_stride = b_stride;
  pro.qk_eps = qk_eps >= 0.f ? qk_eps : -1.f;
  Epilogue epi;
  epi.y = T > 0 ? y : nullptr;
  epi.z = gate;
  epi.z_stride = gate_stride;
  epi.nw = norm_weight;
  epi.eps = norm_eps;
  epi.act = activation;
  return decode_fwd_impl(q, k, v, g, nullptr, initial_state, cu_seqlens, T, N, H, scale, o,
                         final_state, stream, pro, epi);
}

kda_status kda_validate_inputs(const float *g, const float *beta, const int32_t *cu_seqlens,
                               int64_t T, int32_t N, int32_t H, int32_t *flags,
                               hipStream_t stream) {
  kda_status st = check_sizes(T, N, H);
  if (st != KDA_OK) return st;
  if (!cu_seqlens || !flags || !aligned(cu_seqlens, 4) || !aligned(flags, 4))
    return KDA_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!g || !aligned(g, 16))) return KDA_ERR_INVALID_ARGUMENT;
  if (beta && !aligned(beta, 4)) return KDA_ERR_INVALID_ARGUMENT;
  const int64_t tok = T * H * DK;
  if (overlap(flags, 4, g, tok * 4) || overlap(flags, 4, beta, T * H * 4) ||
      overlap(flags, 4, cu_seqlens, ((int64_t)N + 1) * 4))
    return KDA_ERR_INVALID_ARGUMENT;
  ValidateArgs va;
  va.g = g;
  va.beta = T > 0 ? beta : nullptr;
  va.cu = cu_seqlens;
  va.flags = flags;
  va.T = T;
  va.N = N;
  va.H = H;
  return hip_status(launch_validate(va, stream));
}

kda_status kda_gated_rmsnorm(const void *x, int64_t x_stride, const void *gate,
                             int64_t gate_stride, const float *weight, float eps,
                             int32_t activation, int64_t T, int32_t H, void *y,
                             hipStream_t stream) {
  if (T < 0 || H < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (T > INT32_MAX || H > 65535) return KDA_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || eps == INFINITY) return KDA_ERR_INVALID_ARGUMENT;  // NaN, < 0, inf
  if (activation != KDA_ACT_SIGMOID && activation != KDA_ACT_SILU)
    return KDA_ERR_INVALID_ARGUMENT;
  if (T == 0) return KDA_OK;
  const int64_t row = (int64_t)H * DK;
  if (!x || !gate || !weight || !y) return KDA_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(gate, 16) || !aligned(weight, 16) || !aligned(y, 16))
    return KDA_ERR_INVALID_ARGUMENT;
  // 16-byte row segments: strides are whole multiples of 8 elements
  // strides up to 2^31 elements keep (T - 1) * stride (T < 2^31) inside int64
  if (x_stride < row || gate_stride < row || x_stride % 8 || gate_stride % 8 ||
      x_stride > ((int64_t)1 << 31) || gate_stride > ((int64_t)1 << 31))
    return KDA_ERR_INVALID_ARGUMENT;
  const int64_t ybytes = T * row * 2;
  const int64_t xbytes = ((T - 1) * x_stride + row) * 2;
  const int64_t zbytes = ((T - 1) * gate_stride + row) * 2;
  // y may be x itself (in place, contiguous x), and nothing else it reads
  const bool in_place = y == x && x_stride == row;
  if ((!in_place && overlap(y, ybytes, x, xbytes)) || overlap(y, ybytes, gate, zbytes) ||
      overlap(y, ybytes, weight, DK * 4))
    return KDA_ERR_INVALID_ARGUMENT;
  NormArgs na;
  na.x = static_cast<const uint16_t *>(x);
  na.z = static_cast<const uint16_t *>(gate);
  na.w = weight;
  na.y = static_cast<uint16_t *>(y);
  na.x_stride = x_stride;
  na.z_stride = gate_stride;
  na.T = T;
  na.H = H;
  na.eps = eps;
  na.act = activation;
  return hip_status(launch_gated_rmsnorm(na, stream));
}

kda_status kda_chunk_recurrence(const float *initial_state, int64_t T, int32_t N, int32_t H,
                                void *o, float *final_state, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  kda_status st = check_sizes(T, N, H);
  if (st != KDA_OK) return st;
  if ((st = check_outputs(initial_state, T, N, H, o, final_state)) != KDA_OK) return st;
  Ws ws;
  if ((st = carve(workspace, workspace_bytes, T, N, H, ws)) != KDA_OK) return st;
  if (overlap(workspace, ws.L.total, o, T * H * DK * 2) ||
      overlap(workspace, ws.L.total, final_state, (int64_t)N * H * DK * DV * 4) ||
      overlap(workspace, ws.L.total, initial_state, (int64_t)N * H * DK * DV * 4))
    return KDA_ERR_INVALID_ARGUMENT;
  return run_recurrence(initial_state, T, N, H, o, final_state, ws, stream);
}

}  // extern "C"
