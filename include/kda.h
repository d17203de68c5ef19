/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA chunked-prefill forward library.
 *
 * The operation (KDA TPU report, sections 1-2 and 6.2; MI355X serving post,
 * section 1.1): the Kimi Delta Attention gated delta rule with per-channel
 * decay, for every packed sequence s and head h,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * with a [128 (key), 128 (value)] fp32 state per (sequence, head), computed
 * in 64-token chunks (16-token subblocks inside each chunk).  The gate must
 * satisfy -5 <= g <= 0 (the bounded gate, lower_bound = -5): the chunk math
 * relies on it to keep bf16 strip factors within range.
 *
 * Conventions for every entry point below:
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *     row-major, and 16-byte aligned (beta and cu_seqlens: 4-byte aligned).
 *   - The library allocates nothing, never synchronises the device, and only
 *     enqueues work on `stream` (0 = the null stream).
 *   - Host-checkable argument errors are reported before anything is
 *     launched; a launch failure is reported as KDA_ERR_HIP.
 *   - Device-content contracts are the caller's: cu_seqlens starts at 0,
 *     never decreases and ends at T; g lies in [-5, 0].  Malformed
 *     cu_seqlens never make a kernel read or write out of bounds (the chunk
 *     table clamps it into [0, T]) but the results are then unspecified.
 *   - No global mutable state: concurrent calls on different streams with
 *     different workspaces are safe.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, misalignment */
    KDA_ERR_UNSUPPORTED = 2,        /* sizes beyond what the kernels index      */
    KDA_ERR_WORKSPACE_TOO_SMALL = 3,
    KDA_ERR_HIP = 4                 /* a kernel launch failed                   */
} kda_status;

/* Fixed problem geometry of this library. */
#define KDA_HEAD_DIM 128   /* K = V = 128                                   */
#define KDA_CHUNK 64       /* BT: tokens per chunk                           */
#define KDA_SUBBLOCK 16    /* SB: tokens per subblock                        */

/* Human-readable name of a status code (static storage, never NULL). */
const char *kda_status_string(kda_status s);

/*
 * Bytes of workspace kda_chunk_fwd / kda_chunk_intra need for T packed
 * tokens, N sequences and H heads.  The bound uses the worst-case chunk
 * count floor((T + 63 N) / 64), so it depends only on sizes, never on the
 * contents of cu_seqlens.  Returns 0 for invalid sizes (T < 0, N < 1,
 * H < 1).
 */
size_t kda_chunk_fwd_workspace_size(int64_t T, int32_t N, int32_t H);

/*
 * Chunked KDA prefill forward (KDA TPU report section 6: gate cumsum and
 * intra-chunk in one kernel, chunk recurrence and output in another; section
 * 6.5: a flat grid over the chunks that exist).
 *
 *   q, k          bf16 [T, H, 128]; k is expected L2-normalised per token
 *   v             bf16 [T, H, 128]
 *   g             fp32 [T, H, 128]   log-decay per key channel, in [-5, 0]
 *   beta          fp32 [T, H]        write strength
 *   initial_state fp32 [N, H, 128, 128] (key-major: S[key][value]) or NULL,
 *                 which means zeros
 *   cu_seqlens    int32 [N + 1] device array of packed sequence offsets;
 *                 zero-length sequences are allowed
 *   T, N, H       tokens, sequences (N >= 1), heads (1 <= H <= 65535);
 *                 T <= 2^31 - 1 and T * H * 128 must fit in int64
 *   scale         multiplies S^T q (1/sqrt(128) for the usual scaling)
 *   o             bf16 [T, H, 128] output, rounded to nearest even; must not
 *                 overlap any input (q, k, v, g, beta, cu_seqlens,
 *                 initial_state)
 *   final_state   fp32 [N, H, 128, 128] output or NULL (not written); may
 *                 alias initial_state exactly (in-place update) and must
 *                 not overlap any other input
 *   workspace     256-byte aligned device scratch of workspace_bytes >=
 *                 kda_chunk_fwd_workspace_size(T, N, H); its contents on
 *                 entry do not matter and on return are unspecified; it is
 *                 written while the inputs are still being read, so it must
 *                 not overlap o, final_state or any input
 *   Overlaps that break these rules return KDA_ERR_INVALID_ARGUMENT before
 *   anything is launched.
 *   stream        HIP stream the three kernels are enqueued on, in order
 *
 * A sequence's outputs depend only on its own tokens and initial state:
 * they are bitwise identical whichever offset and neighbours it is packed
 * with.  Results are deterministic run to run.
 */
kda_status kda_chunk_fwd(const void *q, const void *k, const void *v,
                         const float *g, const float *beta,
                         const float *initial_state, const int32_t *cu_seqlens,
                         int64_t T, int32_t N, int32_t H, float scale,
                         void *o, float *final_state,
                         void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Chunk-parallel state passing (derived from the chunk recurrence of the KDA
 * TPU report, section 6.2: each chunk maps the state affinely, h' = A_c h +
 * B_c with A_c = Diag(gamma) - kg^T W and B_c = kg^T U, so a run of chunks
 * composes into h' = M h + b).  The same operation as kda_chunk_fwd, for
 * few, long chains: each (sequence, head) chain of n chunks is cut into
 * `segments` runs of ceil(n / segments) chunks.  A first recurrence pass
 * runs segment 0 from the initial state and, in parallel, every middle
 * segment twice, from the identity with U = 0 (giving M) and from zero
 * (giving b); a second pass runs every later segment from its entry state,
 * h_p = M_{p-1} h_{p-1} + b_{p-1} (products on bf16 MFMAs with hi + lo
 * operands).  Three chain-lengths of recurrence work are done instead of
 * one, in about two segment-lengths of latency.
 *
 *   segments   1 .. KDA_MAX_SEGMENTS; 1 is kda_chunk_fwd itself.
 *   workspace  >= kda_chunk_fwd_segmented_workspace_size(T, N, H, segments)
 *              bytes, 256-byte aligned.
 * Everything else as kda_chunk_fwd.  Results differ from kda_chunk_fwd's by
 * rounding only.  A sequence's results depend on its own tokens, its
 * initial state and `segments`, not on its neighbours or offset.
 */
#define KDA_MAX_SEGMENTS 64
size_t kda_chunk_fwd_segmented_workspace_size(int64_t T, int32_t N, int32_t H,
                                              int32_t segments);
kda_status kda_chunk_fwd_segmented(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta,
                                   const float *initial_state, const int32_t *cu_seqlens,
                                   int64_t T, int32_t N, int32_t H, float scale,
                                   int32_t segments, void *o, float *final_state,
                                   void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * kda_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The workspace is a file-scope device
 * array of KDA_NOALLOC_WORKSPACE_BYTES inside the library, one per GPU,
 * allocated when the library's code is loaded on that GPU and held until the
 * process ends; its address is looked up on the first call on each device.
 * The call itself allocates nothing.
 *
 * Arguments, results and errors are those of kda_chunk_fwd.  Sizes whose
 * workspace (kda_chunk_fwd_workspace_size) exceeds the array return
 * KDA_ERR_WORKSPACE_TOO_SMALL before any launch; the headline shape of 4 x
 * 2048 tokens at 16 heads needs 144.3 MiB of it.  KDA_ERR_HIP if the array's
 * address cannot be obtained on the current device.
 *
 * Every call on a GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (other streams, other threads) race and must not be issued;
 * calls in stream order on one stream are safe.  The array keeps the last
 * call's contents, which no call depends on.
 */
#define KDA_NOALLOC_WORKSPACE_BYTES ((size_t)160 << 20)
kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                 const float *g, const float *beta,
                                 const float *initial_state, const int32_t *cu_seqlens,
                                 int64_t T, int32_t N, int32_t H, float scale,
                                 void *o, float *final_state, hipStream_t stream);

/*
 * Token-serial KDA forward for decode and speculative verification (MI355X
 * Kimi K3 post, sections 1.2-1.3: one fused kernel applies each sequence's
 * new tokens, 1 for a decode step or a window of a few for verification,
 * to its recurrent state, which stays on chip).  For every sequence s and
 * head h, and each token t of the sequence in order:
 *     S <- Diag(exp g_t) S;  S <- S + beta_t k_t (v_t - S^T k_t)^T;
 *     o_t = scale S^T q_t.
 * This is the same function kda_chunk_fwd computes, evaluated token by token
 * in fp32 (the two differ only by rounding).  Any sequence length is
 * accepted, but the cost grows with the longest sequence, so it is meant
 * for a handful of tokens per sequence; prefill belongs to kda_chunk_fwd.
 *
 * Arguments, layouts, aliasing and errors are those of kda_chunk_fwd
 * (initial_state NULL means zeros; final_state NULL is not written and may
 * alias initial_state exactly; o and final_state must not overlap any other
 * input, cu_seqlens included, since every workgroup reads cu_seqlens while
 * others write).  final_state NULL with T > 0 is the verification pass of
 * speculative decoding: the window's outputs are formed and no state is
 * kept; the accepted prefix is committed afterwards by a second call over
 * the accepted tokens (cu_seqlens of the accepted lengths) from the same
 * initial state.  It needs no workspace and enqueues one
 * kernel on `stream`.  KDA_ERR_UNSUPPORTED if N * H * 2 exceeds 2^31 - 1.
 */
kda_status kda_decode_fwd(const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          const float *initial_state, const int32_t *cu_seqlens,
                          int64_t T, int32_t N, int32_t H, float scale,
                          void *o, float *final_state, hipStream_t stream);

/*
 * The same two operations with the steps before them fused in ("Kimi K3
 * Prefill PP16" notes, third throughput section, KDA switch table: beta is
 * computed from a strided bf16 slice of the projection output, copy and
 * sigmoid in one kernel; KDA TPU report, section 8: q and k are
 * L2-normalised per token, as the model does):
 *
 *   b         bf16 beta logits; beta[t, h] = sigmoid(b[t * b_stride + h])
 *             in fp32.  b points at the slice's first column (e.g. into a
 *             [T, b_stride] row-major projection output); H <= b_stride <=
 *             2^24; 2-byte aligned.  It replaces the fp32 beta argument.
 *   qk_eps    >= 0: q and k are used as x / sqrt(sum_i x_i^2 + qk_eps) over
 *             the 128 channels of each (token, head), computed in fp32 from
 *             the bf16 inputs (an all-zero row stays zero); < 0: q and k are
 *             used as given.  NaN is KDA_ERR_INVALID_ARGUMENT.
 *
 * All other arguments, and the results, are those of kda_chunk_fwd and
 * kda_decode_fwd.  b must not overlap o.
 */
kda_status kda_chunk_fwd_fused(const void *q, const void *k, const void *v,
                               const float *g, const void *b, int64_t b_stride,
                               float qk_eps, const float *initial_state,
                               const int32_t *cu_seqlens, int64_t T, int32_t N,
                               int32_t H, float scale, void *o, float *final_state,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);
kda_status kda_decode_fwd_fused(const void *q, const void *k, const void *v,
                                const float *g, const void *b, int64_t b_stride,
                                float qk_eps, const float *initial_state,
                                const int32_t *cu_seqlens, int64_t T, int32_t N,
                                int32_t H, float scale, void *o, float *final_state,
                                hipStream_t stream);

/*
 * The gated RMSNorm that follows the operation in the model ("Kimi K3
 * Prefill PP16" notes, third throughput section, KDA switch table: the KDA
 * output tail reads its strided input directly; RMSNorm after Zhang and
 * Sennrich, cited by the KDA TPU report).  Per (token t, head h) row of 128
 * channels:
 *
 *   y[t, h, :] = weight * x / sqrt(mean(x^2) + eps) * act(gate)
 *
 * with act(z) = 1 / (1 + exp(-z)) (KDA_ACT_SIGMOID) or z / (1 + exp(-z))
 * (KDA_ACT_SILU), in fp32, y rounded to bf16 (nearest even).  An all-zero
 * row with eps = 0 stays zero.
 *
 *   x, gate   bf16; row (t, h) at element t * stride + h * 128, with
 *             H * 128 <= x_stride, gate_stride <= 2^31, multiples of 8
 *             (16-byte row segments), e.g. column slices of a row-major
 *             [T, stride] tensor.  16-byte aligned.
 *   weight    fp32 [128], 16-byte aligned.
 *   eps       >= 0 and finite.
 *   y         bf16 [T, H, 128] contiguous, 16-byte aligned.  y == x (with
 *             x_stride = H * 128) updates in place; otherwise y must not
 *             overlap x, gate or weight.
 *
 * T = 0 is a no-op.  Invalid arguments return KDA_ERR_INVALID_ARGUMENT
 * before any launch; T > 2^31 - 1 or H > 65535 return KDA_ERR_UNSUPPORTED.
 */
enum { KDA_ACT_SIGMOID = 0, KDA_ACT_SILU = 1 };
kda_status kda_gated_rmsnorm(const void *x, int64_t x_stride, const void *gate,
                             int64_t gate_stride, const float *weight, float eps,
                             int32_t activation, int64_t T, int32_t H, void *y,
                             hipStream_t stream);

/*
 * A whole decode step of the layer in one kernel: kda_decode_fwd_fused (the
 * prologue: beta from logits, q/k L2 norm) with kda_gated_rmsnorm applied to
 * each output row before it leaves the chip (MI355X Kimi K3 serving post,
 * section 1.3: the decode step fused into one kernel, output normalisation
 * included).  The norm uses o's fp32 row (before o's bf16 rounding).
 *
 *   q ... scale           as in kda_decode_fwd_fused (b required when T > 0).
 *   gate, gate_stride     bf16 gate rows as in kda_gated_rmsnorm (2-byte
 *                         aligned; H * 128 <= gate_stride <= 2^31).
 *   norm_weight           fp32 [128], 4-byte aligned.
 *   norm_eps, activation  as in kda_gated_rmsnorm.
 *   o                     bf16 [T, H, 128], written as by kda_decode_fwd.
 *   y                     bf16 [T, H, 128] (required when T > 0), the
 *                         normalised output; it must not overlap any other
 *                         argument.
 *   final_state           as in kda_decode_fwd.
 *
 * One workgroup per (sequence, head) holds all 128 value columns, where
 * kda_decode_fwd uses two.  KDA_ERR_UNSUPPORTED if N * H * 2 exceeds
 * 2^31 - 1.
 */
kda_status kda_decode_step_fused(const void *q, const void *k, const void *v,
                                 const float *g, const void *b, int64_t b_stride,
                                 float qk_eps, const float *initial_state,
                                 const int32_t *cu_seqlens, int64_t T, int32_t N,
                                 int32_t H, float scale, const void *gate,
                                 int64_t gate_stride, const float *norm_weight,
                                 float norm_eps, int32_t activation, void *o, void *y,
                                 float *final_state, hipStream_t stream);

/*
 * Opt-in check of the contracts on device contents that the entry points
 * above trust (they never read out of bounds on any input, but compute
 * garbage on a broken contract): cu_seqlens monotone with cu[0] = 0 and
 * cu[N] = T; every g inside [-5, 0] (the KDA TPU report's lower bound,
 * section 4); every beta inside [0, 1] (beta may be NULL: not checked).
 * NaN fails both range checks.  Enqueued on `stream`: a kernel clears
 * *flags, a second ORs in KDA_BAD_CU_SEQLENS, KDA_BAD_G and KDA_BAD_BETA
 * for what it finds; read *flags after the stream has run.  flags: device
 * int32 [1], 4-byte aligned, not overlapping the inputs.  g: 16-byte
 * aligned.  Not part of any forward call; it reads g once more.
 */
enum { KDA_BAD_CU_SEQLENS = 1, KDA_BAD_G = 2, KDA_BAD_BETA = 4 };
kda_status kda_validate_inputs(const float *g, const float *beta,
                               const int32_t *cu_seqlens, int64_t T, int32_t N,
                               int32_t H, int32_t *flags, hipStream_t stream);

/*
 * Step-level entry points.  They run the steps of kda_chunk_fwd on their
 * own so that each step can be checked and timed separately; kda_chunk_fwd
 * does not call them.
 */

/*
 * Chunk table (KDA TPU report, section 6.5 flat packed-chunk grid; section
 * 6.4 worked example).  Writes, for cu_seqlens clamped into [0, T]:
 *   chunk_first  int32 [N + 1]: index of each sequence's first chunk, with
 *                chunk_first[N] = number of chunks NC = sum ceil(L_s / 64);
 *   chunk_info   int32 [NCmax, 4] with NCmax = floor((T + 63 N) / 64): for
 *                chunk c < NC (token_start, length, sequence, local_index);
 *                rows c >= NC are (0, 0, -1, -1);
 *   flags        int32 [1]: 0, or 1 if cu_seqlens had to be clamped.
 * Returns KDA_ERR_INVALID_ARGUMENT for null pointers or bad sizes.
 */
kda_status kda_chunk_table(const int32_t *cu_seqlens, int64_t T, int32_t N,
                           int32_t *chunk_first, int32_t *chunk_info,
                           int32_t *flags, hipStream_t stream);

/*
 * Chunk-local gate cumsum (KDA TPU report section 6.1): G[t, h, :] is the
 * inclusive sum of g over the tokens of t's chunk up to and including t,
 * restarting at every chunk and sequence start.  fp32, same layout as g.
 * Uses `workspace` (>= kda_chunk_fwd_workspace_size(T, N, H) bytes) for the
 * chunk table.
 */
kda_status kda_gate_cumsum(const float *g, const int32_t *cu_seqlens,
                           int64_t T, int32_t N, int32_t H, float *G,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Chunk table + intra-chunk kernel only: leaves the per-(head, chunk)
 * intermediates of the fused recurrence in `workspace` (where: see
 * kda_workspace_layout).  Same arguments as kda_chunk_fwd.
 */
kda_status kda_chunk_intra(const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           const int32_t *cu_seqlens, int64_t T, int32_t N,
                           int32_t H, float scale, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Chunk recurrence + output only (KDA TPU report section 6.2: the state
 * stays on chip across a sequence's chunks and the output is formed in the
 * same pass): runs the second half of kda_chunk_fwd on a workspace that
 * kda_chunk_intra has just filled for the same T, N, H and inputs, on the
 * same stream.  kda_chunk_intra followed by kda_chunk_recurrence computes
 * exactly what kda_chunk_fwd computes.  Arguments as in kda_chunk_fwd; the
 * workspace must not overlap o or either state buffer.  A workspace that
 * kda_chunk_intra did not fill gives unspecified results, never an
 * out-of-bounds access.
 */
kda_status kda_chunk_recurrence(const float *initial_state, int64_t T, int32_t N, int32_t H,
                                void *o, float *final_state, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Where things live inside the workspace, for the step-level tests.
 * kda_workspace_layout fills out[0..4] = byte offsets of (flags,
 * chunk_first, chunk_info, first intermediate block) and the block size
 * in bytes; the block of (head h, chunk c) starts at
 * out[3] + (h * NCmax + c) * out[4].  Returns KDA_ERR_INVALID_ARGUMENT for
 * bad sizes.
 */
kda_status kda_workspace_layout(int64_t T, int32_t N, int32_t H, int64_t out[5]);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
