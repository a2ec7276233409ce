/*
 * kda.h - C ABI of the MI355X (gfx950) Kimi Delta Attention hot path.
 *
 * KDA is a linear-attention recurrence whose d_k x d_v state S is edited by
 * the delta rule and forgotten channel by channel:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,            alpha_t = exp(g_t)
 *
 * Sources for the operation (pages, by title and section):
 *  - "From GPT-2 to Kimi K3" (molayo1419.me): section "DeltaNet: memory you
 *    can edit" (read the stored value, write back only the difference);
 *    section "Gated DeltaNet: now it can forget" (decay first, then write;
 *    alpha in [0,1]); section "KDA: Kimi's secret sauce" (alpha becomes a
 *    vector, one forget rate per channel); section on the parallelisation
 *    trick (chunks of C tokens; masked attention inside a chunk, the state and
 *    one matmul between chunks; a Householder-type reparametrisation gives all
 *    deltas of a chunk at once; C = 64 or 128 works best).
 *  - "Kimi Linear architecture" (ttj.ttj.kr): section on linear attention
 *    (chunkwise for training and prefill, a per-token state update for
 *    generation); section "KDA: a memo that erases and rewrites" (per-channel
 *    gate; diagonal-plus-low-rank transition whose low-rank term is tied to
 *    the key).
 *  - "Kimi Delta Attention ... 1M context" (molayo1419.me): paragraph on the
 *    specialised DPLR transition.
 * The write strength beta is not on the pages; it enters as in the transition
 * written above (beta = 1 gives the pages' plain delta rule).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers, row-major and densely packed.
 *    Alignment: every pointer to its element size; in kda_chunk_fwd also
 *    q, k, v and a per-channel g to two elements; in kda_recurrent_step S
 *    to 16 bytes; the workspace to 256 bytes.  The caller allocates and owns every buffer, including
 *    the workspace, and keeps it alive until the work on `stream` completes.
 *    The library allocates nothing and keeps no per-call state (the static
 *    scratch of kda_chunk_fwd_noalloc aside, which the library holds).
 *  - Calls are asynchronous on `stream` (0 = the null stream) and never
 *    synchronise the host.
 *  - Token tensors: q, k, g are [T, H, d_k]; v, o are [T, H, d_v]; beta is
 *    [T, H].  With KDA_GATE_PER_HEAD, g is [T, H] (one log-gate per token and
 *    head, broadcast over the key channels: the Gated DeltaNet special case).
 *  - q, k, v, g, beta and o share the element type `dt`; state tensors are
 *    always fp32, [N, H, d_k, d_v], row c = key channel c.
 *  - No 1/sqrt(d) scale is applied and q, k are used as given (callers
 *    L2-normalise them).  g must be finite and <= 0; other values are
 *    computed without checks and the result is unspecified.  The chunked
 *    path is exact (up to rounding) while the decay accumulated over any
 *    eight consecutive tokens of a sequence stays above e^-80 (e.g. every
 *    g >= -10); stronger decay stays finite but loses accuracy.
 *  - Supported: d_k, d_v in {64, 128}; chunk size C = 64.
 *  - Errors are returned, never thrown.  Argument checks run on the host
 *    before anything is launched: KDA_ERR_INVALID_ARG (null pointer,
 *    misalignment, negative or inconsistent sizes), KDA_ERR_UNSUPPORTED
 *    (d_k or d_v outside {64,128}, unknown dtype or gate mode, or 2^23 or
 *    more (chunk, head) pairs: (ceil(T_total / 64) + N) * H),
 *    KDA_ERR_WORKSPACE (workspace null or smaller than required).  A failed
 *    launch returns KDA_ERR_HIP.  Input values are not inspected.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,
    KDA_ERR_UNSUPPORTED = 2,
    KDA_ERR_WORKSPACE = 3,
    KDA_ERR_HIP = 4,
    KDA_ERR_BAD_SEQLENS = 5,
    KDA_ERR_TIMEOUT = 6,
    KDA_ERR_TOO_LARGE = 7
} kda_status;

typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

typedef enum { KDA_GATE_PER_CHANNEL = 0, KDA_GATE_PER_HEAD = 1 } kda_gate;

/* Human-readable name of a status code (static string, never NULL). */
const char *kda_status_string(kda_status status);

/* Library version, (major << 16) | minor. */
int32_t kda_version(void);

/*
 * Bytes of device workspace kda_chunk_fwd needs for these sizes (0 if the
 * sizes are invalid or unsupported).  T_total counts all packed tokens and N
 * the sequences.  The requirement depends only on the arguments.
 */
size_t kda_chunk_fwd_workspace_size(int64_t T_total, int32_t N, int32_t H,
                                    int32_t d_k, int32_t d_v, kda_dtype dt,
                                    kda_gate gk);

/*
 * Chunkwise-parallel KDA forward (prefill) over a packed batch.
 *
 * Operation: for every sequence n and head h, starting from S0[n,h] (zeros
 * if S0 is NULL), run the recurrence above over the sequence's tokens in
 * order; write o_t for every token and the final state into S_T[n,h].  It is
 * evaluated in chunks of C = 64 tokens that restart at every sequence start
 * (the last chunk of a sequence may be shorter): inside a chunk all deltas
 * come from one unit-lower-triangular solve (the WY/UT form of the product of
 * rank-one corrections), the state crosses chunk boundaries once per chunk.
 *
 *   q, k, v, g, beta  inputs as described above; T_total tokens
 *   S0                fp32 [N, H, d_k, d_v] or NULL (= zeros)
 *   cu_seqlens        int32 device array [N + 1] of sequence offsets
 *                     (cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N] =
 *                     T_total; empty sequences allowed: S_T = S0), or NULL:
 *                     N sequences of T_total / N tokens each (T_total % N
 *                     must be 0).  Device offsets are validated on the
 *                     device; if they are invalid no output is written and
 *                     kda_chunk_fwd_check reports KDA_ERR_BAD_SEQLENS.
 *   N, T_total, H     sequences (>= 1), packed tokens (>= 0), heads (>= 1)
 *   o                 [T_total, H, d_v], element type dt (output)
 *   S_T               fp32 [N, H, d_k, d_v] or NULL; may alias S0 exactly
 *   workspace         device scratch of >= kda_chunk_fwd_workspace_size()
 *                     bytes, 256-byte aligned; its contents on entry do not
 *                     matter and are clobbered
 *   stream            HIP stream the kernels are enqueued on
 *
 * Numerics: bf16 inputs are widened exactly; matrix products run on bf16
 * MFMA with fp32 accumulation (fp32 MFMA for KDA_F32 inputs); the state is
 * carried in fp32 and o is rounded once (round-to-nearest-even for bf16).
 * Two calls with identical arguments give bit-identical results.
 */
kda_status kda_chunk_fwd(const void *q, const void *k, const void *v,
                         const void *g, const void *beta, const float *S0,
                         const int32_t *cu_seqlens, int32_t N, int64_t T_total,
                         int32_t H, int32_t d_k, int32_t d_v, kda_dtype dt,
                         kda_gate gk, void *o, float *S_T, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd from raw projections: the pre-path transforms of
 * kda_prepare_inputs (q, k scaled to unit L2 norm over d_k per token and
 * head, an all-zero row staying zero; g <- -softplus(g); beta <-
 * sigmoid(beta)) are applied inside the intra-chunk kernel as the inputs are
 * read, in fp32, each result rounded once to dt: the values
 * kda_prepare_inputs would write, up to the summation order of the norms.
 * The separate pre-path pass and its round trip through HBM fall away.  "Kimi
 * Linear architecture" (ttj.ttj.kr), section "KDA: a memo that erases and
 * rewrites": one forget rate in (0, 1) per channel; "From GPT-2 to Kimi K3",
 * section "Gated DeltaNet: now it can forget".  v is used as given.
 * Arguments, layouts, workspace, alignment and status codes as for
 * kda_chunk_fwd (q_raw, k_raw, g_raw, beta_raw in the places of q, k, g,
 * beta; a raw gate may take any finite value).
 */
kda_status kda_chunk_fwd_raw(const void *q_raw, const void *k_raw,
                             const void *v, const void *g_raw,
                             const void *beta_raw, const float *S0,
                             const int32_t *cu_seqlens, int32_t N,
                             int64_t T_total, int32_t H, int32_t d_k,
                             int32_t d_v, kda_dtype dt, kda_gate gk, void *o,
                             float *S_T, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Same as kda_chunk_fwd, and also records the four caller-created HIP events
 * events[0..3] on `stream`: before the chunk-map kernel, before the
 * intra-chunk kernel, before the chunk-walk kernel and after it, so that
 * hipEventElapsedTime gives each kernel's duration.  For profiling; `events`
 * must hold four valid hipEvent_t (KDA_ERR_INVALID_ARG if NULL).  If
 * T_total == 0 the intra-chunk kernel is skipped and events[1] and
 * events[2] coincide.
 */
typedef struct ihipEvent_t *hipEvent_t;
kda_status kda_chunk_fwd_instrumented(const void *q, const void *k, const void *v,
                                      const void *g, const void *beta, const float *S0,
                                      const int32_t *cu_seqlens, int32_t N, int64_t T_total,
                                      int32_t H, int32_t d_k, int32_t d_v, kda_dtype dt,
                                      kda_gate gk, void *o, float *S_T, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream,
                                      hipEvent_t *events);

/*
 * kda_chunk_fwd with chunks of C = 128 tokens instead of 64.  "From GPT-2 to
 * Kimi K3" (molayo1419.me), section "The parallelisation trick": chunks of 64
 * or 128 tokens work best.  The chunk algebra is the same with C = 128: one
 * 128 x 128 unit-lower-triangular solve per chunk, half as many steps of the
 * state across chunk boundaries, each twice as long.
 *
 *   Arguments, layouts, numerics and status codes as for kda_chunk_fwd, with
 *   the workspace sized by kda_chunk_fwd_c128_workspace_size (the status of
 *   a call is read back with kda_chunk_fwd_check, as for kda_chunk_fwd).
 *   Supported: KDA_BF16 with d_k, d_v in {64, 128}; KDA_F32 with
 *   d_k = d_v = 64 only (the fp32 operand tiles of 128 rows at d = 128 do
 *   not fit the 160 KB of LDS of a compute unit); KDA_ERR_UNSUPPORTED
 *   otherwise.  Results agree with kda_chunk_fwd to rounding; they are not
 *   bit-identical to it (the sums are grouped differently).
 *   events: NULL, or four caller-created events recorded as for
 *   kda_chunk_fwd_instrumented.
 */
size_t kda_chunk_fwd_c128_workspace_size(int64_t T_total, int32_t N, int32_t H,
                                         int32_t d_k, int32_t d_v, kda_dtype dt,
                                         kda_gate gk);
kda_status kda_chunk_fwd_c128(const void *q, const void *k, const void *v,
                              const void *g, const void *beta, const float *S0,
                              const int32_t *cu_seqlens, int32_t N,
                              int64_t T_total, int32_t H, int32_t d_k,
                              int32_t d_v, kda_dtype dt, kda_gate gk, void *o,
                              float *S_T, void *workspace,
                              size_t workspace_bytes, hipStream_t stream,
                              hipEvent_t *events);

/*
 * kda_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing and frees nothing.
 * Its scratch is a static device array of KDA_NOALLOC_SCRATCH_BYTES inside
 * the library, one copy on every GPU the library runs on, held until the
 * process ends; its address on a device is looked up once, on the first call
 * with that device current.
 *
 *   Arguments, layouts, numerics and results as for kda_chunk_fwd (bit-
 *   identical to it for the same arguments); the caller still allocates the
 *   inputs and the outputs o and S_T.
 *   Limit: problems whose kda_chunk_fwd_workspace_size exceeds
 *   KDA_NOALLOC_SCRATCH_BYTES (128 MiB: about 1,800 (chunk, head) pairs at
 *   d_k = d_v = 128 in bf16, e.g. T = 3,500 tokens over 32 heads) return
 *   KDA_ERR_TOO_LARGE before anything is launched.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents: calls that overlap on one GPU (on different streams, or
 *   from different host threads without ordering) race and give unspecified
 *   results.  Calls on one stream are ordered and safe.  Device-side
 *   rejection of cu_seqlens leaves o and S_T unwritten, as for kda_chunk_fwd;
 *   there is no status query for it.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                 const void *g, const void *beta, const float *S0,
                                 const int32_t *cu_seqlens, int32_t N,
                                 int64_t T_total, int32_t H, int32_t d_k,
                                 int32_t d_v, kda_dtype dt, kda_gate gk, void *o,
                                 float *S_T, hipStream_t stream);

/*
 * Wait for `stream` and report how the last kda_chunk_fwd that used this
 * workspace went on the device: KDA_OK; KDA_ERR_BAD_SEQLENS (the offsets were
 * not 0 = c_0 <= ... <= c_N = T_total; nothing was written); KDA_ERR_TIMEOUT
 * (a bounded wait between the cooperating waves of a workgroup gave up, which
 * only a fault could cause; outputs unspecified); KDA_ERR_HIP if
 * synchronisation fails.  Optional; it synchronises the host.
 */
kda_status kda_chunk_fwd_check(const void *workspace, hipStream_t stream);

/*
 * One recurrent (decode) step for N independent sequences, in place.
 *
 * Operation, per (n, h) with a = exp(g): r = S^T (a*k), s = S^T (a*q),
 * u = beta (v - r), o = s + (q.k) u, S <- Diag(a) S + k u^T; equal to one
 * token of the recurrence above.  S is read once and written once.
 *
 *   q, k, g   [N, H, d_k] (g is [N, H] with KDA_GATE_PER_HEAD), type dt
 *   v         [N, H, d_v], type dt;  beta [N, H], type dt
 *   S         fp32 [N, H, d_k, d_v], updated in place
 *   o         [N, H, d_v], type dt (output)
 */
kda_status kda_recurrent_step(const void *q, const void *k, const void *v,
                              const void *g, const void *beta, float *S,
                              int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                              kda_dtype dt, kda_gate gk, void *o,
                              hipStream_t stream);

/*
 * The steps just before the recurrence, from raw projections, in one pass
 * over HBM:
 *     q <- q / ||q||,  k <- k / ||k||   (per token and head, over d_k; an
 *                                        all-zero row stays zero)
 *     g <- -softplus(g) = -log(1 + e^g) (so alpha = exp(g) = 1 / (1 + e^x)
 *                                        lies in (0, 1))
 *     beta <- sigmoid(beta)
 * "Kimi Linear architecture" (ttj.ttj.kr), section "KDA: a memo that erases
 * and rewrites": one forget rate in (0, 1) per channel; "From GPT-2 to Kimi
 * K3", section "Gated DeltaNet: now it can forget": alpha in [0, 1].  The
 * pages print no parametrisation; this is the plainest one that gives those
 * ranges.  Outputs are ready for kda_chunk_fwd / kda_recurrent_step.
 *
 *   q_raw, k_raw, q, k   [T_total, H, d_k], type dt
 *   g_raw, g             [T_total, H, d_k] ([T_total, H] with KDA_GATE_PER_HEAD)
 *   beta_raw, beta       [T_total, H]
 * Outputs may alias their inputs exactly (in place).  Arithmetic in fp32,
 * outputs rounded once to dt.  d_k in {64, 128}.  q_raw, k_raw, q, k and a
 * per-channel g_raw, g must be 16-byte aligned (KDA_ERR_INVALID_ARG
 * otherwise); T_total * H must stay below 2^32 (KDA_ERR_UNSUPPORTED).
 */
kda_status kda_prepare_inputs(const void *q_raw, const void *k_raw,
                              const void *g_raw, const void *beta_raw,
                              int64_t T_total, int32_t H, int32_t d_k,
                              kda_dtype dt, kda_gate gk, void *q, void *k,
                              void *g, void *beta, hipStream_t stream);

/*
 * kda_recurrent_step with the pre-path transforms of kda_prepare_inputs
 * fused into the step: q_raw, k_raw are normalised, g_raw and beta_raw
 * activated, inside the kernel (in fp32, without rounding the transformed
 * values).  Arguments and layouts as for kda_recurrent_step.
 */
kda_status kda_recurrent_step_raw(const void *q_raw, const void *k_raw,
                                  const void *v, const void *g_raw,
                                  const void *beta_raw, float *S, int32_t N,
                                  int32_t H, int32_t d_k, int32_t d_v,
                                  kda_dtype dt, kda_gate gk, void *o,
                                  hipStream_t stream);

/*
 * Bytes of device workspace kda_chunk_bwd needs to process all H heads at
 * once (0 if the sizes are invalid or unsupported).  About 570 KB per (chunk,
 * head) at d_k = d_v = 128 for KDA_BF16 (593 KB for KDA_F32): the chunk's
 * intermediates are kept, in fp32 except the operands of the two sequential
 * passes over the chunks, which are kept in type dt (for KDA_BF16 in the
 * matrix cores' fragment order, two of them in two layouts).  The value for
 * H = 1 is the least kda_chunk_bwd accepts.
 */
size_t kda_chunk_bwd_workspace_size(int64_t T_total, int32_t N, int32_t H,
                                    int32_t d_k, int32_t d_v, kda_dtype dt,
                                    kda_gate gk);

/*
 * Chunked KDA backward pass over a packed batch: the vector-Jacobian product
 * of the map (q, k, v, g, beta, S0) -> (o, S_T) computed by kda_chunk_fwd,
 * with cotangents dO and dS_T.  That is, for
 *     L = sum_t <dO_t, o_t> + sum_{n,h} <dS_T[n,h], S_T[n,h]>,
 * it writes dq = dL/dq, dk, dv, dg, dbeta and dS0 = dL/dS0.  The chunked form
 * is what the pages present as the training path ("From GPT-2 to Kimi K3",
 * section on the parallelisation trick; "Kimi Linear architecture", section
 * on linear attention: chunkwise for training and prefill).  The chunk
 * algebra of the forward pass is differentiated as written: a reverse walk
 * over the chunks carries the state cotangent, and every chunk then forms its
 * inputs' gradients, including those through the triangular solve and the
 * gate's prefix sums, on its own.
 *
 *   q, k, v, g, beta, S0, cu_seqlens, N, T_total, H, d_k, d_v, dt, gk
 *                     exactly as passed to kda_chunk_fwd (the forward outputs
 *                     are not needed: the pass recomputes what it uses)
 *   dO                [T_total, H, d_v], element type dt
 *   dS_T              fp32 [N, H, d_k, d_v] or NULL (= zeros)
 *   dq, dk, dg        [T_total, H, d_k] (dg is [T_total, H] with
 *                     KDA_GATE_PER_HEAD: the sum over channels), type dt
 *   dv                [T_total, H, d_v], type dt;  dbeta [T_total, H], type dt
 *   dS0               fp32 [N, H, d_k, d_v] or NULL (not written); an empty
 *                     sequence gives dS0 = dS_T
 *   workspace         256-byte aligned, clobbered; at least
 *                     kda_chunk_bwd_workspace_size(..., H = 1, ...) bytes.
 *                     With less than the size for all H heads, the heads are
 *                     processed in the largest groups that fit, one group
 *                     after another on `stream` (same results, more time).
 *                     kda_chunk_fwd_check accepts it too and reports rejected
 *                     cu_seqlens the same way
 *
 * Alignment: every pointer to its element size.  Errors as for
 * kda_chunk_fwd.  Numerics: all arithmetic in fp32, gradients rounded once
 * to dt; the operands of the two sequential passes over the chunks (QG, Kd,
 * W and the intra-chunk P) are rounded to dt as well.  For KDA_BF16 those two
 * passes, and the per-chunk products with the saved states (dW, dQG, dKd, dP),
 * multiply on the bf16 matrix cores with fp32 accumulation, every fp32 operand
 * entering as a sum of two bf16 parts (about 16 significant bits).  Domain:
 * the forward's.  Every decayed operand is referred to the
 * middle row of its own 16-token tile and the decay between tiles is rebuilt
 * from factors <= 1, so the gradients are exact (up to rounding) while the
 * decay accumulated over any eight consecutive tokens stays above e^-80 (e.g.
 * every g >= -10); stronger decay stays finite but loses accuracy.
 */
kda_status kda_chunk_bwd(const void *q, const void *k, const void *v,
                         const void *g, const void *beta, const float *S0,
                         const int32_t *cu_seqlens, int32_t N, int64_t T_total,
                         int32_t H, int32_t d_k, int32_t d_v, kda_dtype dt,
                         kda_gate gk, const void *dO, const float *dS_T,
                         void *dq, void *dk, void *dv, void *dg, void *dbeta,
                         float *dS0, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
