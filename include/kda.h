/*
 * kda.h -- C ABI of libkda, the Kimi Delta Attention (KDA) core for AMD
 * Instinct MI355X (gfx950).
 *
 * What it computes (per sequence and head, S in R^{d_k x d_v}, fp32):
 *
 *   alpha_t = exp(-5 * sigmoid(exp(A_h) * z_t))   per channel     (1)
 *   beta_t  = sigmoid(b_t)                                           (2)
 *   S_t     = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 *             + beta_t k_t v_t^T                                     (3)
 *   o_t     = S_t^T q_t                                              (4)
 *
 * Sources (web pages):
 *   [LA-KDA]   "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制",
 *              blog-3d3.pages.dev/posts/150
 *   [K3-ATTN]  "Kimi K3 注意力机制深度解析：KDA、Gated MLA 与 AttnRes 的混合架构",
 *              forceinjection.github.io/09_inference_system/vllm/module_analysis/kimi_k3_attention.html
 *   [K3-NOTES] "Kimi K3", llm.rainlin.net/llm-inference/kimi-k3
 * (1) is the lower-bounded sigmoid decay of [LA-KDA §5.4]; (2) the write
 * strength of [LA-KDA §5.3]; (3) the recurrence of [LA-KDA §5.2] and
 * [K3-ATTN §2.1]; (4) the read-out of [LA-KDA §5.5].  The prefill entry point
 * uses the chunked form of [LA-KDA §7] with 16-token sub-tiles ([LA-KDA §8]);
 * the decode entry point uses the three-step DPLR update of [K3-ATTN §2.2].
 * Both take the same raw logits and produce the same state semantics, as the
 * chunked and recurrent call sites on [K3-NOTES] ("KDA Prefill 与 Decode
 * Kernel") require.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller, contiguous in
 *     the stated row-major layout and 16-byte aligned (the entry points refuse
 *     a misaligned row tensor -- q, k, v, o, y, gate logits, states, taps --
 *     with KDA_ERR_INVALID_ARG).  The library never allocates, frees or keeps
 *     them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued asynchronously on it; nothing synchronises the host.
 *     No entry point allocates memory, synchronises or clears memory with a
 *     memset: each call is a fixed sequence of kernel launches, so it may be
 *     captured into a HIP graph and replayed (with the same pointers).
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-OK status means nothing was enqueued, except KDA_ERR_HIP, which
 *     reports a failed launch.  No exception crosses the ABI.
 *   - The library holds no mutable global state: calls on different streams
 *     may run concurrently if their buffers do not overlap.  The one
 *     exception is kda_chunk_fwd_noalloc, whose scratch is a per-GPU array
 *     inside the library (see its declaration).
 *   - No query scale is applied: o = S^T q exactly (no formula on the pages
 *     carries one); a caller wanting 1/sqrt(d_k) scales q first.  q and k are
 *     used as given (the pages normalise them upstream, [LA-KDA §5.3]).
 *   - NaN or Inf inputs propagate; they are not detected.
 */
#ifndef LIBKDA_KDA_H
#define LIBKDA_KDA_H

#include <stddef.h>

#if defined(__GNUC__) || defined(__clang__)
#define KDA_API __attribute__((visibility("default")))
#else
#define KDA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,   /* NULL or misaligned pointer, negative or       */
                               /* inconsistent size                             */
    KDA_ERR_UNSUPPORTED = 2,   /* (d_k, d_v, chunk, dtype) not compiled in      */
    KDA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required     */
    KDA_ERR_HIP = 4,           /* a kernel launch failed                         */
    KDA_ERR_SCRATCH = 5        /* kda_chunk_fwd_noalloc: the call needs more     */
                               /* scratch than KDA_NOALLOC_SCRATCH_BYTES        */
} kda_status_t;

/* Element type of q, k, v and o.  Gate logits, beta logits, A and states are
 * always fp32. */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;

/* Human-readable name of a status code (static string, never NULL). */
KDA_API const char* kda_status_string(kda_status_t s);

/*
 * Supported shapes.
 *   kda_chunk_fwd:      d_k == d_v in {16, 32, 64, 128}, chunk in {16, 64},
 *                       dtype fp32 or bf16.  bf16 with d_k = d_v = 128 and
 *                       chunk = 64 runs the MFMA path; every other supported
 *                       combination runs an fp32-arithmetic path.
 *   kda_recurrent_step: d_k == d_v in {16, 32, 64, 128}, fp32 or bf16.
 * Returns 1 when the combination is compiled in, 0 otherwise.
 *
 * Size limits (KDA_ERR_INVALID_ARG beyond them, checked on the host; a
 * dispatch counts its work-items in 32 bits, and the intra-chunk kernels
 * address a chunk's rows with 32-bit offsets):
 *   prefill:  B * T < 2^31;  C_cap * H * 1024 < 2^32 with C_cap = B * ceil(T /
 *             chunk) + N (about 4.2M chunk-heads);  N * H * 2048 < 2^32;
 *             H * max(d_k, d_v) * chunk < 2^32 (H < 524,288 at d = 128,
 *             chunk 64);  on the fp32 layer path also B * T * H * 64 < 2^32.
 *   recurrent calls:  N * H * 256 < 2^32.
 * At d = 128 each limit lies beyond what 288 GB of HBM can hold for the
 * tensors involved, except the head count of very short batches.
 */
KDA_API int kda_chunk_fwd_supported(int dk, int dv, int chunk, kda_dtype_t dtype);
KDA_API int kda_recurrent_step_supported(int dk, int dv, kda_dtype_t dtype);

/*
 * Workspace size in bytes for kda_chunk_fwd with these sizes (N = number of
 * sequences: N == B without cu_seqlens, the length of cu_seqlens minus one
 * with it).  The bound covers both layouts.  Returns 0 for unsupported or
 * invalid sizes.  The workspace is scratch device memory owned by the caller;
 * its contents need no initialisation and are meaningless afterwards, except
 * through kda_chunk_fwd_debug.
 */
KDA_API size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                     int chunk, kda_dtype_t dtype);

/*
 * Prefill: run the recurrence (1)-(4) over whole sequences, chunk by chunk.
 *
 *   q, k         [B, T, H, dk]  dtype
 *   v            [B, T, H, dv]  dtype
 *   g_logits     [B, T, H, dk]  fp32  raw per-channel gate logits z
 *   beta_logits  [B, T, H]      fp32  raw write-strength logits b
 *   A            [H]            fp32  per-head A_h of (1)
 *   h0           [N, H, dk, dv] fp32  initial states, or NULL for zeros
 *   cu_seqlens   [N+1]          int32 device offsets, or NULL
 *   o            [B, T, H, dv]  dtype output
 *   hT           [N, H, dk, dv] fp32  final states, or NULL to skip; may be
 *                                     the same pointer as h0 (in place)
 *
 * Without cu_seqlens the batch holds N = B sequences of T tokens each.  With
 * cu_seqlens, B must be 1, the T tokens are N packed sequences and sequence s
 * is tokens [cu_seqlens[s], cu_seqlens[s+1]).  The offsets stay on the device
 * (the host never reads them); they must satisfy 0 = cu[0] <= cu[1] <= ... <=
 * cu[N] = T.  Offsets that break this are clamped into [0, T] so that no
 * access leaves the buffers, and the results are then unspecified.
 * The state restarts at every sequence from that sequence's h0.  An empty
 * sequence (or T = 0) yields hT = h0 (zeros without h0).  Chunks restart at
 * every sequence start; a sequence whose length is not a multiple of `chunk`
 * ends in a shorter chunk.
 *
 * Workspace: at least kda_chunk_fwd_workspace_bytes(...) bytes, 256-byte
 * aligned.
 */
KDA_API kda_status_t kda_chunk_fwd(const void* q, const void* k, const void* v,
                           const float* g_logits, const float* beta_logits,
                           const float* A, const float* h0, const int* cu_seqlens,
                           int B, int T, int H, int dk, int dv, int N, int chunk,
                           kda_dtype_t dtype, void* o, float* hT,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments, layouts, supported shapes, results and errors, without the
 * workspace.  Its scratch memory is a device array inside the library,
 * KDA_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, held from the
 * library's first use on that GPU until the process ends; the call allocates
 * and frees nothing.
 * Limit: a call whose kda_chunk_fwd_workspace_bytes exceeds
 * KDA_NOALLOC_SCRATCH_BYTES returns KDA_ERR_SCRATCH and enqueues nothing
 * (on the MFMA path about 70,000 token-heads fit: e.g. 4,096 tokens x 16
 * heads; use kda_chunk_fwd with a workspace beyond that).
 * Sharing: every call on one GPU uses that GPU's one array.  Calls that can
 * overlap on one GPU (on different streams, or from different host threads)
 * race on it and give undefined results: serialise them.  Nothing in the
 * array needs to start at zero; each call overwrites what it reads.
 * `stream` must belong to the current device (hipGetDevice) of the calling
 * thread; the first call on a device looks up that device's array once
 * (KDA_ERR_HIP if the lookup fails).
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
KDA_API kda_status_t kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                           const float* g_logits, const float* beta_logits,
                                           const float* A, const float* h0,
                                           const int* cu_seqlens, int B, int T, int H, int dk,
                                           int dv, int N, int chunk, kda_dtype_t dtype, void* o,
                                           float* hT, void* stream);

/*
 * Diagnostic variant of kda_chunk_fwd: identical results, plus per-chunk
 * intermediates of the chunked form ([LA-KDA §7]) for stage-level checks.
 * With Cn = the workspace's chunk capacity (returned through *chunk_capacity
 * by kda_chunk_fwd_debug_floats) and c the chunk length:
 *   dbg_intra  [Cn, H, c*dk + 3*c*c] fp32, per chunk and head in this order:
 *              G [c, dk] (in-chunk cumulative log-decay, inclusive),
 *              A_kk [c, c] (beta-scaled, strictly lower), A_qk [c, c] (lower),
 *              T [c, c] = (I + A_kk)^{-1} Diag(beta);  may be NULL
 *   dbg_state  [Cn, H, dk, dv] fp32, the state entering each chunk; may be NULL
 * Chunks are numbered sequence by sequence in token order.
 */
KDA_API size_t kda_chunk_fwd_debug_floats(int B, int T, int H, int dk, int dv, int N,
                                  int chunk, size_t* dbg_state_floats,
                                  int* chunk_capacity);
KDA_API kda_status_t kda_chunk_fwd_debug(const void* q, const void* k, const void* v,
                                 const float* g_logits, const float* beta_logits,
                                 const float* A, const float* h0,
                                 const int* cu_seqlens, int B, int T, int H,
                                 int dk, int dv, int N, int chunk,
                                 kda_dtype_t dtype, void* o, float* hT,
                                 void* workspace, size_t workspace_bytes,
                                 float* dbg_intra, float* dbg_state, void* stream);

/*
 * Diagnostic variant of kda_chunk_fwd that also records caller-created HIP
 * events on `stream` around its kernels, so a caller can time each stage on
 * the stream the kernels run on: events[0] before the chunk bookkeeping,
 * events[1] after it (the two are back to back for equal-length batches on
 * the MFMA path, whose tables the intra-chunk kernel writes), events[2]
 * after the intra-chunk kernel (gate, A_kk,
 * A_qk, triangular inverse, W, U), events[3] after the state-chain kernel
 * (inter-chunk state and outputs).  `events` points to n_events >= 4
 * hipEvent_t handles (as void*).  With n_events >= 6 on the MFMA path,
 * events[4] is recorded after the segment-transition kernel and events[5]
 * after the segment-composition kernel (both between events[2] and
 * events[3]).  Results are identical to kda_chunk_fwd.
 */
KDA_API kda_status_t kda_chunk_fwd_timed(const void* q, const void* k, const void* v,
                                         const float* g_logits, const float* beta_logits,
                                         const float* A, const float* h0,
                                         const int* cu_seqlens, int B, int T, int H,
                                         int dk, int dv, int N, int chunk,
                                         kda_dtype_t dtype, void* o, float* hT,
                                         void* workspace, size_t workspace_bytes,
                                         void* const* events, int n_events, void* stream);

/*
 * Decode: one token per sequence, state updated in place.
 *
 *   q, k         [N, H, dk]       dtype
 *   v            [N, H, dv]       dtype
 *   g_logits     [N, H, dk]       fp32
 *   beta_logits  [N, H]           fp32
 *   A            [H]              fp32
 *   state        [N, H, dk, dv]   fp32, read and overwritten
 *   o            [N, H, dv]       dtype
 *
 * Each (sequence, head) state is read once and written once: with
 * S' = Diag(alpha) S, the step forms p = S'^T k and r = S'^T q in one pass,
 * then u = beta (v - p), S = S' + k u^T and o = r + (q . k) u, which equals
 * S^T q after the update ([K3-ATTN §2.2], three steps with no d_k x d_k matrix).
 * N = 0 is a no-op.  No workspace.
 */
KDA_API kda_status_t kda_recurrent_step(const void* q, const void* k, const void* v,
                                const float* g_logits, const float* beta_logits,
                                const float* A, float* state, void* o,
                                int N, int H, int dk, int dv, kda_dtype_t dtype,
                                void* stream);

/*
 * Family modes: the other rows of the family table of [LA-KDA §4], run by the
 * same kernels.
 *   KDA_MODE_KDA       (3) as above.
 *   KDA_MODE_GLA       gated linear attention: the erase step is off,
 *                      S_t = Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T.  The
 *                      table's row has no write strength; it is beta = 1
 *                      here (a large beta logit).
 *   KDA_MODE_DELTANET  DeltaNet: alpha = 1,
 *                      S_t = (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T;
 *                      g_logits and A are not read and may be NULL.
 * With both switches of the table off (GLA at alpha = 1) the update is plain
 * linear attention ([LA-KDA §3]); pass very negative gate logits to GLA.
 */
typedef enum { KDA_MODE_KDA = 0, KDA_MODE_GLA = 1, KDA_MODE_DELTANET = 2 } kda_mode_t;

/*
 * kda_chunk_fwd in a family mode: same arguments, layouts, supported shapes,
 * workspace and errors, plus `mode` (KDA_ERR_INVALID_ARG outside the enum).
 * KDA_MODE_KDA gives exactly kda_chunk_fwd.
 */
KDA_API kda_status_t kda_chunk_fwd_mode(const void* q, const void* k, const void* v,
                                        const float* g_logits, const float* beta_logits,
                                        const float* A, const float* h0,
                                        const int* cu_seqlens, int B, int T, int H, int dk,
                                        int dv, int N, int chunk, kda_dtype_t dtype,
                                        kda_mode_t mode, void* o, float* hT, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * kda_recurrent_step in a family mode: same arguments and errors, plus `mode`.
 * KDA_MODE_GLA writes u = beta v without forming S'^T k.
 */
KDA_API kda_status_t kda_recurrent_step_mode(const void* q, const void* k, const void* v,
                                             const float* g_logits, const float* beta_logits,
                                             const float* A, float* state, void* o, int N,
                                             int H, int dk, int dv, kda_dtype_t dtype,
                                             kda_mode_t mode, void* stream);

/*
 * General diagonal-plus-low-rank (DPLR) update.  [K3-ATTN §2.2] writes the
 * KDA step as three steps (decay, a rank-1 correction, the write) and credits
 * binding the diagonal and low-rank terms to one key with halving the chunk
 * matrices.  These entry points lift the binding: the rank-1 correction has
 * its own pair (a_t, b_t) and the write its own key k_t,
 *   S'  = Diag(alpha_t) S_{t-1}          alpha_t as in (1)
 *   S'' = S' + a_t (b_t^T S')
 *   S_t = S'' + k_t v_t^T,   o_t = S_t^T q_t.
 * KDA is the case a = -beta k, b = k with write key beta k.  There is no
 * write-strength logit (it is folded into a and k).  The chunked form needs
 * four C x C matrices (A_ba, A_bk, A_qa, A_qk) where KDA needs two.
 *
 *   q, k, a, b   [B, T, H, dk]  dtype
 *   v            [B, T, H, dv]  dtype
 *   g_logits     [B, T, H, dk]  fp32     A [H] fp32
 *   h0, hT, cu_seqlens, o, the batch layout, empty sequences, chunking and
 *   the workspace rules: as kda_chunk_fwd, with the workspace sized by
 *   kda_dplr_chunk_fwd_workspace_bytes.
 * Supported shapes: as kda_chunk_fwd.  Results are unspecified (not an
 * error) when I - A_ba is ill-conditioned, i.e. when the low-rank steps
 * amplify the state strongly.
 */
KDA_API size_t kda_dplr_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                                  int chunk, kda_dtype_t dtype);
KDA_API kda_status_t kda_dplr_chunk_fwd(const void* q, const void* k, const void* v,
                                        const void* a, const void* b, const float* g_logits,
                                        const float* A, const float* h0,
                                        const int* cu_seqlens, int B, int T, int H, int dk,
                                        int dv, int N, int chunk, kda_dtype_t dtype, void* o,
                                        float* hT, void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * kda_dplr_chunk_fwd that also records caller-created HIP events on `stream`
 * around its stages, as kda_chunk_fwd_timed does (events[0..3]: before the
 * chunk bookkeeping, after it, after the intra-chunk kernel, after the
 * chain; with n_events >= 6 on the MFMA path events[4], events[5] after the
 * segment transition and composition).  Results are identical to
 * kda_dplr_chunk_fwd.
 */
KDA_API kda_status_t kda_dplr_chunk_fwd_timed(const void* q, const void* k, const void* v,
                                              const void* a, const void* b,
                                              const float* g_logits, const float* A,
                                              const float* h0, const int* cu_seqlens, int B,
                                              int T, int H, int dk, int dv, int N, int chunk,
                                              kda_dtype_t dtype, void* o, float* hT,
                                              void* workspace, size_t workspace_bytes,
                                              void* const* events, int n_events, void* stream);

/*
 * One DPLR token per sequence, state updated in place (layouts as
 * kda_recurrent_step, plus a, b [N, H, dk] dtype).  One pass over
 * S' = Diag(alpha) S forms x = S'^T b and r = S'^T q; then
 * S = S' + a x^T + k v^T and o = r + (q . a) x + (q . k) v.
 */
KDA_API kda_status_t kda_dplr_recurrent_step(const void* q, const void* k, const void* v,
                                             const void* a, const void* b,
                                             const float* g_logits, const float* A,
                                             float* state, void* o, int N, int H, int dk,
                                             int dv, kda_dtype_t dtype, void* stream);

/*
 * The KDA layer between its projections: the core with the steps either side
 * of it that act on one token-head row.
 *
 *   before  q, k = L2Norm(Swish(ShortConv(q_in | k_in))),
 *           v = Swish(ShortConv(v_in))                     [LA-KDA §5.3], [K3-ATTN §2.3]
 *   core    the recurrence (1)-(4) of kda_chunk_fwd / kda_recurrent_step
 *   after   y = Sigmoid(gate) * RMSNorm(o) per head        [LA-KDA §5.5], [K3-ATTN §2.3]
 *
 * ShortConv is a depthwise causal convolution with four taps per channel
 * (kernel size 4), taps ordered oldest first, no bias; the three inputs
 * before a sequence's first token come from the carried convolution state
 * (zeros without one) [K3-NOTES].  Swish(x) = x * sigmoid(x).  L2Norm(x) =
 * x / sqrt(sum x^2 + l2_eps) over the head's d channels; RMSNorm(o) =
 * o / sqrt(mean o^2 + rms_eps) * norm_w, with one weight per channel shared
 * by the heads.  Readings of the pages where they are silent: no convolution
 * bias, the epsilons under the square roots, the shared RMSNorm weight.
 *
 * Prefill (d_k = d_v = d; same supported set as kda_chunk_fwd):
 *   q_in, k_in, v_in  [B, T, H, d]      dtype  projections before the convolution
 *   conv_w            [3, H, d, 4]      fp32   taps of q, k, v
 *   conv_state0       [N, 3, 3, H, d]   dtype  per sequence, for q, k, v, the
 *                                              inputs at t-3, t-2, t-1 before
 *                                              its first token; NULL for zeros
 *   conv_stateT       [N, 3, 3, H, d]   dtype  the last three inputs of each
 *                                              sequence (reaching into
 *                                              conv_state0 for sequences shorter
 *                                              than three); NULL to skip; may be
 *                                              conv_state0 (in place)
 *   g_logits, beta_logits, A, h0, cu_seqlens, hT  as for kda_chunk_fwd
 *   gate              [B, T, H, d]      dtype  output-gate logits W_g x
 *   norm_w            [d]               fp32
 *   y                 [B, T, H, d]      dtype  Sigmoid(gate) * RMSNorm(o), before W_o
 * The workspace (kda_layer_fwd_workspace_bytes) holds the core's workspace
 * and the intermediate q, k, v and o.  Outputs of tokens outside every
 * sequence are unspecified.  Errors as for kda_chunk_fwd; negative or
 * non-finite epsilons are KDA_ERR_INVALID_ARG.
 */
KDA_API size_t kda_layer_fwd_workspace_bytes(int B, int T, int H, int d, int N, int chunk,
                                     kda_dtype_t dtype);
KDA_API kda_status_t kda_layer_fwd(const void* q_in, const void* k_in, const void* v_in,
                           const float* conv_w, const void* conv_state0, void* conv_stateT,
                           const float* g_logits, const float* beta_logits, const float* A,
                           const float* h0, const int* cu_seqlens, const void* gate,
                           const float* norm_w, float l2_eps, float rms_eps, int B, int T, int H,
                           int d, int N, int chunk, kda_dtype_t dtype, void* y, float* hT,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode of the same layer, one token per sequence, in one launch
 * ([K3-ATTN §6.3]: convolution, recurrent update and gated RMSNorm fused):
 *   q_in, k_in, v_in, gate  [N, H, d]          dtype
 *   conv_w                  [3, H, d, 4]       fp32
 *   conv_state              [N, 3, 3, H, d]    dtype, read and shifted in place
 *   g_logits [N, H, d], beta_logits [N, H], A [H], state [N, H, d, d]  as for
 *   kda_recurrent_step (state in place)
 *   y                       [N, H, d]          dtype
 * Same supported set as kda_recurrent_step.  N = 0 is a no-op.
 */
KDA_API kda_status_t kda_layer_step(const void* q_in, const void* k_in, const void* v_in,
                            const float* conv_w, void* conv_state, const float* g_logits,
                            const float* beta_logits, const float* A, float* state,
                            const void* gate, const float* norm_w, float l2_eps, float rms_eps,
                            void* y, int N, int H, int d, kda_dtype_t dtype, void* stream);

/*
 * Verify pass over a stored draft window ([K3-ATTN §6.2], ReplaySSM): from the
 * checkpoint `state`, the outputs of all W window tokens of every sequence,
 * exactly as W successive kda_recurrent_step calls would produce them (same
 * step, same operation order: the outputs are bit-identical), while `state`
 * itself is only read.  Once the number of accepted tokens is known,
 * kda_recurrent_fold commits that prefix from the same window.
 *
 *   q, k, g_logits  [N, W, H, dk]   dtype / dtype / fp32
 *   v, o            [N, W, H, dv]   dtype
 *   beta_logits     [N, W, H]       fp32
 *   A               [H]             fp32
 *   state           [N, H, dk, dv]  fp32, read only
 *
 * Each (sequence, head) state is read once for the whole window.  N = 0 or
 * W = 0 is a no-op.  Supported shapes: as kda_recurrent_step.
 */
KDA_API kda_status_t kda_recurrent_verify(const void* q, const void* k, const void* v,
                                          const float* g_logits, const float* beta_logits,
                                          const float* A, const float* state, void* o, int N,
                                          int W, int H, int dk, int dv, kda_dtype_t dtype,
                                          void* stream);

/*
 * Replay fold for speculative decoding ([K3-ATTN §6.2], ReplaySSM): instead
 * of a state snapshot per draft token, the caller keeps each window token's
 * inputs; once the number of accepted tokens is known, this call advances
 * every (sequence, head) state over the first n_accept[s] tokens of its
 * window.  Each token is processed by the same step as kda_recurrent_step, so
 * the result is bit-identical to n_accept[s] kda_recurrent_step calls on the
 * same state with the same k, v, g_logits, beta_logits and A (q only shapes
 * the output of those calls, never the state).  The state is read and written
 * once for the whole window.
 *
 *   k            [N, W, H, dk]    dtype  window keys
 *   v            [N, W, H, dv]    dtype  window values
 *   g_logits     [N, W, H, dk]    fp32   window gate logits
 *   beta_logits  [N, W, H]        fp32   window write-strength logits
 *   A            [H]              fp32
 *   n_accept     [N]              int32, on the device: tokens to replay per
 *                                 sequence; values outside [0, W] are clamped
 *   state        [N, H, dk, dv]   fp32, read and overwritten (untouched where
 *                                 n_accept[s] <= 0)
 *
 * Same supported set as kda_recurrent_step.  N = 0 or W = 0 is a no-op.  No
 * workspace.
 */
KDA_API kda_status_t kda_recurrent_fold(const void* k, const void* v, const float* g_logits,
                                const float* beta_logits, const float* A,
                                const int* n_accept, float* state, int N, int W, int H,
                                int dk, int dv, kda_dtype_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBKDA_KDA_H */
