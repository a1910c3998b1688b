/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library (libkda.so).
 *
 * The operation is the chunked forward pass of KDA as the "Kernel API" table of the
 * FlashKDA README ("MoonshotAI/FlashKDA" repository page) states it (plus, in kda_bwd,
 * its gradients):
 *
 *   fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
 *       initial_state=None, final_state=None, cu_seqlens=None)
 *
 * with the in-kernel gate activation, q/k l2 normalisation and beta sigmoid that the
 * README section "Using FlashKDA as an FLA backend" switches on (use_gate_in_kernel,
 * use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel, safe_gate) and the V-major state
 * layout it selects (transpose_state_layout).  Per (sequence, head) chain, per token:
 *   q^ = q/sqrt(|q|^2+1e-6), k^ = k/sqrt(|k|^2+1e-6), beta = sigmoid(beta_logit),
 *   a_c = lower_bound * sigmoid(exp(A_log[h]) * (g_c + dt_bias[h,c])),
 *   S <- S Diag(exp(a)),  S <- S + beta (v - S k^) k^T,  out = scale * S q^.
 * The library evaluates this in 16-token chunks (FlashKDA article index: "processes
 * 16-token chunks"; "Neumann-series expansion" for the intra-chunk inverse).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers unless the name ends in _host.
 *   - The caller owns every buffer; the library allocates no device memory.  Scratch
 *     space comes from the caller's workspace (size from kda_fwd_workspace_size), except
 *     for kda_fwd_noalloc, which uses a static device array of the library.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs
 *     asynchronously; no entry point synchronises the host except kda_fwd_device_status.
 *   - Arguments are fully validated on the host before anything is launched; on any
 *     error nothing is launched and an error status is returned.  Nothing throws.
 *   - No global mutable state besides kda_fwd_noalloc's scratch and its per-device
 *     address; the other entry points are safe to call from several host threads on
 *     different streams with different workspaces.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128 /* K = V = 128 is the only supported head size (Kernel API table) */
#define KDA_CHUNK 16     /* tokens per chunk */

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* A_log or dt_bias is NULL (in-pass gate), or a token tensor is NULL while T > 0 */
    KDA_ERR_SHAPE = 2,       /* B < 1, T < 0, H < 1, N inconsistent or >= 2^29, or cu_seqlens with B != 1 */
    KDA_ERR_HEAD_DIM = 3,    /* K or V is not 128 */
    KDA_ERR_DTYPE = 4,       /* state dtype unknown, or initial/final state dtypes differ */
    KDA_ERR_LOWER_BOUND = 5, /* lower_bound not finite or outside [-5, 0] */
    KDA_ERR_SCALE = 6,       /* scale not finite */
    KDA_ERR_ALIGN = 7,       /* a pointer misses its alignment (see kda_fwd) */
    KDA_ERR_WORKSPACE = 8,   /* workspace NULL or smaller than kda_fwd_workspace_size */
    KDA_ERR_CU_SEQLENS = 9,  /* cu_seqlens_host given and cu[0] != 0, decreasing, or cu[N] != T */
    KDA_ERR_HIP = 10,        /* a HIP launch or query failed */
    KDA_ERR_ALIAS = 11,      /* out overlaps an input, or final_state overlaps a non-state input */
    KDA_ERR_FLAGS = 12,      /* kda_fwd_ex: unknown bits in the activation switch mask */
    KDA_ERR_SCRATCH = 13     /* kda_fwd_noalloc: the call needs more than KDA_NOALLOC_SCRATCH_BYTES */
} kda_status;

typedef enum kda_state_dtype {
    KDA_STATE_NONE = 0, /* pointer is NULL: no initial state (zeros) / final state not written */
    KDA_STATE_BF16 = 1,
    KDA_STATE_FP32 = 2
} kda_state_dtype;

/*
 * kda_fwd -- chunked KDA forward pass (Kernel API table of the FlashKDA README).
 *
 *   q, k, g   bf16 [B, T, H, 128], contiguous, 16-byte aligned.  Query, key, gate before
 *             activation.
 *   v         bf16 [B, T, H, 128], contiguous, 16-byte aligned.
 *   beta      bf16 [B, T, H], contiguous, 2-byte aligned.  Beta logits (sigmoid applied here).
 *   scale     output scaling factor, finite.
 *   out       bf16 [B, T, H, 128], contiguous, 16-byte aligned; fully overwritten (every
 *             token of every sequence).  Must not overlap any input.
 *   A_log     fp32 [H], 4-byte aligned.   dt_bias  fp32 [H, 128], 16-byte aligned.
 *   lower_bound  gate lower bound in [-5, 0] (the table's stated range); the per-token
 *             log-decay lies in (lower_bound, 0].
 *   initial_state  NULL (zeros) or [N, H, 128(V), 128(K)] of initial_state_dtype, 16-byte aligned.
 *   final_state    NULL (not written) or [N, H, 128(V), 128(K)] of final_state_dtype,
 *             16-byte aligned.  May be the same buffer as initial_state (in-place state carry).
 *             bf16 states are widened on load and rounded (nearest-even) once on store.
 *   initial_state_dtype / final_state_dtype  KDA_STATE_NONE exactly when the pointer is NULL;
 *             when both states are given the two dtypes must be equal (KDA_ERR_DTYPE).
 *   cu_seqlens  NULL, or device int64 [N+1] cumulative sequence lengths (8-byte aligned);
 *             then B must be 1, T is the total length and sequence i is tokens
 *             [cu[i], cu[i+1]).  Without it each of the B batch rows is one sequence (N = B;
 *             pass N = B or N = 0).
 *   cu_seqlens_host  optional host copy of cu_seqlens.  When given, its content is checked
 *             synchronously (KDA_ERR_CU_SEQLENS).  Without it the device checks the content;
 *             an invalid cu_seqlens then turns every sequence into an empty one (out is not
 *             written, final_state = initial_state or zeros) and sets the device status word
 *             that kda_fwd_device_status reads.
 *   B, T, H, N  sizes as above.  K, V must both be 128.
 *   workspace, workspace_bytes  device scratch, 256-byte aligned, at least
 *             kda_fwd_workspace_size(B, T, H, N, cu_seqlens != NULL) bytes.  It must not be
 *             used by another call until this one has finished on the stream.
 *   stream    hipStream_t (NULL = default stream).
 * Returns KDA_OK once the work is enqueued, or the first validation error found.
 */
kda_status kda_fwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                   float scale, void *out, const float *A_log, const float *dt_bias,
                   float lower_bound, const void *initial_state, kda_state_dtype initial_state_dtype,
                   void *final_state, kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                   const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H, int64_t N,
                   int64_t K, int64_t V, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Activation switches for kda_fwd_ex, after the use_gate_in_kernel, use_qk_l2norm_in_kernel
 * and use_beta_sigmoid_in_kernel flags the README section "Using FlashKDA as an FLA backend"
 * passes to chunk_kda (the pages name them and set all three; kda_fwd is the all-set case).
 * A switch that is off means that input arrives already activated:
 *   KDA_GATE_IN_KERNEL off:   g holds the per-token, per-channel natural-log decay a itself
 *                             (bf16 [B, T, H, 128]); the pass uses min(max(a, lower_bound), 0),
 *                             the range the in-pass gate produces.  A_log and dt_bias are
 *                             not read and may be NULL.
 *   KDA_QK_L2NORM_IN_KERNEL off: q and k are used as given (no l2 normalisation).
 *   KDA_BETA_SIGMOID_IN_KERNEL off: beta is the write strength itself (no sigmoid).
 */
#define KDA_GATE_IN_KERNEL 1u
#define KDA_QK_L2NORM_IN_KERNEL 2u
#define KDA_BETA_SIGMOID_IN_KERNEL 4u
#define KDA_ALL_IN_KERNEL 7u

/*
 * kda_fwd_ex -- kda_fwd with the activation switch mask `flags` (KDA_*_IN_KERNEL bits).
 * Same arguments, layouts, ownership and errors as kda_fwd, plus KDA_ERR_FLAGS for bits
 * outside KDA_ALL_IN_KERNEL.  With KDA_GATE_IN_KERNEL clear, A_log and dt_bias may be NULL
 * (they are then not checked for alignment either); lower_bound is still checked and
 * bounds the pre-activated log-decay.  kda_fwd(...) is kda_fwd_ex(..., KDA_ALL_IN_KERNEL).
 */
kda_status kda_fwd_ex(const void *q, const void *k, const void *v, const void *g, const void *beta,
                      float scale, void *out, const float *A_log, const float *dt_bias,
                      float lower_bound, const void *initial_state, kda_state_dtype initial_state_dtype,
                      void *final_state, kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                      const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H, int64_t N,
                      int64_t K, int64_t V, void *workspace, size_t workspace_bytes, void *stream,
                      uint32_t flags);

/*
 * kda_fwd_recurrent -- the same forward pass evaluated token by token (the recurrence the
 * FlashKDA article index calls the linear-time recurrence), for short sequences: the decode
 * step (one token per sequence, state in and out, often in place) and sequences of a few
 * tokens.  Same arguments, layouts, ownership, errors and activation switches as kda_fwd_ex,
 * and the same workspace (kda_fwd_workspace_size).  One workgroup per (sequence, head)
 * keeps the 128 x 128 state in fp32 registers and walks the sequence's tokens in order, so
 * its time grows with the longest sequence; for sequences longer than a few chunks use
 * kda_fwd.  Results agree with kda_fwd to the same tolerance against the fp64 recurrence
 * (this path is all fp32; kda_fwd uses split-bf16 matrix products).
 */
kda_status kda_fwd_recurrent(const void *q, const void *k, const void *v, const void *g, const void *beta,
                             float scale, void *out, const float *A_log, const float *dt_bias,
                             float lower_bound, const void *initial_state,
                             kda_state_dtype initial_state_dtype, void *final_state,
                             kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                             const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H, int64_t N,
                             int64_t K, int64_t V, void *workspace, size_t workspace_bytes, void *stream,
                             uint32_t flags);

/*
 * kda_fwd_recurrent_timed -- kda_fwd_recurrent with stage timing, for measurement: three
 * hipEvent_t handles (created by the caller) recorded on `stream` before the chunk-table
 * kernel, before the recurrent kernel and after it.  Returns KDA_ERR_NULL if any of the
 * three is NULL.
 */
kda_status kda_fwd_recurrent_timed(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, float scale, void *out, const float *A_log,
                                   const float *dt_bias, float lower_bound, const void *initial_state,
                                   kda_state_dtype initial_state_dtype, void *final_state,
                                   kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                                   const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H,
                                   int64_t N, int64_t K, int64_t V, void *workspace,
                                   size_t workspace_bytes, void *stream, uint32_t flags,
                                   void *const *stage_events);

/*
 * kda_fwd_timed -- kda_fwd with stage timing, for measurement.  Same arguments and behaviour
 * as kda_fwd, plus stage_events: five hipEvent_t handles (created by the caller), recorded
 * on `stream`:
 *   [0] before the chunk-table kernel
 *   [1] before the first forward-kernel launch
 *   [2] after it (with the cut plan: after pass A and the transition runs)
 *   [3] after the cut scan (recorded right after [2] when there is none)
 *   [4] after pass B (right after [3] when there is none)
 * With the whole-chain plans (see kda_fwd_workspace_size) the forward kernel runs once;
 * with the cut plan, pass A, the transition runs, the scan and pass B.  hipEventElapsedTime
 * between consecutive events gives each stage's duration.  Returns KDA_ERR_NULL if any of
 * the five handles is NULL.
 */
kda_status kda_fwd_timed(const void *q, const void *k, const void *v, const void *g, const void *beta,
                         float scale, void *out, const float *A_log, const float *dt_bias,
                         float lower_bound, const void *initial_state,
                         kda_state_dtype initial_state_dtype, void *final_state,
                         kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                         const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H, int64_t N,
                         int64_t K, int64_t V, void *workspace, size_t workspace_bytes, void *stream,
                         void *const *stage_events);

/*
 * kda_fwd_noalloc -- kda_fwd_ex for callers that cannot allocate device memory: code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * layouts, ownership, activation switches, results and errors as kda_fwd_ex, without the
 * workspace arguments: the library's own static device scratch of KDA_NOALLOC_SCRATCH_BYTES
 * (64 MiB; one copy on every GPU the library runs on, held until the process ends) serves
 * as the workspace.  The call allocates nothing.
 *   - Returns KDA_ERR_SCRATCH, before any HIP call, when kda_fwd_workspace_size for these
 *     sizes exceeds KDA_NOALLOC_SCRATCH_BYTES (e.g. very many sequences).
 *   - The scratch belongs to the device of `stream` (the current device for NULL); its
 *     address is looked up once per device.  Calls on one GPU share it: two calls that
 *     overlap in time on one GPU (different streams, or host threads) race and give
 *     undefined results; serialise them.  Every word a call reads from the scratch is
 *     written earlier in the same call, so nothing needs clearing between calls.
 *   - kda_fwd_device_status cannot read this call's status word (it is not in a caller's
 *     buffer); validation errors are still returned.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
kda_status kda_fwd_noalloc(const void *q, const void *k, const void *v, const void *g, const void *beta,
                           float scale, void *out, const float *A_log, const float *dt_bias,
                           float lower_bound, const void *initial_state, kda_state_dtype initial_state_dtype,
                           void *final_state, kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                           const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H, int64_t N,
                           int64_t K, int64_t V, void *stream, uint32_t flags);

/*
 * kda_fwd_workspace_size -- bytes of workspace kda_fwd needs: the status word, the
 * per-sequence chunk table (start, length, chunk offset), O(N) bytes, a fixed 2.25 KiB
 * table of the first unit of each workgroup and the unit list (8 bytes per sequence) that
 * spreads the sequences over the workgroups with about equal chunk counts (a long sequence
 * of a varlen batch may run as two units of 64 value columns each), and a fixed 3.25 KiB
 * cut table.  When sequences are long on average (at least 64 chunks of 16 tokens, about
 * ceil(T / 16) / N for varlen) and H <= 128, the cut plan gives each head P = min(256 / H,
 * C / 16) workgroups (C = the head's chunk count, ceil(T / 16) for varlen) that take equal
 * runs of its chunks, cutting sequences where needed (the state after a piece is affine
 * in the state before it); that adds three fp32 128 x 128 states per head and cut,
 * 3 * H * P * 64 KiB, plus 40 bytes per head and cut.  P is a deterministic function of
 * (B, T, H, N, has_cu_seqlens).  The per-chunk operands never leave the chip.  Returns 0
 * for invalid sizes.
 */
size_t kda_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t N, int has_cu_seqlens);

/*
 * kda_bwd -- gradients of kda_fwd_ex's outputs (out and final_state) with respect to its
 * inputs, for training.  The pages describe the forward pass only; this is the reverse-mode
 * derivative of the same per-token recurrence (stated in the comment at the top of this
 * file), under the same activation switches.  All arithmetic is fp32 (the products with the
 * states as three-term bf16 products with fp32 accumulation, about 16 significant bits per
 * factor, as in kda_fwd's chunk recurrence); the inputs q, k, v,
 * g, beta, scale, A_log, dt_bias, lower_bound, initial_state, cu_seqlens, B, T, H, N, K, V
 * and flags mean exactly what they mean for kda_fwd_ex.
 *   dout          bf16 [B, T, H, 128], 16-byte aligned: dL/dout.
 *   dfinal_state  NULL (zero) or fp32 [N, H, 128, 128], 16-byte aligned: dL/dfinal_state.
 *   dq, dk, dv, dg  fp32 [B, T, H, 128], 16-byte aligned, fully written: dL/dq, dL/dk,
 *                 dL/dv and dL/dg (with the gate switch off, g is the log-decay itself and
 *                 its gradient is zero where g lies outside (lower_bound, 0)).
 *   dbeta         fp32 [B, T, H], 4-byte aligned: dL/dbeta (the logit when the sigmoid runs
 *                 in the pass).
 *   dA_log        NULL or fp32 [H]; ddt_bias  NULL or fp32 [H, 128] (16-byte aligned):
 *                 summed over every token of every sequence.  Written only with the gate
 *                 switch on (KDA_GATE_IN_KERNEL); NULL = not written.
 *   dinitial_state  NULL (not written) or fp32 [N, H, 128, 128], 16-byte aligned: dL/d
 *                 initial_state (also when initial_state is NULL, i.e. zero).
 *   workspace     device scratch of at least kda_bwd_workspace_size(...) bytes, 256-byte
 *                 aligned.
 * An invalid cu_seqlens (found on the device) makes every sequence empty, as in kda_fwd:
 * dq, dk, dv, dg and dbeta are not written, dA_log and ddt_bias are zero, and
 * dinitial_state = dfinal_state (or zero); kda_fwd_device_status on the workspace reports it.
 * Outputs must not overlap any input or each other (KDA_ERR_ALIAS).  Same error codes as
 * kda_fwd_ex otherwise.  Work is enqueued on `stream`; nothing is allocated.  The pass runs
 * in 16-token chunks: the state runs forwards and dL/dS backwards over the chunks of each
 * (sequence, head), and the tokens' gradients are formed per chunk in parallel.  Where the
 * sequences are few and long (64 chunks or more on average), both walks are cut into pieces
 * that run in parallel and are joined by an affine scan (with the in-kernel l2norm and
 * sigmoid, a start state's share that has fallen below 2^-30 of a piece's own end state is
 * dropped, as in kda_fwd's cut plan).  Results are deterministic: fixed summation orders,
 * no atomics.
 */
kda_status kda_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta, float scale,
                   const float *A_log, const float *dt_bias, float lower_bound, const void *initial_state,
                   kda_state_dtype initial_state_dtype, const void *dout, const float *dfinal_state, float *dq,
                   float *dk, float *dv, float *dg, float *dbeta, float *dA_log, float *ddt_bias,
                   float *dinitial_state, const int64_t *cu_seqlens, const int64_t *cu_seqlens_host, int64_t B,
                   int64_t T, int64_t H, int64_t N, int64_t K, int64_t V, void *workspace,
                   size_t workspace_bytes, void *stream, uint32_t flags);

/*
 * kda_bwd_workspace_size -- bytes of workspace kda_bwd needs: the chunk table, then per
 * 16-token chunk of each head (counted as ceil(T / 16) per batch row, or ceil(T / 16) + N
 * with cu_seqlens) 33.5 KiB of chunk operands, one fp32 state (64 KiB: the state before the
 * chunk for the even chunks of a sequence, dL/dS after it for the odd ones) and the chunk's
 * V' and dL/dV' (8 KiB each), 16 bytes per chunk of location records and 64 KiB per head of
 * partial sums; when the pass cuts its walks into pieces, also three fp32 states per (piece,
 * head, direction) (pieces of L chunks, L = max(8, ceil(4 H C / 768)) with C the chunk count
 * above; at most ceil(C / L) + N pieces per head, N the number of sequences).  Returns 0 for
 * invalid sizes.
 */
size_t kda_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t N, int has_cu_seqlens);

/* Human-readable name of a kda_status value (static string; never NULL). */
const char *kda_status_string(int status);

/*
 * kda_fwd_device_status -- after kda_fwd on `stream`, wait for the stream and read the
 * device status word from the workspace: 0 = inputs valid and the forward pass ran to
 * completion; otherwise a bit mask (1: cu[0] != 0, 2: cu decreasing somewhere,
 * 4: cu[N] != T, 0x100: a wavefront of the forward kernel gave up waiting for another
 * one -- results invalid; not expected to happen).  Synchronises the stream.
 */
kda_status kda_fwd_device_status(const void *workspace, int32_t *status_out, void *stream);

/*
 * kda_chunk_table -- run only the first stage of kda_fwd: the integer chunk table built
 * from cu_seqlens (or from B and T).  Writes into the workspace and, when the host
 * pointers are non-NULL, copies back (synchronising the stream):
 *   seq_off_host  int64 [N+1]  exclusive prefix sum of ceil(L_i / 16)
 *   n_total_host  int64        total number of chunks
 *   status_host   int32        device status word (as kda_fwd_device_status)
 * Used to check the integer indexing bit for bit.
 */
kda_status kda_chunk_table(const int64_t *cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t N,
                           void *workspace, size_t workspace_bytes, int64_t *seq_off_host,
                           int64_t *n_total_host, int32_t *status_host, void *stream);

/* Library version, major * 10000 + minor * 100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
