/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library (libkda.so).
 *
 * Operation (fireworks.ai, "Kimi K3 on Fireworks: Fast RL at frontier scale",
 * section on Kimi Delta Attention: a linear attention that updates a compact
 * per-head recurrent state with channel-wise gating, linear in sequence length,
 * fixed-size decoding state).  Per sequence and head, with state S (dk x dv,
 * row = key channel) and scale = dk^-1/2 unless given:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(log_alpha_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * S_0 = init_state (zero when NULL); final_state = S_T.  kda_bwd returns the
 * gradients of L = <d_out, o> + <d_final_state, S_T> with respect to every
 * input.  The same page says the training kernel must parallelise chunk-local
 * work while limiting the stalls of the recurrent dependency and the movement
 * of intermediates; the library does chunk-local work in parallel and runs
 * the chunk-to-chunk state recurrence as a separate sequential pass.
 *
 * Layouts (all contiguous, token-major; sequences of a varlen batch packed):
 *   q, k, log_alpha                      : [B, T, H, dk]   (desc.dtype)
 *   v, d_out                             : [B, T, H, dv]   (desc.dtype)
 *   beta                                 : [B, T, H]       (desc.dtype)
 *   dq, dk, dlog_alpha                   : [B, T, H, dk]   (desc.out_dtype)
 *   out, dv                              : [B, T, H, dv]   (desc.out_dtype)
 *   dbeta                                : [B, T, H]       (desc.out_dtype)
 *   init_state, final_state, d_final_state, d_init_state : float32 [N, H, dk, dv]
 *     with N = B, or N = num_seqs when cu_seqlens is given.
 *   cu_seqlens : int32 [num_seqs + 1] in device memory, cu[0] = 0,
 *     non-decreasing, cu[num_seqs] = T; only valid with B == 1.
 *
 * Ownership: every pointer is device memory owned by the caller, including
 * the workspace (size from kda_workspace_bytes).  The library allocates and
 * frees nothing, does not synchronise, and keeps no pointer after a call
 * returns.  All work is enqueued on `stream` in order.
 *
 * Aliasing: final_state may alias init_state (each state slice is read before
 * it is written).  out and the gradient outputs must not overlap any input.
 *
 * Precision: all accumulation is fp32, and states are fp32.  With bf16 inputs
 * the matrix products take fp16 operands (bf16 for the decayed factors); those
 * whose rounding would reach the outputs or gradients beyond the bf16 error
 * bound take a two-term split of the fp32 operand (x = hi + lo): the decayed
 * Gram blocks, the states and U wherever they are multiplied, Kh and U in the
 * training-mode state update, dS' and dU, and dT and Y in the backward's
 * dA = -T^T dT T^T.  Their error is then that of fp32 operands.  The bf16
 * backward multiplies d_out and d_final_state by a power of two that puts their
 * largest magnitude in [0.5, 1) before anything is narrowed to fp16, and every
 * gradient by its inverse (both exact), so the relative error does not depend on
 * the scale of the upstream gradients.  fp32 inputs use fp32 operands; the
 * in-chunk sums of log alpha are taken in fp64 and rounded to fp32 once.  A bf16
 * out_dtype rounds the results once at the end.
 *
 * Errors: arguments are validated on the host before anything is enqueued; on
 * an error nothing is launched.  Launch failures return KDA_ERROR_LAUNCH.
 * Sizes: B*T < 2^31 tokens, H <= 65535, (T/64 + N)*H < 2^31 chunk slots (B*ceil(T/64)*H
 * without cu_seqlens) and N*H < 2^22, with N the number of sequences; larger
 * problems return KDA_ERROR_INVALID_VALUE (kda_workspace_bytes returns 0).
 * The contents of cu_seqlens are a precondition (checked with a synchronous
 * copy only when the environment variable KDA_DEBUG=1).
 *
 * Decay: log_alpha must be <= 0 (-inf allowed: alpha = 0).  Every kernel reads
 * it as max(log_alpha, -16): a token that would keep less than e^-16 (about
 * 1.1e-7, fp32 resolution) of a state row keeps e^-16 of it, and dlog_alpha is
 * 0 for such tokens (the derivative of that floor).  The floor bounds every
 * decay factor the chunked kernels form, so no gate can make them overflow or
 * produce NaN; results move by far less than the error bounds.  A NaN in any
 * input of one (sequence, head) reaches no other (sequence, head).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_SUCCESS = 0,
    KDA_ERROR_INVALID_VALUE = 1,     /* null required pointer, bad shape, bad num_seqs */
    KDA_ERROR_NOT_SUPPORTED = 2,     /* dk or dv not in {64, 128}, unknown dtype */
    KDA_ERROR_MISALIGNED = 3,        /* a pointer not 16-byte aligned */
    KDA_ERROR_WORKSPACE_TOO_SMALL = 4,
    KDA_ERROR_LAUNCH = 5             /* a kernel launch failed (hipGetLastError) */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef struct {
    int32_t B;          /* rows; must be 1 when cu_seqlens is given                         */
    int32_t T;          /* tokens per row (total packed tokens when cu_seqlens is given)    */
    int32_t H;          /* heads                                                            */
    int32_t dk;         /* key/query head dim: 64 or 128                                    */
    int32_t dv;         /* value head dim: 64 or 128                                        */
    int32_t num_seqs;   /* number of packed sequences when cu_seqlens is given, else ignored */
    kda_dtype dtype;    /* storage dtype of q, k, v, log_alpha, beta, d_out                 */
    kda_dtype out_dtype;/* storage dtype of out, dq, dk, dv, dlog_alpha, dbeta; KDA_BF16 is
                           allowed only when dtype is KDA_BF16                               */
    float scale;        /* output scale; 0 means dk^-1/2                                    */
    int32_t flags;      /* KDA_FLAG_* bits below; 0 for a self-contained call               */
} kda_desc;

/* kda_fwd: also leave in the workspace everything kda_bwd would recompute
 * (training step).  The workspace must then have kda_workspace_bytes(desc, 1)
 * bytes.  Not available where kda_bwd is not (fp32 inputs with dk = 128).  With
 * bf16 inputs this pass splits more of its operands than the forward-only pass
 * (the states it keeps feed the gradients), so out and final_state can differ
 * from a call without the flag in the last bits; both are within the same
 * error bound. */
#define KDA_FLAG_SAVE_FOR_BACKWARD 1
/* kda_bwd: the workspace holds what a kda_fwd call with KDA_FLAG_SAVE_FOR_BACKWARD
 * left there, for the same descriptor, inputs (q, k, v, log_alpha, beta,
 * init_state, cu_seqlens) and workspace pointer, with nothing written to the
 * workspace in between; the recomputation of the forward is skipped.  Results
 * are bit-identical to a kda_bwd call without the flag.  Violating the
 * precondition gives wrong gradients; it is not detected. */
#define KDA_FLAG_USE_SAVED 2
/* Fused input preparation (the step upstream of the recurrence in the page's
 * KDA workloads), for kda_fwd, kda_bwd and kda_decode alike:
 * KDA_FLAG_QK_L2NORM: q and k arrive raw; each (token, head) row is scaled to
 *   x / sqrt(sum(x^2) + 1e-6) over the dk channels inside the kernels, and dq,
 *   dk are gradients with respect to the raw rows.  With bf16 inputs the
 *   normalised rows are never rounded to bf16: every use multiplies the raw
 *   row by its 1/|x|.
 * KDA_FLAG_GATE_LOGSIGMOID: log_alpha holds a raw gate x; the kernels use
 *   log alpha = logsigmoid(x) (alpha = sigmoid(x)), and dlog_alpha is the
 *   gradient with respect to x.
 * A backward call must carry the same preparation flags as the forward it
 * differentiates (and, with KDA_FLAG_USE_SAVED, as the saving forward);
 * kda_workspace_bytes accounts for them. */
#define KDA_FLAG_QK_L2NORM 4
#define KDA_FLAG_GATE_LOGSIGMOID 8

/* Bytes of device workspace kda_fwd (backward = 0) or kda_bwd (backward != 0)
 * needs for this problem; 0 if the descriptor is invalid. */
size_t kda_workspace_bytes(const kda_desc *desc, int backward);

/* Forward pass: out (and final_state unless NULL).  init_state may be NULL (zero). */
kda_status kda_fwd(const kda_desc *desc, const void *q, const void *k, const void *v,
                   const void *log_alpha, const void *beta, const float *init_state,
                   void *out, float *final_state, const int32_t *cu_seqlens,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Forward pass for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as kda_fwd, without the workspace: the library
 * takes it from a device array of KDA_NOALLOC_SCRATCH_BYTES that it holds on
 * every GPU it runs on until the process ends (allocated when the library's
 * device code is loaded on that GPU, never by this call).  A problem whose
 * kda_workspace_bytes(desc, 0) exceeds that returns KDA_ERROR_WORKSPACE_TOO_SMALL
 * with the sizes in kda_last_error(); KDA_FLAG_SAVE_FOR_BACKWARD is rejected
 * (KDA_ERROR_INVALID_VALUE).  All calls on one GPU share the array: calls that
 * may overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller.  The call enqueues on `stream` and allocates nothing. */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20)
kda_status kda_fwd_noalloc(const kda_desc *desc, const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *beta, const float *init_state,
                           void *out, float *final_state, const int32_t *cu_seqlens, void *stream);

/* Backward pass: recomputes the forward internally, unless desc->flags has
 * KDA_FLAG_USE_SAVED (see above).  d_final_state may be NULL (zero);
 * d_init_state may be NULL (not written). */
kda_status kda_bwd(const kda_desc *desc, const void *q, const void *k, const void *v,
                   const void *log_alpha, const void *beta, const float *init_state,
                   const int32_t *cu_seqlens, const void *d_out, const float *d_final_state,
                   void *dq, void *dk, void *dv, void *dlog_alpha, void *dbeta,
                   float *d_init_state, void *workspace, size_t workspace_bytes, void *stream);

/* Decode / replay step (same page: KDA keeps a fixed-size decoding state; its
 * section on speculative decoding keeps that state consistent after rejected
 * draft tokens by replaying the accepted tokens' state-update inputs from a
 * committed state, with no per-candidate snapshot).
 *
 * Advances B = desc->B sequences by T = desc->T tokens each (0 <= T <=
 * KDA_DECODE_MAX_TOKENS), one token at a time, from states kept in a pool:
 *   q, k, log_alpha : [B, T, H, dk] (desc->dtype);  v : [B, T, H, dv];  beta : [B, T, H]
 *   out             : [B, T, H, dv] (desc->out_dtype), every token's o_t
 *   state_pool      : float32 [pool_size, H, dk, dv], updated in place
 *   state_indices   : int32 [B] in device memory, pool slot of each sequence;
 *                     NULL means slot b (then pool_size >= B).  A value outside
 *                     [0, pool_size) marks a padding entry: its outputs are
 *                     written as 0 and no state is read or written.
 *   num_commit      : int32 [B] in device memory, NULL meaning T for all.  The
 *                     state after the first num_commit[b] tokens (clamped to
 *                     [0, T]) is written back to the slot; 0 leaves it
 *                     untouched.  Outputs always follow all T tokens.
 * A verification pass over draft tokens commits 0; the replay of the accepted
 * prefix commits its length (or passes only the accepted tokens).
 * desc->num_seqs is ignored; desc->flags may hold only the preparation flags.  Non-padding slots must
 * be distinct within one call (two sequences on one slot race).  No
 * workspace: the call uses only the buffers passed in.  The 16-byte alignment
 * rule applies to q, k, v, log_alpha, out and state_pool; state_indices and
 * num_commit need 4-byte alignment. */
#define KDA_DECODE_MAX_TOKENS 16
kda_status kda_decode(const kda_desc *desc, const void *q, const void *k, const void *v,
                      const void *log_alpha, const void *beta, float *state_pool, int32_t pool_size,
                      const int32_t *state_indices, const int32_t *num_commit, void *out, void *stream);

/* Short causal convolution with a carried state.  The same page's section on
 * disaggregated prefill and decode lists, among what a KDA layer hands from one
 * serving pool to another, a convolution state beside the recurrent state; the
 * page defines neither.  Read here as a causal depthwise convolution of width
 * W along time over each of D channels, whose state is the sequence's last
 * W - 1 inputs:
 *
 *     z[t, c] = bias[c] + sum_{j<W} weight[c, j] * X[t - (W-1) + j, c]
 *     y[t, c] = z[t, c]                      (KDA_CONV_IDENTITY)
 *     y[t, c] = z[t, c] * sigmoid(z[t, c])   (KDA_CONV_SILU)
 *
 * X is the sequence's input preceded by its W - 1 state rows (state row i
 * stands for time i - (W - 1); zero when init_state is NULL).  final_state is
 * the last W - 1 rows of that extended input (for a sequence shorter than
 * W - 1 it still holds some initial-state rows).
 *
 * Layouts (contiguous, token-major):
 *   x, dy                    : [B, T, D] (or packed [1, T, D] with cu_seqlens), desc.dtype
 *   y, dx                    : like x, desc.out_dtype
 *   weight, dweight          : float32 [D, W];  bias, dbias : float32 [D]
 *   init_state, final_state, d_final_state, d_init_state : float32 [N, W - 1, D]
 *   cu_seqlens               : int32 [num_seqs + 1] in device memory (as for kda_fwd)
 * Supported: W in {2, 3, 4}; D a positive multiple of 8.  All pointers are
 * device memory owned by the caller; 16-byte alignment is required of x, y,
 * dy, dx, the states and the pool; 4-byte alignment of weight, bias, dweight,
 * dbias and the int32 arrays.  Validation happens before any launch; the
 * calls enqueue on `stream`, allocate nothing and do not synchronise.
 * final_state may alias init_state; nothing else may overlap. */
typedef enum { KDA_CONV_IDENTITY = 0, KDA_CONV_SILU = 1 } kda_conv_activation;

typedef struct {
    int32_t B;            /* rows (decode: sequences); 1 when cu_seqlens is given   */
    int32_t T;            /* tokens per row (total packed tokens with cu_seqlens)   */
    int32_t D;            /* channels                                               */
    int32_t W;            /* kernel width: 2, 3 or 4                                */
    int32_t num_seqs;     /* packed sequences when cu_seqlens is given              */
    kda_dtype dtype;      /* x, dy                                                  */
    kda_dtype out_dtype;  /* y, dx (KDA_BF16 only with bf16 inputs)                 */
    int32_t activation;   /* kda_conv_activation                                    */
} kda_conv_desc;

/* Bytes of device workspace kda_conv_bwd needs (partial sums of dweight and
 * dbias over tiles of 256 tokens); kda_conv_fwd and kda_conv_decode need none.
 * 0 if the descriptor is invalid or there is nothing to reduce. */
size_t kda_conv_workspace_bytes(const kda_conv_desc *desc);

/* Forward: y, and final_state unless NULL.  bias and init_state may be NULL. */
kda_status kda_conv_fwd(const kda_conv_desc *desc, const void *x, const float *weight, const float *bias,
                        const float *init_state, void *y, float *final_state, const int32_t *cu_seqlens,
                        void *stream);

/* Backward: gradients of <dy, y> + <d_final_state, final_state>.  dx and
 * dweight are required; dbias and d_init_state may be NULL (not written);
 * d_final_state may be NULL (zero).  d_init_state must not alias
 * d_final_state.  dweight and dbias are sums over all tokens in a fixed order
 * (bitwise reproducible). */
kda_status kda_conv_bwd(const kda_conv_desc *desc, const void *x, const float *weight, const float *bias,
                        const float *init_state, const int32_t *cu_seqlens, const void *dy,
                        const float *d_final_state, void *dx, float *dweight, float *dbias,
                        float *d_init_state, void *workspace, size_t workspace_bytes, void *stream);

/* Decode / replay step of the convolution, the companion of kda_decode: x
 * [B, T, D] (T >= 0 tokens per sequence), y [B, T, D]; state_pool float32
 * [pool_size, W - 1, D] updated in place; state_indices and num_commit as in
 * kda_decode (NULL: slot b; NULL: commit all T; a slot outside
 * [0, pool_size) is padding: zero outputs, no state touched; the slot
 * receives the state after the first num_commit[b] tokens, clamped to
 * [0, T]).  Non-padding slots must be distinct within one call. */
kda_status kda_conv_decode(const kda_conv_desc *desc, const void *x, const float *weight, const float *bias,
                           float *state_pool, int32_t pool_size, const int32_t *state_indices,
                           const int32_t *num_commit, void *y, void *stream);

/* Static description of a status code. */
const char *kda_status_string(kda_status status);

/* Which kernel launch failed, and the HIP error it gave, when the last
 * kda_fwd/kda_bwd call on this host thread returned KDA_ERROR_LAUNCH
 * ("" if no launch failed).  The string belongs to the library and stays
 * valid until the thread's next kda_fwd/kda_bwd call. */
const char *kda_last_error(void);

/* Measurement support (for benchmarks and profilers; not needed to compute).
 * kda_timing_enable(1) makes every later kernel launch of kda_fwd/kda_bwd
 * record a hipEvent pair around itself on the call's stream (clearing any
 * accumulated times); kda_timing_enable(0) stops recording.  kda_timing_read
 * waits for the recorded events, adds their durations into per-kernel totals
 * and copies up to max_entries (name, total milliseconds, launch count)
 * triples into the caller's arrays, returning the number of kernels with
 * totals.  Names are static strings.  Events are created on first use and
 * kept for reuse; both calls are host-thread safe.  Returns -1 if a HIP
 * event call fails. */
void kda_timing_enable(int enable);
int kda_timing_read(int max_entries, const char **names, double *total_ms, int *launches);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
