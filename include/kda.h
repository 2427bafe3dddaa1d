/*
 * kda.h -- C ABI of libkda, Kimi Delta Attention (KDA) prefill and decode on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Kimi (AI)", section "Kimi Delta Attention (KDA)"):
 * per (sequence, head) a memory matrix S of d_v x d_k float32 values -- rows
 * index value channels, columns key channels, as in the naive linear-attention
 * equation S_t = sum_i v_i k_i^T of that section -- is carried through the
 * section's three steps for every token t:
 *     forget gating    S~  = diag(alpha_t) S_{t-1}     (alpha_t scales rows)
 *     predict          v~  = S~ k_t
 *     memory updating  S_t = S~ + beta_t (v_t - v~) k_t^T
 * and the output is the linear-attention read-out o_t = S_t q_t, taken with
 * the updated state.  No 1/sqrt(d_k) or other scaling is applied to q or k.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, owned by the caller, contiguous
 *     in the layouts given below and 16-byte aligned, except beta and
 *     cu_seqlens, which need 4-byte alignment.  The library keeps no device
 *     memory of its own between calls, except the workspace array of
 *     kda_prefill_noalloc once that entry point has been used on a device.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream) and return as soon as the work is enqueued.  The library is
 *     reentrant; calls on different streams may run concurrently if their
 *     buffers do not overlap.
 *   - Arguments are validated on the host before any HIP call.  An invalid
 *     argument returns an error status and enqueues nothing.  A failed kernel
 *     launch returns KDA_ERR_DEVICE.  On any error the contents of the
 *     outputs are undefined.  Nothing aborts the process.
 *   - NaN and Inf inputs are not checked; they propagate.
 *   - d_k and d_v must each be 64 or 128.
 *   - alpha is taken as given (the gate after its activation), in [0, 1];
 *     alpha == 0 forgets a row (or, for the key-channel variants, a column)
 *     entirely and is handled exactly by every entry point.  The bf16 prefill's
 *     chunked form scales values by the inverse of a row's decay within a
 *     64-token chunk; a (sequence, head, 64-row block) in which some row decays
 *     by more than 2^-100 within one chunk (alpha == 0 included) is recomputed
 *     token by token, from S0, inside the same call.  That costs time, never
 *     accuracy.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misalignment, bad cu_seqlens shape */
    KDA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. d_k = 96) */
    KDA_ERR_DEVICE = 3,           /* a HIP call or kernel launch failed */
    KDA_ERR_WORKSPACE = 4         /* workspace missing or smaller than kda_prefill_workspace_size */
} kda_status;

typedef enum {
    KDA_DTYPE_F32 = 0,  /* q, k, v and o are float32 */
    KDA_DTYPE_BF16 = 1  /* q, k, v and o are bfloat16; o is rounded to nearest even */
} kda_dtype;

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* kda_status_string(kda_status s);

/*
 * Bytes of device workspace kda_prefill (and its gate variants) needs for these
 * sizes (0 is possible).  Returns 0 as well for sizes that kda_prefill would
 * reject.  The size depends on the sizes only, never on cu_seqlens.
 *   KDA_DTYPE_F32:  the longest-first schedule of the packed sequences
 *                   (n_seq int32, rounded up to 256 bytes).
 *   KDA_DTYPE_BF16: the schedule, the first chunk of every sequence
 *                   ((n_seq + 1) int32), one int32 per (sequence, head, 64
 *                   value rows) marking blocks that need the token-by-token
 *                   recomputation, and the solved within-chunk system
 *                   A = (I + L)^{-1} diag(beta) of every (chunk, head) -- 12 KiB
 *                   each, for at most n_tok / 64 + n_seq chunks of 64 tokens.
 *                   Calls with few (sequence, head) pairs and long sequences
 *                   (d_k = d_v) are split into G segments per sequence that are
 *                   scanned in parallel and composed; for those the schedule and
 *                   offsets cover n_seq G segments, plus the segments' token
 *                   offsets, and three fp32 states of d_v x d_k and a d_v-vector
 *                   per (segment, head).  Every part is rounded up to 256 bytes.
 */
size_t kda_prefill_workspace_size(int32_t n_seq, int32_t n_tok, int32_t n_heads,
                                  int32_t d_k, int32_t d_v, kda_dtype dt);

/*
 * Prefill: runs every token of n_seq packed sequences through the recurrence
 * (chunkwise: each chunk of consecutive tokens is solved in parallel, the
 * state is carried from chunk to chunk), writes every output o_t and the final
 * state of every (sequence, head).
 *
 *   q, k        [n_tok, n_heads, d_k]   dtype dt
 *   v           [n_tok, n_heads, d_v]   dtype dt
 *   alpha       [n_tok, n_heads, d_v]   float32, forget gate per value channel
 *   beta        [n_tok, n_heads]        float32, one scalar per (token, head)
 *   S0          [n_seq, n_heads, d_v, d_k] float32 row-major, or NULL = zeros
 *   cu_seqlens  device int32 [n_seq+1]: sequence n owns tokens
 *               cu_seqlens[n] .. cu_seqlens[n+1]-1.  Must start at 0, be
 *               nondecreasing and end at n_tok (not checked on the device:
 *               the host never reads it, so no synchronisation is implied).
 *               NULL = n_seq sequences of n_tok/n_seq tokens each (n_tok must
 *               then be a multiple of n_seq).  Empty sequences are allowed and
 *               give S_T = S0.
 *   o           [n_tok, n_heads, d_v]   dtype dt (written)
 *   S_T         [n_seq, n_heads, d_v, d_k] float32 (written), or NULL.  May be
 *               the same buffer as S0 (in-place continuation); any other
 *               overlap between inputs and outputs is not allowed.
 *   workspace   device scratch of at least kda_prefill_workspace_size(...)
 *               bytes (may be NULL when that size is 0); its contents need no
 *               initialisation and are clobbered.  It may not overlap any other
 *               argument.  Calls that share one workspace must be ordered
 *               (the same stream, or events between them).
 * n_seq >= 1, n_tok >= 0, n_heads >= 1.
 */
kda_status kda_prefill(const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta,
                       const float* S0, const int32_t* cu_seqlens,
                       int32_t n_seq, int32_t n_tok, int32_t n_heads,
                       int32_t d_k, int32_t d_v, kda_dtype dt,
                       void* o, float* S_T,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory -- code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc: kda_prefill with the
 * workspace taken from a device array that the library itself holds (one per
 * device, KDA_PREFILL_NOALLOC_MAX_WORKSPACE bytes, reserved when the library
 * first uses it on that device and kept until the process ends).  The call
 * itself allocates nothing.
 *   Every argument, layout, convention and result is that of kda_prefill; the
 *   outputs are bit-identical to kda_prefill's with a workspace of its own.
 *   Returns KDA_ERR_WORKSPACE, before any HIP call, when
 *   kda_prefill_workspace_size(...) for these sizes exceeds the maximum
 *   (the batched workload of 4 x 8192 tokens, 32 heads, d = 128, bf16, needs
 *   203 MB), and KDA_ERR_DEVICE if the array's address cannot be obtained.
 *   The array is shared by every call on the device and keeps whatever the
 *   last call left (nothing in it needs clearing): calls that may overlap in
 *   time on one device -- different streams, or different threads without
 *   ordering -- race on it and must not be made.
 */
#define KDA_PREFILL_NOALLOC_MAX_WORKSPACE ((size_t)256 << 20)

kda_status kda_prefill_noalloc(const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta,
                               const float* S0, const int32_t* cu_seqlens,
                               int32_t n_seq, int32_t n_tok, int32_t n_heads,
                               int32_t d_k, int32_t d_v, kda_dtype dt,
                               void* o, float* S_T, void* stream);

/*
 * Decode step: one new token for each of `batch` sequences (recurrent form,
 * constant memory per sequence -- the section's "linear time and constant
 * memory").  The state is read once and written once, in place.
 *
 *   q, k    [batch, n_heads, d_k]  dtype dt
 *   v       [batch, n_heads, d_v]  dtype dt
 *   alpha   [batch, n_heads, d_v]  float32
 *   beta    [batch, n_heads]       float32
 *   S       [batch, n_heads, d_v, d_k] float32, in/out: S_{t-1} in, S_t out
 *   o       [batch, n_heads, d_v]  dtype dt (written): o_t = S_t q_t
 * batch >= 0 (0 enqueues nothing), n_heads >= 1.  S must not overlap any
 * other argument.
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta,
                           float* S, void* o,
                           int32_t batch, int32_t n_heads, int32_t d_k, int32_t d_v,
                           kda_dtype dt, void* stream);

/*
 * Scalar-gate variants.  The transcript page ("Per dins de Kimi K3 ..."), where
 * it introduces KDA, describes it as Gated DeltaNet with the decay control
 * replaced by a per-channel one: Gated DeltaNet forgets with one gate for the
 * whole state, and the delta rule without a gate is the case alpha = 1.  These
 * two entry points run that family on the same kernels: the update is the one
 * above with diag(alpha_t) replaced by the scalar alpha_t (or by the identity).
 *
 *   alpha   [n_tok, n_heads] float32 (prefill) or [batch, n_heads] (decode):
 *           one gate per (token, head), applied to every row of S; 4-byte
 *           aligned.  NULL: no forget gate (alpha = 1), the delta rule.
 * Every other argument, the workspace (kda_prefill_workspace_size), the
 * layouts, the conventions and the errors are those of kda_prefill and
 * kda_decode_step, including the handling of strong decay described at the
 * top of this file.
 */
kda_status kda_prefill_scalar_gate(const void* q, const void* k, const void* v,
                                   const float* alpha, const float* beta,
                                   const float* S0, const int32_t* cu_seqlens,
                                   int32_t n_seq, int32_t n_tok, int32_t n_heads,
                                   int32_t d_k, int32_t d_v, kda_dtype dt,
                                   void* o, float* S_T,
                                   void* workspace, size_t workspace_bytes, void* stream);

kda_status kda_decode_step_scalar_gate(const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       float* S, void* o,
                                       int32_t batch, int32_t n_heads, int32_t d_k, int32_t d_v,
                                       kda_dtype dt, void* stream);

/*
 * Key-channel-gate variants: the forget gate applied to the key side,
 * S~ = S_{t-1} diag(alpha_t) with alpha_t in R^{d_k} (column j scaled by
 * alpha_t[j]), then predict, update and read-out as above.  This is the
 * reading of the section's forget-gating step under which the per-channel decay
 * falls on key channels (the transcript page's "channel by channel" control
 * does not say which side); kda_prefill follows the equation as the section
 * writes it, with the gate on rows.
 *
 *   alpha   [n_tok, n_heads, d_k] float32 (prefill) or [batch, n_heads, d_k]
 *           (decode), 16-byte aligned.
 *   workspace  at least kda_prefill_key_gate_workspace_size(...) bytes.
 * Every other argument, the layouts, the conventions and the errors are those
 * of kda_prefill and kda_decode_step.  float32 input runs token by token.
 * bf16 input runs chunkwise: within a 64-token chunk the decay acts on the
 * contraction index of K K^T, so each chunk solves its own decayed system
 * (I + strictly_lower(diag(beta) M))^{-1} diag(beta), M[t,r] = sum_j k_t[j] k_r[j]
 * alpha_{r+1..t}[j], with 16-token sub-chunks bounding every exponent; a chunk
 * in which some key channel decays by more than 2^-64 within 8 consecutive
 * tokens (alpha = 0 included) sends its (sequence, head) to a token-by-token
 * recomputation from S0, so the result is exact for any alpha in [0, 1].
 */
size_t kda_prefill_key_gate_workspace_size(int32_t n_seq, int32_t n_tok, int32_t n_heads,
                                           int32_t d_k, int32_t d_v, kda_dtype dt);

kda_status kda_prefill_key_gate(const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta,
                                const float* S0, const int32_t* cu_seqlens,
                                int32_t n_seq, int32_t n_tok, int32_t n_heads,
                                int32_t d_k, int32_t d_v, kda_dtype dt,
                                void* o, float* S_T,
                                void* workspace, size_t workspace_bytes, void* stream);

kda_status kda_decode_step_key_gate(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta,
                                    float* S, void* o,
                                    int32_t batch, int32_t n_heads, int32_t d_k, int32_t d_v,
                                    kda_dtype dt, void* stream);

/*
 * Backward of the prefill (training): the gradients of a scalar loss L with
 * respect to q, k, v, alpha, beta and S0, given dO = dL/do and dS_T = dL/dS_T.
 * The transcript page ("Per dins de Kimi K3 ..."), where it turns to
 * training, says the model is trained with the chunk-wise parallel algorithm;
 * the gradients follow from the per-token steps of page "Kimi (AI)", section
 * "Kimi Delta Attention (KDA)", by the chain rule.
 *   bf16 inputs with the value-channel, scalar or no gate run chunkwise on
 *   matrix cores: a forward pass keeps the state entering every 64-token chunk,
 *   a reverse scan forms the gradient of the state leaving every chunk, and one
 *   workgroup per (chunk, head) then forms every gradient of the chunk (the
 *   chunk's transposed UT-form algebra).  A (sequence, head) with a chunk beyond
 *   the forward's decay range, a gate below 2^-5 (dalpha = dg / alpha would
 *   magnify rounding) or a |beta| below 2^-20 is recomputed instead by:
 *   the token-recurrent backward, which serves fp32 inputs and the gate on key
 *   channels too: the chain rule in reverse token order, states recomputed from
 *   checkpoints every 16 tokens.
 * Both keep their states in the workspace.
 *
 *   q, k, v, alpha, beta, S0, cu_seqlens, n_seq, n_tok, n_heads, d_k, d_v, dt:
 *               as for kda_prefill (the forward inputs of the call)
 *   dO          [n_tok, n_heads, d_v]   float32, 4-byte aligned
 *   dS_T        [n_seq, n_heads, d_v, d_k] float32, or NULL = zeros
 *   dq, dk      [n_tok, n_heads, d_k]   float32 (written)
 *   dv          [n_tok, n_heads, d_v]   float32 (written), 4-byte aligned
 *   dalpha      shaped as alpha, float32 (written), 4-byte aligned
 *   dbeta       [n_tok, n_heads]        float32 (written), 4-byte aligned
 *   dS0         [n_seq, n_heads, d_v, d_k] float32 (written), or NULL
 *   workspace   device scratch of at least kda_prefill_backward_workspace_size
 *               bytes (never NULL), clobbered.
 * dq, dk, dbeta (and a scalar gate's dalpha) are sums over the value rows; the
 * chunked path forms them whole in one workgroup, the token-recurrent path adds
 * them up with float atomics, so there their last bits can differ from run to
 * run.
 * No output may overlap an input, another output or the workspace.  The
 * arithmetic is fp32 for either input dtype.
 */
size_t kda_prefill_backward_workspace_size(int32_t n_seq, int32_t n_tok, int32_t n_heads,
                                           int32_t d_k, int32_t d_v);

kda_status kda_prefill_backward(const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta,
                                const float* S0, const int32_t* cu_seqlens,
                                const float* dO, const float* dS_T,
                                int32_t n_seq, int32_t n_tok, int32_t n_heads,
                                int32_t d_k, int32_t d_v, kda_dtype dt,
                                float* dq, float* dk, float* dv, float* dalpha, float* dbeta,
                                float* dS0, void* workspace, size_t workspace_bytes, void* stream);

/* The same with one gate per (token, head): alpha and dalpha [n_tok, n_heads];
 * alpha NULL = no gate (then dalpha is not written and may be NULL). */
kda_status kda_prefill_backward_scalar_gate(const void* q, const void* k, const void* v,
                                            const float* alpha, const float* beta,
                                            const float* S0, const int32_t* cu_seqlens,
                                            const float* dO, const float* dS_T,
                                            int32_t n_seq, int32_t n_tok, int32_t n_heads,
                                            int32_t d_k, int32_t d_v, kda_dtype dt,
                                            float* dq, float* dk, float* dv, float* dalpha,
                                            float* dbeta, float* dS0, void* workspace,
                                            size_t workspace_bytes, void* stream);

/* The same with the gate on key channels (as kda_prefill_key_gate): alpha and
 * dalpha [n_tok, n_heads, d_k] float32, alpha 16-byte aligned; dalpha_t is a
 * sum over the value rows, added up with float atomics like dq. */
kda_status kda_prefill_backward_key_gate(const void* q, const void* k, const void* v,
                                         const float* alpha, const float* beta,
                                         const float* S0, const int32_t* cu_seqlens,
                                         const float* dO, const float* dS_T,
                                         int32_t n_seq, int32_t n_tok, int32_t n_heads,
                                         int32_t d_k, int32_t d_v, kda_dtype dt,
                                         float* dq, float* dk, float* dv, float* dalpha,
                                         float* dbeta, float* dS0, void* workspace,
                                         size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
