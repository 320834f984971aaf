/*
 * gdn2.h -- C ABI of the Gated DeltaNet-2 forward-pass library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation.  Per head, per token t, with a state S in R^{dk x dv} whose
 * rows are key channels ("Gated DeltaNet-2: Decoupling Erase and Write in
 * Linear Attention" analysis at iplexlaw.co.kr, section "Independent
 * decisions on two axes"):
 *     e_t = b_t (.) k_t           z_t = w_t (.) v_t
 *     Sbar = Diag(alpha_t) S_{t-1}          (decay on key channels)
 *     r_t = Sbar^T e_t                      (old read through the erase key)
 *     S_t = Sbar + k_t (z_t - r_t)^T        (delta update)
 *     o_t = S_t^T q_t                       (output from the state AFTER the update)
 * The same page, section "Token processing and parallel training", gives the
 * chunkwise WY form with 64-token chunks used for long inputs
 * (gdn2_chunk_fwd); the "DeltaNet" entity trail at mindpattern.ai (finding
 * "You Could Have Come Up With Kimi Delta Attention") states that the fused
 * recurrent decode form (gdn2_recurrent_step) computes the same result.
 *
 * Conventions shared by every entry point.
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates no memory, keeps no state between calls and is thread-safe.
 *  - Tensors are contiguous, row-major, with the innermost index last.
 *  - dtype (gdn2_dtype) applies to q, k, v, b, w and o.  alpha and the
 *    recurrent state are always FP32.  bf16 outputs are rounded to nearest
 *    even.  Arithmetic is FP32 (decay, cumulative decay, solve and state);
 *    bf16 inputs feed bf16 matrix-core products with FP32 accumulation.
 *  - Inputs are gate VALUES, not logits: 0 <= alpha <= 1; b, w are used as
 *    given (no clamp, so an erase gate in [0, 2] works).  There is no query
 *    scale: callers pre-scale q.  Every entry point clamps alpha per token
 *    and key channel to [2^-15, 1] (alpha below 2^-15 acts as 2^-15).
 *  - Pointers to q, k, v, b, w, o, alpha and states must be 16-byte aligned.
 *  - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *    and return without synchronising.  Argument errors are reported
 *    synchronously, before anything is enqueued; device faults surface at the
 *    caller's next synchronisation.  Results are bitwise reproducible from
 *    run to run (no atomics, fixed reduction order).
 *  - Supported head sizes: dk in {32, 64, 128}, dv in {32, 64, 128}.
 */
#ifndef GDN2_H
#define GDN2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn2_status {
    GDN2_OK = 0,
    GDN2_ERR_NULL_POINTER = 1, /* a required pointer is NULL                         */
    GDN2_ERR_BAD_SHAPE = 2,    /* a size is <= 0 (or < 0 for T), or inconsistent     */
    GDN2_ERR_UNSUPPORTED = 3,  /* head size not instantiated                         */
    GDN2_ERR_BAD_DTYPE = 4,    /* dtype is not a gdn2_dtype value                    */
    GDN2_ERR_MISALIGNED = 5,   /* a tensor pointer is not 16-byte aligned            */
    GDN2_ERR_ALIAS = 6,        /* an output overlaps an input it may not overlap     */
    GDN2_ERR_WORKSPACE = 7,    /* workspace smaller than the query function's answer */
    GDN2_ERR_HIP = 8,          /* the HIP runtime reported an error at launch        */
    /* not statuses: with these every int32 value is a valid gdn2_status, so
       unknown codes are safe to pass */
    GDN2_STATUS_MIN_ENUM = -0x7fffffff - 1,
    GDN2_STATUS_MAX_ENUM = 0x7fffffff
} gdn2_status;

typedef enum gdn2_dtype {
    GDN2_DTYPE_F32 = 0,
    GDN2_DTYPE_BF16 = 1,
    /* not dtypes (GDN2_ERR_BAD_DTYPE): with these every int32 value is a valid
       gdn2_dtype, so bad codes are safe to pass */
    GDN2_DTYPE_MIN_ENUM = -0x7fffffff - 1,
    GDN2_DTYPE_MAX_ENUM = 0x7fffffff
} gdn2_dtype;

/*
 * Gate layouts, a bitwise OR of gdn2_gate_flags ("gates" below).  The same
 * analysis (section "Independent decisions on two axes") obtains Kimi Delta
 * Attention by tying the erase and write gates to one scalar per token and
 * head, and Gated DeltaNet by also making the decay one scalar per token and
 * head; its ablations (section "Ablations and training throughput") average
 * one of the two gates over its channels.  A scalar gate is passed compactly,
 * one value per token and head ([..] below: the tensor's leading dimensions,
 * [B, T, H] or [N, H]), which saves its memory traffic, and acts on every
 * channel of its axis:
 *   GDN2_GATES_SCALAR_ERASE  b is [..] (dtype) in place of [.., dk]
 *   GDN2_GATES_SCALAR_WRITE  w is [..] (dtype) in place of [.., dv]
 *   GDN2_GATES_TIED          w is ignored (may be NULL); b also serves as the
 *                            write gate.  Requires SCALAR_ERASE and excludes
 *                            SCALAR_WRITE.
 *   GDN2_GATES_SCALAR_DECAY  alpha is [..] (FP32) in place of [.., dk]
 * GDN2_GATES_FULL (0) is the Gated DeltaNet-2 layout of gdn2_chunk_fwd and
 * gdn2_recurrent_step.  GDN2_GATES_KDA and GDN2_GATES_GDN name the two
 * reductions.  Averaging a channel-wise gate is the caller's (it belongs with
 * the gate projection); the result is passed as the scalar gate.
 */
typedef enum gdn2_gate_flags {
    GDN2_GATES_FULL = 0,
    GDN2_GATES_SCALAR_ERASE = 1,
    GDN2_GATES_SCALAR_WRITE = 2,
    GDN2_GATES_TIED = 4,
    GDN2_GATES_SCALAR_DECAY = 8,
    GDN2_GATES_KDA = 5,  /* SCALAR_ERASE | TIED                 */
    GDN2_GATES_GDN = 13  /* SCALAR_ERASE | TIED | SCALAR_DECAY  */
} gdn2_gate_flags;

/*
 * Chunkwise forward over whole sequences ("Token processing and parallel
 * training": chunks of 64 tokens; inside a chunk the running per-channel
 * decay, in FP32, is folded into unequal row and column factors, leaving a
 * lower-triangular solve and dense products; the state passes from chunk to
 * chunk in FP32).
 *
 *   q, k, b : [B, T, H, dk]  dtype          v, w, o : [B, T, H, dv]  dtype
 *   alpha   : [B, T, H, dk]  FP32
 *   initial_state : [N, H, dk, dv] FP32, or NULL for zeros.
 *   final_state   : [N, H, dk, dv] FP32, or NULL if not wanted.  May be the
 *                   same pointer as initial_state (updated in place); any
 *                   other overlap with an input is GDN2_ERR_ALIAS.
 *   cu_seqlens    : NULL, or DEVICE int32 [num_seqs + 1] with cu_seqlens[0] = 0,
 *                   non-decreasing, cu_seqlens[num_seqs] = T.  Then B must be
 *                   1, the batch row holds num_seqs packed sequences, sequence
 *                   n owns tokens [cu_seqlens[n], cu_seqlens[n+1]) and state
 *                   row n (N = num_seqs).  Without it N = B and num_seqs is
 *                   ignored.  Offsets are clamped to [0, T] on the device, so
 *                   a malformed array cannot make the kernel read or write
 *                   outside the tensors; it only gives meaningless results.
 *   T may be 0 (then only final_state = initial_state is written).
 *   workspace / workspace_bytes: NULL, or device scratch of at least
 *                   gdn2_chunk_fwd_workspace_bytes(...) bytes, 16-byte aligned,
 *                   contents on entry irrelevant.  With it, calls with few
 *                   (sequence, head) chains run the segmented path below;
 *                   with NULL they run the single pass.  Smaller than
 *                   required: GDN2_ERR_WORKSPACE.  It must not overlap any
 *                   argument (GDN2_ERR_ALIAS).
 * o must not overlap any input.
 *
 * Segmented path (bf16, dk = 128, dv a multiple of 64, no cu_seqlens, few
 * chains).  The single pass runs one workgroup per (chain, 64 value
 * columns), walking its chain chunk by chunk, so B x H x dv / 64 small
 * leaves most of the GPU idle.  Each batch row is then cut into P segments
 * of whole chunks.  Over a segment the state map is affine, S_out = M S_in +
 * N (the same fact that carries the state from chunk to chunk), so: pass 1
 * runs segments 0 .. P - 2 in parallel, each from a zero state (segment 0
 * from initial_state) with dk extra columns that start from the identity and
 * take no writes, giving N and M; a combine step forms the true incoming
 * state of every later segment; pass 2 runs segments 1 .. P - 1 from those.
 * The result is the same mathematics, rounded differently.
 */
gdn2_status gdn2_chunk_fwd(const void* q, const void* k, const void* v,
                           const float* alpha, const void* b, const void* w,
                           const float* initial_state, float* final_state, void* o,
                           const int32_t* cu_seqlens,
                           int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                           int32_t num_seqs, gdn2_dtype dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn2_chunk_fwd with the gate layout `gates` (a bitwise OR of
 * gdn2_gate_flags, shapes as listed there; GDN2_GATES_FULL is identical to
 * gdn2_chunk_fwd).  Other bits, or TIED without SCALAR_ERASE or with
 * SCALAR_WRITE, give GDN2_ERR_BAD_SHAPE.
 */
gdn2_status gdn2_chunk_fwd_gates(const void* q, const void* k, const void* v,
                                 const float* alpha, const void* b, const void* w,
                                 const float* initial_state, float* final_state, void* o,
                                 const int32_t* cu_seqlens,
                                 int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                 int32_t num_seqs, gdn2_dtype dtype, int32_t gates,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for the segmented path of gdn2_chunk_fwd / _gates: 0 when that
 * path does not apply to these sizes (then the call needs no workspace).
 * num_seqs: the packed sequence count with cu_seqlens, else 0 (the
 * segmented path takes no packed input; it needs T >= 1024).  P segments of
 * L tokens (L a multiple of 64, at least 256; P at least 3 and small enough
 * that pass 1 fills the device's compute units once) need B x P x H x dk x (dv + dk) +
 * B x P x H x dk x dv FP32 values, each part rounded up to 256 bytes. */
size_t gdn2_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                      int32_t num_seqs, gdn2_dtype dtype);

/*
 * One fused recurrent step (decode) for N independent sequences: each
 * (sequence, head) state is read once and written once, in place.
 *
 *   q, k, b : [N, H, dk] dtype     v, w, o : [N, H, dv] dtype
 *   alpha   : [N, H, dk] FP32
 *   state   : [N, H, dk, dv] FP32, read and overwritten with the new state.
 * o must not overlap any input or the state.
 */
gdn2_status gdn2_recurrent_step(const void* q, const void* k, const void* v,
                                const float* alpha, const void* b, const void* w,
                                float* state, void* o,
                                int32_t N, int32_t H, int32_t dk, int32_t dv,
                                gdn2_dtype dtype, void* stream);

/*
 * gdn2_recurrent_step with the gate layout `gates` (as for
 * gdn2_chunk_fwd_gates; [..] is [N, H]).
 */
gdn2_status gdn2_recurrent_step_gates(const void* q, const void* k, const void* v,
                                      const float* alpha, const void* b, const void* w,
                                      float* state, void* o,
                                      int32_t N, int32_t H, int32_t dk, int32_t dv,
                                      gdn2_dtype dtype, int32_t gates, void* stream);

/*
 * The fused recurrent form over T tokens per sequence in one call (short
 * prompts, several tokens to verify, decode after a chunkwise prefill): the
 * recurrence token by token, each (sequence, head) state read once and
 * written once, in place.  The same mathematics as gdn2_chunk_fwd ("DeltaNet"
 * entity trail at mindpattern.ai, finding "You Could Have Come Up With Kimi
 * Delta Attention"), so a final state of gdn2_chunk_fwd continues here.  For
 * T >= 24 with bf16 inputs, dk = 128 and dv a multiple of 64 the call runs the
 * chunkwise matrix-core kernel on the [N, T, H, .] inputs (the same
 * mathematics; it is faster from about 20 tokens on); otherwise one token at
 * a time with the state in registers.
 *
 *   q, k, b : [N, T, H, dk] dtype     v, w, o : [N, T, H, dv] dtype
 *   alpha   : [N, T, H, dk] FP32
 *   gates   : a gate layout as for gdn2_chunk_fwd_gates ([..] is [N, T, H]);
 *             GDN2_GATES_FULL for the layout above
 *   state   : [N, H, dk, dv] FP32, read and overwritten with the state after
 *             token T - 1.  T = 0 leaves it unchanged and launches nothing.
 * gdn2_recurrent_step is this call with T = 1.  o must not overlap any input
 * or the state; the state must not overlap an input.
 */
gdn2_status gdn2_recurrent_fwd(const void* q, const void* k, const void* v,
                               const float* alpha, const void* b, const void* w,
                               float* state, void* o,
                               int32_t N, int32_t T, int32_t H, int32_t dk, int32_t dv,
                               gdn2_dtype dtype, int32_t gates, void* stream);

/*
 * Chunkwise backward pass: the gradients of gdn2_chunk_fwd (full gate layout)
 * for the loss <d_o, o> + <d_final_state, final_state>, accumulated through
 * the gated keys and values with the channel-wise decay inside the sums
 * ("Token processing and parallel training": the backward pass cannot pull
 * the channel-wise factors out as it could a scalar beta).  alpha is clamped
 * to [2^-15, 1] as in the forward pass, and dalpha is zero where the clamp is
 * active.
 *
 * Two paths.  bf16 inputs with dk = dv = 128 (T > 0) take the matrix-core
 * path: 64-token chunks, bf16 products with FP32 accumulation, FP32 decay,
 * states and state gradients (stored in bf16 between its kernels).  It needs
 * every key channel to decay by at least 2^-64 over every 64-token chunk
 * (the split of the pairwise decay factors stays in range); when some chunk
 * decays faster, the FP32 path below runs instead, on the same workspace,
 * decided on the device without a host round trip.  All other calls take the
 * FP32 path: 32-token chunks, FP32 arithmetic throughout, exact pairwise
 * factors where the split would leave the FP32 range.  After a matrix-core
 * shaped call the first int32 of the workspace is 0 when the matrix-core path
 * produced the results and 1 when the FP32 path did.
 *
 *   q, k, v, alpha, b, w, initial_state, cu_seqlens, B, T, H, dk, dv,
 *   num_seqs, dtype: the forward call's arguments (initial_state may be NULL).
 *   d_o           : [B, T, H, dv] dtype, the gradient of o.
 *   d_final_state : [N, H, dk, dv] FP32, or NULL for zero.
 *   dq, dk, db    : [B, T, H, dk] dtype      dv, dw : [B, T, H, dv] dtype
 *   dalpha        : [B, T, H, dk] FP32
 *   d_initial_state : [N, H, dk, dv] FP32, or NULL if not wanted; may be the
 *                   same pointer as d_final_state (replaced in place).
 *   workspace     : device memory of at least gdn2_chunk_bwd_workspace_bytes
 *                   (same sizes; num_seqs = the packed sequence count with
 *                   cu_seqlens, else 0), 16-byte aligned; its contents on
 *                   entry do not matter.  Too small or NULL: GDN2_ERR_WORKSPACE.
 * Every output, and the workspace, must not overlap an input or another
 * output (GDN2_ERR_ALIAS).  Results are bitwise reproducible.
 */
gdn2_status gdn2_chunk_bwd(const void* q, const void* k, const void* v,
                           const float* alpha, const void* b, const void* w,
                           const float* initial_state, const void* d_o, const float* d_final_state,
                           void* dq, void* dk, void* dv, float* dalpha, void* db, void* dw,
                           float* d_initial_state, const int32_t* cu_seqlens,
                           int32_t B, int32_t T, int32_t H, int32_t dk_size, int32_t dv_size,
                           int32_t num_seqs, gdn2_dtype dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace needed by gdn2_chunk_bwd.  FP32 path, with C = B x (ceil(T / 32)
 * + num_seqs) x H chunk slots: 2 x C x dk x dv x 4 bytes of states,
 * 2 x B x T x H x dv x 4 bytes of rows and C x (2048 + 97 dk) x 4 bytes of
 * per-chunk triangular algebra, each rounded up to 256 bytes (0 when T = 0).
 * Matrix-core shaped calls (bf16, dk = dv = 128, T > 0): 256 bytes more than
 * the larger of that and, with C64 = B x (ceil(T / 64) + num_seqs) x H,
 * 2 x C64 x 128 x 128 x 2 bytes of states plus 2 x C64 x 64 x 128 x 2 bytes of
 * rows (each rounded up to 256 bytes).  Returns 0 for invalid sizes. */
size_t gdn2_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t dk_size, int32_t dv_size,
                                      int32_t num_seqs, gdn2_dtype dtype);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * gdn2_chunk_bwd with its workspace taken from a fixed device array that the
 * library owns, so the call allocates nothing (no hipMalloc, no hipFree, no
 * allocating library routine).  Arguments, outputs, checks and results are
 * those of gdn2_chunk_bwd (bitwise the same), without the workspace
 * arguments.
 *
 * Limit: the workspace gdn2_chunk_bwd_workspace_bytes reports for the call
 * must not exceed gdn2_chunk_bwd_noalloc_max_workspace_bytes() (256 MiB),
 * else GDN2_ERR_WORKSPACE, before anything is enqueued.  For example
 * B = 1, T = 2048, H = 16, dk = dv = 128 fits; the B = 8, T = 4096 training
 * shape (3.4 GB) does not.
 *
 * The array: each GPU the library runs on holds its own 256 MiB copy from the
 * moment the library's code is loaded there until the process ends; its
 * address is looked up on the call's current device at the first call there.
 * Every call on one GPU shares that GPU's array and nothing in it needs to
 * start at zero.  Calls that overlap on one GPU (two streams, two host
 * threads) race on the array: serialise them.  A failed address lookup
 * returns GDN2_ERR_HIP.
 */
gdn2_status gdn2_chunk_bwd_noalloc(const void* q, const void* k, const void* v,
                                   const float* alpha, const void* b, const void* w,
                                   const float* initial_state, const void* d_o,
                                   const float* d_final_state,
                                   void* dq, void* dk, void* dv, float* dalpha, void* db, void* dw,
                                   float* d_initial_state, const int32_t* cu_seqlens,
                                   int32_t B, int32_t T, int32_t H, int32_t dk_size, int32_t dv_size,
                                   int32_t num_seqs, gdn2_dtype dtype, void* stream);

/* Capacity of the library-owned workspace of gdn2_chunk_bwd_noalloc, in bytes. */
size_t gdn2_chunk_bwd_noalloc_max_workspace_bytes(void);

/*
 * Token-mixer prologue: q, k, v, b, w for the recurrence from the projection
 * outputs, in one pass ("Token processing and parallel training": short
 * causal convolution, SiLU and L2 normalisation on the query and key paths,
 * convolution and SiLU on the value path; "Independent decisions on two
 * axes": sigmoid erase and write gates).  Per channel c of head h and token t
 * of a sequence starting at bos:
 *     y_t = sum_{i<K} W[h d + c][i] x_{t-K+1+i}   (inputs before bos come from
 *                                                  the carried state)
 *     q = q_scale * y_q' / sqrt(|y_q'|^2 + eps_l2) with y_q' = SiLU(y_q)
 *     k = y_k' / sqrt(|y_k'|^2 + eps_l2)            with y_k' = SiLU(y_k)
 *     v = SiLU(y_v),  b = sigmoid(b_logit),  w = sigmoid(w_logit)
 * (the norms over the head's dk channels).
 *
 *   xq, xk, b_logit : [B, T, H, dk] dtype     xv, w_logit : [B, T, H, dv] dtype
 *   conv_q, conv_k  : [H * dk][K] FP32        conv_v      : [H * dv][K] FP32
 *                     (tap K - 1 multiplies the current token)
 *   conv_state_in   : [N, H * (2 dk + dv), K - 1] FP32, the K - 1 inputs before
 *                     each sequence, oldest first (channels: q, then k, then v);
 *                     NULL = zeros
 *   conv_state_out  : same layout, each sequence's last K - 1 inputs, or NULL.
 *                     It may equal conv_state_in only when every sequence is
 *                     one token (T = 1 without cu_seqlens: a decode step).
 *   q, k, b         : [B, T, H, dk] dtype      v, w : [B, T, H, dv] dtype
 *   cu_seqlens, num_seqs: as for gdn2_chunk_fwd (the convolution restarts at
 *                     every sequence).  1 <= kernel_size <= 16, eps_l2 >= 0.
 * Outputs must not overlap inputs or each other (GDN2_ERR_ALIAS).
 */
gdn2_status gdn2_mixer_prologue(const void* xq, const void* xk, const void* xv,
                                const float* conv_q, const float* conv_k, const float* conv_v,
                                const void* b_logit, const void* w_logit,
                                const float* conv_state_in, float* conv_state_out,
                                void* q, void* k, void* v, void* b, void* w,
                                const int32_t* cu_seqlens,
                                int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                int32_t kernel_size, int32_t num_seqs, float q_scale, float eps_l2,
                                gdn2_dtype dtype, void* stream);

/*
 * Token-mixer epilogue, after the recurrence (same section: RMS
 * normalisation, then an output gate distinct from the write gate):
 *     y = o / sqrt(mean(o^2) + eps) * weight * act(gate)
 * per row of dv values.  o, gate, y: [rows, dv] dtype; weight: [dv] FP32;
 * gate_act 0 = sigmoid, 1 = SiLU; eps > 0.  y must not overlap an input.
 */
gdn2_status gdn2_mixer_epilogue(const void* o, const void* gate, const float* weight, void* y,
                                int64_t rows, int32_t dv, float eps, int32_t gate_act,
                                gdn2_dtype dtype, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* gdn2_status_string(gdn2_status status);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int32_t gdn2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
