/*
 * kda.h - C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) core.
 *
 * KDA is the per-channel gated delta rule.  For one sequence and one head,
 * with a d_k x d_v fp32 state S (element S[c][j]: c key channel, j value
 * channel) and, per token t, alpha_t = exp(g_t) (one decay per key channel):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * The code audit of the Kimi remote modelling code (finding
 * "dual-kda-execution-regimes") splits it into a chunked form for
 * training/prefill and a fused recurrent form for one-token cached decode;
 * kda_chunk_prefill and kda_recurrent_decode are those two forms, and
 * kda_gate produces their g and beta inputs.  The Kimi K3 artifact audit
 * (§4.1 KDA tensor table, §5.2 shape table, §7.1 FlashKDA interface) fixes
 * the shapes: 96 heads of 128 dims, per-head A_log, per-(head,channel)
 * dt_bias, bf16 q/k/v, fp32 A_log/dt_bias, variable-length batches and
 * initial/final recurrent state.
 *
 * Conventions for every entry point:
 *   - Tensors are dense, row-major (last index fastest), on the current HIP
 *     device, and must not overlap unless stated.  The library never
 *     allocates, frees or copies memory and never synchronises the stream
 *     (outside the KDA_DEBUG mode below).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = legacy default
 *     stream) and runs asynchronously; outputs are ready when the stream is.
 *   - Each call validates all arguments first.  On any status other than
 *     KDA_OK returned before launch, nothing was launched and no output was
 *     written.  KDA_ERR_LAUNCH means the kernel launch itself failed.
 *   - kda_last_error() returns a thread-local message for the last failure.
 *   - The recurrence's domain: g <= 0 and beta in [0, 1] (the gate produces
 *     exactly these), q, k, v and states finite.  The chunked prefill computes
 *     its matrix products on fp16 operands, so q, k, v and state entries must
 *     stay well inside fp16 range (|x| < 2^15); with unit-norm q and k that
 *     holds for any realistic v and state.  Any g <= 0 is accepted: the
 *     chunked prefill floors the per-token decay factor exp(g) at 2^-15.5
 *     (2.2e-5), which keeps every factor it forms in fp32 range for decays
 *     as strong as the Kimi K3 artifact audit's printed parameter maxima
 *     produce (§5.1: A_log up to 2.47, dt_bias up to 0.18), and moves o and
 *     the state by far less than their rounding error.
 *   - Values outside that domain are not checked and propagate into the
 *     outputs, unless the environment variable KDA_DEBUG is "1" (read on
 *     every call).  Then every call first scans its inputs (q, k, v and
 *     states finite, g <= 0, beta in [0, 1], gate logits not NaN, A_log and
 *     dt_bias finite) and returns KDA_ERR_DOMAIN, launching nothing and
 *     writing nothing, if any value breaks its rule; after its kernels it
 *     scans every output and returns KDA_ERR_NONFINITE if any value is NaN
 *     or infinite (a g of -inf, the gate's limit for an infinite logit, is
 *     allowed).  kda_last_error() names each offending tensor and the count.
 *     Debug calls wait for their stream and are serialised by a process-wide
 *     lock.  The Model-Optimizer PR #2749 review (the KDA beta fix) describes
 *     the failure this makes visible: a recurrence fed unsquashed beta
 *     diverges, and the only symptom downstream is a NaN.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad scale       */
  KDA_ERR_SHAPE = 2,       /* inconsistent sizes (e.g. A_log not [H] or [H,d]) */
  KDA_ERR_DTYPE = 3,       /* dtype code not supported for this argument   */
  KDA_ERR_UNSUPPORTED = 4, /* valid but not implemented (e.g. d != 128)    */
  KDA_ERR_ALIGNMENT = 5,   /* pointer not 16-byte aligned                  */
  KDA_ERR_WORKSPACE = 6,   /* workspace missing or too small               */
  KDA_ERR_LAUNCH = 7,      /* the HIP launch failed (see kda_last_error)   */
  KDA_ERR_DOMAIN = 8,      /* KDA_DEBUG=1: an input outside the domain; nothing launched */
  KDA_ERR_NONFINITE = 9    /* KDA_DEBUG=1: a NaN or inf in an output (outputs written)   */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Thread-local text of the last non-OK status ("" if none). */
const char* kda_last_error(void);

/* Library version string. */
const char* kda_version(void);

/*
 * kda_gate - log-decay and beta gate (one elementwise pass).
 *
 *   g[t,h,c]  = -exp(A_log[h]) * softplus(x[t,h,c] + dt_bias[h,c])
 *   beta[t,h] = sigmoid(b[t,h])                     (computed in fp32)
 *
 * A_log holds one value per head and dt_bias one per (head, channel): the
 * artifact audit's §5.2 shape table lists A_log as [H] in the model config,
 * remote code and FlashKDA's host check, and dt_bias [12288] = [96,128].
 * The checkpoint's own A_log is [128]; that section leaves open whether it
 * is a per-channel parameter and advises against guessing a reshape.  So
 * the library takes A_log per head (A_log_len == H) or, given explicitly,
 * per (head, channel) (A_log_len == H*d, [H, d] row-major, exp(A_log[h,c])
 * in place of exp(A_log[h])), and refuses every other length, the bare
 * [128] among them (KDA_ERR_SHAPE).
 * beta is squashed here, once, in fp32 (Model-Optimizer PR #2749 review,
 * the KDA beta fix); the prefill and decode calls take it post-sigmoid and
 * never apply a sigmoid themselves.
 *
 *   x        [n_tok, H, d]  gate logits, dtype x_dt (KDA_F32 or KDA_BF16)
 *   b        [n_tok, H]     beta logits, dtype b_dt (KDA_F32 or KDA_BF16)
 *   A_log    [A_log_len]    fp32, A_log_len == H, or H*d for [H, d]
 *   dt_bias  [dt_bias_len]  fp32, dt_bias_len must equal H*d
 *   g_out    [n_tok, H, d]  fp32 output
 *   beta_out [n_tok, H]     fp32 output
 * Requires d % 4 == 0, d <= 1024 and 16-byte aligned x/g_out (8-byte for bf16 x).
 * n_tok == 0 is a no-op.
 */
kda_status kda_gate(const void* x, kda_dtype x_dt, const void* b, kda_dtype b_dt,
                    const float* A_log, int64_t A_log_len, const float* dt_bias,
                    int64_t dt_bias_len, float* g_out, float* beta_out, int64_t n_tok,
                    int32_t H, int32_t d, void* stream);

/*
 * kda_gate_backward - gradient of kda_gate.
 *
 * For the loss sum(dg * g) + sum(dbeta * beta) with g, beta as kda_gate
 * forms them from the same x, b, A_log and dt_bias (A_log [H] or [H, d]):
 *   dx[t,h,c]    = dg * (-exp(A_log) sigmoid(x + dt_bias))        fp32 [n_tok, H, d]
 *   db[t,h]      = dbeta * beta (1 - beta)                        fp32 [n_tok, H]
 *   ddt_bias[h,c] = sum_t dx[t,h,c]                               fp32 [H, d]
 *   dA_log       = sum of dg * g over the entries sharing the parameter
 *                  (A_log's shape: [H] or [H, d])                 fp32
 * This is the chain rule through the gate of the artifact audit's §4.1 /
 * §5.2 parameters, so that kda_chunk_prefill_backward's dg and dbeta reach
 * the gated call's raw inputs.  The token sums go through the workspace
 * (kda_gate_backward_workspace_bytes: two fp32 partial sums per 32-token run,
 * head and channel) in a fixed order, so the result is deterministic.
 * Requires d % 4 == 0, d <= 1024; 16-byte aligned x (8 for bf16), dg, dx,
 * dt_bias; the rest aligned to their element size.  Refusals as kda_gate,
 * plus a NULL or short workspace (KDA_ERR_WORKSPACE).
 */
kda_status kda_gate_backward(const void* x, kda_dtype x_dt, const void* b, kda_dtype b_dt,
                             const float* A_log, int64_t A_log_len, const float* dt_bias,
                             int64_t dt_bias_len, const float* dg, const float* dbeta, float* dx,
                             float* db, float* dA_log, float* ddt_bias, int64_t n_tok,
                             int32_t H, int32_t d, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Workspace bytes of kda_gate_backward; 0 for invalid arguments. */
size_t kda_gate_backward_workspace_bytes(int64_t n_tok, int32_t H, int32_t d);

/*
 * kda_chunk_prefill - chunked KDA over a packed variable-length batch.
 *
 * Sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of the packed
 * token axis.  Each (sequence, head) starts from initial_state[n,h] (zeros
 * if initial_state is NULL), runs the recurrence above over its tokens in
 * chunks of 64 that never cross a sequence boundary (the tail chunk is
 * partial), writes o for every token and, if final_state is not NULL, the
 * state after its last token.  A zero-length sequence copies its initial
 * state to its final state.
 *
 *   q, k        [T_tot, H, dk]   dtype qkv_dt (KDA_BF16 or KDA_F32)
 *   v           [T_tot, H, dv]   dtype qkv_dt
 *   g           [T_tot, H, dk]   fp32 log-decay (<= 0)
 *   beta        [T_tot, H]       fp32, post-sigmoid
 *   cu_seqlens  [N+1] int32, device copy (read by the kernels)
 *   cu_seqlens_host [N+1] int32, host copy or NULL.  When given it is
 *               validated (cu[0]=0, non-decreasing, cu[N]=T_tot) and must
 *               equal the device copy; it also sizes the work to the longest
 *               sequence.  Without it every sequence is assumed to be up to
 *               T_tot long.  The kernels clamp every sequence range into
 *               [0, T_tot], so no value can make them read or write out of
 *               bounds.
 *   initial_state [N, H, dk, dv] fp32 or NULL; final_state [N, H, dk, dv]
 *               fp32 or NULL; they may be the same buffer (in-place update).
 *   o           [T_tot, H, dv]   dtype o_dt (KDA_BF16 or KDA_F32)
 *   workspace   device scratch of workspace_bytes bytes, 256-byte aligned,
 *               owned by the caller, not read before it is written; it must
 *               not overlap any other argument and must not be used by
 *               anything else until the stream has finished this call.
 *               kda_chunk_prefill_workspace_bytes(N, H, dk, dv, 1) is the
 *               minimum (KDA_ERR_WORKSPACE below it).  The chunks of all
 *               sequences are processed in passes of as many chunks per
 *               sequence as the workspace holds (two launches per pass), so
 *               a workspace for the longest sequence's chunk count runs the
 *               whole batch in one pass.
 * Requires dk == dv == 128 (else KDA_ERR_UNSUPPORTED), N >= 1, H >= 1,
 * 16-byte aligned tensors.  Matrix products run as fp16 MFMA tiles with fp32
 * accumulation (bf16 inputs convert to fp16 exactly inside fp16's range); X
 * and Delta enter the products as hi+lo fp16 pairs, the state as one fp16
 * value (it stays fp32 in the accumulators).  Against an fp64 recurrence
 * the final state agrees to about 3.4e-4 of its Frobenius norm and o to
 * about 3.4e-3 of its RMS (measured on the full-size workloads; the stated
 * bounds are 1e-3 and 5e-3).  A bf16 o is the round-to-nearest-even
 * rounding of the fp32 o, bit for bit.
 */
kda_status kda_chunk_prefill(const void* q, const void* k, const void* v, kda_dtype qkv_dt,
                             const float* g, const float* beta, const int32_t* cu_seqlens,
                             const int32_t* cu_seqlens_host, int32_t N,
                             const float* initial_state, float* final_state, void* o,
                             kda_dtype o_dt, int64_t T_tot, int32_t H, int32_t dk,
                             int32_t dv, float scale, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * kda_chunk_prefill_gated - kda_gate fused into kda_chunk_prefill, with the
 * states in a pool of slots (fp32 or bf16) shared with
 * kda_recurrent_decode_gated.
 *
 * The same recurrence, outputs, workspace and rules as kda_chunk_prefill,
 * but the decay and beta come as the gate's raw inputs (the arguments of
 * kda_gate): x [T_tot, H, dk] gate logits (x_dt KDA_F32 or KDA_BF16), b
 * [T_tot, H] beta logits (b_dt), A_log [H] or [H, dk] (16-byte aligned),
 * dt_bias [H, dk].  g and beta are
 * formed in registers and g never goes to memory.
 *
 * States: initial_state and final_state are pools [num_slots, H, dk, dv] of
 * state_dt (KDA_F32 or KDA_BF16), either NULL (zero entry states / no exit
 * states), possibly the same pool (an in-place update).  Sequence n reads and
 * writes slot state_indices[n] (int32, device), or slot n when state_indices
 * is NULL (then num_slots >= N).  A sequence whose slot lies outside
 * [0, num_slots) (a padding entry such as -1) starts from a zero state and
 * writes no final state; its o is computed.  Two sequences must not share a
 * slot that is written.  A bf16 entry state is widened exactly; the walk
 * keeps the state in fp32 (also between passes) and rounds the exit state
 * to bf16 once, to nearest even.  The artifact audit's §7.4 times FlashKDA's
 * prefill with BF16, no and FP32 state modes; the code audit's
 * repeated-cache-concatenation finding recommends indexed writes into
 * preallocated storage, which the slots provide, so a prefill hands its
 * states to the gated decode without copies or conversions.  g is summed into the
 * cumulative decay straight in log2 units with the plain hardware exp2/log2
 * (absolute error about exp(A_log) 2^-23 per token, against a few ulp for
 * kda_gate), so results agree with kda_gate followed by kda_chunk_prefill to
 * rounding, not bit for bit.  FlashKDA's interface (Kimi K3 artifact audit,
 * §7.1) likewise
 * takes the gate's inputs.  Refusals: those of kda_gate for A_log /
 * dt_bias, then those of kda_chunk_prefill; x must be 16-byte aligned;
 * state_dt not KDA_F32 / KDA_BF16 (KDA_ERR_DTYPE), num_slots < 0
 * (KDA_ERR_INVALID_ARG), num_slots < N with states but no indices
 * (KDA_ERR_SHAPE), a final-state pool overlapping q, k, v, o, the workspace
 * or the indices (KDA_ERR_INVALID_ARG).  The indices themselves are device
 * data and are bounds-checked by the kernel.
 */
kda_status kda_chunk_prefill_gated(const void* q, const void* k, const void* v, kda_dtype qkv_dt,
                                   const void* x, kda_dtype x_dt, const void* b, kda_dtype b_dt,
                                   const float* A_log, int64_t A_log_len, const float* dt_bias,
                                   int64_t dt_bias_len, const int32_t* cu_seqlens,
                                   const int32_t* cu_seqlens_host, int32_t N,
                                   const void* initial_state, void* final_state,
                                   kda_dtype state_dt, int64_t num_slots,
                                   const int32_t* state_indices, void* o, kda_dtype o_dt,
                                   int64_t T_tot, int32_t H, int32_t dk, int32_t dv, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill_gated_static - kda_chunk_prefill_gated with no workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, results and refusals are those of kda_chunk_prefill_gated.  The
 * workspace is a device array inside the library of
 * KDA_PREFILL_STATIC_SCRATCH_BYTES (256 MiB) per GPU, created when the library
 * is loaded and held until the process ends; the call allocates and frees
 * nothing.  A batch needs kda_chunk_prefill_workspace_bytes(N, H, 128, 128, 1)
 * bytes for one chunk per pass (N * H <= 2,131 (sequence, head) pairs): a
 * larger one is refused with KDA_ERR_WORKSPACE before any HIP call.  Smaller
 * batches run the chunk axis in as few passes as the array allows (45 chunks
 * of 64 tokens per pass at N = 1, H = 96; 4 at N = 8).  Every call on one
 * GPU uses that GPU's one
 * array: calls that overlap in time on one GPU (two streams, two host threads)
 * race and must be serialised by the caller.  Nothing in the array is read
 * before the same call writes it.
 */
#define KDA_PREFILL_STATIC_SCRATCH_BYTES (256u << 20)
kda_status kda_chunk_prefill_gated_static(
    const void* q, const void* k, const void* v, kda_dtype qkv_dt, const void* x, kda_dtype x_dt,
    const void* b, kda_dtype b_dt, const float* A_log, int64_t A_log_len, const float* dt_bias,
    int64_t dt_bias_len, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t N,
    const void* initial_state, void* final_state, kda_dtype state_dt, int64_t num_slots,
    const int32_t* state_indices, void* o, kda_dtype o_dt, int64_t T_tot, int32_t H, int32_t dk,
    int32_t dv, float scale, void* stream);

/*
 * kda_chunk_prefill_backward - gradients of kda_chunk_prefill.
 *
 * For the forward of kda_chunk_prefill with the same q, k, v, g, beta,
 * cu_seqlens, initial_state and scale, and the loss
 *   sum(d_o * o) + sum(d_final_state * final_state),
 * writes its gradients with respect to q, k, v, g, beta and the initial state:
 *   dq, dk [T_tot, H, dk] fp32, dv [T_tot, H, dv] fp32, dg [T_tot, H, dk] fp32,
 *   dbeta [T_tot, H] fp32, d_initial_state [N, H, dk, dv] fp32 (NULL: not wanted;
 *   it is the gradient of the zero state when initial_state is NULL).
 * d_o [T_tot, H, dv] has dtype do_dt (KDA_F32 or KDA_BF16); d_o and
 * d_final_state may be NULL (zero).  The chunked form is the training path of
 * the code audit's chunked KDA; this is the reverse-mode of the chunk
 * identities (per chunk: the triangular inverse, the decay-weighted K K^T and
 * Q K^T, the state products), in fp32: the forward states are recomputed
 * chunk by chunk and the state gradient walks the chunks backwards.  The
 * result equals the gradient of the fp64 recurrence up to fp32 rounding.  g
 * enters with the forward's per-token floor (exp(g) >= 2^-15.5; see the
 * conventions above), so the gradient is that of the floored recurrence the
 * forward computes: dg is 0 for a token and channel where the floor acts.
 * The workspace (kda_chunk_prefill_backward_workspace_bytes) holds per (chunk,
 * head) the chunk's intermediate matrices, the recomputed entry state and the
 * state gradient, 344,576 bytes, for P = (T_tot / 64 + N) * H (chunk slot,
 * head) pairs, plus min(P, 8192) scratch slots of 196,608 bytes for the
 * gradient kernel (one workgroup per slot in a launch); the call never
 * allocates.  Requires dk == dv == 128; refusals as for
 * kda_chunk_prefill (the workspace check uses the backward size), plus NULL
 * or unaligned gradients (16-byte, dbeta 4-byte).  Asynchronous on stream.
 */
kda_status kda_chunk_prefill_backward(const void* q, const void* k, const void* v,
                                      kda_dtype qkv_dt, const float* g, const float* beta,
                                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                      int32_t N, const float* initial_state, const void* d_o,
                                      kda_dtype do_dt, const float* d_final_state, float* dq,
                                      float* dk, float* dv, float* dg, float* dbeta,
                                      float* d_initial_state, int64_t T_tot, int32_t H,
                                      int32_t dk_dim, int32_t dv_dim, float scale,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of kda_chunk_prefill_backward; 0 for unsupported arguments. */
size_t kda_chunk_prefill_backward_workspace_bytes(int64_t T_tot, int32_t N, int32_t H,
                                                  int32_t dk, int32_t dv);

/*
 * kda_chunk_prefill_workspace_bytes - workspace size for kda_chunk_prefill
 * processing up to chunks_per_pass chunks (of 64 tokens) of every sequence per
 * pass: a state carry of N*H*dk*dv*4 bytes plus N*H*chunks_per_pass images
 * of 60,416 bytes.  Returns 0 for unsupported or non-positive arguments.
 */
size_t kda_chunk_prefill_workspace_bytes(int32_t N, int32_t H, int32_t dk, int32_t dv,
                                         int32_t chunks_per_pass);

/*
 * kda_recurrent_decode - one token per sequence, state updated in place.
 *
 *   q, k  [N, H, dk], v [N, H, dv]   dtype qkv_dt (KDA_BF16 or KDA_F32)
 *   g     [N, H, dk] fp32, beta [N, H] fp32 (post-sigmoid)
 *   state [N, H, dk, dv] fp32, read and overwritten with S_t
 *   o     [N, H, dv] dtype o_dt
 * Requires dk == dv == 128.  state must not overlap q/k/v/g/beta/o.
 * All arithmetic is fp32.
 */
kda_status kda_recurrent_decode(const void* q, const void* k, const void* v, kda_dtype qkv_dt,
                                const float* g, const float* beta, float* state, void* o,
                                kda_dtype o_dt, int32_t N, int32_t H, int32_t dk, int32_t dv,
                                float scale, void* stream);

/*
 * kda_recurrent_decode_gated - the one-token step of kda_recurrent_decode for
 * serving: the gate fused in, the states in a pool of slots, fp32 or bf16.
 *
 *   q, k  [N, H, dk], v [N, H, dv]   dtype qkv_dt
 *   x     [N, H, dk] gate logits (x_dt), b [N, H] beta logits (b_dt),
 *         A_log [H] or [H, dk] fp32, dt_bias [H, dk] fp32: g and beta are formed per
 *         key channel with kda_gate's arithmetic and never stored
 *   state [num_slots, H, dk, dv] dtype state_dt, read and overwritten in place
 *   state_indices [N] int32 device array: sequence n uses state slot
 *         state_indices[n]; NULL means slot n (then num_slots >= N)
 *   o     [N, H, dv] dtype o_dt
 * A sequence whose slot lies outside [0, num_slots) (a padding entry, e.g.
 * -1) is skipped: its o is written as zeros and no state is read or written.
 * Two sequences of one call must not share a slot (their updates would race).
 * With state_dt KDA_BF16 every step rounds the updated state to bf16 (round to
 * nearest even); the arithmetic of the step is fp32 either way.  The gate's
 * inputs are FlashKDA's (Kimi K3 artifact audit, §7.1: bf16 inputs, fp32
 * A_log / dt_bias, a bf16 state mode, §7.4); the step is the code audit's fused
 * recurrent decode regime.  Requires dk == dv == 128.  Refusals: A_log_len
 * other than H or H*dk, or dt_bias_len != H*dk (KDA_ERR_SHAPE), num_slots < N without
 * indices (KDA_ERR_SHAPE), unaligned or overlapping tensors; the indices
 * themselves are device data and are bounds-checked by the kernel.
 */
kda_status kda_recurrent_decode_gated(const void* q, const void* k, const void* v,
                                      kda_dtype qkv_dt, const void* x, kda_dtype x_dt,
                                      const void* b, kda_dtype b_dt, const float* A_log,
                                      int64_t A_log_len, const float* dt_bias,
                                      int64_t dt_bias_len, void* state, kda_dtype state_dt,
                                      int64_t num_slots, const int32_t* state_indices, void* o,
                                      kda_dtype o_dt, int32_t N, int32_t H, int32_t dk,
                                      int32_t dv, float scale, void* stream);

/* activation after the short convolution */
enum { KDA_ACT_NONE = 0, KDA_ACT_SILU = 1 };

/*
 * kda_shortconv_l2norm - the KDA layer's prologue to the core: for each of
 * the q, k and v projections a causal depthwise convolution of kernel 4 per
 * channel, then (optionally) SiLU, then for q and k an L2 normalisation over
 * the d channels of every (token, head):
 *
 *   y[t, c] = sum_{i=0..3} w[c, i] x[t - 3 + i, c]
 *   y       = silu(y) = y / (1 + exp(-y))       if activation == KDA_ACT_SILU
 *   q, k    : y / sqrt(sum_c y[t, h, c]^2 + eps)
 *
 *   xq, xk, xv  [T_tot, H, d] dtype in_dt (packed varlen by cu_seqlens)
 *   wq, wk, wv  [H*d, 4] fp32 each, w_len = H*d*4 values: the checkpoint's
 *               q/k/v_conv1d.weight [H*d, 1, 4] (Kimi K3 artifact audit,
 *               §4.1: 12288 = 96 x 128 channels, kernel size 4); no bias
 *   yq, yk, yv  [T_tot, H, d] dtype out_dt
 *   conv_state_in / conv_state_out  [N, 3 (q, k, v), 3 (taps, oldest first),
 *               H*d] fp32: the 3 inputs before / the last 3 inputs of each
 *               sequence (NULL in: zeros; NULL out: not written).  A sequence
 *               shorter than 3 tokens carries the older state entries on, so
 *               a prefill followed by one-token calls with the state equals
 *               one longer prefill.  In place (in == out) is allowed only when
 *               every sequence has at most one token (the decode step).
 * The pages give the weight shapes only: the activation and eps are the
 * caller's (SiLU and 1e-6 are the usual choices).  Requires d == 128.
 * Refusals: w_len != H*d*4 (KDA_ERR_SHAPE), bad cu_seqlens_host,
 * overlapping outputs and inputs, unaligned tensors.
 */
kda_status kda_shortconv_l2norm(const void* xq, const void* xk, const void* xv, kda_dtype in_dt,
                                const float* wq, const float* wk, const float* wv, int64_t w_len,
                                int32_t activation, float eps, const int32_t* cu_seqlens,
                                const int32_t* cu_seqlens_host, int32_t N,
                                const float* conv_state_in, float* conv_state_out, void* yq,
                                void* yk, void* yv, kda_dtype out_dt, int64_t T_tot, int32_t H,
                                int32_t d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
