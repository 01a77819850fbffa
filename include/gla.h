/*
 * gla.h -- C ABI of the MI355X (gfx950) chunkwise gated-linear-attention library
 *          (libgla_mi355x.so).
 *
 * The operation (page "Gated Linear Attention Transformers with Hardware-Efficient
 * Training", atlas.scime.ai summary, section Approach): a linear-attention recurrent
 * state with the data-dependent low-rank gate G_t = alpha_t^T 1, evaluated with the
 * pages' I/O-aware chunkwise algorithm.  Per batch b and head h:
 *
 *     S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,     o_t = q_t S_t,     S_{-1} = S0,
 *     alpha_t = exp(log_alpha_t)  (0 < alpha <= 1, i.e. log_alpha <= 0),
 *
 * with S a dk x dv matrix.  The backward returns the gradient of a loss L through its
 * incoming gradients dO = dL/do and dS_T = dL/dS_T; the gate gradient uses the pages'
 * closed form (Approach: no per-step states are needed), the reverse cumulative sum
 * over time of q*dq - k*dk plus rowsum(dS_T * S_T).
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major, contiguous device buffers:
 *      q, k, dq, dk                          [B, H, T, dk]
 *      log_alpha, dlog_alpha                 [B, H, T, dk], or [B, H, T] with
 *                                            gate_shape GLA_GATE_SCALAR
 *      v, o, dO, dv                          [B, H, T, dv]
 *      S0, S_T, dS_T, dS0                    [B, H, dk, dv]   always float32
 *    The element type of the [B,H,T,*] tensors is desc->dtype (GLA_F32 or GLA_BF16).
 *    Base pointers must be 16-byte aligned.
 *  - The caller owns every buffer.  The library never allocates device memory: scratch
 *    space comes from the caller's workspace `ws` of at least gla_workspace_bytes()
 *    bytes (16-byte aligned; its contents on entry do not matter).
 *  - Outputs are overwritten, never accumulated, and must not alias any input.
 *  - Calls enqueue kernels on `stream` (a hipStream_t; NULL is the default stream) and
 *    return before they finish.  The library keeps no global mutable state (apart from
 *    the scratch array of gla_chunk_fwd_noalloc and its per-device address, set once),
 *    so calls are reentrant; two calls that share a workspace must be ordered on one
 *    stream.
 *  - Nullable pointers (marked) mean "zero" for inputs and "not wanted" for outputs.
 *  - Errors are reported by status code; no C++ exception crosses this boundary.  All
 *    argument checks run on the host before any launch, and on an error no output is
 *    touched.  Kernel-launch failures surface as GLA_ERR_DEVICE.
 *  - Preconditions that are not checked by default: log_alpha finite and <= 0 (gate
 *    logits: finite; a value breaking it gives unspecified output), inputs finite.  With
 *    GLA_DEBUG_CHECKS=1 in the environment (read once, at the first call),
 *    gla_chunk_fwd / gla_chunk_bwd (and their _traced and _noalloc forms) first count the
 *    gate elements that break it on the device (gla_check_gates, in a 256-byte region
 *    that the workspace always reserves), synchronize the stream, and return
 *    GLA_ERR_INVALID_ARG before any launch that touches an output if there are any.
 */
#ifndef GLA_MI355X_H
#define GLA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GLA_OK = 0,
  GLA_ERR_INVALID_ARG = 1,   /* NULL required pointer, negative size, bad enum, ...   */
  GLA_ERR_UNSUPPORTED = 2,   /* valid request outside what the kernels implement      */
  GLA_ERR_WORKSPACE = 3,     /* workspace NULL or smaller than gla_workspace_bytes()  */
  GLA_ERR_DEVICE = 4         /* a HIP call or kernel launch failed                    */
} gla_status_t;

typedef enum { GLA_F32 = 0, GLA_BF16 = 1 } gla_dtype_t;

/* How inter-chunk states are handled in the forward (Approach section: materialized or
 * non-materialized inter-chunk states).
 *  GLA_STATES_MATERIALIZED: every chunk-start state S_[i] is written to the workspace
 *    by the state-scan kernel, then a chunk-parallel kernel forms the outputs.
 *  GLA_STATES_RECOMPUTE: the state stays on chip; one kernel walks the chunks of a
 *    (batch, head, dv-slice) and emits the outputs directly (no per-chunk state tensor
 *    in memory).
 * The backward always recomputes the chunk-start states from the inputs (the API is
 * stateless); the mode only changes the forward. */
typedef enum { GLA_STATES_MATERIALIZED = 0, GLA_STATES_RECOMPUTE = 1 } gla_state_mode_t;

/* Passes of gla_validate / gla_workspace_bytes.  2 is gla_chunk_states; FWD_SAVE and
 * BWD_SAVED are the training pair gla_chunk_fwd_save / gla_chunk_bwd_saved. */
typedef enum {
  GLA_PASS_FWD = 0,
  GLA_PASS_BWD = 1,
  GLA_PASS_FWD_SAVE = 3,
  GLA_PASS_BWD_SAVED = 4
} gla_pass_t;

/* What the log_alpha argument of every entry point holds (Approach section: the gate is
 * data-dependent).
 *  GLA_GATE_LOG_ALPHA: log_alpha itself (finite, <= 0).
 *  GLA_GATE_LOGITS: gate logits x; the layer uses log_alpha = logsigmoid(x) / gate_tau
 *    (alpha = sigmoid(x)^(1/gate_tau), gate_tau > 0), formed inside the kernels that read
 *    the gates, and the backward's dlog_alpha output is the gradient with respect to x,
 *    dL/dlog_alpha * sigmoid(-x) / gate_tau. */
typedef enum { GLA_GATE_LOG_ALPHA = 0, GLA_GATE_LOGITS = 1 } gla_gate_t;

/* Shape of the gate (Experiments section of the same summary: its ablations compare the
 * fine-grained gate with a data-dependent scalar gate and with a data-independent scalar
 * decay, RetNet-style).
 *  GLA_GATE_PER_KEY: one gate per key dimension, log_alpha [B, H, T, dk] (the layer).
 *  GLA_GATE_SCALAR: one gate per token and head, log_alpha [B, H, T], shared by every
 *    row of the state: S_t = alpha_t S_{t-1} + k_t^T v_t.  A data-independent decay
 *    (RetNet-style, one constant per head) is the case of a value constant along t.
 *    dlog_alpha is [B, H, T]: the sum over the key dimension of the per-key gradient
 *    (times sigmoid(-x) / gate_tau with GLA_GATE_LOGITS).
 * gate (the meaning of the values) and gate_shape combine freely. */
typedef enum { GLA_GATE_PER_KEY = 0, GLA_GATE_SCALAR = 1 } gla_gate_shape_t;

/* Arithmetic of the diagonal 16 x 16 sub-blocks of the intra-chunk matrix A (Approach
 * section: with two-level chunking *most* intra-chunk products run on the half-precision
 * matrix units; the plainest reading of "most" is that the products between different
 * sub-chunks do, while the sub-blocks on the diagonal stay in full precision).
 *  GLA_DIAG_F32: fp32 throughout.  When the spread of the chunk-local cumulative log-gate
 *    inside every 16-row sub-block is at most 96 (in log2 units, per key dimension) the
 *    sub-block is an fp32 matrix product (v_mfma_f32_16x16x4_f32) of q and k rebased at
 *    the sub-block's first row: every factor exp(g_t - g_rho), exp(g_rho - g_s) is then a
 *    normal fp32 number, so each term carries fp32 rounding only.  Otherwise the exact
 *    log-space sum of q_td k_sd exp(g_td - g_sd) per (t, s, d) in fp32.  The default.
 *  GLA_DIAG_BF16: the same rebased product with bf16 operands (one bf16 MFMA per 32 key
 *    dimensions instead of eight fp32 ones); the operand rounding (2^-9 relative per
 *    factor) matches that of the off-diagonal sub-blocks.  Opt-in, for speed; bf16
 *    inputs only (fp32 inputs always take GLA_DIAG_F32). */
typedef enum { GLA_DIAG_F32 = 0, GLA_DIAG_BF16 = 1 } gla_diag_t;

typedef struct {
  int32_t B, H, T;     /* batch, heads, sequence length (any of them may be 0)          */
  int32_t dk, dv;      /* key and value head dimensions                                  */
  int32_t chunk;       /* chunk size C of the chunkwise form                             */
  int32_t subchunk;    /* secondary (sub-)chunk size c of the intra-chunk part           */
  int32_t dtype;       /* gla_dtype_t                                                    */
  int32_t state_mode;  /* gla_state_mode_t                                               */
  int32_t gate;        /* gla_gate_t (zero: log_alpha given directly)                      */
  float gate_tau;      /* temperature of GLA_GATE_LOGITS (> 0, finite); unused otherwise   */
  int32_t gate_shape;  /* gla_gate_shape_t (zero: one gate per key dimension)              */
  int32_t diag;        /* gla_diag_t (zero: fp32 diagonal sub-blocks)                      */
} gla_desc_t;

/* Supported by this build (else GLA_ERR_UNSUPPORTED):
 *   chunk in {64, 128}; subchunk == 16; dk in {64, 128, 192, 256};
 *   dv a multiple of 64 up to 1024; fp32 only with chunk 64; B*H <= 65535;
 *   B*H*T < 2^31; ceil(T/chunk) <= 65535; any T >= 0 (a ragged last chunk is masked). */

/* Human-readable name of a status code (static string, never NULL). */
const char* gla_status_string(gla_status_t status);

/* Library version as 10000*major + 100*minor + patch. */
int32_t gla_version(void);

/* Host-only validation of a descriptor for a pass (no device call).  Returns GLA_OK,
 * GLA_ERR_INVALID_ARG (desc NULL, a negative size, chunk or subchunk < 1,
 * chunk % subchunk != 0, unknown dtype/mode/pass/gate/gate_shape/diag, GLA_GATE_LOGITS with
 * gate_tau not a positive finite number) or GLA_ERR_UNSUPPORTED. */
gla_status_t gla_validate(const gla_desc_t* desc, int32_t pass);

/* Workspace bytes needed by gla_chunk_fwd (pass = GLA_PASS_FWD), gla_chunk_bwd
 * (GLA_PASS_BWD), gla_chunk_states (pass = 2), gla_chunk_fwd_save (GLA_PASS_FWD_SAVE) or
 * gla_chunk_bwd_saved (GLA_PASS_BWD_SAVED) for `desc`; writes them to *bytes.  Host-only;
 * same errors as gla_validate, plus GLA_ERR_INVALID_ARG for bytes == NULL. */
gla_status_t gla_workspace_bytes(const gla_desc_t* desc, int32_t pass, size_t* bytes);

/* Gate precondition check (the layer reads log_alpha as finite and <= 0, gate logits as
 * finite; see the gate fields of gla_desc_t): *n_bad (host) = the number of elements of
 * log_alpha ([B,H,T,dk], or [B,H,T] with scalar gates; element type desc->dtype) that
 * break it.  ws: device scratch of at least 8 bytes (its first 8 bytes are overwritten).
 * Synchronous: the stream is synchronized before return.  Errors: as gla_validate;
 * GLA_ERR_INVALID_ARG for n_bad == NULL or a NULL or misaligned log_alpha (B*H*T > 0);
 * GLA_ERR_WORKSPACE for ws == NULL or ws_bytes < 8. */
gla_status_t gla_check_gates(const gla_desc_t* desc, const void* log_alpha, void* ws,
                             size_t ws_bytes, int64_t* n_bad, void* stream);

/* Gate log-cumsum (the first step of the chunkwise form, Approach section):
 *   g[b,h,t,:] = sum of log_alpha[b,h,u,:] over u from the start of t's chunk to t,
 *   gamma[b,h,i,:] = g at the last row of chunk i (a ragged last chunk ends at T-1).
 * g: float32 [B,H,T,dk]; gamma: float32 [B,H,ceil(T/chunk),dk] (with a scalar gate the
 * dk entries of a row are equal). */
gla_status_t gla_gate_cumsum(const gla_desc_t* desc, const void* log_alpha,
                             float* g, float* gamma, void* stream);

/* Inter-chunk state recurrence with materialized states (Approach section):
 *   S_[0] = S0,  S_[i+1] = diag(exp(gamma_i)) S_[i] + (K_i * exp(gamma_i - g_i))^T V_i,
 * writes states[b,h,i,:,:] = S_[i] for i < N = ceil(T/chunk) (float32
 * [B,H,N,dk,dv]) and S_T = S_[N] (nullable).  S0 nullable (zero). */
gla_status_t gla_chunk_states(const gla_desc_t* desc, const void* k, const void* v,
                              const void* log_alpha, const float* S0, float* states,
                              float* S_T, void* ws, size_t ws_bytes, void* stream);

/* Forward of the layer.  Inputs q, k, v, log_alpha, S0 (nullable: zero).
 * Outputs o (required) and S_T (nullable). */
gla_status_t gla_chunk_fwd(const gla_desc_t* desc, const void* q, const void* k,
                           const void* v, const void* log_alpha, const float* S0,
                           void* o, float* S_T, void* ws, size_t ws_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * computation and kernels as gla_chunk_fwd, with its scratch space taken from a fixed
 * device array of GLA_NOALLOC_SCRATCH_BYTES inside the library instead of a workspace.
 * The caller still passes every input and output.  The array is placed on a device at
 * the first call there and held until the process ends; every call on one device uses
 * that device's array, so calls that overlap on one device (other streams, other host
 * threads) race on it and must be ordered by the caller.  Its contents on entry do not
 * matter (every byte the kernels read is written first in the same call).  A problem
 * whose gla_workspace_bytes(desc, GLA_PASS_FWD) exceeds GLA_NOALLOC_SCRATCH_BYTES is
 * GLA_ERR_WORKSPACE, returned before the device is touched; other errors as for
 * gla_chunk_fwd.  No device memory is allocated or freed by this call. */
#define GLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gla_status_t gla_chunk_fwd_noalloc(const gla_desc_t* desc, const void* q, const void* k,
                                   const void* v, const void* log_alpha, const float* S0,
                                   void* o, float* S_T, void* stream);

/* Backward of the layer for the loss gradient (dO, dS_T).  Inputs q, k, v, log_alpha,
 * S0 (nullable), dO (required), dS_T (nullable: zero).  Outputs dq, dk, dv,
 * dlog_alpha (required) and dS0 (nullable). */
gla_status_t gla_chunk_bwd(const gla_desc_t* desc, const void* q, const void* k,
                           const void* v, const void* log_alpha, const float* S0,
                           const void* dO, const float* dS_T, void* dq, void* dk,
                           void* dv, void* dlog_alpha, float* dS0, void* ws,
                           size_t ws_bytes, void* stream);

/* Training pair: a forward that keeps what the backward would otherwise recompute, and a
 * backward that starts from it (page "Gated Linear Attention Transformers with
 * Hardware-Efficient Training", atlas.scime.ai summary, Approach: what to keep from the
 * forward pass and what to recompute in the backward is a trade of memory against work;
 * the chunk states themselves are still recomputed by the backward's scans).
 *
 * gla_chunk_fwd_save: gla_chunk_fwd with the recomputed-states forward only
 * (state_mode GLA_STATES_RECOMPUTE, else GLA_ERR_UNSUPPORTED), whose intra-chunk kernel also
 * writes the backward's intra-chunk operands into `saved` (device, 16-byte aligned, at least
 * gla_saved_bytes(desc) bytes, caller-owned; contents opaque): the decayed causal matrix A,
 * Q*e^g token-major and transposed, K*e^(gamma-g) token-major and transposed (the
 * transposed ones as the backward's scans read them: bf16 inputs as a bf16 high part and
 * bf16 remainder) and e^gamma.  o and S_T are bit for bit those of gla_chunk_fwd (with bf16
 * inputs the forward's later kernels read the high parts of the transposed keys alone,
 * the bf16 rounding gla_chunk_fwd stores).
 * ws: at least gla_workspace_bytes(desc, GLA_PASS_FWD_SAVE) bytes.
 *
 * gla_chunk_bwd_saved: gla_chunk_bwd without its intra-chunk kernel, reading those operands
 * from `saved` as written by gla_chunk_fwd_save for the same desc and the same q, k,
 * log_alpha (not checked; anything else gives wrong gradients).  The results are the bits
 * gla_chunk_bwd returns for the same inputs.  ws: at least
 * gla_workspace_bytes(desc, GLA_PASS_BWD_SAVED) bytes.
 *
 * Errors: as gla_chunk_fwd / gla_chunk_bwd; GLA_ERR_WORKSPACE also for a NULL or short
 * `saved` (B*H*T > 0).  The stream orders the pair: saved is written by the forward's
 * first kernel and read by the backward's kernels. */
gla_status_t gla_saved_bytes(const gla_desc_t* desc, size_t* bytes);

gla_status_t gla_chunk_fwd_save(const gla_desc_t* desc, const void* q, const void* k,
                                const void* v, const void* log_alpha, const float* S0,
                                void* o, float* S_T, void* saved, size_t saved_bytes,
                                void* ws, size_t ws_bytes, void* stream);

gla_status_t gla_chunk_bwd_saved(const gla_desc_t* desc, const void* q, const void* k,
                                 const void* v, const void* log_alpha, const float* S0,
                                 const void* dO, const float* dS_T, void* dq, void* dk,
                                 void* dv, void* dlog_alpha, float* dS0, const void* saved,
                                 size_t saved_bytes, void* ws, size_t ws_bytes,
                                 void* stream);

/* Recurrent evaluation, for decoding (page "Gated Slot Attention for Efficient
 * Linear-Time Sequence Modeling", mlsanity.com summary, Abstract: linear attention and its
 * gated variants infer recurrently; here the layer's own recurrence, one state per
 * (b, h) carried from token to token).  For every (b, h) and t = 0 .. T-1 in order:
 *     S <- diag(exp(log_alpha[b,h,t,:])) S + k[b,h,t,:]^T v[b,h,t,:],
 *     o[b,h,t,:] = q[b,h,t,:] S,
 * with S float32 [B,H,dk,dv], read and updated in place (required; it is both input and
 * output, the one exception to the no-alias rule).  q, k, log_alpha [B,H,T,dk] ([B,H,T]
 * with a scalar gate) and v [B,H,T,dv] are inputs, o [B,H,T,dv] the output (all
 * desc->dtype).  T is typically 1:
 * one new token per sequence; the state is read and written once per call whatever T
 * is, every step in fp32.  desc->chunk, subchunk and state_mode are not used, and no
 * workspace is needed.  B*H == 0 or T == 0 is a no-op.
 * Supported: dk a multiple of 32 in [32, 256]; dv a multiple of 32 in [32, 1024];
 * B*H*(dv/32) and B*H*T below 2^31 (else GLA_ERR_UNSUPPORTED).  A NULL or misaligned
 * pointer is GLA_ERR_INVALID_ARG. */
gla_status_t gla_decode(const gla_desc_t* desc, const void* q, const void* k, const void* v,
                        const void* log_alpha, float* S, void* o, void* stream);

/* Gated Slot Attention (page "Gated Slot Attention for Efficient Linear-Time Sequence
 * Modeling", mlsanity.com summary, Abstract: m memory slots forgotten by a GLA-style gate,
 * read with a softmax; two GLA passes joined by a softmax).  Per batch b and head h, with
 * per-slot gates alpha_t = exp(log_alpha[b,h,t,:]) in (0,1]^m and w_t = 1 - alpha_t:
 *
 *     Kt_t = diag(alpha_t) Kt_{t-1} + w_t^T k_t,   Vt_t = diag(alpha_t) Vt_{t-1} + w_t^T v_t,
 *     o_t  = softmax(Kt_t q_t)^T Vt_t     (softmax over the m slots; Kt, Vt start at zero)
 *
 * q, k [B,H,T,dk], v, o, dO, dv [B,H,T,dv], log_alpha, dlog_alpha [B,H,T,slots], all of
 * element type desc->dtype, contiguous, 16-byte aligned, caller-owned.  GLA_F32: fp32
 * throughout.  GLA_BF16: the first pass (slot scores) in fp32 on fp32 copies of q, k and
 * log_alpha; softmax(scores) and 1 - alpha enter the second pass (the layer's bf16 path)
 * rounded to bf16, whose gradients return in bf16; the softmax backward, the first pass's
 * backward and the gate-gradient sum in fp32; outputs rounded to nearest even.
 * Scratch comes from `ws` (gla_gsa_workspace_bytes); no state is carried in or out.
 * Supported: dk and slots in {64, 128, 192, 256}, dv a multiple of 64 up to 1024,
 * B*H <= 65535, B*H*T < 2^31; B*H*T == 0 is a no-op.  Errors as for the layer's entry
 * points; everything is checked on the host before any launch. */
typedef struct {
  int32_t B, H, T;
  int32_t dk, dv;
  int32_t slots;   /* m, the number of memory slots */
  int32_t dtype;   /* gla_dtype_t: GLA_F32 or GLA_BF16 */
} gla_gsa_desc_t;

gla_status_t gla_gsa_validate(const gla_gsa_desc_t* desc);
/* pass: GLA_PASS_FWD or GLA_PASS_BWD. */
gla_status_t gla_gsa_workspace_bytes(const gla_gsa_desc_t* desc, int32_t pass, size_t* bytes);
/* o (required) from q, k, v, log_alpha. */
gla_status_t gla_gsa_fwd(const gla_gsa_desc_t* desc, const void* q, const void* k,
                         const void* v, const void* log_alpha, void* o, void* ws,
                         size_t ws_bytes, void* stream);
/* dq, dk, dv, dlog_alpha (all required) for the loss gradient dO; recomputes the forward. */
gla_status_t gla_gsa_bwd(const gla_gsa_desc_t* desc, const void* q, const void* k,
                         const void* v, const void* log_alpha, const void* dO, void* dq,
                         void* dk, void* dv, void* dlog_alpha, void* ws, size_t ws_bytes,
                         void* stream);

/* Stage tracing, for profiling.  The *_traced variants behave exactly like
 * gla_chunk_fwd / gla_chunk_bwd / gla_chunk_fwd_save / gla_chunk_bwd_saved and
 * additionally record caller-created hipEvent_t
 * handles on `stream`: events[j] right before the j-th kernel launch and events[n] after
 * the last, where n is the stage count from gla_trace_stages (events == NULL records
 * nothing; a NULL entry records nothing at its boundary, so two events time one stage
 * with the least disturbance).  The elapsed time between events[j] and events[j+1] is the
 * duration of stage j.  n_events smaller than n + 1 is GLA_ERR_INVALID_ARG (checked
 * before any launch).
 *
 * gla_trace_stages returns n for a pass (GLA_PASS_FWD, GLA_PASS_BWD, GLA_PASS_FWD_SAVE,
 * GLA_PASS_BWD_SAVED; with_dS_T: whether the backward gets a dS_T) and writes up to
 * max_names static stage names to `names` (nullable); -1 on a NULL desc or a bad pass.
 * The forward that saves has the recompute forward's stages (its intra-chunk kernel
 * writes more), the backward from saved operands the backward's without intra.  The
 * stages are
 *   forward, materialized: intra (it forms the gate cumsum itself), state_scan (in
 *                          sequence segments when few workgroups would walk the whole
 *                          sequence), output
 *   forward, recompute:    intra, seg_state (bf16, at least 4 chunks: the states at the
 *                          starts of the sequence segments that the fused kernel walks in
 *                          parallel, and their chaining; no launch otherwise), fwd_fused
 *   backward:              intra, state_scans (the forward and the reverse scan, in one
 *                          launch, or in sequence segments when few workgroups would walk
 *                          them), [state_dot when dS_T is given], gate_tot, bwd_dqk_dv
 *                          (dq/dk/dlog_alpha and dv workgroups: one launch at chunk 64,
 *                          two at chunk 128), and with
 *                          scalar gates gate_reduce (the gradient summed over dk) */
int32_t gla_trace_stages(const gla_desc_t* desc, int32_t pass, int32_t with_dS_T,
                         const char** names, int32_t max_names);

gla_status_t gla_chunk_fwd_traced(const gla_desc_t* desc, const void* q, const void* k,
                                  const void* v, const void* log_alpha, const float* S0,
                                  void* o, float* S_T, void* ws, size_t ws_bytes, void* stream,
                                  void** events, int32_t n_events);

gla_status_t gla_chunk_bwd_traced(const gla_desc_t* desc, const void* q, const void* k,
                                  const void* v, const void* log_alpha, const float* S0,
                                  const void* dO, const float* dS_T, void* dq, void* dk,
                                  void* dv, void* dlog_alpha, float* dS0, void* ws,
                                  size_t ws_bytes, void* stream, void** events,
                                  int32_t n_events);

gla_status_t gla_chunk_fwd_save_traced(const gla_desc_t* desc, const void* q, const void* k,
                                       const void* v, const void* log_alpha, const float* S0,
                                       void* o, float* S_T, void* saved, size_t saved_bytes,
                                       void* ws, size_t ws_bytes, void* stream, void** events,
                                       int32_t n_events);

gla_status_t gla_chunk_bwd_saved_traced(const gla_desc_t* desc, const void* q, const void* k,
                                        const void* v, const void* log_alpha, const float* S0,
                                        const void* dO, const float* dS_T, void* dq, void* dk,
                                        void* dv, void* dlog_alpha, float* dS0,
                                        const void* saved, size_t saved_bytes, void* ws,
                                        size_t ws_bytes, void* stream, void** events,
                                        int32_t n_events);

#ifdef __cplusplus
}
#endif

#endif /* GLA_MI355X_H */
