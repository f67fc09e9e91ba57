/*
 * gdn2.h -- C ABI of the MI355X (gfx950) Gated DeltaNet-2 core library, libgdn2.so.
 *
 * The method (burn-gdn2 0.1.5 docs page, section "Architecture"): per sequence and per
 * value head, a matrix state S in R^{d_k x d_v} follows
 *
 *     S_t = (I - k_t (b_t . k_t)^T) diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T
 *     o_t = q_t^T S_t
 *
 * with alpha_t the channel-wise decay and b_t the erase gate on the key axis, and w_t the
 * write gate on the value axis. The same page names two ways to run it, and this library
 * exports one call for each:
 *   - gdn2_chunk_fwd       the chunked WY-decomposition forward ("Chunk" mode, training and
 *                          prefill; chunk_size defaults to 64 on that page);
 *   - gdn2_recurrent_step  one fused token-by-token step ("FusedRecurrent" mode, decode),
 *                          which reads and writes a persistent state in place as the
 *                          GDN decode verify page (LocalAI mirror), section 2, describes.
 * Around them (each declared below with its own description):
 *   - gdn2_recurrent_fwd        several tokens per call against a pool of fp32 or bf16
 *                               states, with optional fused prologue and epilogue;
 *   - gdn2_chunk_bwd, gdn2_chunk_bwd_states
 *                               the gradients of the chunked forward (recomputing the
 *                               chunk states, or from those a training forward saved);
 *   - gdn2_map_gates, gdn2_map_gates_bwd
 *                               the inputs of other delta-rule variants (KDA, GDN,
 *                               FG2-GDN, FG2-GDN+) mapped onto these, and their gradients
 *                               mapped back;
 *   - gdn2_chunk_fwd_noalloc    the chunked forward on a static device workspace, for
 *                               callers that cannot allocate.
 *
 * Conventions (the pages are silent on these; this is the reading the library implements):
 *   - o_t reads the state AFTER the update of token t.
 *   - The decay argument carries log(alpha) <= 0, in the input dtype; the kernels take exp.
 *   - No query scaling (a caller wanting 1/sqrt(d_k) pre-scales q; o is linear in q).
 *   - Grouped value attention: value head h reads key head h / (h_v / h_k)
 *     (burn-gdn2 "num_v_heads"; the llama.cpp notes' 48 value heads over 16 key groups).
 *   - The negative-eigenvalue option of burn-gdn2 (allow_neg_eigval, "b x 2") is the
 *     caller's b in (0,2); the library has no flag for it.
 *
 * Layouts (all contiguous, last dimension fastest):
 *   q, k          [B, T, h_k, d_k]      input dtype
 *   v, w, o       [B, T, h_v, d_v]      input dtype (o is written in the input dtype)
 *   log_alpha, b  [B, T, h_v, d_k]      input dtype
 *   S0, S_T, S    [N, h_v, d_k, d_v]    fp32 always, d_v fastest
 * A packed (variable-length) batch uses B = 1, T = total tokens and cu_seqlens (int32,
 * N + 1 offsets, device memory): sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1.
 * Without cu_seqlens the batch is dense: N = B sequences of T tokens each.
 *
 * Ownership: the caller allocates every buffer (inputs, outputs, workspace, state). The
 * library allocates no device memory and keeps no state between calls apart from the
 * thread-local error message.
 *
 * Streams: every call only enqueues work on `stream` (a hipStream_t; NULL is the default
 * stream) and returns without synchronising. No call reads device memory on the host.
 * The work enqueued is kernel launches only (no allocation, copy, fill or host
 * synchronisation), so a caller may capture the calls into a HIP graph and replay it; a
 * replay reads and writes the buffers given at capture time.
 *
 * Errors: arguments are validated on the host before anything is enqueued; a failed check
 * returns a status code and launches nothing. A failed launch returns GDN2_ERR_HIP. A short
 * message for the last failure of the calling thread is available from gdn2_last_error().
 * Device-side contents (cu_seqlens values, NaN/Inf in the data) are not checked: NaN and
 * Inf propagate into the affected (sequence, head) outputs.
 */
#ifndef GDN2_H
#define GDN2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN2_ABI_VERSION 9

typedef enum gdn2_status {
    GDN2_OK = 0,
    GDN2_ERR_NULL_ARG = 1,      /* a required pointer is NULL */
    GDN2_ERR_BAD_SHAPE = 2,     /* a dimension is out of range or inconsistent */
    GDN2_ERR_UNSUPPORTED = 3,   /* valid but not built: head dims, chunk size, dtype */
    GDN2_ERR_WORKSPACE = 4,     /* workspace missing or smaller than required */
    GDN2_ERR_HIP = 5            /* the HIP runtime reported an error */
} gdn2_status;

typedef enum gdn2_dtype {
    GDN2_F32 = 0,               /* fp32 inputs and o; fp32 arithmetic throughout */
    GDN2_BF16 = 1               /* bf16 inputs and o; bf16 matrix-core operands, fp32
                                   accumulation, fp32 state */
} gdn2_dtype;

typedef enum gdn2_state_dtype {
    GDN2_STATE_F32 = 0,         /* fp32 recurrent state */
    GDN2_STATE_BF16 = 1         /* bf16 recurrent state: widened to fp32 for the update inside
                                   a call, rounded to nearest even when written back */
} gdn2_state_dtype;

/*
 * Optional fusions of the stages the burn-gdn2 page (section "Architecture") draws around
 * the recurrence: the L2-Norm of q and k before it, and the Gated RMS Norm with a SiLU
 * gate after it (its Configuration table gives norm_eps = 1e-5). Pass NULL for none.
 *
 *   qk_l2norm    nonzero: every q and k vector (one token of one key head, d_k values) is
 *                replaced by x / sqrt(sum_c x_c^2 + l2norm_eps) before it is used
 *   l2norm_eps   >= 0 (1e-6 is a usual choice; with 0 an all-zero vector gives NaN)
 *   gate         NULL, or a device tensor shaped like o ([.., h_v, d_v], input dtype): the
 *                output becomes  o / sqrt(mean_c o_c^2 + norm_eps) * norm_weight * silu(gate)
 *                per (token, value head), silu(g) = g / (1 + exp(-g)); must not alias o
 *   norm_weight  device fp32 [d_v], required with a gate (shared by all value heads)
 *   norm_eps     >= 0
 *
 * gdn2_recurrent_fwd only: the short causal depthwise convolution that the same diagram
 * puts before the L2-Norm (burn-gdn2 use_short_conv; the GDN decode verify page, section 1,
 * give its kernel width 4, and section 2 its state of the last 3 inputs per channel, kept
 * in the recurrent cache and read and written back every step). The convolved channels are
 * q, k and v, C = 2 h_k d_k + h_v d_v of them in that order (q of key head 0..h_k-1, then
 * k likewise, then v of value head 0..h_v-1, each head's d values contiguous):
 *   conv_weight  NULL: no convolution. Else device fp32 [C][4]; tap 3 multiplies the
 *                current token, tap 0 the input three tokens back
 *   conv_state   device fp32 [num_slots][3][C], the last three inputs of each channel
 *                (oldest first), on the same slots as the recurrent state; read and updated
 *                in place
 *   conv_silu    nonzero: y = silu(conv(x)); zero: y = conv(x)
 * The convolved q and k are what the L2-norm (if on) and the recurrence see.
 *
 *   gate_mode    0: b and w are the GDN-2 gates. A gdn2_gate_mode (see gdn2_map_gates):
 *                the call runs that variant with its gate mapping fused into the kernels,
 *                reading the variant's own gates (no mapping pass, no mapped tensors):
 *                  GDN2_GATES_KDA       b = beta [.., h_v]; w unused (may be NULL)
 *                  GDN2_GATES_GDN       as KDA, and log_alpha [.., h_v] (one per head)
 *                  GDN2_GATES_FG2       b = beta [.., h_v, d_k], d_v = d_k; w unused
 *                  GDN2_GATES_FG2_PLUS  b = beta [.., h_v, d_k], w = beta_v [.., h_v, d_v]
 *                The FG2 modes scale the keys by sqrt(beta) inside the kernels, so they
 *                take neither qk_l2norm nor the short convolution (GDN2_ERR_UNSUPPORTED).
 *
 * gdn2_chunk_fwd only (the recurrent calls return GDN2_ERR_UNSUPPORTED when it is set):
 *   chunk_states NULL, or device fp32 [num_chunks][h_v][d_k][d_v]: the state entering
 *                every chunk of every sequence, the quantity the chunked form hands from one
 *                chunk to the next (burn-gdn2 docs page, "Architecture", Chunk WY mode): a
 *                training backward recomputes each chunk from it, and a serving cache can
 *                resume any sequence at a chunk boundary from it. Chunk j of sequence n is
 *                entry n * ceil(T / chunk_size) + j of a dense batch, and entry
 *                sum_{m < n} ceil(len_m / chunk_size) + j of a packed one (len_m =
 *                cu_seqlens[m+1] - cu_seqlens[m]); entry j holds the state after the first
 *                j * chunk_size tokens of the sequence (entry 0: S0, or zeros). The caller
 *                owns it; it must not overlap any input, output or the workspace.
 */
typedef struct gdn2_fusion {
    int32_t qk_l2norm;
    float l2norm_eps;
    const void *gate;
    const float *norm_weight;
    float norm_eps;
    const float *conv_weight;
    float *conv_state;
    int32_t conv_silu;
    int32_t gate_mode;
    float *chunk_states;
} gdn2_fusion;

typedef struct gdn2_dims {
    int32_t batch;      /* dense: number of sequences B. packed: must be 1.
                           recurrent step: number of sequences N. */
    int32_t seqlen;     /* dense: tokens per sequence T (>= 0). packed: total tokens.
                           recurrent step: must be 1. */
    int32_t num_seqs;   /* packed: N, the number of sequences (cu_seqlens has N+1 entries).
                           dense and recurrent step: ignored. */
    int32_t h_k;        /* key/query heads (>= 1) */
    int32_t h_v;        /* value heads, a multiple of h_k */
    int32_t d_k;        /* key head dim: 64 or 128 */
    int32_t d_v;        /* value head dim: 64 or 128 */
    int32_t dtype;      /* gdn2_dtype */
} gdn2_dims;

/* Library ABI version (GDN2_ABI_VERSION of the build). */
int32_t gdn2_abi_version(void);

/* Static text for a status code. */
const char *gdn2_status_string(int32_t status);

/* Message of the last failing call made by this thread ("" if none). */
const char *gdn2_last_error(void);

/*
 * Bytes of device workspace gdn2_chunk_fwd needs for these dims and chunk size, or 0 if
 * the dims or the chunk size are invalid. For a packed batch the size uses the upper bound
 * ceil(T / chunk_size) + N on the number of chunks, so it depends only on the dims.
 */
size_t gdn2_chunk_fwd_workspace_bytes(const gdn2_dims *dims, int32_t chunk_size);

/*
 * Chunked WY forward over a whole batch (burn-gdn2 docs page, "Chunk" mode of the
 * Architecture section; chunk_size as in its Configuration table).
 *
 *   q, k, v, log_alpha, b, w   device inputs in the layouts above (dims->dtype)
 *   S0          device fp32 [N, h_v, d_k, d_v] initial states, or NULL for zero states
 *   cu_seqlens  device int32 [N+1] for a packed batch, or NULL for a dense batch.
 *               Precondition (not checked on the device): cu_seqlens[0] = 0,
 *               non-decreasing, cu_seqlens[N] = T. Zero-length sequences are allowed and
 *               return S_T = S0 (or zeros).
 *   chunk_size  32, 64 or 128 tokens per chunk of the WY form (results do not depend on
 *               it beyond rounding). Every dtype and head-dim pair is built at every size.
 *   o           device output [B, T, h_v, d_v] in the input dtype; must not alias inputs
 *   S_T         device fp32 [N, h_v, d_k, d_v] final states, or NULL to skip them. S_T may
 *               be the same buffer as S0 (in-place continuation); no other aliasing.
 *   workspace   device buffer of at least gdn2_chunk_fwd_workspace_bytes() bytes, 256-byte
 *               aligned; its contents on entry are ignored and are clobbered.
 *   fusion      NULL, or the optional q/k L2-norm and gated output norm (gdn2_fusion);
 *               the gate is [B, T, h_v, d_v]. A short convolution is not built for this
 *               call (GDN2_ERR_UNSUPPORTED)
 *   stream      hipStream_t the work is enqueued on
 * Returns GDN2_OK or an error status (nothing is enqueued on a validation error).
 */
gdn2_status gdn2_chunk_fwd(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *b, const void *w,
                           const float *S0, const int32_t *cu_seqlens, int32_t chunk_size,
                           void *o, float *S_T, const gdn2_dims *dims,
                           void *workspace, size_t workspace_bytes,
                           const gdn2_fusion *fusion, void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. gdn2_chunk_fwd with the same arguments
 * minus the workspace, which comes instead from a static device array of
 * GDN2_STATIC_WORKSPACE_BYTES (128 MiB) that the library holds on every GPU it runs on
 * until the process ends. The call allocates nothing (no hipMalloc, no allocating library
 * routine); the caller still allocates the inputs and outputs.
 *   - Calls whose gdn2_chunk_fwd_workspace_bytes() exceeds GDN2_STATIC_WORKSPACE_BYTES
 *     return GDN2_ERR_WORKSPACE and enqueue nothing (128 MiB holds, for instance, a bf16
 *     batch of 4,096 tokens x 16 heads at d = 128 with chunk_size 64).
 *   - Every call on one GPU uses that GPU's one array, and the array keeps the last call's
 *     contents (none of which a later call reads). Calls that can overlap in time on one
 *     GPU -- issued to different streams with no ordering between them -- race on the
 *     array and give undefined results; order them on one stream (or with events).
 *   - The device is the stream's (the current device for a NULL stream). The first call on
 *     a device looks the array's address up once (hipGetSymbolAddress); later calls reuse it.
 * Results are those of gdn2_chunk_fwd (the same kernels run).
 */
#define GDN2_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)

gdn2_status gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                   const void *log_alpha, const void *b, const void *w,
                                   const float *S0, const int32_t *cu_seqlens,
                                   int32_t chunk_size, void *o, float *S_T,
                                   const gdn2_dims *dims, const gdn2_fusion *fusion,
                                   void *stream);

/*
 * Bytes of device workspace gdn2_chunk_bwd needs for these dims and chunk size, or 0 if
 * the dims are invalid (same upper bound on the chunks of a packed batch as the forward).
 */
size_t gdn2_chunk_bwd_workspace_bytes(const gdn2_dims *dims, int32_t chunk_size);

/*
 * Gradients of gdn2_chunk_fwd (without fusion options, GDN-2 gates) with respect to every
 * input and the initial state, taken through the chunked form of the burn-gdn2 docs page
 * ("Architecture", Chunk mode; its Chunk WY training path): the forward is re-run to store
 * the state entering every chunk, then one pass runs the state gradient backward over the
 * chunks, and one pass per chunk forms the input gradients. Built for bf16 inputs (bf16
 * matrix-core products, fp32 accumulation) and fp32 inputs (fp32 products) at every
 * supported head-dim pair.
 *
 *   q .. w, S0, cu_seqlens, dims   as for gdn2_chunk_fwd
 *   chunk_size  32, 64 or 128: the chunk size of the forward call whose gradients these are.
 *               The chunked form computes the same function at every chunk size, so the
 *               gradients do not depend on it; all three are computed with 64-token chunks
 *               (the same bits). Other values return GDN2_ERR_UNSUPPORTED.
 *   dO          device [B, T, h_v, d_v] in the input dtype: dL/do
 *   dS_T        device fp32 [N, h_v, d_k, d_v]: dL/dS_T, or NULL for zero
 *   dq, dk      device fp32 [B, T, h_k, d_k]   (value heads that share a key head add up,
 *               with fp32 atomics: when h_v > h_k the summation order, and so the last bits,
 *               may differ between runs; with h_v == h_k they are stored, and every call
 *               gives the same bits)
 *   dv, dw      device fp32 [B, T, h_v, d_v]
 *   dlog_alpha, db   device fp32 [B, T, h_v, d_k]
 *   dS0         device fp32 [N, h_v, d_k, d_v]: dL/dS0 (written also when S0 is NULL)
 *   workspace   at least gdn2_chunk_bwd_workspace_bytes() bytes, 256-byte aligned
 * Outputs must not alias inputs or each other. Every output is overwritten.
 * Returns GDN2_OK or an error status (nothing is enqueued on a validation error).
 */
gdn2_status gdn2_chunk_bwd(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *b, const void *w,
                           const float *S0, const int32_t *cu_seqlens, int32_t chunk_size,
                           const void *dO, const float *dS_T, float *dq, float *dk, float *dv,
                           float *dw, float *dlog_alpha, float *db, float *dS0,
                           const gdn2_dims *dims, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * gdn2_chunk_bwd for a forward that saved the state entering every chunk (its
 * gdn2_fusion.chunk_states, taken with chunk_size 64 on the same inputs, S0 and layout):
 * the chunked form hands exactly that state from one chunk to the next (burn-gdn2 docs page,
 * "Architecture", Chunk WY training path), so the backward uses it instead of re-running
 * the serial pass over the chunks. Gradients equal gdn2_chunk_bwd's (the same bits when no
 * value heads share a key head). chunk_size must be 64 (GDN2_ERR_UNSUPPORTED otherwise);
 * with fp32 inputs the states are recomputed and chunk_states is only checked.
 *
 *   chunk_states  device fp32 [num_chunks][h_v][d_k][d_v], the layout of
 *                 gdn2_fusion.chunk_states; read only; must not alias an output
 *   other arguments, the workspace size and the error behaviour as for gdn2_chunk_bwd
 */
gdn2_status gdn2_chunk_bwd_states(const void *q, const void *k, const void *v,
                                  const void *log_alpha, const void *b, const void *w,
                                  const float *S0, const int32_t *cu_seqlens, int32_t chunk_size,
                                  const float *chunk_states, const void *dO, const float *dS_T,
                                  float *dq, float *dk, float *dv, float *dw, float *dlog_alpha,
                                  float *db, float *dS0, const gdn2_dims *dims, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * One decode step for N sequences, one token each (burn-gdn2 "FusedRecurrent" mode; the
 * GDN decode verify page, section 2, describes the same fused state read-update-write).
 *
 *   q, k          device [N, h_k, d_k]   (dims->batch = N, dims->seqlen = 1)
 *   v, w          device [N, h_v, d_v]
 *   log_alpha, b  device [N, h_v, d_k]
 *   S             device fp32 [N, h_v, d_k, d_v], read and updated in place
 *   o             device [N, h_v, d_v] in the input dtype; must not alias any input or S
 *   stream        hipStream_t
 * Each state is read from memory once and written once.
 */
gdn2_status gdn2_recurrent_step(const void *q, const void *k, const void *v,
                                const void *log_alpha, const void *b, const void *w,
                                float *S, void *o, const gdn2_dims *dims, void *stream);

/*
 * Multi-token recurrent forward against a state cache (burn-gdn2 "FusedRecurrent" mode run
 * over T tokens). The GDN decode verify page (LocalAI mirror) describes, in section 2, the
 * recurrent cache whose slots hold one state per sequence and are read and written back
 * every step, and a fused kernel that keeps its share of a state in registers across the
 * tokens of the call; section 4 names a bf16 state as the way to cut the state traffic.
 * T > 1 serves short multi-token steps (draft tokens of speculative decoding, short
 * prefills) at the state traffic of one step.
 *
 * Sequence n runs tokens 0..T-1 in order, starting from the state in its slot, and the
 * slot holds the state after token T-1 on return. Every state is read from memory once and
 * written once per call, whatever T is.
 *
 *   q, k          device [N, T, h_k, d_k]   (dims->batch = N >= 0, dims->seqlen = T >= 1)
 *   v, w          device [N, T, h_v, d_v]
 *   log_alpha, b  device [N, T, h_v, d_k]   (input dtype dims->dtype for all six)
 *   state         device [num_slots, h_v, d_k, d_v] in state_dtype (gdn2_state_dtype),
 *                 read and updated in place
 *   state_idx     device int32 [N]: the slot of sequence n; or NULL, meaning slot n (then
 *                 num_slots must be >= N). An entry outside [0, num_slots) marks a padding
 *                 sequence: its slot is neither read nor written and its o rows are zeros.
 *                 Precondition (not checked on the device): the valid entries are
 *                 distinct; two sequences on one slot race.
 *   o             device [N, T, h_v, d_v] in the input dtype; must not alias an input or
 *                 the state
 *   fusion        NULL, or the optional short convolution, q/k L2-norm and gated output
 *                 norm (gdn2_fusion); the gate is [N, T, h_v, d_v]. Padding sequences still
 *                 get zero o rows, and their conv state is untouched.
 *   stream        hipStream_t
 * With T = 1, state_idx = NULL and an fp32 state this is gdn2_recurrent_step.
 */
gdn2_status gdn2_recurrent_fwd(const void *q, const void *k, const void *v,
                               const void *log_alpha, const void *b, const void *w,
                               void *state, int32_t state_dtype, const int32_t *state_idx,
                               int32_t num_slots, void *o, const gdn2_dims *dims,
                               const gdn2_fusion *fusion, void *stream);

/*
 * Gate mappings: other members of the gated delta-rule family as GDN-2 inputs. The
 * burn-gdn2 page ("Architecture") introduces the channel-wise b_t and w_t as the
 * replacement of the scalar gate of Kimi Delta Attention; the FG2-GDN page (section 2)
 * writes its update with keys and values scaled by sqrt(beta). Each mode below is exactly
 * GDN-2 with mapped inputs (per value head h, key head h / (h_v / h_k)):
 *
 *   GDN2_GATES_KDA       S = (I - beta k k^T) diag(alpha) S + beta k v^T
 *                        beta  [rows, h_v] (one value per token and value head)
 *                        -> b_out [rows, h_v, d_k] = beta, w_out [rows, h_v, d_v] = beta;
 *                        q, k, v and log_alpha are used as they are
 *   GDN2_GATES_GDN       as KDA with a scalar decay: log_alpha [rows, h_v]
 *                        -> also log_alpha_out [rows, h_v, d_k] = log_alpha
 *   GDN2_GATES_FG2       S = (I - k~ k~^T) diag(alpha) S + k~ v~^T, k~ = sqrt(beta) . k,
 *                        v~ = sqrt(beta) . v; beta [rows, h_v, d_k]; needs d_v = d_k
 *                        -> k_out [rows, h_v, d_k] = k~, v_out [rows, h_v, d_v] = v~,
 *                           b_out = w_out = 1
 *   GDN2_GATES_FG2_PLUS  as FG2 with the erase scale beta [rows, h_v, d_k] on the keys and
 *                        the write scale beta_v [rows, h_v, d_v] on the values:
 *                        S = (I - k~ k~^T) diag(alpha) S + k~ (sqrt(beta_v) . v)^T
 *                        -> k_out = sqrt(beta) . k, b_out = 1, w_out = sqrt(beta_v);
 *                           v is used as it is
 *
 * rows = dims->batch x dims->seqlen tokens in the layout of the call that follows (dense,
 * packed or recurrent); dims is that call's dims. In the FG2 modes k_out is per value head,
 * so the follow-up call takes h_k = h_v, with q_out [rows, h_v, d_k] (q replicated per
 * value head) in place of q; q_out is required when h_v > h_k and may be NULL (q used as it
 * is) when h_v = h_k. All tensors are in dims->dtype. Pointers a mode does not use are
 * ignored. The outputs a mode writes must not alias its inputs or each other. An
 * elementwise pass on `stream` (HBM-bound); nothing else is computed.
 */
typedef enum gdn2_gate_mode {
    GDN2_GATES_KDA = 1,
    GDN2_GATES_FG2 = 2,
    GDN2_GATES_FG2_PLUS = 3,
    GDN2_GATES_GDN = 4
} gdn2_gate_mode;

gdn2_status gdn2_map_gates(int32_t mode, const gdn2_dims *dims, const void *q, const void *k,
                           const void *v, const void *log_alpha, const void *beta,
                           const void *beta_v, void *q_out, void *k_out, void *v_out,
                           void *log_alpha_out, void *b_out, void *w_out, void *stream);

/*
 * Gradients through gdn2_map_gates: the chain rule of its mapping (the mappings are those
 * of gdn2_map_gates, after the burn-gdn2 "Architecture" section and the FG2-GDN summary,
 * section 2). Given the gradients of a loss with respect to the GDN-2 inputs the mapping
 * wrote (for instance from gdn2_chunk_bwd run on them), it writes the gradients with
 * respect to the variant's own inputs. Only the gradients the mapping changes are written;
 * every other gradient of the variant is the mapped one itself:
 *   GDN2_GATES_KDA       dbeta [rows, h_v] = sum over d_k of db_m + sum over d_v of dw_m;
 *                        dq, dk, dv, dlog_alpha are dq_m, dk_m, dv_m, dla_m
 *   GDN2_GATES_GDN       as KDA, and dlog_alpha [rows, h_v] = sum over d_k of dla_m
 *   GDN2_GATES_FG2       dk [rows, h_k, d_k] = sum over the key head's value heads of
 *                        sqrt(beta) . dk_m; dv [rows, h_v, d_v] = sqrt(beta) . dv_m;
 *                        dbeta [rows, h_v, d_k] = (dk_m . k + dv_m . v) / (2 sqrt(beta));
 *                        dq [rows, h_k, d_k] = sum over the value heads of dq_m when
 *                        h_v > h_k (when h_v = h_k, dq is dq_m); dlog_alpha is dla_m;
 *                        db_m and dw_m are not read (b = w = 1 are constants)
 *   GDN2_GATES_FG2_PLUS  dk and dq as FG2; dbeta = dk_m . k / (2 sqrt(beta));
 *                        dbeta_v [rows, h_v, d_v] = dw_m / (2 sqrt(beta_v)); dv and
 *                        dlog_alpha are dv_m and dla_m
 *
 *   mode, dims          as for gdn2_map_gates (rows = dims->batch x dims->seqlen)
 *   k, v, beta, beta_v  the forward's inputs of gdn2_map_gates, device, dims->dtype
 *   dq_m, dk_m          device fp32 [rows, h', d_k]: dL/dq', dL/dk' of the mapped inputs
 *                       (h' = h_v in the FG2 modes, whose mapped keys are per value head)
 *   dv_m, dw_m          device fp32 [rows, h_v, d_v];  dla_m, db_m  device fp32 [rows, h_v, d_k]
 *   dq .. dbeta_v       device fp32 outputs, in the shapes listed above
 * Pointers a mode does not read or write are ignored. In the FG2 modes beta (and beta_v)
 * must be > 0 (the derivative of the square root); a zero gives inf or NaN there. Outputs
 * must not alias the inputs or each other. One elementwise pass on `stream` (HBM-bound).
 */
gdn2_status gdn2_map_gates_bwd(int32_t mode, const gdn2_dims *dims, const void *k,
                               const void *v, const void *beta, const void *beta_v,
                               const float *dq_m, const float *dk_m, const float *dv_m,
                               const float *dla_m, const float *db_m, const float *dw_m,
                               float *dq, float *dk, float *dv, float *dlog_alpha,
                               float *dbeta, float *dbeta_v, void *stream);

/*
 * Host helper: checks a HOST copy of cu_seqlens (N+1 entries) against total tokens T.
 * Returns GDN2_OK when cu[0] = 0, cu is non-decreasing and cu[N] = T, else
 * GDN2_ERR_BAD_SHAPE (GDN2_ERR_NULL_ARG for a NULL pointer). Touches no device.
 */
gdn2_status gdn2_check_cu_seqlens(const int32_t *cu_seqlens_host, int32_t num_seqs,
                                  int32_t total_tokens);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
