// gdn2_api.cpp -- the extern "C" boundary of libgdn2: argument validation, workspace sizing
// and dispatch to the gfx950 kernels. Every check runs on the host before anything is
// enqueued, so a rejected call has no effect on the device.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

#include "gdn2.h"
#include "gdn2_internal.h"

namespace {

thread_local char g_last_error[256] = "";

gdn2_status fail(gdn2_status st, const char *msg) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
    return st;
}

gdn2_status fail_hip(hipError_t e, const char *where) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
    return GDN2_ERR_HIP;
}

bool head_dim_ok(int d) { return d == 64 || d == 128; }

// Checks shared by both entry points. `tokens` is the token count the layouts span.
gdn2_status check_heads(const gdn2_dims *d) {
    if (d->dtype != GDN2_F32 && d->dtype != GDN2_BF16)
        return fail(GDN2_ERR_UNSUPPORTED, "dtype must be GDN2_F32 or GDN2_BF16");
    if (d->h_k < 1 || d->h_v < 1) return fail(GDN2_ERR_BAD_SHAPE, "h_k and h_v must be >= 1");
    if (d->h_v % d->h_k != 0) return fail(GDN2_ERR_BAD_SHAPE, "h_v must be a multiple of h_k");
    if (d->d_k < 1 || d->d_v < 1) return fail(GDN2_ERR_BAD_SHAPE, "d_k and d_v must be >= 1");
    if (!head_dim_ok(d->d_k) || !head_dim_ok(d->d_v))
        return fail(GDN2_ERR_UNSUPPORTED, "d_k and d_v must each be 64 or 128");
    return GDN2_OK;
}

constexpr int64_t kMaxElems = (int64_t{1} << 40);   // bound on any tensor's element count

bool eps_ok(float e) { return e >= 0.f && e <= 1e30f; }   // also rejects NaN

// Checks the optional fusion options and copies them into the launch arguments.
gdn2_status take_fusion(const gdn2_fusion *f, const void *o, const gdn2_dims *d,
                        gdn2::Fusion *out) {
    *out = gdn2::Fusion{};
    if (!f) return GDN2_OK;
    if (f->gate_mode < 0 || f->gate_mode > GDN2_GATES_GDN)
        return fail(GDN2_ERR_UNSUPPORTED, "gate_mode must be 0 or a gdn2_gate_mode");
    const bool fg2 = f->gate_mode == GDN2_GATES_FG2 || f->gate_mode == GDN2_GATES_FG2_PLUS;
    if (fg2 && (f->qk_l2norm || f->conv_weight))
        return fail(GDN2_ERR_UNSUPPORTED,
                    "the FG2 gate modes take neither the q/k L2-norm nor the convolution");
    if (f->gate_mode == GDN2_GATES_FG2 && d->d_v != d->d_k)
        return fail(GDN2_ERR_BAD_SHAPE, "GDN2_GATES_FG2 needs d_v = d_k");
    if (f->qk_l2norm && !eps_ok(f->l2norm_eps))
        return fail(GDN2_ERR_BAD_SHAPE, "l2norm_eps must be finite and >= 0");
    if (f->gate) {
        if (!f->norm_weight) return fail(GDN2_ERR_NULL_ARG, "a gate needs norm_weight");
        if (!eps_ok(f->norm_eps)) return fail(GDN2_ERR_BAD_SHAPE, "norm_eps must be finite and >= 0");
        if (f->gate == o) return fail(GDN2_ERR_BAD_SHAPE, "the gate must not alias o");
    }
    if (f->conv_weight && !f->conv_state)
        return fail(GDN2_ERR_NULL_ARG, "a short convolution needs conv_state");
    if (f->conv_weight && (f->conv_state == o || static_cast<const void *>(f->conv_weight) == o))
        return fail(GDN2_ERR_BAD_SHAPE, "the convolution buffers must not alias o");
    out->qk_norm = f->qk_l2norm != 0;
    out->cw = f->conv_weight;
    out->cst = f->conv_state;
    out->csilu = f->conv_silu != 0;
    out->l2eps = f->l2norm_eps;
    out->gate = f->gate;
    out->nw = f->norm_weight;
    out->neps = f->norm_eps;
    if (f->chunk_states && static_cast<const void *>(f->chunk_states) == o)
        return fail(GDN2_ERR_BAD_SHAPE, "chunk_states must not alias o");
    out->gmode = f->gate_mode;
    out->cks = f->chunk_states;
    return GDN2_OK;
}

// The w argument is unused by the gate modes that derive w from b.
bool needs_w(const gdn2::Fusion &fu) {
    return fu.gmode == 0 || fu.gmode == GDN2_GATES_FG2_PLUS;
}

}  // namespace

namespace gdn2 {
gdn2_status report(gdn2_status st, const char *msg) { return fail(st, msg); }
gdn2_status report_hip(hipError_t e, const char *where) { return fail_hip(e, where); }
}  // namespace gdn2

extern "C" {

int32_t gdn2_abi_version(void) { return GDN2_ABI_VERSION; }

const char *gdn2_status_string(int32_t s) {
    switch (s) {
        case GDN2_OK: return "ok";
        case GDN2_ERR_NULL_ARG: return "a required pointer is NULL";
        case GDN2_ERR_BAD_SHAPE: return "invalid or inconsistent dimensions";
        case GDN2_ERR_UNSUPPORTED: return "unsupported configuration";
        case GDN2_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN2_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *gdn2_last_error(void) { return g_last_error; }

// The chunked backward takes the chunk size of the forward whose gradients it forms (32, 64
// or 128). The gradients do not depend on it, and every chunk size is computed with 64-token
// chunks, for both dtypes at every supported head-dim pair.
static gdn2_status check_bwd_built(const gdn2_dims *d, int32_t chunk_size) {
    if (!d) return fail(GDN2_ERR_NULL_ARG, "dims is NULL");
    if (!gdn2::chunk_size_built(chunk_size))
        return fail(GDN2_ERR_UNSUPPORTED, "chunk_size must be 32, 64 or 128");
    return GDN2_OK;
}

static gdn2_status check_chunk_dims(const gdn2_dims *d, int32_t chunk_size, bool packed) {
    if (!d) return fail(GDN2_ERR_NULL_ARG, "dims is NULL");
    gdn2_status st = check_heads(d);
    if (st != GDN2_OK) return st;
    if (chunk_size < 1) return fail(GDN2_ERR_BAD_SHAPE, "chunk_size must be >= 1");
    if (!gdn2::chunk_size_built(chunk_size))
        return fail(GDN2_ERR_UNSUPPORTED, "chunk_size must be 32, 64 or 128");
    if (d->seqlen < 0) return fail(GDN2_ERR_BAD_SHAPE, "seqlen must be >= 0");
    if (packed) {
        if (d->batch != 1) return fail(GDN2_ERR_BAD_SHAPE, "packed batches need batch = 1");
        if (d->num_seqs < 1) return fail(GDN2_ERR_BAD_SHAPE, "num_seqs must be >= 1");
    } else if (d->batch < 1) {
        return fail(GDN2_ERR_BAD_SHAPE, "batch must be >= 1");
    }
    const int64_t tokens = static_cast<int64_t>(d->batch) * d->seqlen;
    if (tokens > INT32_MAX) return fail(GDN2_ERR_BAD_SHAPE, "more than 2^31-1 tokens");
    const int64_t hd = static_cast<int64_t>(d->h_v) * (d->d_k > d->d_v ? d->d_k : d->d_v);
    if (tokens * hd > kMaxElems) return fail(GDN2_ERR_BAD_SHAPE, "tensors too large");
    const int64_t nseq = packed ? d->num_seqs : d->batch;
    if (nseq * d->h_v * d->d_k * d->d_v > kMaxElems)
        return fail(GDN2_ERR_BAD_SHAPE, "state tensor too large");
    return GDN2_OK;
}

size_t gdn2_chunk_fwd_workspace_bytes(const gdn2_dims *dims, int32_t chunk_size) {
    if (!dims) return 0;
    const bool packed = dims->num_seqs > 0 && dims->batch == 1;
    // A dense call ignores num_seqs; size for whichever layout the caller may use.
    if (check_chunk_dims(dims, chunk_size, false) != GDN2_OK &&
        check_chunk_dims(dims, chunk_size, packed) != GDN2_OK)
        return 0;
    const bool bf = dims->dtype == GDN2_BF16;
    const size_t dense = gdn2::chunk_workspace_bytes(chunk_size, dims->batch, dims->seqlen,
                                                      dims->num_seqs, dims->h_v, dims->d_k,
                                                      dims->d_v, bf, false);
    const size_t pk = packed ? gdn2::chunk_workspace_bytes(chunk_size, dims->batch, dims->seqlen,
                                                           dims->num_seqs, dims->h_v, dims->d_k,
                                                           dims->d_v, bf, true)
                             : 0;
    return dense > pk ? dense : pk;
}

gdn2_status gdn2_chunk_fwd(const void *q, const void *k, const void *v, const void *log_alpha,
                           const void *b, const void *w, const float *S0,
                           const int32_t *cu_seqlens, int32_t chunk_size, void *o, float *S_T,
                           const gdn2_dims *dims, void *workspace, size_t workspace_bytes,
                           const gdn2_fusion *fusion, void *stream) {
    const bool packed = cu_seqlens != nullptr;
    gdn2_status st = check_chunk_dims(dims, chunk_size, packed);
    if (st != GDN2_OK) return st;
    gdn2::Fusion fu;
    st = take_fusion(fusion, o, dims, &fu);
    if (st != GDN2_OK) return st;
    if (fu.cw)
        return fail(GDN2_ERR_UNSUPPORTED, "the short convolution is built for gdn2_recurrent_fwd only");
    const int64_t tokens = static_cast<int64_t>(dims->batch) * dims->seqlen;
    if (tokens > 0 && (!q || !k || !v || !log_alpha || !b || (!w && needs_w(fu)) || !o))
        return fail(GDN2_ERR_NULL_ARG, "q, k, v, log_alpha, b, w and o are required");
    const bool bf = dims->dtype == GDN2_BF16;
    const size_t need = gdn2::chunk_workspace_bytes(chunk_size, dims->batch, dims->seqlen,
                                                    dims->num_seqs, dims->h_v, dims->d_k,
                                                    dims->d_v, bf, packed);
    if (need > 0 && !workspace) return fail(GDN2_ERR_WORKSPACE, "workspace is NULL");
    if (workspace_bytes < need) return fail(GDN2_ERR_WORKSPACE, "workspace is too small");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(GDN2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (o && (o == q || o == k || o == v || o == log_alpha || o == b || o == w))
        return fail(GDN2_ERR_BAD_SHAPE, "o must not alias an input");
    if (fu.cks) {
        const void *c = fu.cks;
        if (c == q || c == k || c == v || c == log_alpha || c == b || c == w || c == S0 ||
            c == S_T || c == workspace || c == cu_seqlens)
            return fail(GDN2_ERR_BAD_SHAPE, "chunk_states must not alias an input or output");
    }

    gdn2::ChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.b = b; a.w = w;
    a.S0 = S0; a.cu_seqlens = cu_seqlens; a.o = o; a.S_T = S_T;
    a.workspace = static_cast<char *>(workspace);
    a.batch = dims->batch; a.seqlen = dims->seqlen; a.num_seqs = packed ? dims->num_seqs : 0;
    a.h_k = dims->h_k; a.h_v = dims->h_v; a.d_k = dims->d_k; a.d_v = dims->d_v;
    a.chunk = chunk_size;
    a.bf16 = bf;
    a.fu = fu;
    const hipError_t e = gdn2::launch_chunk_fwd(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, "gdn2_chunk_fwd launch");
    g_last_error[0] = '\0';
    return GDN2_OK;
}

size_t gdn2_chunk_bwd_workspace_bytes(const gdn2_dims *dims, int32_t chunk_size) {
    if (!dims) return 0;
    if (check_bwd_built(dims, chunk_size) != GDN2_OK) return 0;
    const bool packed = dims->num_seqs > 0 && dims->batch == 1;
    if (check_chunk_dims(dims, chunk_size, false) != GDN2_OK &&
        check_chunk_dims(dims, chunk_size, packed) != GDN2_OK)
        return 0;
    const bool bf = dims->dtype == GDN2_BF16;
    const size_t dense = gdn2::chunk_bwd_workspace_bytes(dims->batch, dims->seqlen, dims->num_seqs,
                                                          dims->h_v, dims->d_k, dims->d_v, bf, false);
    const size_t pk = packed ? gdn2::chunk_bwd_workspace_bytes(dims->batch, dims->seqlen,
                                                               dims->num_seqs, dims->h_v, dims->d_k,
                                                               dims->d_v, bf, true)
                             : 0;
    return dense > pk ? dense : pk;
}

static gdn2_status chunk_bwd_common(const void *q, const void *k, const void *v,
                                    const void *log_alpha, const void *b, const void *w,
                                    const float *S0, const int32_t *cu_seqlens, int32_t chunk_size,
                                    const float *chunk_states, bool given, const void *dO,
                                    const float *dS_T, float *dq, float *dk, float *dv, float *dw,
                                    float *dlog_alpha, float *db, float *dS0, const gdn2_dims *dims,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    const bool packed = cu_seqlens != nullptr;
    gdn2_status st = check_chunk_dims(dims, chunk_size, packed);
    if (st != GDN2_OK) return st;
    st = check_bwd_built(dims, chunk_size);
    if (st != GDN2_OK) return st;
    if (given && chunk_size != gdn2::kChunk)
        return fail(GDN2_ERR_UNSUPPORTED, "chunk_states are those of a chunk_size 64 forward");
    const int64_t tokens = static_cast<int64_t>(dims->batch) * dims->seqlen;
    const int N = packed ? dims->num_seqs : dims->batch;
    if (tokens > 0 && (!q || !k || !v || !log_alpha || !b || !w || !dO || !dq || !dk || !dv ||
                       !dw || !dlog_alpha || !db))
        return fail(GDN2_ERR_NULL_ARG, "the inputs, dO and every token gradient are required");
    if (N > 0 && !dS0) return fail(GDN2_ERR_NULL_ARG, "dS0 is required");
    if (given && tokens > 0 && !chunk_states) return fail(GDN2_ERR_NULL_ARG, "chunk_states is NULL");
    const void *outs[] = {dq, dk, dv, dw, dlog_alpha, db, dS0};
    const void *ins[] = {q, k, v, log_alpha, b, w, S0, cu_seqlens, dO, dS_T, workspace, chunk_states};
    for (const void *x : outs) {
        if (!x) continue;
        for (const void *y : ins)
            if (x == y) return fail(GDN2_ERR_BAD_SHAPE, "an output aliases an input or the workspace");
        int same = 0;
        for (const void *y : outs) same += x == y;
        if (same > 1) return fail(GDN2_ERR_BAD_SHAPE, "two outputs alias");
    }
    const bool bf = dims->dtype == GDN2_BF16;
    const size_t need = gdn2::chunk_bwd_workspace_bytes(dims->batch, dims->seqlen, dims->num_seqs,
                                                        dims->h_v, dims->d_k, dims->d_v, bf, packed);
    if (need > 0 && !workspace) return fail(GDN2_ERR_WORKSPACE, "workspace is NULL");
    if (workspace_bytes < need) return fail(GDN2_ERR_WORKSPACE, "workspace is too small");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(GDN2_ERR_WORKSPACE, "workspace must be 256-byte aligned");

    gdn2::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.b = b; a.w = w;
    a.S0 = S0; a.cu_seqlens = cu_seqlens; a.dO = dO; a.dS_T = dS_T;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dw = dw; a.dla = dlog_alpha; a.db = db; a.dS0 = dS0;
    a.workspace = static_cast<char *>(workspace);
    a.batch = dims->batch; a.seqlen = dims->seqlen; a.num_seqs = packed ? dims->num_seqs : 0;
    a.h_k = dims->h_k; a.h_v = dims->h_v; a.d_k = dims->d_k; a.d_v = dims->d_v;
    a.bf16 = bf;
    a.ck_in = given && bf ? chunk_states : nullptr;   // fp32 inputs recompute them
    const hipError_t e = gdn2::launch_chunk_bwd(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, "gdn2_chunk_bwd launch");
    g_last_error[0] = '\0';
    return GDN2_OK;
}

gdn2_status gdn2_chunk_bwd(const void *q, const void *k, const void *v, const void *log_alpha,
                           const void *b, const void *w, const float *S0,
                           const int32_t *cu_seqlens, int32_t chunk_size, const void *dO,
                           const float *dS_T, float *dq, float *dk, float *dv, float *dw,
                           float *dlog_alpha, float *db, float *dS0, const gdn2_dims *dims,
                           void *workspace, size_t workspace_bytes, void *stream) {
    return chunk_bwd_common(q, k, v, log_alpha, b, w, S0, cu_seqlens, chunk_size, nullptr, false,
                            dO, dS_T, dq, dk, dv, dw, dlog_alpha, db, dS0, dims, workspace,
                            workspace_bytes, stream);
}

gdn2_status gdn2_chunk_bwd_states(const void *q, const void *k, const void *v,
                                  const void *log_alpha, const void *b, const void *w,
                                  const float *S0, const int32_t *cu_seqlens, int32_t chunk_size,
                                  const float *chunk_states, const void *dO, const float *dS_T,
                                  float *dq, float *dk, float *dv, float *dw, float *dlog_alpha,
                                  float *db, float *dS0, const gdn2_dims *dims, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return chunk_bwd_common(q, k, v, log_alpha, b, w, S0, cu_seqlens, chunk_size, chunk_states,
                            true, dO, dS_T, dq, dk, dv, dw, dlog_alpha, db, dS0, dims, workspace,
                            workspace_bytes, stream);
}

static gdn2_status recurrent_common(const void *q, const void *k, const void *v,
                                    const void *log_alpha, const void *b, const void *w,
                                    void *S, int32_t state_dtype, const int32_t *idx,
                                    int32_t num_slots, void *o, const gdn2_dims *dims,
                                    const gdn2_fusion *fusion, void *stream,
                                    const char *where) {
    if (!dims) return fail(GDN2_ERR_NULL_ARG, "dims is NULL");
    gdn2_status st = check_heads(dims);
    if (st != GDN2_OK) return st;
    gdn2::Fusion fu;
    st = take_fusion(fusion, o, dims, &fu);
    if (st != GDN2_OK) return st;
    if (fu.cks) return fail(GDN2_ERR_UNSUPPORTED, "chunk_states is an output of gdn2_chunk_fwd only");
    if (state_dtype != GDN2_STATE_F32 && state_dtype != GDN2_STATE_BF16)
        return fail(GDN2_ERR_UNSUPPORTED, "state_dtype must be GDN2_STATE_F32 or GDN2_STATE_BF16");
    if (dims->seqlen < 1) return fail(GDN2_ERR_BAD_SHAPE, "seqlen (tokens per sequence) must be >= 1");
    if (dims->batch < 0) return fail(GDN2_ERR_BAD_SHAPE, "batch must be >= 0");
    if (num_slots < 0) return fail(GDN2_ERR_BAD_SHAPE, "num_slots must be >= 0");
    if (!idx && num_slots < dims->batch)
        return fail(GDN2_ERR_BAD_SHAPE, "without state_idx, num_slots must be >= batch");
    const int64_t per_state = static_cast<int64_t>(dims->h_v) * dims->d_k * dims->d_v;
    if (static_cast<int64_t>(num_slots) * per_state > kMaxElems)
        return fail(GDN2_ERR_BAD_SHAPE, "state tensor too large");
    if (static_cast<int64_t>(dims->batch) * dims->h_v > INT32_MAX)
        return fail(GDN2_ERR_BAD_SHAPE, "too many states");
    const int64_t tokens = static_cast<int64_t>(dims->batch) * dims->seqlen;
    const int64_t hd = static_cast<int64_t>(dims->h_v) * (dims->d_k > dims->d_v ? dims->d_k : dims->d_v);
    if (tokens > INT32_MAX || tokens * hd > kMaxElems)
        return fail(GDN2_ERR_BAD_SHAPE, "tensors too large");
    if (dims->batch == 0) {
        g_last_error[0] = '\0';
        return GDN2_OK;
    }
    if (!q || !k || !v || !log_alpha || !b || (!w && needs_w(fu)) || !o || (num_slots > 0 && !S))
        return fail(GDN2_ERR_NULL_ARG, "q, k, v, log_alpha, b, w, the state and o are required");
    if (o == q || o == k || o == v || o == log_alpha || o == b || o == w || o == S)
        return fail(GDN2_ERR_BAD_SHAPE, "o must not alias an input or the state");

    gdn2::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.b = b; a.w = w;
    a.S = S; a.idx = idx; a.o = o;
    a.num_seqs = dims->batch; a.ntok = dims->seqlen; a.num_slots = num_slots;
    a.h_k = dims->h_k; a.h_v = dims->h_v; a.d_k = dims->d_k; a.d_v = dims->d_v;
    a.bf16 = dims->dtype == GDN2_BF16;
    a.state_bf16 = state_dtype == GDN2_STATE_BF16;
    a.fu = fu;
    const hipError_t e = gdn2::launch_decode(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, where);
    g_last_error[0] = '\0';
    return GDN2_OK;
}

gdn2_status gdn2_recurrent_step(const void *q, const void *k, const void *v,
                                const void *log_alpha, const void *b, const void *w, float *S,
                                void *o, const gdn2_dims *dims, void *stream) {
    if (!dims) return fail(GDN2_ERR_NULL_ARG, "dims is NULL");
    if (dims->seqlen != 1) return fail(GDN2_ERR_BAD_SHAPE, "recurrent step needs seqlen = 1");
    return recurrent_common(q, k, v, log_alpha, b, w, S, GDN2_STATE_F32, nullptr,
                            dims->batch < 0 ? 0 : dims->batch, o, dims, nullptr, stream,
                            "gdn2_recurrent_step launch");
}

gdn2_status gdn2_recurrent_fwd(const void *q, const void *k, const void *v,
                               const void *log_alpha, const void *b, const void *w,
                               void *state, int32_t state_dtype, const int32_t *state_idx,
                               int32_t num_slots, void *o, const gdn2_dims *dims,
                               const gdn2_fusion *fusion, void *stream) {
    return recurrent_common(q, k, v, log_alpha, b, w, state, state_dtype, state_idx,
                            num_slots, o, dims, fusion, stream, "gdn2_recurrent_fwd launch");
}

gdn2_status gdn2_map_gates(int32_t mode, const gdn2_dims *dims, const void *q, const void *k,
                           const void *v, const void *log_alpha, const void *beta,
                           const void *beta_v, void *q_out, void *k_out, void *v_out,
                           void *log_alpha_out, void *b_out, void *w_out, void *stream) {
    if (!dims) return fail(GDN2_ERR_NULL_ARG, "dims is NULL");
    gdn2_status st = check_heads(dims);
    if (st != GDN2_OK) return st;
    if (mode != GDN2_GATES_KDA && mode != GDN2_GATES_FG2 && mode != GDN2_GATES_FG2_PLUS &&
        mode != GDN2_GATES_GDN)
        return fail(GDN2_ERR_UNSUPPORTED, "mode must be a gdn2_gate_mode");
    const bool fg2 = mode == GDN2_GATES_FG2 || mode == GDN2_GATES_FG2_PLUS;
    if (mode == GDN2_GATES_FG2 && dims->d_v != dims->d_k)
        return fail(GDN2_ERR_BAD_SHAPE, "GDN2_GATES_FG2 scales v by sqrt(beta): d_v must equal d_k");
    if (dims->batch < 0 || dims->seqlen < 0) return fail(GDN2_ERR_BAD_SHAPE, "batch and seqlen must be >= 0");
    const int64_t rows = static_cast<int64_t>(dims->batch) * dims->seqlen;
    const int64_t hd = static_cast<int64_t>(dims->h_v) * (dims->d_k > dims->d_v ? dims->d_k : dims->d_v);
    if (rows > INT32_MAX || rows * hd > kMaxElems) return fail(GDN2_ERR_BAD_SHAPE, "tensors too large");
    if (rows == 0) {
        g_last_error[0] = '\0';
        return GDN2_OK;
    }
    const bool share = dims->h_v > dims->h_k;       // value heads share key heads
    if (!beta || !b_out || !w_out) return fail(GDN2_ERR_NULL_ARG, "beta, b_out and w_out are required");
    if (mode == GDN2_GATES_GDN && (!log_alpha || !log_alpha_out))
        return fail(GDN2_ERR_NULL_ARG, "GDN2_GATES_GDN needs log_alpha and log_alpha_out");
    if (fg2 && (!k || !k_out)) return fail(GDN2_ERR_NULL_ARG, "the FG2 modes need k and k_out");
    if (mode == GDN2_GATES_FG2 && (!v || !v_out)) return fail(GDN2_ERR_NULL_ARG, "GDN2_GATES_FG2 needs v and v_out");
    if (mode == GDN2_GATES_FG2_PLUS && !beta_v) return fail(GDN2_ERR_NULL_ARG, "GDN2_GATES_FG2_PLUS needs beta_v");
    if (fg2 && share && !q_out)
        return fail(GDN2_ERR_NULL_ARG, "the FG2 modes need q_out when value heads share key heads");
    if (fg2 && q_out && !q) return fail(GDN2_ERR_NULL_ARG, "q_out needs q");
    // the outputs this mode writes must not overlap each other or any input
    const void *ins[6] = {q, k, v, log_alpha, beta, beta_v};
    void *outs[6] = {fg2 ? q_out : nullptr, fg2 ? k_out : nullptr,
                     mode == GDN2_GATES_FG2 ? v_out : nullptr,
                     mode == GDN2_GATES_GDN ? log_alpha_out : nullptr, b_out, w_out};
    for (int i = 0; i < 6; ++i) {
        if (!outs[i]) continue;
        for (int j = 0; j < 6; ++j)
            if (ins[j] && outs[i] == ins[j]) return fail(GDN2_ERR_BAD_SHAPE, "an output aliases an input");
        for (int j = i + 1; j < 6; ++j)
            if (outs[i] == outs[j]) return fail(GDN2_ERR_BAD_SHAPE, "two outputs are the same buffer");
    }
    gdn2::GateArgs a;
    a.mode = mode;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.beta_v = beta_v;
    a.q_out = fg2 ? q_out : nullptr; a.k_out = k_out; a.v_out = v_out;
    a.log_alpha_out = log_alpha_out; a.b_out = b_out; a.w_out = w_out;
    a.rows = rows; a.h_k = dims->h_k; a.h_v = dims->h_v; a.d_k = dims->d_k; a.d_v = dims->d_v;
    a.bf16 = dims->dtype == GDN2_BF16;
    const hipError_t e = gdn2::launch_map_gates(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, "gdn2_map_gates launch");
    g_last_error[0] = '\0';
    return GDN2_OK;
}

gdn2_status gdn2_map_gates_bwd(int32_t mode, const gdn2_dims *dims, const void *k,
                               const void *v, const void *beta, const void *beta_v,
                               const float *dq_m, const float *dk_m, const float *dv_m,
                               const float *dla_m, const float *db_m, const float *dw_m,
                               float *dq, float *dk, float *dv, float *dlog_alpha, float *dbeta,
                               float *dbeta_v, void *stream) {
    if (!dims) return fail(GDN2_ERR_NULL_ARG, "dims is NULL");
    gdn2_status st = check_heads(dims);
    if (st != GDN2_OK) return st;
    if (mode != GDN2_GATES_KDA && mode != GDN2_GATES_FG2 && mode != GDN2_GATES_FG2_PLUS &&
        mode != GDN2_GATES_GDN)
        return fail(GDN2_ERR_UNSUPPORTED, "mode must be a gdn2_gate_mode");
    const bool fg2 = mode == GDN2_GATES_FG2 || mode == GDN2_GATES_FG2_PLUS;
    if (mode == GDN2_GATES_FG2 && dims->d_v != dims->d_k)
        return fail(GDN2_ERR_BAD_SHAPE, "GDN2_GATES_FG2 scales v by sqrt(beta): d_v must equal d_k");
    if (dims->batch < 0 || dims->seqlen < 0) return fail(GDN2_ERR_BAD_SHAPE, "batch and seqlen must be >= 0");
    const int64_t rows = static_cast<int64_t>(dims->batch) * dims->seqlen;
    const int64_t hd = static_cast<int64_t>(dims->h_v) * (dims->d_k > dims->d_v ? dims->d_k : dims->d_v);
    if (rows > INT32_MAX || rows * hd > kMaxElems) return fail(GDN2_ERR_BAD_SHAPE, "tensors too large");
    if (rows == 0) {
        g_last_error[0] = '\0';
        return GDN2_OK;
    }
    const bool share = dims->h_v > dims->h_k;
    // what each mode reads and writes
    const void *ins[10] = {k, v, beta, beta_v, dq_m, dk_m, dv_m, dla_m, db_m, dw_m};
    const bool need_in[10] = {fg2, mode == GDN2_GATES_FG2, fg2, mode == GDN2_GATES_FG2_PLUS,
                              fg2 && share, fg2, mode == GDN2_GATES_FG2, mode == GDN2_GATES_GDN,
                              !fg2, !fg2 || mode == GDN2_GATES_FG2_PLUS};
    float *outs[6] = {fg2 && share ? dq : nullptr, fg2 ? dk : nullptr,
                      mode == GDN2_GATES_FG2 ? dv : nullptr, mode == GDN2_GATES_GDN ? dlog_alpha : nullptr,
                      dbeta, mode == GDN2_GATES_FG2_PLUS ? dbeta_v : nullptr};
    const bool need_out[6] = {fg2 && share, fg2, mode == GDN2_GATES_FG2, mode == GDN2_GATES_GDN, true,
                              mode == GDN2_GATES_FG2_PLUS};
    for (int i = 0; i < 10; ++i)
        if (need_in[i] && !ins[i]) return fail(GDN2_ERR_NULL_ARG, "an input this mode reads is NULL");
    for (int i = 0; i < 6; ++i)
        if (need_out[i] && !outs[i]) return fail(GDN2_ERR_NULL_ARG, "an output this mode writes is NULL");
    for (int i = 0; i < 6; ++i) {
        if (!outs[i]) continue;
        for (int j = 0; j < 10; ++j)
            if (need_in[j] && static_cast<const void *>(outs[i]) == ins[j])
                return fail(GDN2_ERR_BAD_SHAPE, "an output aliases an input");
        for (int j = i + 1; j < 6; ++j)
            if (outs[i] == outs[j]) return fail(GDN2_ERR_BAD_SHAPE, "two outputs are the same buffer");
    }
    gdn2::GateBwdArgs a;
    a.mode = mode;
    a.k = k; a.v = v; a.beta = beta; a.beta_v = beta_v;
    a.dq_m = dq_m; a.dk_m = dk_m; a.dv_m = dv_m; a.dla_m = dla_m; a.db_m = db_m; a.dw_m = dw_m;
    a.dq = outs[0]; a.dk = outs[1]; a.dv = outs[2]; a.dla = outs[3]; a.dbeta = outs[4]; a.dbeta_v = outs[5];
    a.rows = rows; a.h_k = dims->h_k; a.h_v = dims->h_v; a.d_k = dims->d_k; a.d_v = dims->d_v;
    a.bf16 = dims->dtype == GDN2_BF16;
    const hipError_t e = gdn2::launch_map_gates_bwd(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, "gdn2_map_gates_bwd launch");
    g_last_error[0] = '\0';
    return GDN2_OK;
}

gdn2_status gdn2_check_cu_seqlens(const int32_t *cu, int32_t num_seqs, int32_t total_tokens) {
    if (!cu) return fail(GDN2_ERR_NULL_ARG, "cu_seqlens is NULL");
    if (num_seqs < 1) return fail(GDN2_ERR_BAD_SHAPE, "num_seqs must be >= 1");
    if (cu[0] != 0) return fail(GDN2_ERR_BAD_SHAPE, "cu_seqlens[0] must be 0");
    for (int32_t n = 0; n < num_seqs; ++n)
        if (cu[n + 1] < cu[n]) return fail(GDN2_ERR_BAD_SHAPE, "cu_seqlens must not decrease");
    if (cu[num_seqs] != total_tokens)
        return fail(GDN2_ERR_BAD_SHAPE, "cu_seqlens[num_seqs] must equal the token count");
    g_last_error[0] = '\0';
    return GDN2_OK;
}

}  // extern "C"
