// gdn2_internal.h -- host-side launch interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn2.h"

namespace gdn2 {

// Records a failure message for gdn2_last_error() on this thread and returns `st`.
gdn2_status report(gdn2_status st, const char *msg);
gdn2_status report_hip(hipError_t e, const char *where);

constexpr int kChunk = 64;   // chunk size of the chunked forward

// Optional fusions (gdn2_fusion): q/k L2-norm before the recurrence, gated RMS norm after.
struct Fusion {
    bool qk_norm = false;
    float l2eps = 0.f;
    const void *gate = nullptr;      // [.., h_v, d_v] input dtype, or NULL
    const float *nw = nullptr;       // [d_v] fp32
    float neps = 0.f;
    const float *cw = nullptr;       // short convolution taps [C][4] fp32, or NULL
    float *cst = nullptr;            // conv state [num_slots][3][C] fp32
    bool csilu = false;
    int gmode = 0;                   // GateMode of the b / w arguments (0: GDN-2 gates)
    float *cks = nullptr;            // chunked forward: state entering every chunk, or NULL
    void *cks16 = nullptr;           // the same as bf16 fragments (64-token path), or NULL
    void *cku16 = nullptr;           // U of every chunk as bf16 fragments (64-token path), or NULL
    char *bops = nullptr;            // with o == NULL: the backward's reverse-pass operands
    const void *bdo = nullptr;       // dO for bops
    void *tmat = nullptr;            // chunked forward, bf16: T = (I + A)^-1 per record, or NULL
    const float *ck_in = nullptr;    // with bops (64-token path): the state entering every chunk,
                                     // given (fp32, the layout of cks): no chain, no segment pass
};

struct DecodeArgs {
    const void *q, *k, *v, *log_alpha, *b, *w;
    void *S;                 // state pool [num_slots][h_v][d_k][d_v], fp32 or bf16
    const int32_t *idx;      // slot of each sequence, or NULL (slot n)
    void *o;
    int num_seqs, ntok, num_slots, h_k, h_v, d_k, d_v;
    bool bf16;               // input dtype
    bool state_bf16;         // state dtype
    Fusion fu;
};

struct ChunkArgs {
    const void *q, *k, *v, *log_alpha, *b, *w;
    const float *S0;
    const int32_t *cu_seqlens;   // NULL: dense
    void *o;
    float *S_T;
    char *workspace;
    int batch, seqlen, num_seqs, h_k, h_v, d_k, d_v;
    int chunk = kChunk;          // chunk size: 32, 64 or 128
    bool bf16;
    Fusion fu;
};

// Workspace layout of the chunked forward (all offsets 256-byte aligned):
//   [chunk map: int32[num_seqs + 1], packed batches only]
//   [per (chunk, value head) record of chunk_record_bytes()]
size_t chunk_record_bytes(int chunk, int d_k, int d_v, bool bf16);
int64_t chunk_upper_bound(int chunk, int batch, int seqlen, int num_seqs, bool packed);
size_t chunk_map_bytes(int num_seqs, bool packed);
size_t chunk_workspace_bytes(int chunk, int batch, int seqlen, int num_seqs, int h_v, int d_k,
                             int d_v, bool bf16, bool packed);
bool chunk_size_built(int chunk);

// Chunked backward (gdn2_chunk_bwd). Workspace: the forward's, then the state entering every
// chunk (fp32), a scratch o, then a per-record fp32 scratch.
struct BwdArgs {
    const void *q, *k, *v, *log_alpha, *b, *w;
    const float *S0;
    const int32_t *cu_seqlens;
    const void *dO;
    const float *dS_T;
    float *dq, *dk, *dv, *dw, *dla, *db, *dS0;
    char *workspace;
    int batch, seqlen, num_seqs, h_k, h_v, d_k, d_v;
    bool bf16;
    const float *ck_in = nullptr;    // the state entering every 64-token chunk, from the forward
                                     // (bf16 inputs: used instead of the re-run's chain), or NULL
};
size_t chunk_bwd_workspace_bytes(int batch, int seqlen, int num_seqs, int h_v, int d_k, int d_v,
                                 bool bf16, bool packed);
hipError_t launch_chunk_bwd(const BwdArgs &a, hipStream_t st);
// bf16 inputs (gdn2_bwd16.hip): the backward on bf16 matrix cores, with its own workspace.
size_t chunk_bwd16_workspace_bytes(int batch, int seqlen, int num_seqs, int h_v, int d_k, int d_v,
                                   bool packed);
hipError_t launch_chunk_bwd16(const BwdArgs &a, hipStream_t st);

// Gate mappings of other delta-rule variants onto the GDN-2 inputs (gdn2_map_gates).
enum GateMode { GATES_GDN2 = 0, GATES_KDA = 1, GATES_FG2 = 2, GATES_FG2_PLUS = 3, GATES_GDN = 4 };

struct GateArgs {
    int mode;
    const void *q, *k, *v, *log_alpha, *beta, *beta_v;
    void *q_out, *k_out, *v_out, *log_alpha_out, *b_out, *w_out;
    int64_t rows;            // tokens: batch x seqlen
    int h_k, h_v, d_k, d_v;
    bool bf16;
};

// The chain rule back through a gate mapping (gdn2_map_gates_bwd): the forward's k, v,
// beta, beta_v (input dtype), the fp32 gradients of the mapped inputs, the fp32 outputs.
struct GateBwdArgs {
    int mode;
    const void *k, *v, *beta, *beta_v;
    const float *dq_m, *dk_m, *dv_m, *dla_m, *db_m, *dw_m;
    float *dq, *dk, *dv, *dla, *dbeta, *dbeta_v;
    int64_t rows;
    int h_k, h_v, d_k, d_v;
    bool bf16;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st);
hipError_t launch_map_gates(const GateArgs &a, hipStream_t st);
hipError_t launch_map_gates_bwd(const GateBwdArgs &a, hipStream_t st);
hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t st);

}  // namespace gdn2
