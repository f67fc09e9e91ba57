// gdn2_bwd.hip -- chunked backward of Gated DeltaNet-2 (gradients of the chunked forward).
//
// Method: the chunked WY form of the burn-gdn2 docs page, section "Architecture" (Chunk
// mode), differentiated chunk by chunk. Within a chunk of C = 64 tokens entering with state
// S and leaving with S', with g the cumulative log decay over the chunk, gamma = exp(g),
// gamma_L its last row, E[r,i,c] = exp(g_r[c] - g_i[c]) for i <= r:
//   A[r,i]  = sum_c b_r k_r k_i E (i < r),   M[r,i] = sum_c q_r k_i E (i <= r),   Tm = (I + A)^-1
//   Y = gamma.b.k,  X = w.v,  W~ = Tm Y,  U~ = Tm X,  U = U~ - W~ S
//   Qg = gamma.q,  Kg = exp(gL - g).k,  O = Qg S + M U,  S' = gamma_L S + Kg^T U
// Given dO and dS' = dL/dS', per chunk from the last:
//   dU = M^T dO + Kg dS',   dS = gamma_L dS' + Qg^T dO - W~^T dU            (to the chunk before)
//   dM = lower(dO U^T), dQg = dO S^T, dKg = U dS'^T, dW~ = -dU S^T, dX = Tm^T dU,
//   dY = Tm^T dW~, dT = dU X^T + dW~ Y^T, dA = strictly-lower(-Tm^T dT Tm^T),
// then the chain rule through E, Y, Qg, Kg and gamma_L to q, k, b and g, and
// dlog_alpha_i = sum_{r >= i} dg_r within the chunk.
//
// Kernels (one call of gdn2_chunk_bwd, after a chunked forward that writes the state
// entering every chunk):
//   bwd_factors_kernel  per (chunk, value head) record, in parallel: g, A, M, Tm, W~, U~,
//                       Qg, Kg and the dO terms of the chain, M^T dO and Qg^T dO
//   bwd_chain_kernel    per (sequence, value head, 64 columns), four waves of 16 columns,
//                       sequential over the chunks from the last: dU of every chunk and the
//                       dS' it leaves, then dS0
//   bwd_grads_kernel    per record, in parallel: every input gradient of the chunk
// The record kernels keep their intermediates in a per-record fp32 scratch of the workspace
// and stage each product's operands in LDS; their products are fp32 matrix-core tiles
// (16x16x4), as are the reverse pass's. This is the path for fp32 inputs (every head-dim
// pair); bf16 inputs take gdn2_bwd16.hip. q and k gradients of value heads that
// share a key head are summed with fp32 atomics; with one value head per key head they are
// stored.
#include "gdn2_common.h"
#include "gdn2_internal.h"
#include "gdn2_mfma.h"

namespace gdn2 {

namespace {

constexpr int C = kChunk;
constexpr int kBwdThreads = 512;

// Per-record fp32 scratch (offsets in floats).
template <int DK, int DV>
struct BLay {
    static constexpr size_t CK = static_cast<size_t>(C) * DK, CV = static_cast<size_t>(C) * DV;
    static constexpr size_t KV = static_cast<size_t>(DK) * DV, CC = static_cast<size_t>(C) * C;
    // [C][DK] tiles
    static constexpr size_t G = 0, K = CK, Q = 2 * CK, BK = 3 * CK, Y = 4 * CK, WT = 5 * CK,
                            KG = 6 * CK, QG = 7 * CK, DQG = 8 * CK, DKG = 9 * CK, DW = 10 * CK,
                            DY = 11 * CK;
    // [C][DV] tiles
    static constexpr size_t X = 12 * CK, UT = X + CV, E1 = X + 2 * CV, DU = X + 3 * CV,
                            U = X + 4 * CV, DX = X + 5 * CV;
    // [DK][DV]
    static constexpr size_t E2 = X + 6 * CV, DSN = E2 + KV;
    // [C][C]
    static constexpr size_t A = DSN + KV, TM = A + CC, M = A + 2 * CC, DM = A + 3 * CC,
                            DT = A + 4 * CC, TMP = A + 5 * CC, DA = A + 6 * CC;
    // [DK]
    static constexpr size_t GL = A + 7 * CC, DGL = GL + DK;
    static constexpr size_t FLOATS = DGL + DK;
};

// LDS copies of g, k, q and b.k of one record with row stride SP floats (DK + 1 where the
// lanes of a wave read one channel of consecutive rows, so that they hit different banks).
template <int DK, int SP_ = DK + 1>
struct KeyTiles {
    static constexpr int SP = SP_;
    static constexpr int BYTES = 4 * C * SP * 4;
    float *g, *k, *q, *bk;
    __device__ explicit KeyTiles(char *base) {
        float *f = reinterpret_cast<float *>(base);
        g = f;
        k = f + C * SP;
        q = f + 2 * C * SP;
        bk = f + 3 * C * SP;
    }
};

struct BwdParams {
    const void *q, *k, *v, *la, *b, *w, *dO;
    const float *dS_T;                 // [N][h_v][DK][DV], or NULL
    const int32_t *cu, *map;           // packed batches: offsets and chunk map, else NULL
    const float *ck;                   // state entering every chunk, [record][DK][DV]
    float *scr;                        // per-record scratch
    float *dq, *dk, *dv, *dw, *dla, *db, *dS0;
    int num_seqs, seqlen, nc_dense, h_k, h_v, group;
};

// chunk -> (sequence n, chunk j of it, token range); false past the last chunk
__device__ __forceinline__ bool locate(const BwdParams &p, int chunk, int &n, int &j,
                                       int64_t &start, int64_t &end) {
    if (p.cu == nullptr) {
        n = chunk / p.nc_dense;
        j = chunk - n * p.nc_dense;
        start = static_cast<int64_t>(n) * p.seqlen;
        end = start + p.seqlen;
        return n < p.num_seqs;
    }
    if (chunk >= p.map[p.num_seqs]) return false;
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.map[mid] <= chunk) lo = mid; else hi = mid - 1;
    }
    n = lo;
    j = chunk - p.map[n];
    start = p.cu[n];
    end = p.cu[n + 1];
    return true;
}

// out[M x N] from sum_k a(m, k) b(k, n) (all sizes multiples of 16), 16x16 tiles spread
// over the workgroup's waves; each tile's operands are all loaded before its products.
// Lane (li, lg) gives a(m0 + li, k0 + 4 lg + s) and b(k0 + 4 lg + s, n0 + li); it
// receives out[m0 + 4 lg + ii][n0 + li].
template <int M, int N, int K, class FA, class FB, class FS>
__device__ void block_mm(FA a, FB b, FS store) {
    constexpr int TN = N / 16, TILES = (M / 16) * TN, KS = K / 16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int nw = blockDim.x >> 6;
    for (int t = wave; t < TILES; t += nw) {
        const int m0 = (t / TN) * 16, n0 = (t - (t / TN) * TN) * 16;
        f32x4 av[KS], bv[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                av[ks][s] = a(m0 + li, 16 * ks + 4 * lg + s);
                bv[ks][s] = b(16 * ks + 4 * lg + s, n0 + li);
            }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mma_k16_f32(av[ks], bv[ks], acc);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) store(m0 + 4 * lg + ii, n0 + li, acc[ii]);
    }
}

// The same product with both operands first copied to LDS, each element read once. The copy
// walks each source along its contiguous axis: TA when a is contiguous along m (else along
// k), TB when b is contiguous along k (else along n), and each thread issues all of its
// loads before its first LDS store, so that the copy costs one memory round trip rather
// than one per element. lds holds at least (M (K + 4) + K (N + 4)) floats. Runs on
// kBwdThreads threads; ends with a barrier, after which lds may be reused.
template <int M, int N, int K, bool TA, bool TB, class FA, class FB, class FS>
__device__ void block_mm_lds(float *lds, FA a, FB b, FS store) {
    constexpr int SA = K + 4, SB = N + 4, NT = kBwdThreads;
    constexpr int NA = M * K / NT, NB = K * N / NT;
    static_assert(NA * NT == M * K && NB * NT == K * N, "operands split evenly over the threads");
    float *As = lds, *Bs = lds + M * SA;
    const int tid = threadIdx.x;
    float ra[NA], rb[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int e = tid + i * NT, m = TA ? e % M : e / K, k = TA ? e / M : e % K;
        ra[i] = a(m, k);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int e = tid + i * NT, k = TB ? e % K : e / N, n = TB ? e / K : e % N;
        rb[i] = b(k, n);
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int e = tid + i * NT, m = TA ? e % M : e / K, k = TA ? e / M : e % K;
        As[m * SA + k] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int e = tid + i * NT, k = TB ? e % K : e / N, n = TB ? e / K : e % N;
        Bs[k * SB + n] = rb[i];
    }
    __syncthreads();
    block_mm<M, N, K>([&](int m, int k) { return As[m * SA + k]; },
                      [&](int k, int n) { return Bs[k * SB + n]; }, store);
    __syncthreads();
}

// Clears the atomically accumulated dq and dk.
__global__ void zero_kernel(float *a, float *b, int64_t n) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        a[i] = 0.f;
        b[i] = 0.f;
    }
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) void bwd_factors_kernel(BwdParams p) {
    using L_ = BLay<DK, DV>;
    const int rec = blockIdx.x, chunk = rec / p.h_v, h = rec - chunk * p.h_v;
    int n, j;
    int64_t start, end;
    if (!locate(p, chunk, n, j, start, end)) return;
    const int64_t t0 = start + static_cast<int64_t>(j) * C;
    const int Lr = static_cast<int>(min<int64_t>(C, end - t0));
    const int hk = h / p.group, tid = threadIdx.x;
    const T *q = static_cast<const T *>(p.q), *k = static_cast<const T *>(p.k);
    const T *v = static_cast<const T *>(p.v), *la = static_cast<const T *>(p.la);
    const T *b = static_cast<const T *>(p.b), *w = static_cast<const T *>(p.w);
    const T *dO = static_cast<const T *>(p.dO);
    float *s = p.scr + static_cast<size_t>(rec) * L_::FLOATS;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    KeyTiles<DK> lt(smem);
    constexpr int SP = KeyTiles<DK>::SP;

    // token vectors (rows >= Lr are identity tokens: k = q = b = w.v = 0, log alpha = 0),
    // (row, channel) entries tid + i * kBwdThreads; every load is issued before the stores
    {
        constexpr int NE = C * DK / kBwdThreads, NX = C * DV / kBwdThreads;
        static_assert(NE * kBwdThreads == C * DK && NX * kBwdThreads == C * DV, "even split");
        float kk[NE], qq[NE], bb[NE], ll[NE], xw[NX], xv[NX];
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int e = tid + i * kBwdThreads, r = e / DK, c = e - r * DK;
            kk[i] = qq[i] = bb[i] = ll[i] = 0.f;
            if (r < Lr) {
                const size_t ok = (static_cast<size_t>(t0 + r) * p.h_k + hk) * DK + c;
                const size_t og = (static_cast<size_t>(t0 + r) * p.h_v + h) * DK + c;
                kk[i] = io<T>::ld(k + ok);
                qq[i] = io<T>::ld(q + ok);
                bb[i] = io<T>::ld(b + og);
                ll[i] = io<T>::ld(la + og);
            }
        }
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int e = tid + i * kBwdThreads, r = e / DV, c = e - r * DV;
            xw[i] = xv[i] = 0.f;
            if (r < Lr) {
                const size_t ov = (static_cast<size_t>(t0 + r) * p.h_v + h) * DV + c;
                xw[i] = io<T>::ld(w + ov);
                xv[i] = io<T>::ld(v + ov);
            }
        }
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int e = tid + i * kBwdThreads, r = e / DK, c = e - r * DK;
            s[L_::K + e] = kk[i];
            s[L_::Q + e] = qq[i];
            s[L_::BK + e] = bb[i] * kk[i];
            lt.k[r * SP + c] = kk[i];
            lt.q[r * SP + c] = qq[i];
            lt.bk[r * SP + c] = bb[i] * kk[i];
            lt.g[r * SP + c] = ll[i];
        }
#pragma unroll
        for (int i = 0; i < NX; ++i) s[L_::X + tid + i * kBwdThreads] = xw[i] * xv[i];
    }
    __syncthreads();
    // the cumulative decay, one channel per thread
    for (int c = tid; c < DK; c += kBwdThreads) {
        float acc = 0.f;
        for (int r = 0; r < C; ++r) {
            acc += lt.g[r * SP + c];
            lt.g[r * SP + c] = acc;
            s[L_::G + r * DK + c] = acc;
        }
        s[L_::GL + c] = acc;
    }
    __syncthreads();
    // gamma.b.k, gamma.q and exp(g_L - g).k
    for (int e = tid; e < C * DK; e += kBwdThreads) {
        const int r = e / DK, c = e - r * DK;
        const float g = lt.g[r * SP + c], gL = lt.g[(C - 1) * SP + c];
        const float ga = __expf(g);
        s[L_::Y + e] = ga * lt.bk[r * SP + c];
        s[L_::QG + e] = ga * lt.q[r * SP + c];
        s[L_::KG + e] = __expf(gL - g) * lt.k[r * SP + c];
    }
    // A and M on the matrix cores, per 16x16 block (row block R, column block I <= R) with
    // the reference row rho = 16 R + 7: sum_c (x_r exp(g_r - g_rho)) (k_i exp(g_rho - g_i)),
    // x = b.k for A (i < r) and q for M (i <= r); blocks above the diagonal are zero.
    {
        const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
        constexpr int NW = kBwdThreads / 64;
        for (int u = wave; u < 16; u += NW) {
            const int R = u >> 2, I = u & 3, rho = 16 * R + 7;
            f32x4 acc_a = {0.f, 0.f, 0.f, 0.f}, acc_m = acc_a;
            if (I <= R) {
                const int r = 16 * R + li, i = 16 * I + li;
                for (int ks = 0; ks < DK / 16; ++ks) {
                    f32x4 aa, am, bv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 16 * ks + 4 * lg + e;
                        const float grho = lt.g[rho * SP + c];
                        const float fr = __expf(lt.g[r * SP + c] - grho);
                        aa[e] = lt.bk[r * SP + c] * fr;
                        am[e] = lt.q[r * SP + c] * fr;
                        bv[e] = lt.k[i * SP + c] * __expf(grho - lt.g[i * SP + c]);
                    }
                    acc_a = mma_k16_f32(aa, bv, acc_a);
                    acc_m = mma_k16_f32(am, bv, acc_m);
                }
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int r = 16 * R + 4 * lg + ii, i = 16 * I + li;
                s[L_::A + r * C + i] = i < r ? acc_a[ii] : 0.f;
                s[L_::M + r * C + i] = i <= r ? acc_m[ii] : 0.f;
            }
        }
    }
    __syncthreads();
    // Tm = (I + A)^-1 by forward substitution (A strictly lower: row r of column col is
    // [r == col] - sum_{i<r} A[r][i] Tm[i][col], zero above the diagonal by itself), with A in
    // LDS (the key tiles are no longer needed). Eight lanes per column: lane l keeps
    // Tm[i][col] for i = l mod 8 in registers and sums those terms of each row; the eight
    // partial sums meet by lane exchanges.
    float *lA = reinterpret_cast<float *>(smem), *lT = lA + C * C;
    for (int e = tid; e < C * C; e += kBwdThreads) lA[e] = s[L_::A + e];
    __syncthreads();
    {
        static_assert(C * 8 == kBwdThreads, "eight lanes per column of Tm");
        const int col = tid >> 3, l = tid & 7;
        float tr[C / 8];
#pragma unroll
        for (int ib = 0; ib < C / 8; ++ib) tr[ib] = 0.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float part = 0.f;
#pragma unroll
            for (int ib = 0; 8 * ib < r; ++ib)
                if (8 * ib + l < r) part += lA[r * C + 8 * ib + l] * tr[ib];
            part += __shfl_xor(part, 1);
            part += __shfl_xor(part, 2);
            part += __shfl_xor(part, 4);
            const float t = (r == col ? 1.f : 0.f) - part;
            if ((r & 7) == l) {
                tr[r >> 3] = t;
                lT[r * C + col] = t;
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += kBwdThreads) s[L_::TM + e] = lT[e];
    __syncthreads();
    const float *sc = s;
    float *lf = reinterpret_cast<float *>(smem);       // product staging from here on
    block_mm_lds<C, DK, C, false, false>(lf, [&](int m, int kk) { return sc[L_::TM + m * C + kk]; },
             [&](int kk, int nn) { return sc[L_::Y + kk * DK + nn]; },
             [&](int m, int nn, float x) { s[L_::WT + m * DK + nn] = x; });
    block_mm_lds<C, DV, C, false, false>(lf, [&](int m, int kk) { return sc[L_::TM + m * C + kk]; },
             [&](int kk, int nn) { return sc[L_::X + kk * DV + nn]; },
             [&](int m, int nn, float x) { s[L_::UT + m * DV + nn] = x; });
    auto dO_at = [&](int r, int c) {
        return r < Lr ? io<T>::ld(dO + (static_cast<size_t>(t0 + r) * p.h_v + h) * DV + c) : 0.f;
    };
    block_mm_lds<C, DV, C, true, false>(lf, [&](int m, int kk) { return sc[L_::M + kk * C + m]; }, dO_at,
             [&](int m, int nn, float x) { s[L_::E1 + m * DV + nn] = x; });
    block_mm_lds<DK, DV, C, true, false>(lf, [&](int m, int kk) { return sc[L_::QG + kk * DK + m]; }, dO_at,
             [&](int m, int nn, float x) { s[L_::E2 + m * DV + nn] = x; });
}

__device__ __forceinline__ void dma16(const void *src, void *lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16, 0, 0);
}
// s_waitcnt with vmcnt(0) only
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS stage of one chunk for the reverse pass (W~ and Kg as fp32 tiles, or with bf16
// inputs as split operand fragments of the same size, then g_L): W~ and Kg ([C][DK] each, adjacent in the
// record scratch), then g_L.
template <int DK>
struct ChainStage {
    static constexpr int TILES = 2 * C * DK * 4;              // bytes of W~ and Kg
    static constexpr int BYTES = TILES + DK * 4;
};

// Four waves per workgroup, each owning 16 state columns of one (sequence, value head);
// the workgroup stages each chunk's W~, Kg and g_L in LDS (double-buffered, direct
// global-to-LDS loads issued one chunk ahead), and each wave prefetches its columns of
// M^T dO and Qg^T dO into registers one chunk ahead. The products are fp32 matrix-core tiles.
template <int DK, int DV>
__global__ __launch_bounds__(256) void bwd_chain_kernel(BwdParams p) {
    using L_ = BLay<DK, DV>;
    using CS = ChainStage<DK>;
    constexpr int RT = DK / 16, NS = DV / 16, WPP = NS / 4, UT = C / 16;
    static_assert(NS % 4 == 0, "four 16-column slices per workgroup");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int unit = blockIdx.x, pair = unit / WPP, part = unit - pair * WPP;
    const int n = pair / p.h_v, h = pair - n * p.h_v;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int col = 16 * (4 * part + wave) + li;
    int64_t start, end;
    int cbase;
    if (p.cu == nullptr) {
        start = static_cast<int64_t>(n) * p.seqlen;
        end = start + p.seqlen;
        cbase = n * p.nc_dense;
    } else {
        start = p.cu[n];
        end = p.cu[n + 1];
        cbase = p.map[n];
    }
    const int nchunks = static_cast<int>((end - start + C - 1) / C);
    auto scratch = [&](int c) {
        return p.scr + (static_cast<size_t>(cbase + c) * p.h_v + h) * L_::FLOATS;
    };
    auto stage = [&](int c, char *dst) {            // this wave's share of chunk c's copies
        const char *src = reinterpret_cast<const char *>(scratch(c) + L_::WT);
        for (int blk = wave; blk < CS::TILES / 1024; blk += 4)
            dma16(src + blk * 1024 + lane * 16, dst + blk * 1024);
        if (wave == 3 && lane < DK / 4)
            dma16(reinterpret_cast<const char *>(scratch(c) + L_::GL) + lane * 16, dst + CS::TILES);
    };
    float e1n[UT][4], e2n[RT][4];                   // this lane's M^T dO and Qg^T dO, next chunk
    auto prefetch = [&](int c) {
        const float *s = scratch(c);
#pragma unroll
        for (int ut = 0; ut < UT; ++ut)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) e1n[ut][ii] = s[L_::E1 + (16 * ut + 4 * lg + ii) * DV + col];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                e2n[rt][ii] = s[L_::E2 + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col];
    };

    f32x4 D[RT];                                    // dS' rows 16 rt + 4 lg + ii, column col
    const size_t sbase = (static_cast<size_t>(n) * p.h_v + h) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            D[rt][ii] = p.dS_T ? p.dS_T[sbase + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] : 0.f;
    if (nchunks > 0) {
        prefetch(nchunks - 1);
        stage(nchunks - 1, smem);
    }
    for (int c = nchunks - 1; c >= 0; --c) {
        const char *buf = smem + ((nchunks - 1 - c) & 1) * CS::BYTES;
        wait_vmem();                                // this wave's copies and prefetches landed
        __syncthreads();                            // everyone's; the other buffer is free
        float e1[UT][4], e2[RT][4];
#pragma unroll
        for (int ut = 0; ut < UT; ++ut)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) e1[ut][ii] = e1n[ut][ii];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) e2[rt][ii] = e2n[rt][ii];
        if (c > 0) {
            prefetch(c - 1);
            stage(c - 1, smem + ((nchunks - c) & 1) * CS::BYTES);
        }
        const float *wt = reinterpret_cast<const float *>(buf);
        const float *kg = wt + C * DK;
        const float *gl = wt + 2 * C * DK;
        float *s = scratch(c);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                s[L_::DSN + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] = D[rt][ii];
        // dU = M^T dO + Kg dS'
        f32x4 U4[UT];
#pragma unroll
        for (int ut = 0; ut < UT; ++ut) {
            f32x4 acc = {e1[ut][0], e1[ut][1], e1[ut][2], e1[ut][3]};
#pragma unroll
            for (int kt = 0; kt < RT; ++kt) {
                const f32x4 av = *reinterpret_cast<const f32x4 *>(&kg[(16 * ut + li) * DK + 16 * kt + 4 * lg]);
                acc = mma_k16_f32(av, D[kt], acc);
            }
            U4[ut] = acc;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) s[L_::DU + (16 * ut + 4 * lg + ii) * DV + col] = acc[ii];
        }
        // dS = gamma_L dS' + Qg^T dO - W~^T dU
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 acc;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                acc[ii] = __expf(gl[16 * rt + 4 * lg + ii]) * D[rt][ii] + e2[rt][ii];
#pragma unroll
            for (int kt = 0; kt < UT; ++kt) {
                f32x4 av;
#pragma unroll
                for (int e = 0; e < 4; ++e) av[e] = -wt[(16 * kt + 4 * lg + e) * DK + 16 * rt + li];
                acc = mma_k16_f32(av, U4[kt], acc);
            }
            D[rt] = acc;
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            p.dS0[sbase + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] = D[rt][ii];
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) void bwd_grads_kernel(BwdParams p) {
    using L_ = BLay<DK, DV>;
    const int rec = blockIdx.x, chunk = rec / p.h_v, h = rec - chunk * p.h_v;
    int n, j;
    int64_t start, end;
    if (!locate(p, chunk, n, j, start, end)) return;
    const int64_t t0 = start + static_cast<int64_t>(j) * C;
    const int Lr = static_cast<int>(min<int64_t>(C, end - t0));
    const int hk = h / p.group, tid = threadIdx.x;
    const T *b = static_cast<const T *>(p.b), *w = static_cast<const T *>(p.w);
    const T *v = static_cast<const T *>(p.v), *dO = static_cast<const T *>(p.dO);
    float *s = p.scr + static_cast<size_t>(rec) * L_::FLOATS;
    const float *sc = s;
    const float *S = p.ck + static_cast<size_t>(rec) * DK * DV;     // state entering the chunk
    extern __shared__ __attribute__((aligned(16))) char smem[];
    KeyTiles<DK, DK> lt(smem);                      // lanes run along channels: no padding
    constexpr int SP = DK;
    float *lDA = reinterpret_cast<float *>(smem + KeyTiles<DK, DK>::BYTES), *lDM = lDA + C * C;
    float *lf = reinterpret_cast<float *>(smem);       // product staging, then the tiles
    auto dO_at = [&](int r, int c) {
        return r < Lr ? io<T>::ld(dO + (static_cast<size_t>(t0 + r) * p.h_v + h) * DV + c) : 0.f;
    };

    // U = U~ - W~ S
    block_mm_lds<C, DV, DK, false, false>(lf, [&](int m, int kk) { return sc[L_::WT + m * DK + kk]; },
             [&](int kk, int nn) { return S[kk * DV + nn]; },
             [&](int m, int nn, float x) { s[L_::U + m * DV + nn] = sc[L_::UT + m * DV + nn] - x; });
    __syncthreads();
    // dM = lower(dO U^T), dQg = dO S^T, dKg = U dS'^T, dW~ = -dU S^T, dX = Tm^T dU
    block_mm_lds<C, C, DV, false, true>(lf, dO_at, [&](int kk, int nn) { return sc[L_::U + nn * DV + kk]; },
             [&](int m, int nn, float x) { s[L_::DM + m * C + nn] = nn <= m ? x : 0.f; });
    block_mm_lds<C, DK, DV, false, true>(lf, dO_at, [&](int kk, int nn) { return S[nn * DV + kk]; },
             [&](int m, int nn, float x) { s[L_::DQG + m * DK + nn] = x; });
    block_mm_lds<C, DK, DV, false, true>(lf, [&](int m, int kk) { return sc[L_::U + m * DV + kk]; },
             [&](int kk, int nn) { return sc[L_::DSN + nn * DV + kk]; },
             [&](int m, int nn, float x) { s[L_::DKG + m * DK + nn] = x; });
    block_mm_lds<C, DK, DV, false, true>(lf, [&](int m, int kk) { return sc[L_::DU + m * DV + kk]; },
             [&](int kk, int nn) { return S[nn * DV + kk]; },
             [&](int m, int nn, float x) { s[L_::DW + m * DK + nn] = -x; });
    block_mm_lds<C, DV, C, true, false>(lf, [&](int m, int kk) { return sc[L_::TM + kk * C + m]; },
             [&](int kk, int nn) { return sc[L_::DU + kk * DV + nn]; },
             [&](int m, int nn, float x) { s[L_::DX + m * DV + nn] = x; });
    {                                                   // dL/d gamma_L (before the exp)
        constexpr int PARTS = kBwdThreads / DK, PV = DV / PARTS;
        static_assert(PARTS == 4 || PARTS == 8, "four or eight threads per key channel");
        const int c = tid / PARTS, part = tid - c * PARTS;
        const size_t o = static_cast<size_t>(c) * DV + part * PV;
        float acc = 0.f;
#pragma unroll
        for (int vv = 0; vv < PV; ++vv) acc += sc[L_::DSN + o + vv] * S[o + vv];
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        if (PARTS == 8) acc += __shfl_xor(acc, 4);
        if (part == 0) s[L_::DGL + c] = acc;
    }
    __syncthreads();
    // dY = Tm^T dW~, dT = dU X^T + dW~ Y^T
    block_mm_lds<C, DK, C, true, false>(lf, [&](int m, int kk) { return sc[L_::TM + kk * C + m]; },
             [&](int kk, int nn) { return sc[L_::DW + kk * DK + nn]; },
             [&](int m, int nn, float x) { s[L_::DY + m * DK + nn] = x; });
    block_mm_lds<C, C, DV, false, true>(lf, [&](int m, int kk) { return sc[L_::DU + m * DV + kk]; },
             [&](int kk, int nn) { return sc[L_::X + nn * DV + kk]; },
             [&](int m, int nn, float x) { s[L_::DT + m * C + nn] = x; });
    __syncthreads();
    block_mm_lds<C, C, DK, false, true>(lf, [&](int m, int kk) { return sc[L_::DW + m * DK + kk]; },
             [&](int kk, int nn) { return sc[L_::Y + nn * DK + kk]; },
             [&](int m, int nn, float x) { s[L_::DT + m * C + nn] += x; });
    __syncthreads();
    // dA = strictly-lower(-Tm^T dT Tm^T)
    block_mm_lds<C, C, C, true, false>(lf, [&](int m, int kk) { return sc[L_::TM + kk * C + m]; },
             [&](int kk, int nn) { return sc[L_::DT + kk * C + nn]; },
             [&](int m, int nn, float x) { s[L_::TMP + m * C + nn] = x; });
    __syncthreads();
    block_mm_lds<C, C, C, false, true>(lf, [&](int m, int kk) { return sc[L_::TMP + m * C + kk]; },
             [&](int kk, int nn) { return sc[L_::TM + nn * C + kk]; },
             [&](int m, int nn, float x) { s[L_::DA + m * C + nn] = nn < m ? -x : 0.f; });
    __syncthreads();
    for (int e = tid; e < C * DK; e += kBwdThreads) {
        const int r = e / DK, c = e - r * DK;
        lt.g[r * SP + c] = sc[L_::G + e];
        lt.k[r * SP + c] = sc[L_::K + e];
        lt.q[r * SP + c] = sc[L_::Q + e];
        lt.bk[r * SP + c] = sc[L_::BK + e];
    }
    for (int e = tid; e < C * C; e += kBwdThreads) {
        lDA[e] = sc[L_::DA + e];
        lDM[e] = sc[L_::DM + e];
    }
    __syncthreads();
    // The decay sums on the matrix cores, per 16-row block B with reference row rho = 16 B + 7
    // (exp(g_r - g_i) = exp(g_r - g_rho) exp(g_rho - g_i), every factor within 8 tokens of
    // decay or <= 1):
    //   P1[x] = sum_{i<x}  dA[x,i] k_i E[x,i],   P3[x] = sum_{i<=x} dM[x,i] k_i E[x,i]   (x in B)
    //   P2[x] = sum_{r>x}  dA[r,x] bk_r E[r,x],  P4[x] = sum_{r>=x} dM[r,x] q_r E[r,x]  (x in B)
    // dA and dM carry their triangular masks, so each block runs over whole 16-row k blocks.
    // One wave per (row block, 16 key channels) forms all four (B + 1 plus 4 - B k blocks,
    // the same work for every unit), then takes them through E, Y, Qg and Kg to q, k, b and
    // g for its 16 x 16 entries: lane (li, lg) holds rows 16 B + 4 lg + ii of channel
    // n0 + li. Its scratch loads are issued before the products.
    float *dq = p.dq, *dk = p.dk;
    {
        const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
        constexpr int NW = kBwdThreads / 64, CT = DK / 16;
        for (int u = wave; u < 4 * CT; u += NW) {
            const int B = u / CT, n0 = (u - B * CT) * 16, rho = 16 * B + 7, c = n0 + li;
            float dy[4], dqg[4], dkg[4], bb[4];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int x = 16 * B + 4 * lg + ii;
                dy[ii] = sc[L_::DY + x * DK + c];
                dqg[ii] = sc[L_::DQG + x * DK + c];
                dkg[ii] = sc[L_::DKG + x * DK + c];
                bb[ii] = x < Lr ? io<T>::ld(b + (static_cast<size_t>(t0 + x) * p.h_v + h) * DK + c) : 0.f;
            }
            const float glc = sc[L_::GL + c];
            const float grho = lt.g[rho * SP + c];
            f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a3 = a1, a2 = a1, a4 = a1;
            for (int kb = 0; kb <= B; ++kb) {           // P1, P3: k over rows 0 .. 16 B + 15
                f32x4 d1, d3, bv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * kb + 4 * lg + e;
                    d1[e] = lDA[(16 * B + li) * C + i];
                    d3[e] = lDM[(16 * B + li) * C + i];
                    bv[e] = lt.k[i * SP + c] * __expf(grho - lt.g[i * SP + c]);
                }
                a1 = mma_k16_f32(d1, bv, a1);
                a3 = mma_k16_f32(d3, bv, a3);
            }
            for (int kb = B; kb < C / 16; ++kb) {       // P2, P4: k over rows 16 B .. C - 1
                f32x4 d2, d4, b2, b4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * kb + 4 * lg + e;
                    d2[e] = lDA[r * C + 16 * B + li];
                    d4[e] = lDM[r * C + 16 * B + li];
                    const float f = __expf(lt.g[r * SP + c] - grho);
                    b2[e] = lt.bk[r * SP + c] * f;
                    b4[e] = lt.q[r * SP + c] * f;
                }
                a2 = mma_k16_f32(d2, b2, a2);
                a4 = mma_k16_f32(d4, b4, a4);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int x = 16 * B + 4 * lg + ii;
                const float gx = lt.g[x * SP + c];
                const float f0 = __expf(gx - grho), f1 = __expf(grho - gx);
                const float p1 = a1[ii] * f0, p3 = a3[ii] * f0, p2 = a2[ii] * f1, p4 = a4[ii] * f1;
                const float ga = __expf(gx), fk = __expf(glc - gx);
                const float kk = lt.k[x * SP + c], qq = lt.q[x * SP + c], bk = lt.bk[x * SP + c];
                const float dbk = p1 + ga * dy[ii];
                const float dgv = bk * p1 - kk * p2 + qq * p3 - kk * p4 + ga * bk * dy[ii] +
                                  ga * qq * dqg[ii] - fk * kk * dkg[ii];
                s[L_::DY + x * DK + c] = dgv;          // this lane's own entries, read above
                s[L_::DKG + x * DK + c] = fk * kk * dkg[ii];
                if (x < Lr) {
                    const size_t ok = (static_cast<size_t>(t0 + x) * p.h_k + hk) * DK + c;
                    const size_t og = (static_cast<size_t>(t0 + x) * p.h_v + h) * DK + c;
                    if (p.group == 1) {
                        dq[ok] = p3 + ga * dqg[ii];
                        dk[ok] = p4 + p2 + fk * dkg[ii] + bb[ii] * dbk;
                    } else {
                        atomicAdd(dq + ok, p3 + ga * dqg[ii]);
                        atomicAdd(dk + ok, p4 + p2 + fk * dkg[ii] + bb[ii] * dbk);
                    }
                    p.db[og] = kk * dbk;
                }
            }
        }
    }
    for (int e = tid; e < C * DV; e += kBwdThreads) {
        const int x = e / DV, c = e - x * DV;
        if (x < Lr) {
            const size_t ov = (static_cast<size_t>(t0 + x) * p.h_v + h) * DV + c;
            const float dx = sc[L_::DX + x * DV + c];
            p.dv[ov] = io<T>::ld(w + ov) * dx;
            p.dw[ov] = io<T>::ld(v + ov) * dx;
        }
    }
    __syncthreads();
    // d log alpha: reverse cumulative sum of dg, with the gamma_L terms on the last row
    // PARTS threads per key channel, RP rows each: every load first, then the partial sums
    // meet by lane exchanges (the DKG terms over all rows, the dg sums of later parts)
    {
        constexpr int PARTS = kBwdThreads / DK, RP = C / PARTS;
        static_assert(PARTS * DK == kBwdThreads && (PARTS == 4 || PARTS == 8), "parts per channel");
        const int c = tid / PARTS, part = tid - c * PARTS, x0 = part * RP;
        float dgv[RP], dkt[RP];
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            dgv[i] = sc[L_::DY + (x0 + i) * DK + c];
            dkt[i] = sc[L_::DKG + (x0 + i) * DK + c];
        }
        const float base = __expf(sc[L_::GL + c]) * sc[L_::DGL + c];
        float all = 0.f, own = 0.f;
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            all += dkt[i];
            own += dgv[i];
        }
        all += __shfl_xor(all, 1);
        all += __shfl_xor(all, 2);
        if (PARTS == 8) all += __shfl_xor(all, 4);
        float later = 0.f;
#pragma unroll
        for (int q = 0; q < PARTS; ++q) {
            const float o = __shfl(own, q, PARTS);
            if (q > part) later += o;
        }
        float acc = base + all + later;
#pragma unroll
        for (int i = RP - 1; i >= 0; --i) {
            acc += dgv[i];
            if (x0 + i < Lr) p.dla[(static_cast<size_t>(t0 + x0 + i) * p.h_v + h) * DK + c] = acc;
        }
    }
}

template <typename T, int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t st) {
    static_assert(BLay<DK, DV>::FLOATS == 12 * static_cast<size_t>(C) * DK + 6 * static_cast<size_t>(C) * DV +
                      2 * static_cast<size_t>(DK) * DV + 7 * static_cast<size_t>(C) * C + 2 * DK,
                  "the per-record scratch matches chunk_bwd_workspace_bytes");
    const bool packed = a.cu_seqlens != nullptr;
    const int N = packed ? a.num_seqs : a.batch;
    const int64_t nrec = chunk_upper_bound(kChunk, a.batch, a.seqlen, a.num_seqs, packed) * a.h_v;
    char *base = a.workspace;
    const size_t fwd_ws = chunk_workspace_bytes(kChunk, a.batch, a.seqlen, a.num_seqs, a.h_v, DK, DV,
                                                a.bf16, packed);
    float *ck = reinterpret_cast<float *>(base + fwd_ws);
    char *o_scratch = base + (fwd_ws + static_cast<size_t>(nrec) * DK * DV * 4 + 255) / 256 * 256;
    const size_t o_bytes = (static_cast<size_t>(a.batch) * a.seqlen * a.h_v * DV * sizeof(T) + 255) / 256 * 256;
    float *scr = reinterpret_cast<float *>(o_scratch + o_bytes);

    ChunkArgs f;
    f.q = a.q; f.k = a.k; f.v = a.v; f.log_alpha = a.log_alpha; f.b = a.b; f.w = a.w;
    f.S0 = a.S0; f.cu_seqlens = a.cu_seqlens; f.o = o_scratch; f.S_T = nullptr;
    f.workspace = base;
    f.batch = a.batch; f.seqlen = a.seqlen; f.num_seqs = a.num_seqs;
    f.h_k = a.h_k; f.h_v = a.h_v; f.d_k = DK; f.d_v = DV; f.bf16 = a.bf16;
    f.fu = Fusion{};
    f.fu.cks = ck;
    hipError_t e = launch_chunk_fwd(f, st);
    if (e != hipSuccess) return e;

    BwdParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.la = a.log_alpha; p.b = a.b; p.w = a.w; p.dO = a.dO;
    p.dS_T = a.dS_T;
    p.cu = a.cu_seqlens;
    p.map = packed ? reinterpret_cast<const int32_t *>(base) : nullptr;
    p.ck = ck;
    p.scr = scr;
    p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dw = a.dw; p.dla = a.dla; p.db = a.db; p.dS0 = a.dS0;
    p.num_seqs = N; p.seqlen = a.seqlen;
    p.nc_dense = (a.seqlen + C - 1) / C;
    p.h_k = a.h_k; p.h_v = a.h_v; p.group = a.h_v / a.h_k;
    const int64_t qk = static_cast<int64_t>(a.batch) * a.seqlen * a.h_k * DK;
    if (qk > 0 && p.group > 1) {
        const int64_t blocks = (qk + 255) / 256;
        hipLaunchKernelGGL(zero_kernel, dim3(blocks < 4096 ? blocks : 4096), dim3(256), 0, st,
                           a.dq, a.dk, qk);
    }
    constexpr int klds = KeyTiles<DK>::BYTES;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(bwd_factors_kernel<T, DK, DV>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, klds);
    if (e != hipSuccess) return e;
    constexpr int glds = KeyTiles<DK, DK>::BYTES + 2 * C * C * 4;
    constexpr auto mm = [](int M, int N, int K) { return 4 * (M * (K + 4) + K * (N + 4)); };
    static_assert(mm(C, DK, C) <= klds && mm(C, DV, C) <= klds && mm(DK, DV, C) <= klds,
                  "the staged products of the factors kernel fit in its LDS");
    static_assert(mm(C, DV, DK) <= glds && mm(C, C, DV) <= glds && mm(C, DK, DV) <= glds &&
                      mm(C, DK, C) <= glds && mm(C, C, DK) <= glds && mm(C, C, C) <= glds,
                  "the staged products of the gradients kernel fit in its LDS");
    static_assert(glds <= 160 * 1024 && klds <= 160 * 1024, "LDS");
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(bwd_grads_kernel<T, DK, DV>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, glds);
    if (e != hipSuccess) return e;
    if (nrec > 0) {
        hipLaunchKernelGGL((bwd_factors_kernel<T, DK, DV>), dim3(nrec), dim3(kBwdThreads), klds, st, p);
    }
    const int64_t units = static_cast<int64_t>(N) * a.h_v * (DV / 64);
    if (units > 0) {
        const int lds = 2 * ChainStage<DK>::BYTES;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(bwd_chain_kernel<DK, DV>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_chain_kernel<DK, DV>), dim3(units), dim3(256), lds, st, p);
    }
    if (nrec > 0) {
        hipLaunchKernelGGL((bwd_grads_kernel<T, DK, DV>), dim3(nrec), dim3(kBwdThreads), glds, st, p);
    }
    return hipGetLastError();
}


}  // namespace

size_t chunk_bwd_workspace_bytes(int batch, int seqlen, int num_seqs, int h_v, int d_k, int d_v,
                                 bool bf16, bool packed) {
    if (bf16) return chunk_bwd16_workspace_bytes(batch, seqlen, num_seqs, h_v, d_k, d_v, packed);
    const int64_t nrec = chunk_upper_bound(kChunk, batch, seqlen, num_seqs, packed) * h_v;
    // (the floats of BLay<d_k, d_v>)
    const size_t per = 4 * (12 * static_cast<size_t>(C) * d_k + 6 * static_cast<size_t>(C) * d_v +
                            2 * static_cast<size_t>(d_k) * d_v + 7 * static_cast<size_t>(C) * C + 2 * d_k);
    const size_t o_bytes = (static_cast<size_t>(batch) * seqlen * h_v * d_v * (bf16 ? 2 : 4) + 255) / 256 * 256;
    const size_t head = (chunk_workspace_bytes(kChunk, batch, seqlen, num_seqs, h_v, d_k, d_v, bf16, packed) +
                         static_cast<size_t>(nrec) * d_k * d_v * 4 + 255) / 256 * 256;
    return head + o_bytes + static_cast<size_t>(nrec) * per;
}

hipError_t launch_chunk_bwd(const BwdArgs &a, hipStream_t st) {
    if (a.bf16) return launch_chunk_bwd16(a, st);
    if (a.d_k == 64 && a.d_v == 64) return launch_bwd_t<float, 64, 64>(a, st);
    if (a.d_k == 128 && a.d_v == 128) return launch_bwd_t<float, 128, 128>(a, st);
    if (a.d_k == 128 && a.d_v == 64) return launch_bwd_t<float, 128, 64>(a, st);
    if (a.d_k == 64 && a.d_v == 128) return launch_bwd_t<float, 64, 128>(a, st);
    return hipErrorInvalidValue;            // refused by the API layer before the launch
}

}  // namespace gdn2
