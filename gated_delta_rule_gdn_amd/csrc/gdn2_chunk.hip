// gdn2_chunk.hip -- chunked WY forward of Gated DeltaNet-2 on gfx950.
//
// Method: burn-gdn2 0.1.5 docs page, section "Architecture" (the per-token recurrence and
// its "Chunk WY" training path); the FG^2-GDN summary (section 2C) notes that the
// identity-plus-rank-1 (DPLR) transition is what lets the WY representation apply.
// Within a chunk of C = 64 tokens entering with state S (token vectors are rows,
// g_r = sum_{i<=r} log alpha_i per key channel, gamma = exp(g)):
//   A[r,i]  = sum_c b_r k_r k_i exp(g_r - g_i)      (i < r)       strictly lower
//   M[r,i]  = sum_c q_r k_i exp(g_r - g_i)          (i <= r)      lower, with diagonal
//   T       = (I + A)^{-1}
//   W~      = T (gamma . b . k),   U~ = T (w . v)                  (WY factors)
//   U       = U~ - W~ S                                             (erase-corrected writes)
//   O       = (gamma . q) S + M U
//   S_next  = diag(gamma_C) S + ((gamma_C / gamma) . k)^T U
// (derived from the recurrence by unrolling it over the chunk; checked against the
// token-by-token recurrence in fp64 by the test suite).
//
// Kernels:
//   K0 chunk_map_kernel    packed batches: chunk offsets per sequence (no host sync).
//   K1 chunk_prep_kernel   one workgroup per (chunk, value head), fully parallel: the
//                          cumulative log decay, A and M on the matrix cores, the 16x16
//                          diagonal inverses of (I + A), a blocked forward substitution for
//                          W~ and U~, and the per-chunk operands of K2, written to the
//                          workspace already in matrix-core fragment order.
//   K2 chunk_state_kernel  one wave per (sequence, value head, 16 columns of S), sequential
//                          over the chunks of its sequence with its slice of S held in
//                          registers in fp32; writes o and S_T.
//
// Numerics: exp(g_r - g_i) is split as exp(g_r - ref) * exp(ref - g_i). For a block of
// rows r in 16-token sub-chunk R against columns in an earlier sub-chunk, ref is the
// cumulative decay at the end of sub-chunk R-1, so both factors are <= 1 and cannot
// overflow (an underflowed factor means a negligible true product). Diagonal 16x16 blocks
// use the middle token of the sub-chunk, so each factor spans at most 8 tokens of decay.
// Padding rows of a partial chunk are identity tokens (k = q = b = 0, w.v = 0,
// log alpha = 0), which leave the state unchanged.
#include "gdn2_common.h"
#include "gdn2_internal.h"
#include "gdn2_mfma.h"

namespace gdn2 {

template <bool BF> struct Op;
template <> struct Op<true> {     // bf16 operands, K = 32 per fragment block
    using type = bf16_t;
    static constexpr int KT = 32, EPL = 8, E = 2;
};
template <> struct Op<false> {    // fp32 operands, K = 16 per fragment block
    using type = float;
    static constexpr int KT = 16, EPL = 4, E = 4;
};

// Per (chunk, value head) workspace record. A-operand matrices are stored as 1 KB fragment
// blocks (64 lanes x 16 B) in (row tile, k tile) order, in perm order (gdn2_mfma.h):
//   Wn  = -W~          [C][DK]   (K2: U = U~ + Wn S)
//   Qg  = gamma . q     [C][DK]   (K2: O = Qg S + M U)
//   KgT = ((gamma_C / gamma) . k)^T  [DK][C]  (K2: S = gamma_C S + KgT U)
//   M                   [C][C]
// U~ is stored as output tiles (D layout), column tile major; gamma_C as fp32 [DK].
template <int DK, int DV, bool BF>
struct Rec {
    static constexpr size_t E = Op<BF>::E;
    static constexpr size_t Wn = 0;
    static constexpr size_t Qg = Wn + kChunk * DK * E;
    static constexpr size_t KgT = Qg + kChunk * DK * E;
    static constexpr size_t M = KgT + DK * kChunk * E;
    static constexpr size_t Ut = M + kChunk * kChunk * E;
    static constexpr size_t gC = Ut + kChunk * DV * E;
    static constexpr size_t bytes = (gC + DK * 4 + 255) / 256 * 256;
    static constexpr int NKT_DK = DK / Op<BF>::KT;     // k tiles over d_k
    static constexpr int NKT_C = kChunk / Op<BF>::KT;  // k tiles over the chunk
    static constexpr size_t UT_TILE = 64 * 4 * E;       // one D-layout tile
};

struct ChunkParams {
    const void *q, *k, *v, *log_alpha, *b, *w;
    const float *S0;
    const int32_t *cu;
    const int32_t *map;
    void *o;
    float *S_T;
    char *rec;           // first per-(chunk, head) record
    int seqlen, num_seqs, h_k, h_v, group, nc_dense, num_pairs, nslices;
};

// Locates chunk `chunk` of the batch: sequence n, its chunk index j, and token range.
__device__ __forceinline__ bool locate_chunk(const ChunkParams &p, int chunk, int &n, int &j,
                                             int64_t &start, int64_t &end) {
    if (p.cu == nullptr) {
        n = chunk / p.nc_dense;
        j = chunk - n * p.nc_dense;
        start = static_cast<int64_t>(n) * p.seqlen;
        end = start + p.seqlen;
        return true;
    }
    if (chunk >= p.map[p.num_seqs]) return false;
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {                       // largest n with map[n] <= chunk
        const int mid = (lo + hi + 1) >> 1;
        if (p.map[mid] <= chunk) lo = mid; else hi = mid - 1;
    }
    n = lo;
    j = chunk - p.map[n];
    start = p.cu[n];
    end = p.cu[n + 1];
    return true;
}

// K0: chunk offsets of a packed batch, map[n] = sum_{m<n} ceil(len_m / C).
__global__ void chunk_map_kernel(const int32_t *__restrict__ cu, int32_t *__restrict__ map,
                                 int num_seqs) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        int acc = 0;
        map[0] = 0;
        for (int n = 0; n < num_seqs; ++n) {
            int len = cu[n + 1] - cu[n];
            len = len < 0 ? 0 : len;
            acc += (len + kChunk - 1) / kChunk;
            map[n + 1] = acc;
        }
    }
}

template <bool BF>
__device__ __forceinline__ u32x4 pack16(const float *v) {
    u32x4 r;
    if constexpr (BF) {
        r.x = pack_bf16x2(v[0], v[1]);
        r.y = pack_bf16x2(v[2], v[3]);
        r.z = pack_bf16x2(v[4], v[5]);
        r.w = pack_bf16x2(v[6], v[7]);
    } else {
        r.x = __float_as_uint(v[0]);
        r.y = __float_as_uint(v[1]);
        r.z = __float_as_uint(v[2]);
        r.w = __float_as_uint(v[3]);
    }
    return r;
}

// ---------------------------------------------------------------------------------------
// K1: per (chunk, value head) WY factors and K2 operands.
// ---------------------------------------------------------------------------------------
template <typename T, bool BF, int DK, int DV>
__global__ __launch_bounds__(512) void chunk_prep_kernel(ChunkParams p) {
    using R_ = Rec<DK, DV, BF>;
    using OT = typename Op<BF>::type;
    constexpr int C = kChunk, NT = 512, NW = NT / 64;
    constexpr int KT = Op<BF>::KT, EPL = Op<BF>::EPL;
    constexpr int VEC = 16 / sizeof(T);          // raw elements per 16-byte load
    constexpr int CP = C + 1;                    // padded row stride of A and M
    constexpr int PARTS = NT / DK;               // cumsum: token parts per channel
    constexpr int RPP = C / PARTS;               // rows per part
    static_assert(sizeof(T) == sizeof(OT), "raw and operand types share LDS staging");

    __shared__ __attribute__((aligned(16))) T s_k[C * DK];
    __shared__ __attribute__((aligned(16))) T s_q[C * DK];   // later: -W~ staging
    __shared__ __attribute__((aligned(16))) T s_b[C * DK];
    __shared__ __attribute__((aligned(16))) T s_v[C * DV];
    __shared__ __attribute__((aligned(16))) T s_w[C * DV];
    __shared__ __attribute__((aligned(16))) float s_g[C * DK];
    __shared__ float s_part[PARTS * DK];
    __shared__ float s_A[C * CP];
    __shared__ float s_M[C * CP];
    __shared__ float s_T[4 * 16 * 16];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int chunk = blockIdx.x, h = blockIdx.y, hk = h / p.group;
    int n, j;
    int64_t start, end;
    if (!locate_chunk(p, chunk, n, j, start, end)) return;
    const int64_t t0 = start + static_cast<int64_t>(j) * C;
    const int L = static_cast<int>(min<int64_t>(C, end - t0));
    char *rec = p.rec + (static_cast<size_t>(chunk) * p.h_v + h) * R_::bytes;

    // ---- phase 0: stage raw tiles, zero A/M, cumulative log decay ----
    {
        const T *kp = static_cast<const T *>(p.k), *qp = static_cast<const T *>(p.q);
        const T *bp = static_cast<const T *>(p.b);
        const T *vp = static_cast<const T *>(p.v), *wp = static_cast<const T *>(p.w);
        constexpr int VK = DK / VEC, VV = DV / VEC;
        for (int idx = tid; idx < C * VK; idx += NT) {
            const int r = idx / VK, cv = idx - r * VK;
            u32x4 kv = {0u, 0u, 0u, 0u}, qv = kv, bv = kv;
            if (r < L) {
                const size_t ok = (static_cast<size_t>(t0 + r) * p.h_k + hk) * DK + cv * VEC;
                const size_t ob = (static_cast<size_t>(t0 + r) * p.h_v + h) * DK + cv * VEC;
                kv = *reinterpret_cast<const u32x4 *>(kp + ok);
                qv = *reinterpret_cast<const u32x4 *>(qp + ok);
                bv = *reinterpret_cast<const u32x4 *>(bp + ob);
            }
            *reinterpret_cast<u32x4 *>(&s_k[r * DK + cv * VEC]) = kv;
            *reinterpret_cast<u32x4 *>(&s_q[r * DK + cv * VEC]) = qv;
            *reinterpret_cast<u32x4 *>(&s_b[r * DK + cv * VEC]) = bv;
        }
        for (int idx = tid; idx < C * VV; idx += NT) {
            const int r = idx / VV, cv = idx - r * VV;
            u32x4 vv = {0u, 0u, 0u, 0u}, wv = vv;
            if (r < L) {
                const size_t ov = (static_cast<size_t>(t0 + r) * p.h_v + h) * DV + cv * VEC;
                vv = *reinterpret_cast<const u32x4 *>(vp + ov);
                wv = *reinterpret_cast<const u32x4 *>(wp + ov);
            }
            *reinterpret_cast<u32x4 *>(&s_v[r * DV + cv * VEC]) = vv;
            *reinterpret_cast<u32x4 *>(&s_w[r * DV + cv * VEC]) = wv;
        }
        for (int idx = tid; idx < C * CP; idx += NT) {
            s_A[idx] = 0.f;
            s_M[idx] = 0.f;
        }
        const T *lap = static_cast<const T *>(p.log_alpha);
        const int c = tid % DK, part = tid / DK;
        float acc = 0.f;
        for (int rr = 0; rr < RPP; ++rr) {
            const int r = part * RPP + rr;
            const float x = (r < L)
                ? io<T>::ld(lap + (static_cast<size_t>(t0 + r) * p.h_v + h) * DK + c) : 0.f;
            acc += x;
            s_g[r * DK + c] = acc;
        }
        s_part[part * DK + c] = acc;
        __syncthreads();
        float pre = 0.f;
        for (int pp = 0; pp < part; ++pp) pre += s_part[pp * DK + c];
        for (int rr = 0; rr < RPP; ++rr) s_g[(part * RPP + rr) * DK + c] += pre;
        __syncthreads();
        if (tid < DK) {
            reinterpret_cast<float *>(rec + R_::gC)[tid] = __expf(s_g[(C - 1) * DK + tid]);
        }
    }

    // ---- phase 1a: A and M, 16x16 blocks (R >= I) on the matrix cores ----
    for (int pr = wave; pr < 10; pr += NW) {
        const int R = pr >= 6 ? 3 : (pr >= 3 ? 2 : (pr >= 1 ? 1 : 0));
        const int I = pr - R * (R + 1) / 2;
        const bool diag = (R == I);
        const int refrow = diag ? 16 * R + 7 : 16 * R - 1;   // R >= 1 when off-diagonal
        const int r = 16 * R + li;                           // A-operand row (token)
        const int i = 16 * I + li;                           // B-operand column (token)
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = accA;
#pragma unroll
        for (int kt = 0; kt < DK / KT; ++kt) {
            if constexpr (BF) {
                float ak[8], aq[8], bk[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int c = kt * 32 + 8 * lg + jj;
                    const float ref = s_g[refrow * DK + c];
                    const float ef = __expf(s_g[r * DK + c] - ref);
                    const float ec = __expf(ref - s_g[i * DK + c]);
                    const float kr = io<T>::ld(&s_k[r * DK + c]);
                    ak[jj] = io<T>::ld(&s_b[r * DK + c]) * kr * ef;
                    aq[jj] = io<T>::ld(&s_q[r * DK + c]) * ef;
                    bk[jj] = io<T>::ld(&s_k[i * DK + c]) * ec;
                }
                const u32x4 B = pack16<true>(bk);
                accA = mma_k32(pack16<true>(ak), B, accA);
                accM = mma_k32(pack16<true>(aq), B, accM);
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int c = kt * 16 + 4 * lg + s;
                    const float ref = s_g[refrow * DK + c];
                    const float ef = __expf(s_g[r * DK + c] - ref);
                    const float ec = __expf(ref - s_g[i * DK + c]);
                    const float kr = io<T>::ld(&s_k[r * DK + c]);
                    const float bk = io<T>::ld(&s_k[i * DK + c]) * ec;
                    accA = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        io<T>::ld(&s_b[r * DK + c]) * kr * ef, bk, accA, 0, 0, 0);
                    accM = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        io<T>::ld(&s_q[r * DK + c]) * ef, bk, accM, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int row = 16 * R + 4 * lg + ii, col = 16 * I + li;
            float a = accA[ii], m = accM[ii];
            if (diag) {
                if (col >= row) a = 0.f;
                if (col > row) m = 0.f;
            }
            s_A[row * CP + col] = a;
            s_M[row * CP + col] = m;
        }
    }

    // ---- phase 1b: Qg and KgT fragment blocks (elementwise) ----
    {
        constexpr int NBQ = (C / 16) * R_::NKT_DK;      // Qg blocks
        constexpr int NBK = (DK / 16) * R_::NKT_C;      // KgT blocks
        u32x4 *qg = reinterpret_cast<u32x4 *>(rec + R_::Qg);
        u32x4 *kg = reinterpret_cast<u32x4 *>(rec + R_::KgT);
        for (int idx = tid; idx < (NBQ + NBK) * 64; idx += NT) {
            const int blk = idx >> 6, l = idx & 63, lli = l & 15, llg = l >> 4;
            float vals[EPL];
            if (blk < NBQ) {
                const int rt = blk / R_::NKT_DK, kt = blk - rt * R_::NKT_DK;
                const int r = 16 * rt + lli;
#pragma unroll
                for (int jj = 0; jj < EPL; ++jj) {
                    const int c = kt * KT + perm_k<BF>(llg, jj);
                    vals[jj] = __expf(s_g[r * DK + c]) * io<T>::ld(&s_q[r * DK + c]);
                }
                qg[blk * 64 + l] = pack16<BF>(vals);
            } else {
                const int b2 = blk - NBQ;
                const int rt = b2 / R_::NKT_C, kt = b2 - rt * R_::NKT_C;
                const int ch = 16 * rt + lli;
                const float gl = s_g[(C - 1) * DK + ch];
#pragma unroll
                for (int jj = 0; jj < EPL; ++jj) {
                    const int tok = kt * KT + perm_k<BF>(llg, jj);
                    vals[jj] = __expf(gl - s_g[tok * DK + ch]) * io<T>::ld(&s_k[tok * DK + ch]);
                }
                kg[b2 * 64 + l] = pack16<BF>(vals);
            }
        }
    }
    __syncthreads();

    // ---- phase 2: wave 0 inverts the four 16x16 diagonal blocks of (I + A); the other
    //      waves write M in fragment order ----
    if (wave == 0) {
        const int R = lane >> 4, jc = lane & 15;      // column jc of T_RR
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == jc) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) acc += s_A[(16 * R + r) * CP + 16 * R + m] * x[m];
            if (r > jc) x[r] = -acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s_T[(R * 16 + r) * 16 + jc] = x[r];
    } else {
        constexpr int NBM = (C / 16) * R_::NKT_C;
        u32x4 *mg = reinterpret_cast<u32x4 *>(rec + R_::M);
        for (int idx = tid - 64; idx < NBM * 64; idx += NT - 64) {
            const int blk = idx >> 6, l = idx & 63, lli = l & 15, llg = l >> 4;
            const int rt = blk / R_::NKT_C, kt = blk - rt * R_::NKT_C;
            const int r = 16 * rt + lli;
            float vals[EPL];
#pragma unroll
            for (int jj = 0; jj < EPL; ++jj) vals[jj] = s_M[r * CP + kt * KT + perm_k<BF>(llg, jj)];
            mg[blk * 64 + l] = pack16<BF>(vals);
        }
    }
    __syncthreads();

    // ---- phase 3: blocked forward substitution, Y_R = T_RR (X_R - sum_{I<R} A_RI Y_I),
    //      for X = gamma.b.k (Y = W~) and X = w.v (Y = U~); one 16-column tile per pass ----
    {
        constexpr int NCTW = DK / 16, NCT = DK / 16 + DV / 16;
        OT *s_W = reinterpret_cast<OT *>(s_q);           // -W~ staging, [C][DK]
        for (int ctile = wave; ctile < NCT; ctile += NW) {
            const bool isW = ctile < NCTW;
            const int ct = isW ? ctile : ctile - NCTW;
            const int col = 16 * ct + li;
            f32x4 Y[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                f32x4 Z;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int r = 16 * R + 4 * lg + ii;
                    Z[ii] = isW ? __expf(s_g[r * DK + col]) * io<T>::ld(&s_b[r * DK + col]) *
                                      io<T>::ld(&s_k[r * DK + col])
                                : io<T>::ld(&s_w[r * DV + col]) * io<T>::ld(&s_v[r * DV + col]);
                }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int I = 0; I < R; ++I) {
                    const float *ap = &s_A[(16 * R + li) * CP + 16 * I + 4 * lg];
                    const f32x4 a = {ap[0], ap[1], ap[2], ap[3]};
                    if constexpr (BF) acc = mma_k16_bf16(f4_to_b16(a), f4_to_b16(Y[I]), acc);
                    else acc = mma_k16_f32(a, Y[I], acc);
                }
                Z -= acc;
                const f32x4 t = *reinterpret_cast<const f32x4 *>(&s_T[(R * 16 + li) * 16 + 4 * lg]);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                if constexpr (BF) Y[R] = mma_k16_bf16(f4_to_b16(t), f4_to_b16(Z), zero);
                else Y[R] = mma_k16_f32(t, Z, zero);
            }
            if (!isW) {
                char *ut = rec + R_::Ut;
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    const size_t off = (static_cast<size_t>(ct) * 4 + R) * R_::UT_TILE;
                    if constexpr (BF) {
                        reinterpret_cast<u32x2 *>(ut + off)[lane] = f4_to_b16(Y[R]);
                    } else {
                        reinterpret_cast<f32x4 *>(ut + off)[lane] = Y[R];
                    }
                }
            } else {
#pragma unroll
                for (int R = 0; R < 4; ++R)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        io<OT>::st(&s_W[(16 * R + 4 * lg + ii) * DK + col], -Y[R][ii]);
            }
        }
    }
    __syncthreads();

    // ---- phase 4: -W~ in fragment order ----
    {
        constexpr int NBW = (C / 16) * R_::NKT_DK;
        const OT *s_W = reinterpret_cast<const OT *>(s_q);
        u32x4 *wg = reinterpret_cast<u32x4 *>(rec + R_::Wn);
        for (int idx = tid; idx < NBW * 64; idx += NT) {
            const int blk = idx >> 6, l = idx & 63, lli = l & 15, llg = l >> 4;
            const int rt = blk / R_::NKT_DK, kt = blk - rt * R_::NKT_DK;
            const int r = 16 * rt + lli;
            float vals[EPL];
#pragma unroll
            for (int jj = 0; jj < EPL; ++jj)
                vals[jj] = io<OT>::ld(&s_W[r * DK + kt * KT + perm_k<BF>(llg, jj)]);
            wg[blk * 64 + l] = pack16<BF>(vals);
        }
    }
}

// ---------------------------------------------------------------------------------------
// K2: inter-chunk state pass. Each wave owns 16 columns of S (all d_k rows) as DK/16
// output tiles in fp32 registers and walks the chunks of its sequence in order.
// ---------------------------------------------------------------------------------------
template <typename T, bool BF, int DK, int DV>
__global__ __launch_bounds__(256) void chunk_state_kernel(ChunkParams p) {
    using R_ = Rec<DK, DV, BF>;
    constexpr int C = kChunk, RT = DK / 16;
    constexpr int NKD = R_::NKT_DK, NKC = R_::NKT_C;
    const int nw = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;

    // XCD-aware decode: the column slices of one (sequence, head) pair share an XCD, so
    // its workspace records are fetched into one L2.
    const int bid = blockIdx.x, xcd = bid & 7, rest = bid >> 3;
    const int slice = rest % p.nslices;
    const int pair = (rest / p.nslices) * 8 + xcd;
    if (pair >= p.num_pairs) return;
    const int n = pair / p.h_v, h = pair - n * p.h_v;
    const int ct = slice * nw + wave;
    const int col = 16 * ct + li;

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

    f32x4 S[RT];
    const size_t sbase = static_cast<size_t>(pair) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            S[rt][ii] = p.S0 ? p.S0[sbase + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col]
                             : 0.f;

    T *op = static_cast<T *>(p.o);
    for (int c = 0; c < nchunks; ++c) {
        const char *rec = p.rec + (static_cast<size_t>(cbase + c) * p.h_v + h) * R_::bytes;
        const u32x4 *wn = reinterpret_cast<const u32x4 *>(rec + R_::Wn);
        const u32x4 *qg = reinterpret_cast<const u32x4 *>(rec + R_::Qg);
        const u32x4 *kg = reinterpret_cast<const u32x4 *>(rec + R_::KgT);
        const u32x4 *mq = reinterpret_cast<const u32x4 *>(rec + R_::M);
        const char *ut = rec + R_::Ut;
        const float *gc = reinterpret_cast<const float *>(rec + R_::gC);

        // B operands from the state (rows = d_k)
        u32x4 SB[BF ? NKD : 1];
        if constexpr (BF) {
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) SB[kt] = dpair_to_b32(S[2 * kt], S[2 * kt + 1]);
        }
        // U = U~ + Wn S
        f32x4 U[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const size_t toff = (static_cast<size_t>(ct) * 4 + rt) * R_::UT_TILE;
            if constexpr (BF) {
                const u32x2 u = reinterpret_cast<const u32x2 *>(ut + toff)[lane];
                U[rt] = f32x4{bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
            } else {
                U[rt] = reinterpret_cast<const f32x4 *>(ut + toff)[lane];
            }
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) {
                const u32x4 a = wn[(rt * NKD + kt) * 64 + lane];
                if constexpr (BF) U[rt] = mma_k32(a, SB[kt], U[rt]);
                else U[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a), S[kt], U[rt]);
            }
        }
        u32x4 UB[BF ? NKC : 1];
        if constexpr (BF) {
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) UB[kt] = dpair_to_b32(U[2 * kt], U[2 * kt + 1]);
        }
        // O = Qg S + M U
        f32x4 O[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) {
                const u32x4 a = qg[(rt * NKD + kt) * 64 + lane];
                if constexpr (BF) O[rt] = mma_k32(a, SB[kt], O[rt]);
                else O[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a), S[kt], O[rt]);
            }
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) {
                const u32x4 a = mq[(rt * NKC + kt) * 64 + lane];
                if constexpr (BF) O[rt] = mma_k32(a, UB[kt], O[rt]);
                else O[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a), U[kt], O[rt]);
            }
        }
        // S = gamma_C S + KgT U
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4 g4 = *reinterpret_cast<const f32x4 *>(gc + 16 * rt + 4 * lg);
            S[rt] *= g4;
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) {
                const u32x4 a = kg[(rt * NKC + kt) * 64 + lane];
                if constexpr (BF) S[rt] = mma_k32(a, UB[kt], S[rt]);
                else S[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a), U[kt], S[rt]);
            }
        }
        // o rows of this chunk (identity padding rows are skipped)
        const int64_t t0 = start + static_cast<int64_t>(c) * C;
        const int L = static_cast<int>(min<int64_t>(C, end - t0));
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int row = 16 * rt + 4 * lg + ii;
                if (row < L)
                    io<T>::st(op + (static_cast<size_t>(t0 + row) * p.h_v + h) * DV + col,
                              O[rt][ii]);
            }
    }
    if (p.S_T) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                p.S_T[sbase + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] = S[rt][ii];
    }
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
size_t chunk_record_bytes(int d_k, int d_v, bool bf16) {
    const size_t E = bf16 ? 2 : 4;
    const size_t gc = E * (3 * kChunk * d_k + kChunk * kChunk + kChunk * d_v);
    return (gc + static_cast<size_t>(d_k) * 4 + 255) / 256 * 256;
}

int64_t chunk_upper_bound(int batch, int seqlen, int num_seqs, bool packed) {
    const int64_t per = (static_cast<int64_t>(seqlen) + kChunk - 1) / kChunk;
    return packed ? per + num_seqs : per * batch;
}

size_t chunk_map_bytes(int num_seqs, bool packed) {
    return packed ? (static_cast<size_t>(num_seqs + 1) * 4 + 255) / 256 * 256 : 0;
}

size_t chunk_workspace_bytes(int batch, int seqlen, int num_seqs, int h_v, int d_k, int d_v,
                             bool bf16, bool packed) {
    return chunk_map_bytes(num_seqs, packed) +
           static_cast<size_t>(chunk_upper_bound(batch, seqlen, num_seqs, packed)) * h_v *
               chunk_record_bytes(d_k, d_v, bf16);
}

bool chunk_dims_built(int d_k, int d_v, bool bf16) {
    if (bf16) return (d_k == 64 || d_k == 128) && (d_v == 64 || d_v == 128);
    return d_k == 64 && d_v == 64;
}

template <typename T, bool BF, int DK, int DV>
static hipError_t launch_chunk_t(const ChunkArgs &a, hipStream_t st) {
    static_assert(Rec<DK, DV, BF>::bytes > 0, "");
    const bool packed = a.cu_seqlens != nullptr;
    const int N = packed ? a.num_seqs : a.batch;
    ChunkParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.log_alpha = a.log_alpha; p.b = a.b; p.w = a.w;
    p.S0 = a.S0; p.cu = a.cu_seqlens; p.o = a.o; p.S_T = a.S_T;
    const size_t mapb = chunk_map_bytes(a.num_seqs, packed);
    p.map = packed ? reinterpret_cast<const int32_t *>(a.workspace) : nullptr;
    p.rec = a.workspace + mapb;
    p.seqlen = a.seqlen; p.num_seqs = N; p.h_k = a.h_k; p.h_v = a.h_v;
    p.group = a.h_v / a.h_k;
    p.nc_dense = (a.seqlen + kChunk - 1) / kChunk;
    p.num_pairs = N * a.h_v;
    if (packed) {
        hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(64), 0, st, a.cu_seqlens,
                           reinterpret_cast<int32_t *>(a.workspace), N);
    }
    const int64_t nchunks = chunk_upper_bound(a.batch, a.seqlen, N, packed);
    if (nchunks > 0) {
        hipLaunchKernelGGL((chunk_prep_kernel<T, BF, DK, DV>), dim3(nchunks, a.h_v), dim3(512),
                           0, st, p);
    }
    // K2: waves per workgroup chosen so that small batches still spread over the CUs.
    int nw = 1;
    const int ctiles = DV / 16;
    while (nw < 4 && ctiles % (2 * nw) == 0 && static_cast<int64_t>(p.num_pairs) * ctiles /
                                                   (2 * nw) >= 1024)
        nw *= 2;
    p.nslices = ctiles / nw;
    const int64_t pairs8 = (static_cast<int64_t>(p.num_pairs) + 7) / 8 * 8;
    const int64_t blocks = pairs8 * p.nslices;
    if (blocks > 0) {
        hipLaunchKernelGGL((chunk_state_kernel<T, BF, DK, DV>), dim3(blocks), dim3(64 * nw), 0,
                           st, p);
    }
    return hipGetLastError();
}

template <typename T, bool BF>
static hipError_t launch_chunk_dt(const ChunkArgs &a, hipStream_t st) {
    if constexpr (BF) {
        if (a.d_k == 128 && a.d_v == 128) return launch_chunk_t<T, BF, 128, 128>(a, st);
        if (a.d_k == 64 && a.d_v == 64) return launch_chunk_t<T, BF, 64, 64>(a, st);
        if (a.d_k == 128 && a.d_v == 64) return launch_chunk_t<T, BF, 128, 64>(a, st);
        return launch_chunk_t<T, BF, 64, 128>(a, st);
    } else {
        return launch_chunk_t<T, BF, 64, 64>(a, st);
    }
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t st) {
    return a.bf16 ? launch_chunk_dt<bf16_t, true>(a, st) : launch_chunk_dt<float, false>(a, st);
}

}  // namespace gdn2
