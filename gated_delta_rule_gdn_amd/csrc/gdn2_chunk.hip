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
//                          cumulative log decay, A and M on the matrix cores, T = (I + A)^{-1}
//                          by 16x16 blocks (diagonal blocks by forward substitution, the rest
//                          by fp32 matrix-core products), the WY factors as tile GEMMs, and
//                          the per-chunk operands of K2, written to the workspace already in
//                          matrix-core fragment order.
//   K2 chunk_state_kernel  one wave per (sequence, value head, 16 columns of S), sequential
//                          over the chunks of its sequence with its slice of S held in
//                          registers in fp32 and the chunk operands prefetched into LDS one
//                          chunk ahead; writes o and S_T.
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
// K1: per (chunk, value head) WY factors and K2 operands, as a persistent kernel.
//
// One 512-thread workgroup per CU walks the (chunk, value head) records in chunk-major order
// (record = chunk * h_v + h, stride = grid size). While a record is computed from LDS, the
// raw k, q, b, log alpha tiles of the next one are already in flight into registers, and
// its w.v operands are requested as soon as the current U~ tiles are done, so global memory
// latency overlaps the math. LDS (about 125 KB at d = 128): raw k, q, b, log alpha with
// padded rows, g = cumulative log decay (fp32), and the lower 16x16 blocks of A and of
// T = (I + A)^{-1} (fp32, fragment order).
//
// Phases per record:
//   0  raw tiles -> LDS, cumulative sum of log alpha, gamma_C
//   1  A^T and M^T blocks (the transposed products leave each lane's results in the
//      row-per-lane fragment order the consumers read); M goes to the workspace
//  2a wave 0: 16x16 diagonal inverses T_RR by forward substitution; waves 1-7: Qg, KgT
//  2b off-diagonal T blocks by levels, T_RI = -T_RR sum_{I<=m<R} A_Rm T_mI (fp32 MFMA)
//   3  W~^T = X^T T^T (X = gamma.b.k) and U~ = T (w.v) as tile GEMMs, one column tile of
//      each per wave, written to the workspace in the orders K2 reads
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int lower_blk(int R, int I) { return R * (R + 1) / 2 + I; }

// Element (r, c) of a 16x16 fp32 block stored in fragment order (lane 16 g + r holds
// X[r][4 g .. 4 g + 3]).
__device__ __forceinline__ int frag_idx(int r, int c) { return 4 * (16 * (c >> 2) + r) + (c & 3); }

struct PrepLoc {
    int64_t t0;     // first token of the chunk
    int L;          // valid rows
    int h, hk;
    size_t rec;     // record index
};

template <typename T, bool BF, int DK, int DV>
__global__ __launch_bounds__(512, 1) void chunk_prep_kernel(ChunkParams p) {
    using R_ = Rec<DK, DV, BF>;
    constexpr int C = kChunk, NT = 512, NW = NT / 64;
    constexpr int KT = Op<BF>::KT;            // k per matrix-core tile: 32 (bf16) / 16 (fp32)
    constexpr int KS = BF ? 8 : 4;            // consecutive k values a lane holds per tile
    constexpr int VEC = 16 / sizeof(T);
    constexpr int SK = DK + VEC;              // padded row stride of the raw tiles (elements)
    constexpr int SG = DK + 4;                // padded row stride of s_g (floats)
    constexpr int VK = DK / VEC;              // 16-byte vectors per raw row
    constexpr int RAWV = C * VK / NT;         // raw vectors per thread per tensor
    constexpr int PARTS = NT / DK;            // cumulative sum: token parts per channel
    constexpr int RPP = C / PARTS;
    constexpr int NKC = R_::NKT_C, NKTC = C / KT;
    constexpr int VV = DV / VEC;              // 16-byte vectors per raw value row
    constexpr int RAWW = C * VV / NT;         // raw w / v vectors per thread
    static_assert(RAWV >= 1 && RAWV * NT == C * VK, "raw tile split");
    static_assert(RAWW >= 1 && RAWW * NT == C * VV, "raw tile split");
    constexpr int SL = (DK > DV ? DK : DV) + VEC;   // row stride of the log alpha / w.v tile

    __shared__ __attribute__((aligned(16))) T s_k[C * SK];
    __shared__ __attribute__((aligned(16))) T s_q[C * SK];
    __shared__ __attribute__((aligned(16))) T s_b[C * SK];
    __shared__ __attribute__((aligned(16))) T s_la[C * SL];  // log alpha, then w.v
    __shared__ __attribute__((aligned(16))) float s_g[C * SG];
    __shared__ __attribute__((aligned(16))) float s_A[10 * 256];
    __shared__ __attribute__((aligned(16))) float s_T[10 * 256];
    __shared__ float s_part[PARTS * DK];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const T *kp = static_cast<const T *>(p.k), *qp = static_cast<const T *>(p.q);
    const T *bp = static_cast<const T *>(p.b), *lap = static_cast<const T *>(p.log_alpha);
    const T *vp = static_cast<const T *>(p.v), *wp = static_cast<const T *>(p.w);

    const int total_chunks = p.cu ? p.map[p.num_seqs] : p.num_seqs * p.nc_dense;
    const int nitems = total_chunks * p.h_v;

    auto locate = [&](int item, PrepLoc &lc) {
        const int chunk = item / p.h_v;
        lc.h = item - chunk * p.h_v;
        lc.hk = lc.h / p.group;
        int n, j;
        int64_t start, end;
        locate_chunk(p, chunk, n, j, start, end);
        lc.t0 = start + static_cast<int64_t>(j) * C;
        lc.L = static_cast<int>(min<int64_t>(C, end - lc.t0));
        lc.rec = static_cast<size_t>(item);
    };
    // raw k, q, b, log alpha vectors of a record (rows >= L are zero: identity tokens)
    u32x4 rk[RAWV], rq[RAWV], rb[RAWV], rl[RAWV], rw[RAWW], rv[RAWW];
    auto load_raw = [&](const PrepLoc &lc) {
#pragma unroll
        for (int e = 0; e < RAWW; ++e) {
            const int vi = tid + NT * e, r = vi / VV, cv = vi - r * VV;
            const u32x4 z = {0u, 0u, 0u, 0u};
            rw[e] = z; rv[e] = z;
            if (r < lc.L) {
                const size_t ov = (static_cast<size_t>(lc.t0 + r) * p.h_v + lc.h) * DV + cv * VEC;
                rw[e] = *reinterpret_cast<const u32x4 *>(wp + ov);
                rv[e] = *reinterpret_cast<const u32x4 *>(vp + ov);
            }
        }
#pragma unroll
        for (int e = 0; e < RAWV; ++e) {
            const int vi = tid + NT * e, r = vi / VK, cv = vi - r * VK;
            const u32x4 z = {0u, 0u, 0u, 0u};
            rk[e] = z; rq[e] = z; rb[e] = z; rl[e] = z;
            if (r < lc.L) {
                const size_t ok = (static_cast<size_t>(lc.t0 + r) * p.h_k + lc.hk) * DK + cv * VEC;
                const size_t og = (static_cast<size_t>(lc.t0 + r) * p.h_v + lc.h) * DK + cv * VEC;
                rk[e] = *reinterpret_cast<const u32x4 *>(kp + ok);
                rq[e] = *reinterpret_cast<const u32x4 *>(qp + ok);
                rb[e] = *reinterpret_cast<const u32x4 *>(bp + og);
                rl[e] = *reinterpret_cast<const u32x4 *>(lap + og);
            }
        }
    };
    int item = blockIdx.x;
    PrepLoc cur;
    if (item < nitems) {
        locate(item, cur);
        load_raw(cur);
    }
    for (; item < nitems; item += gridDim.x) {
        const int next = item + gridDim.x;
        const bool has_next = next < nitems;
        PrepLoc nxt = cur;
        if (has_next) locate(next, nxt);
        char *rec = p.rec + cur.rec * R_::bytes;

        // ---- phase 0 ----
#pragma unroll
        for (int e = 0; e < RAWV; ++e) {
            const int vi = tid + NT * e, r = vi / VK, cv = vi - r * VK;
            *reinterpret_cast<u32x4 *>(&s_k[r * SK + cv * VEC]) = rk[e];
            *reinterpret_cast<u32x4 *>(&s_q[r * SK + cv * VEC]) = rq[e];
            *reinterpret_cast<u32x4 *>(&s_b[r * SK + cv * VEC]) = rb[e];
            *reinterpret_cast<u32x4 *>(&s_la[r * SL + cv * VEC]) = rl[e];
        }
        __syncthreads();
        {
            const int c = tid % DK, part = tid / DK;
            float x[RPP];
            float acc = 0.f;
#pragma unroll
            for (int rr = 0; rr < RPP; ++rr) {
                acc += io<T>::ld(&s_la[(part * RPP + rr) * SL + c]);
                x[rr] = acc;
            }
            s_part[part * DK + c] = acc;
            __syncthreads();
            float pre = 0.f;
            for (int pp = 0; pp < part; ++pp) pre += s_part[pp * DK + c];
#pragma unroll
            for (int rr = 0; rr < RPP; ++rr) s_g[(part * RPP + rr) * SG + c] = x[rr] + pre;
            // w.v, rounded to the operand type (the rounding its matrix-core use applies),
            // into the log alpha tile, which is no longer read
#pragma unroll
            for (int e = 0; e < RAWW; ++e) {
                const int vi = tid + NT * e, r = vi / VV, cv = vi - r * VV;
                float prod[16 / sizeof(T)];
                if constexpr (BF) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        prod[2 * q4] = bf16_lo(rw[e][q4]) * bf16_lo(rv[e][q4]);
                        prod[2 * q4 + 1] = bf16_hi(rw[e][q4]) * bf16_hi(rv[e][q4]);
                    }
                } else {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        prod[q4] = __uint_as_float(rw[e][q4]) * __uint_as_float(rv[e][q4]);
                }
                *reinterpret_cast<u32x4 *>(&s_la[r * SL + cv * VEC]) = pack16<BF>(prod);
            }
            __syncthreads();
            if (has_next) load_raw(nxt);       // next record's raw tiles, in flight from here
            if (tid < DK)
                reinterpret_cast<float *>(rec + R_::gC)[tid] = __expf(s_g[(C - 1) * SG + tid]);
        }

        // ---- phase 1: A^T and M^T blocks (R >= I); zero upper blocks of M ----
        char *mrec = rec + R_::M;
        for (int pr = wave; pr < 10; pr += NW) {
            const int R = pr >= 6 ? 3 : (pr >= 3 ? 2 : (pr >= 1 ? 1 : 0));
            const int I = pr - R * (R + 1) / 2;
            const bool diag = (R == I);
            const int refrow = diag ? 16 * R + 7 : 16 * R - 1;
            const int ri = 16 * I + li;              // A operand: column-side token i
            const int rr = 16 * R + li;              // B operand: row-side token r
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = accA;
#pragma unroll
            for (int kt = 0; kt < DK / KT; ++kt) {
                const int c0 = kt * KT + KS * lg;
                float kb[KS], ka[KS], qa[KS];
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const int c = c0 + s;
                    const float ref = s_g[refrow * SG + c];
                    const float ec = __expf(ref - s_g[ri * SG + c]);
                    const float ef = __expf(s_g[rr * SG + c] - ref);
                    kb[s] = io<T>::ld(&s_k[ri * SK + c]) * ec;
                    ka[s] = io<T>::ld(&s_b[rr * SK + c]) * io<T>::ld(&s_k[rr * SK + c]) * ef;
                    qa[s] = io<T>::ld(&s_q[rr * SK + c]) * ef;
                }
                if constexpr (BF) {
                    const u32x4 a = pack16<true>(kb);
                    accA = mma_k32(a, pack16<true>(ka), accA);
                    accM = mma_k32(a, pack16<true>(qa), accM);
                } else {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        accA = __builtin_amdgcn_mfma_f32_16x16x4f32(kb[s], ka[s], accA, 0, 0, 0);
                        accM = __builtin_amdgcn_mfma_f32_16x16x4f32(kb[s], qa[s], accM, 0, 0, 0);
                    }
                }
            }
            // lane holds A[r = 16R + li][i = 16I + 4 lg + ii] (and M): fragment order already
            f32x4 a4, m4;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int il = 4 * lg + ii;
                a4[ii] = (diag && il >= li) ? 0.f : accA[ii];
                m4[ii] = (diag && il > li) ? 0.f : accM[ii];
            }
            *reinterpret_cast<f32x4 *>(&s_A[lower_blk(R, I) * 256 + 4 * lane]) = a4;
            if constexpr (BF) {
                reinterpret_cast<u32x2 *>(mrec)[(((R * NKC + (I >> 1)) * 64 + lane) << 1) + (I & 1)] =
                    f4_to_b16(m4);
            } else {
                reinterpret_cast<f32x4 *>(mrec)[(R * NKC + I) * 64 + lane] = m4;
            }
        }
        for (int u = wave; u < 6; u += NW) {
            // (R, I) with I > R, in the order (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
            const int R2 = u < 3 ? 0 : (u < 5 ? 1 : 2);
            const int I2 = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
            if constexpr (BF) {
                const u32x2 z = {0u, 0u};
                reinterpret_cast<u32x2 *>(mrec)[(((R2 * NKC + (I2 >> 1)) * 64 + lane) << 1) + (I2 & 1)] = z;
            } else {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                reinterpret_cast<f32x4 *>(mrec)[(R2 * NKC + I2) * 64 + lane] = z;
            }
        }
        __syncthreads();

        // ---- phase 2a: diagonal inverses (wave 0) || Qg and KgT (waves 1-7) ----
        if (wave == 0) {
            const int R = lane >> 4, jc = lane & 15;      // column jc of T_RR
            const float *Ab = &s_A[lower_blk(R, R) * 256];
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == jc) ? 1.f : 0.f;
#pragma unroll
            for (int r = 1; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) acc += Ab[frag_idx(r, m)] * x[m];
                if (r > jc) x[r] = -acc;
            }
            float *Tb = &s_T[lower_blk(R, R) * 256];
#pragma unroll
            for (int r = 0; r < 16; ++r) Tb[frag_idx(r, jc)] = x[r];
        } else {
            constexpr int NBQ = (C / 16) * R_::NKT_DK;      // Qg blocks
            constexpr int NBK = (DK / 16) * R_::NKT_C;      // KgT blocks
            constexpr int EPL = Op<BF>::EPL;
            u32x4 *qg = reinterpret_cast<u32x4 *>(rec + R_::Qg);
            u32x4 *kg = reinterpret_cast<u32x4 *>(rec + R_::KgT);
            for (int idx = tid - 64; idx < (NBQ + NBK) * 64; idx += NT - 64) {
                const int blk = idx >> 6, l = idx & 63, lli = l & 15, llg = l >> 4;
                float vals[EPL];
                if (blk < NBQ) {
                    const int rt = blk / R_::NKT_DK, kt = blk - rt * R_::NKT_DK;
                    const int r = 16 * rt + lli;
#pragma unroll
                    for (int jj = 0; jj < EPL; ++jj) {
                        const int c = kt * KT + perm_k<BF>(llg, jj);
                        vals[jj] = __expf(s_g[r * SG + c]) * io<T>::ld(&s_q[r * SK + c]);
                    }
                    qg[blk * 64 + l] = pack16<BF>(vals);
                } else {
                    const int b2 = blk - NBQ;
                    const int rt = b2 / R_::NKT_C, kt = b2 - rt * R_::NKT_C;
                    const int ch = 16 * rt + lli;
                    const float gl = s_g[(C - 1) * SG + ch];
#pragma unroll
                    for (int jj = 0; jj < EPL; ++jj) {
                        const int tok = kt * KT + perm_k<BF>(llg, jj);
                        vals[jj] = __expf(gl - s_g[tok * SG + ch]) * io<T>::ld(&s_k[tok * SK + ch]);
                    }
                    kg[b2 * 64 + l] = pack16<BF>(vals);
                }
            }
        }
        __syncthreads();

        // ---- phase 2b: off-diagonal blocks of T by levels d = R - I ----
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            if (wave < 4 - d) {
                const int R = d + wave, I = R - d;
                f32x4 P = {0.f, 0.f, 0.f, 0.f};
                for (int m = I; m < R; ++m) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(&s_A[lower_blk(R, m) * 256 + 4 * lane]);
                    const float *Tm = &s_T[lower_blk(m, I) * 256];
                    f32x4 bT;                      // B operand: T_mI[4 lg + s][li]
#pragma unroll
                    for (int s = 0; s < 4; ++s) bT[s] = Tm[frag_idx(4 * lg + s, li)];
                    P = mma_k16_f32(a, bT, P);
                }
                const f32x4 tRR = *reinterpret_cast<const f32x4 *>(&s_T[lower_blk(R, R) * 256 + 4 * lane]);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 Tn = mma_k16_f32(tRR, P, zero);   // lane: (T_RR P)[4 lg + ii][li]
                float *Tb = &s_T[lower_blk(R, I) * 256];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) Tb[frag_idx(4 * lg + ii, li)] = -Tn[ii];
            }
            __syncthreads();
        }

        // ---- phase 3: W~^T = X^T T^T (X = gamma.b.k) and U~ = T (w.v) ----
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const bool isW = which == 0;
            if (wave >= (isW ? DK : DV) / 16) continue;
            const int ct = wave;
            const int c = 16 * ct + li;
            float xv[NKTC][KS];
#pragma unroll
            for (int kt = 0; kt < NKTC; ++kt)
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const int tok = kt * KT + KS * lg + s;
                    if (isW) {
                        xv[kt][s] = __expf(s_g[tok * SG + c]) * io<T>::ld(&s_b[tok * SK + c]) *
                                    io<T>::ld(&s_k[tok * SK + c]);
                    } else {
                        xv[kt][s] = io<T>::ld(&s_la[tok * SL + c]);     // w.v
                    }
                }
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < NKTC; ++kt) {
                    if (kt * KT > 16 * R + 15) break;
                    float tv[KS];                  // T[16R + li][kt*KT + KS*lg + s]
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const int tok = kt * KT + KS * lg + s;
                        const int I = tok >> 4;
                        tv[s] = (I <= R) ? s_T[lower_blk(R, I) * 256 + frag_idx(li, tok & 15)] : 0.f;
                    }
                    if constexpr (BF) {
                        if (isW) acc = mma_k32(pack16<true>(xv[kt]), pack16<true>(tv), acc);
                        else acc = mma_k32(pack16<true>(tv), pack16<true>(xv[kt]), acc);
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            acc = isW ? __builtin_amdgcn_mfma_f32_16x16x4f32(xv[kt][s], tv[s], acc, 0, 0, 0)
                                      : __builtin_amdgcn_mfma_f32_16x16x4f32(tv[s], xv[kt][s], acc, 0, 0, 0);
                    }
                }
                if (isW) {
                    // lane: W~[16R + li][16 ct + 4 lg + ii] -> -W~ in K2's fragment order
                    const f32x4 wn = -acc;
                    char *wr = rec + R_::Wn;
                    if constexpr (BF) {
                        reinterpret_cast<u32x2 *>(wr)[(((R * R_::NKT_DK + (ct >> 1)) * 64 + lane) << 1) +
                                                      (ct & 1)] = f4_to_b16(wn);
                    } else {
                        reinterpret_cast<f32x4 *>(wr)[(R * R_::NKT_DK + ct) * 64 + lane] = wn;
                    }
                } else {
                    // lane: U~[16R + 4 lg + ii][16 ct + li], an output tile (D layout)
                    char *ut = rec + R_::Ut + (static_cast<size_t>(ct) * 4 + R) * R_::UT_TILE;
                    if constexpr (BF) reinterpret_cast<u32x2 *>(ut)[lane] = f4_to_b16(acc);
                    else reinterpret_cast<f32x4 *>(ut)[lane] = acc;
                }
            }
        }
        __syncthreads();                       // LDS is reused by the next record
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------------------
// K2: inter-chunk state pass. Each compute wave owns 16 columns of S (all d_k rows) as DK/16
// output tiles in fp32 registers and walks the chunks of its sequence in order. The waves
// of a workgroup share one (sequence, head). Per chunk:
//   * the record (operands common to all columns, gamma_C, each wave's U~ slice) is copied
//     into a double-buffered LDS stage one chunk ahead by kLoaders extra loader waves with
//     direct global-to-LDS loads: one wave cannot keep enough copies in flight to move a
//     record per chunk step, several can. Loaders wait for their own copies, then meet
//     the compute waves at the per-chunk barrier (a plain s_barrier, no memory fence);
//   * each matrix-core phase first reads all its A fragments from LDS, then issues the
//     products with the independent accumulator chains interleaved;
//   * o of a chunk is transposed through LDS and stored with 16-byte writes one chunk later.
// ---------------------------------------------------------------------------------------
template <int DK, int DV, bool BF>
struct StageLayout {
    using R_ = Rec<DK, DV, BF>;
    static constexpr size_t SHARED = R_::Ut;                 // Wn, Qg, KgT, M
    static constexpr size_t GCB = DK * 4;                    // gamma_C
    static constexpr size_t UTS = 4 * R_::UT_TILE;           // one wave's U~ slice
    static constexpr size_t OTILE = kChunk * 16 * 4;         // one wave's o transpose area
    __host__ __device__ static constexpr size_t buffer_bytes(int nw) {
        return SHARED + GCB + nw * UTS;
    }
    __host__ __device__ static constexpr size_t lds_bytes(int nw) {
        return 2 * buffer_bytes(nw) + nw * OTILE;
    }
    static_assert(2 * (SHARED + GCB + UTS) + OTILE <= 160 * 1024,
                  "double buffer must fit in LDS");
};

__device__ __forceinline__ void dma16(const void *src, void *lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16, 0, 0);
}

// s_waitcnt with vmcnt(0) only (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt with lgkmcnt(0) only
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier without a memory fence (so it never waits for outstanding loads). The
// empty asm statements keep the compiler from moving memory accesses across it; every wave
// waits for its own copies with wait_vmem() before arriving when it needs them.
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

constexpr int kLoaders = 4;           // loader waves per state-pass workgroup

template <typename T, bool BF, int DK, int DV>
__global__ __launch_bounds__(512) void chunk_state_kernel(ChunkParams p) {
    using R_ = Rec<DK, DV, BF>;
    using SL = StageLayout<DK, DV, BF>;
    constexpr int C = kChunk, RT = DK / 16;
    constexpr int KT = Op<BF>::KT;
    constexpr int NKD = R_::NKT_DK, NKC = R_::NKT_C;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int nw = (blockDim.x >> 6) - kLoaders;   // compute waves; the rest load
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const size_t BUF = SL::buffer_bytes(nw);
    char *otile_base = smem + 2 * BUF;

    // XCD-aware decode: the column slices of one (sequence, head) pair share an XCD, so
    // its workspace records are fetched into one L2.
    const int bid = blockIdx.x, xcd = bid & 7, rest = bid >> 3;
    const int slice = rest % p.nslices;
    const int pair = (rest / p.nslices) * 8 + xcd;
    if (pair >= p.num_pairs) return;
    const int n = pair / p.h_v, h = pair - n * p.h_v;

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
    auto record = [&](int c) {
        return p.rec + (static_cast<size_t>(cbase + c) * p.h_v + h) * R_::bytes;
    };

    if (wave >= nw) {
        // ---- loader waves: copy chunk c + 1 into the other stage during chunk c
        const int ldr = wave - nw;
        auto issue = [&](int c, char *dst) {
            const char *rec = record(c);
            for (int blk = ldr; blk < static_cast<int>(SL::SHARED / 1024); blk += kLoaders)
                dma16(rec + blk * 1024 + lane * 16, dst + blk * 1024);
            if (ldr == kLoaders - 1 && lane < static_cast<int>(SL::GCB / 16))
                dma16(rec + R_::gC + lane * 16, dst + SL::SHARED);
            // the compute waves' U~ slices: column tiles slice*nw .. slice*nw + nw - 1 are
            // contiguous in the record, and so are their stage slots
            const char *us = rec + R_::Ut + static_cast<size_t>(slice) * nw * SL::UTS;
            char *ud = dst + SL::SHARED + SL::GCB;
            for (int b = ldr; b < static_cast<int>(nw * SL::UTS / 1024); b += kLoaders)
                dma16(us + b * 1024 + lane * 16, ud + b * 1024);
        };
        if (nchunks > 0) issue(0, smem);
        for (int c = 0; c < nchunks; ++c) {
            wait_vmem();                    // this loader's copies for chunk c have landed
            raw_barrier();                  // chunk c is staged; chunk c-1 fully consumed
            if (c + 1 < nchunks) issue(c + 1, smem + ((c + 1) & 1) * BUF);
        }
        return;
    }

    const int ct = slice * nw + wave;
    const int col = 16 * ct + li;
    f32x4 S[RT];
    const size_t sbase = static_cast<size_t>(pair) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            S[rt][ii] = p.S0 ? p.S0[sbase + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col]
                             : 0.f;

    // o of chunk c is written to this wave's LDS tile at the end of chunk c and stored to
    // memory during chunk c + 1 as 16-byte rows.
    T *op = static_cast<T *>(p.o);
    T *otile = reinterpret_cast<T *>(otile_base + wave * SL::OTILE);
    constexpr int OPR = 16 * sizeof(T) / 16;        // 16-byte pieces per 16-column row
    int64_t t0prev = 0;
    int Lprev = 0;
    auto store_o = [&]() {
#pragma unroll
        for (int e = 0; e < C * OPR / 64; ++e) {
            const int pidx = lane + 64 * e, row = pidx / OPR, piece = pidx - row * OPR;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(&otile[row * 16 + piece * (16 / sizeof(T))]);
            if (row < Lprev)
                *reinterpret_cast<u32x4 *>(op + (static_cast<size_t>(t0prev + row) * p.h_v + h) * DV +
                                           16 * ct + piece * (16 / sizeof(T))) = v;
        }
    };

    for (int c = 0; c < nchunks; ++c) {
        char *cur = smem + (c & 1) * BUF;
        raw_barrier();                      // chunk c is staged; chunk c-1 fully consumed
        if (c > 0) store_o();

        const u32x4 *wn = reinterpret_cast<const u32x4 *>(cur + R_::Wn);
        const u32x4 *qg = reinterpret_cast<const u32x4 *>(cur + R_::Qg);
        const u32x4 *kg = reinterpret_cast<const u32x4 *>(cur + R_::KgT);
        const u32x4 *mq = reinterpret_cast<const u32x4 *>(cur + R_::M);
        const float *gc = reinterpret_cast<const float *>(cur + SL::SHARED);
        const char *ut = cur + SL::SHARED + SL::GCB + wave * SL::UTS;

        u32x4 SB[BF ? NKD : 1];
        if constexpr (BF) {
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) SB[kt] = dpair_to_b32(S[2 * kt], S[2 * kt + 1]);
        }
        // U = U~ + Wn S
        f32x4 U[4];
        {
            u32x4 a[4][NKD];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int kt = 0; kt < NKD; ++kt) a[rt][kt] = wn[(rt * NKD + kt) * 64 + lane];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if constexpr (BF) {
                    const u32x2 u = reinterpret_cast<const u32x2 *>(ut + rt * R_::UT_TILE)[lane];
                    U[rt] = f32x4{bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
                } else {
                    U[rt] = reinterpret_cast<const f32x4 *>(ut + rt * R_::UT_TILE)[lane];
                }
            }
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    if constexpr (BF) U[rt] = mma_k32(a[rt][kt], SB[kt], U[rt]);
                    else U[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a[rt][kt]), S[kt], U[rt]);
                }
        }
        u32x4 UB[BF ? NKC : 1];
        if constexpr (BF) {
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) UB[kt] = dpair_to_b32(U[2 * kt], U[2 * kt + 1]);
        }
        // O = Qg S + M U   (M is lower triangular: k tiles above the diagonal are skipped)
        f32x4 O[4];
        {
            u32x4 a[4][NKD], m[4][NKC];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int kt = 0; kt < NKD; ++kt) a[rt][kt] = qg[(rt * NKD + kt) * 64 + lane];
#pragma unroll
                for (int kt = 0; kt < NKC; ++kt)
                    if (kt * KT <= 16 * rt + 15) m[rt][kt] = mq[(rt * NKC + kt) * 64 + lane];
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    if constexpr (BF) O[rt] = mma_k32(a[rt][kt], SB[kt], O[rt]);
                    else O[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a[rt][kt]), S[kt], O[rt]);
                }
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    if (kt * KT > 16 * rt + 15) continue;
                    if constexpr (BF) O[rt] = mma_k32(m[rt][kt], UB[kt], O[rt]);
                    else O[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, m[rt][kt]), U[kt], O[rt]);
                }
        }
        // S = gamma_C S + KgT U
        {
            u32x4 a[RT][NKC];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kt = 0; kt < NKC; ++kt) a[rt][kt] = kg[(rt * NKC + kt) * 64 + lane];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 g4 = *reinterpret_cast<const f32x4 *>(gc + 16 * rt + 4 * lg);
                S[rt] *= g4;
            }
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    if constexpr (BF) S[rt] = mma_k32(a[rt][kt], UB[kt], S[rt]);
                    else S[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a[rt][kt]), U[kt], S[rt]);
                }
        }
        // o rows of this chunk into the wave's LDS tile (row-major [C][16]); stored next chunk
        wait_lds();
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                io<T>::st(&otile[(16 * rt + 4 * lg + ii) * 16 + li], O[rt][ii]);
        t0prev = start + static_cast<int64_t>(c) * C;
        Lprev = static_cast<int>(min<int64_t>(C, end - t0prev));
    }
    if (nchunks > 0) {
        wait_lds();
        store_o();
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

// Compute units of the current device (the persistent prep kernel runs one workgroup per
// CU). Queried once per device and cached.
static int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
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
        const int64_t items = nchunks * a.h_v;
        const int grid = static_cast<int>(items < device_cu_count() ? items : device_cu_count());
        hipLaunchKernelGGL((chunk_prep_kernel<T, BF, DK, DV>), dim3(grid), dim3(512), 0, st, p);
    }
    // K2: compute waves per workgroup (plus one prefetch wave). More waves share one copy of
    // each chunk's operands in LDS; fewer spread a small batch over more CUs.
    using SLy = StageLayout<DK, DV, BF>;
    constexpr size_t kMaxLds = 160 * 1024;          // LDS per workgroup on gfx950
    int nw = 1;
    const int ctiles = DV / 16;
    while (nw < 4 && ctiles % (2 * nw) == 0 &&
           static_cast<int64_t>(p.num_pairs) * ctiles / (2 * nw) >= 256 &&
           SLy::lds_bytes(2 * nw) <= kMaxLds)
        nw *= 2;
    p.nslices = ctiles / nw;
    const size_t lds = SLy::lds_bytes(nw);
    auto kern = chunk_state_kernel<T, BF, DK, DV>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const int64_t pairs8 = (static_cast<int64_t>(p.num_pairs) + 7) / 8 * 8;
    const int64_t blocks = pairs8 * p.nslices;
    if (blocks > 0) {
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * (nw + kLoaders)), lds, st, p);
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
