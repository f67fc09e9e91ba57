// gdn2_prep.hip -- the intra-chunk pass of the chunked WY forward (the prep kernel) on gfx950.
//
// Method: burn-gdn2 0.1.5 docs page, section "Architecture" (the recurrence and its "Chunk
// WY" training path). For a chunk of C tokens (rows r, i; g_r = sum_{i<=r} log alpha_i per
// key channel, gamma = exp(g)) the state pass needs, per (chunk, value head):
//   A  = strict_lower(K^ K-bar^T)  with A[r,i] = sum_c b_r k_r k_i exp(g_r - g_i)
//   M  = lower_incl(Q^ K-bar^T)    with M[r,i] = sum_c q_r k_i exp(g_r - g_i)
//   T  = (I + A)^{-1}
//   Wn = -T (gamma . b . k),  U~ = T (w . v),  Qg = gamma . q,
//   KgT = ((gamma_C / gamma) . k)^T,  gamma_C
// (the record layout of gdn2_chunk.h).
//
// One workgroup per record, small enough in LDS that two records run on a CU at once for
// C <= 64 (the rounds of one hide the latency of the other's): eight waves at C = 64 (and
// for bf16 records at C = 128), where a round covers two matrix-core k tiles, four waves
// over one k tile per round otherwise (PrepShape below). The key channels are
// processed in rounds of k tiles (32 bf16 / 16 fp32 channels each):
//   scan    every lane holds one token of a 16-token sub-chunk and 8 (bf16) or 4 (fp32)
//           channels; the cumulative log decay inside each sub-chunk is an in-row scan of the
//           16 lanes (DPP row shifts), in log2 units; sub-chunk sums go through LDS
//   round   K^ = b k 2^(c_r - c_mid), Q^ = q 2^(c_r - c_mid), K-bar = k 2^(c_mid - c_r) with
//           c the in-sub-chunk cumsum and c_mid its value at the sub-chunk's middle token (no
//           factor spans more than 8 tokens of decay), written to LDS tiles; A and M
//           accumulate on the matrix cores in registers over the rounds, block pair by block
//           pair, the off-diagonal pairs with the per-channel factor 2^(g_mid_R - g_mid_I) <= 1
//   solve   T = (I + A)^{-1} on 16x16 blocks stored as a packed lower triangle: diagonal
//           blocks by forward substitution, the rest level by level on fp32 matrix cores
//   WY      W~^T = X^T T^T (X = gamma . b . k, kept in registers from the rounds) and
//           U~ = T (w . v), one channel block per round, written in the record's order.
// Padding rows of a partial chunk are identity tokens (k = q = b = 0, w.v = 0,
// log alpha = 0).
#include "gdn2_chunk.h"

namespace gdn2 {

// The (R, I) block pairs of the lower triangle (R >= I) of NS 16-token sub-chunks, numbered
// off-diagonal pairs first ((1,0), (2,0), (2,1), (3,0), ...), then the diagonal; wave w
// takes pairs w, w + NWV, ...
__device__ __forceinline__ void pair_of(int idx, int ns, int &R, int &I) {
    const int noff = ns * (ns - 1) / 2;
    if (idx >= noff) {
        R = I = idx - noff;
        return;
    }
    int r = 1;
    while (r * (r + 1) / 2 <= idx) ++r;
    R = r;
    I = idx - r * (r - 1) / 2;
}

// Index of block (R, I), R >= I, in the packed lower triangle.
__host__ __device__ constexpr int tri_blk(int R, int I) { return R * (R + 1) / 2 + I; }

// Inclusive prefix sum over the 16 lanes of each DPP row (lanes outside the row read 0).
__device__ __forceinline__ float row_scan16(float x) {
    int v = __builtin_bit_cast(int, x);
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true));
    v = __builtin_bit_cast(int, x);
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true));
    v = __builtin_bit_cast(int, x);
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true));
    v = __builtin_bit_cast(int, x);
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true));
    return x;
}

// NWV waves per workgroup; CPR channel blocks (matrix-core k tiles) per round. Every item of
// a round is one 16-token sub-chunk x one channel block; item it of round r covers
// sub-chunk it % NS and block r CPR + it / NS, and wave w takes items w, w + NWV, ...
template <typename T, bool BF, int C, int DK, int DV, int GM, int NWV, int CPR, bool NTR>
__global__ __launch_bounds__(64 * NWV) void prep_kernel(ChunkParams p) {
    using R_ = Rec<C, DK, DV, BF>;
    constexpr int NT = 64 * NWV;
    constexpr int NS = C / 16;                 // 16-token sub-chunks
    constexpr int VEC = 16 / sizeof(T);        // elements per 16-byte vector
    constexpr int CB = 4 * VEC;                // channels per block: one k tile
    constexpr int KT = Op<BF>::KT;
    static_assert(KT == CB, "a channel block is one matrix-core k tile");
    constexpr int NJ = DK / CB, NJV = DV / CB;
    static_assert(NJ % CPR == 0 && NJV % CPR == 0, "whole rounds");
    constexpr int NR = NJ / CPR, NRV = NJV / CPR;   // key and value rounds
    constexpr int IPR = NS * CPR;              // items per round
    constexpr int IPW = (IPR + NWV - 1) / NWV; // items per wave per round (at most)
    constexpr int NPAIR = NS * (NS + 1) / 2, NOFF = NS * (NS - 1) / 2;
    constexpr int PPW = (NPAIR + NWV - 1) / NWV;    // block pairs per wave (at most)
    constexpr int RW = CPR * CB;               // channels per round
    constexpr int SB = RW + VEC;               // tile row stride (elements), 16 B of padding
    constexpr int TILE = C * SB;
    constexpr bool DBUF = C <= 64 && NWV == 4; // double-buffered round tiles
    constexpr int NBUF = DBUF ? 2 : 1;
    constexpr int BSTR = 20, BS = 16 * BSTR;   // fp32 16x16 block: row stride, size (floats)
    constexpr int NKD = R_::NKT_DK, NKC = R_::NKT_C;
    constexpr int CT = CB / 16;                // 16-channel tiles per block
    constexpr int RCT = CPR * CT;              // 16-channel tiles per round
    constexpr int STB = C + 8;                 // row stride of the bf16 copy of T
    constexpr bool b_scalar = GM == GATES_KDA || GM == GATES_GDN;
    constexpr bool la_scalar = GM == GATES_GDN;
    constexpr bool fg2 = GM == GATES_FG2 || GM == GATES_FG2_PLUS;
    static_assert(NBUF * 3 * TILE >= 2 * TILE, "two X / w.v tiles fit in the round tiles");
    static_assert(!BF || C * STB * 2 <= NPAIR * BS * 4, "bf16 T fits over A");
    static_assert(NWV % RCT == 0, "the WY rounds deal whole channel tiles to the waves");

    __shared__ float s_tot[NS * DK];           // sum of the log2 decay over each sub-chunk
    __shared__ float s_cmid[NS * DK];          // in-sub-chunk cumsum at its middle token
    __shared__ float s_fkg[NS * DK];           // 2^(g_C - g_mid_R)
    __shared__ float s_fmid[NS * DK];          // 2^(g_mid_R)
    __shared__ float s_foff[(NOFF > 0 ? NOFF : 1) * DK];   // 2^(g_mid_R - g_mid_I), R > I
    __shared__ __attribute__((aligned(16))) T s_tile[NBUF * 3 * TILE];
    __shared__ __attribute__((aligned(16))) float s_A[NPAIR * BS];
    // bf16 records at C = 128 keep the fp32 T over the round tiles (dead between the last
    // round and the WY rounds) so that eight waves fit the LDS; the WY rounds read the bf16
    // copy of T only
    constexpr bool TALIAS = BF && C == 128;
    static_assert(!TALIAS || NBUF * 3 * TILE * sizeof(T) >= NPAIR * BS * sizeof(float), "T fits the tiles");
    __shared__ __attribute__((aligned(16))) float s_Tst[TALIAS ? 4 : NPAIR * BS];
    float *const s_T = TALIAS ? reinterpret_cast<float *>(s_tile) : s_Tst;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;   // matrix-core lane roles (= t, gi below)
    const int t = li, gi = lg;                  // elementwise roles: token in sub-chunk, group

    // Records in (chunk, value head) order. With grouped heads (xgroup = G), blocks of one
    // XCD (b mod 8) take the G records of a (chunk, key head) one after another, so that
    // their q and k rows are fetched into that XCD's L2 once (a bijection on the records).
    int item = blockIdx.x;
    if (p.xgroup > 1) {
        const int xr = item >> 3;
        item = ((xr / p.xgroup) * 8 + (item & 7)) * p.xgroup + xr % p.xgroup;
    }
    const int chunk = item / p.h_v, h = item - chunk * p.h_v, hk = h / p.group;
    int n, jc;
    int64_t start, end;
    if (!locate_chunk(p, chunk, n, jc, start, end)) return;      // uniform: past the last chunk
    const int64_t t0 = start + static_cast<int64_t>(jc) * C;
    const int L = static_cast<int>(min<int64_t>(C, end - t0));
    char *rec = p.rec + static_cast<size_t>(item) * R_::bytes;

    const T *kp = static_cast<const T *>(p.k), *qp = static_cast<const T *>(p.q);
    const T *bp = static_cast<const T *>(p.b), *lap = static_cast<const T *>(p.log_alpha);
    const T *vp = static_cast<const T *>(p.v), *wp = static_cast<const T *>(p.w);

    // item m of this wave in a round: its index in the round (valid when < IPR), sub-chunk
    // and channel block within the round
    auto it_of = [&](int m) { return wave + NWV * m; };
    auto live = [&](int m) { return it_of(m) < IPR; };
    auto subR = [&](int m) { return it_of(m) % NS; };
    auto blk = [&](int m) { return it_of(m) / NS; };
    auto row_ok = [&](int m) { return live(m) && 16 * subR(m) + t < L; };
    auto tok = [&](int m) { return t0 + 16 * subR(m) + t; };
    auto bcast = [](const T *x) {      // a 16-byte vector of VEC copies of one element
        uint32_t u;
        if constexpr (sizeof(T) == 4) u = __float_as_uint(io<T>::ld(x));
        else u = static_cast<uint32_t>(x->bits) * 0x10001u;
        return u32x4{u, u, u, u};
    };
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    // ---- k, q, b of a round, prefetched one round ahead ----
    u32x4 rk[2][IPW], rq[2][IPW], rb[2][IPW];
    auto load_round = [&](int r, int slot) {
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            rk[slot][m] = zero4;
            rq[slot][m] = zero4;
            rb[slot][m] = zero4;
            if (row_ok(m)) {
                const int c0 = CB * (r * CPR + blk(m)) + VEC * gi;
                const size_t okq = (static_cast<size_t>(tok(m)) * p.h_k + hk) * DK + c0;
                rk[slot][m] = *reinterpret_cast<const u32x4 *>(kp + okq);
                rq[slot][m] = *reinterpret_cast<const u32x4 *>(qp + okq);
                if constexpr (b_scalar)
                    rb[slot][m] = bcast(bp + static_cast<size_t>(tok(m)) * p.h_v + h);
                else
                    rb[slot][m] = *reinterpret_cast<const u32x4 *>(
                        bp + (static_cast<size_t>(tok(m)) * p.h_v + h) * DK + c0);
            }
        }
    };
    load_round(0, 0);

    // ---- scan: in-sub-chunk cumulative log2 decay of every item of every round ----
    float cs[NR][IPW][VEC];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            u32x4 raw = zero4;
            if (row_ok(m)) {
                if constexpr (la_scalar) raw = bcast(lap + static_cast<size_t>(tok(m)) * p.h_v + h);
                else raw = *reinterpret_cast<const u32x4 *>(
                         lap + (static_cast<size_t>(tok(m)) * p.h_v + h) * DK +
                         CB * (r * CPR + blk(m)) + VEC * gi);
            }
            unpack16<BF>(raw, cs[r][m]);
        }
    // q/k L2-norm factors (a uniform branch): sums of squares over all d_k channels of the
    // token; a token's channels are spread over the items of one sub-chunk (in this wave
    // and others), so the partial sums meet in LDS (s_A is free until the rounds end)
    float fk[IPW], fq[IPW];
#pragma unroll
    for (int m = 0; m < IPW; ++m) fk[m] = fq[m] = 1.f;
    if (p.qkn) {
        float *s_nk = s_A, *s_nq = s_A + C;
        for (int i = tid; i < 2 * C; i += NT) s_A[i] = 0.f;
        lds_barrier();
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            if (!live(m)) continue;
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                u32x4 k4 = zero4, q4 = zero4;
                if (row_ok(m)) {
                    const size_t okq = (static_cast<size_t>(tok(m)) * p.h_k + hk) * DK +
                                       CB * (r * CPR + blk(m)) + VEC * gi;
                    k4 = *reinterpret_cast<const u32x4 *>(kp + okq);
                    q4 = *reinterpret_cast<const u32x4 *>(qp + okq);
                }
                float kk[VEC], qq[VEC];
                unpack16<BF>(k4, kk);
                unpack16<BF>(q4, qq);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    sk += kk[e] * kk[e];
                    sq += qq[e] * qq[e];
                }
            }
            sk += __shfl_xor(sk, 16);
            sk += __shfl_xor(sk, 32);
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            if (gi == 0) {
                atomicAdd(&s_nk[16 * subR(m) + t], sk);
                atomicAdd(&s_nq[16 * subR(m) + t], sq);
            }
        }
        lds_barrier();
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            if (!live(m)) continue;
            fk[m] = rsqrtf(s_nk[16 * subR(m) + t] + p.l2eps);
            fq[m] = rsqrtf(s_nq[16 * subR(m) + t] + p.l2eps);
        }
        lds_barrier();                         // s_A is reused for A
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            if (!live(m)) continue;            // uniform over the wave
            const int R = subR(m), c0 = CB * (r * CPR + blk(m)) + VEC * gi;
#pragma unroll
            for (int e = 0; e < VEC; ++e) cs[r][m][e] = row_scan16(cs[r][m][e] * kLog2e);
            if (t == 15) {
#pragma unroll
                for (int e = 0; e < VEC; e += 4)
                    *reinterpret_cast<f32x4 *>(&s_tot[R * DK + c0 + e]) =
                        f32x4{cs[r][m][e], cs[r][m][e + 1], cs[r][m][e + 2], cs[r][m][e + 3]};
            }
            if (t == 7) {
#pragma unroll
                for (int e = 0; e < VEC; e += 4)
                    *reinterpret_cast<f32x4 *>(&s_cmid[R * DK + c0 + e]) =
                        f32x4{cs[r][m][e], cs[r][m][e + 1], cs[r][m][e + 2], cs[r][m][e + 3]};
            }
        }
    lds_barrier();

    // ---- per-channel factors (one thread per channel) and gamma_C ----
    for (int c = tid; c < DK; c += NT) {
        float gmid[NS];
        float run = 0.f;
#pragma unroll
        for (int R = 0; R < NS; ++R) {
            gmid[R] = run + s_cmid[R * DK + c];
            run += s_tot[R * DK + c];
        }
        st_rec<NTR>(&reinterpret_cast<float *>(rec + R_::gC)[c], exp2_hw(run));
#pragma unroll
        for (int R = 0; R < NS; ++R) {
            s_fkg[R * DK + c] = exp2_hw(run - gmid[R]);
            s_fmid[R * DK + c] = exp2_hw(gmid[R]);
        }
#pragma unroll
        for (int R = 1; R < NS; ++R)
#pragma unroll
            for (int I = 0; I < R; ++I)
                s_foff[(R * (R - 1) / 2 + I) * DK + c] = exp2_hw(gmid[R] - gmid[I]);
    }
    // this lane's values relative to its sub-chunk's middle token: cs <- c_r - c_mid
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            if (!live(m)) continue;
            const int R = subR(m), c0 = CB * (r * CPR + blk(m)) + VEC * gi;
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                const f32x4 cm = *reinterpret_cast<const f32x4 *>(&s_cmid[R * DK + c0 + e]);
#pragma unroll
                for (int q = 0; q < 4; ++q) cs[r][m][e + q] -= cm[q];
            }
        }
    lds_barrier();                             // the per-channel factors are written
    // 2^(g at the middle token of sub-chunk R) for channels c0 .. c0 + VEC - 1
    auto fmid_of = [&](int R, int c0, float *out) {
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            const f32x4 f = *reinterpret_cast<const f32x4 *>(&s_fmid[R * DK + c0 + e]);
#pragma unroll
            for (int q = 0; q < 4; ++q) out[e + q] = f[q];
        }
    };

    // ---- rounds over the key channels: operand tiles, A and M on the matrix cores ----
    f32x4 accA[PPW], accM[PPW];
#pragma unroll
    for (int pi = 0; pi < PPW; ++pi) accA[pi] = accM[pi] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 X[NR][IPW];                          // gamma . b . k of this lane, for the WY pass
    char *qgrec = rec + R_::Qg;
    u32x4 *kgrec = reinterpret_cast<u32x4 *>(rec + R_::KgT);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int slot = r & 1, buf = DBUF ? (r & 1) : 0;
        if (r + 1 < NR) load_round(r + 1, slot ^ 1);
        T *tkh = s_tile + buf * 3 * TILE, *tqh = tkh + TILE, *tkb = tkh + 2 * TILE;
        if constexpr (!DBUF) {
            if (r > 0) lds_barrier();          // the previous round's products are done
        }
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            if (!live(m)) continue;
            const int R = subR(m), row = 16 * R + t, j = r * CPR + blk(m);
            const int c0 = CB * j + VEC * gi;
            float kk[VEC], qq[VEC], bb[VEC], kh[VEC], qh[VEC], kb[VEC], xx[VEC], qg[VEC], fm[VEC];
            fmid_of(R, c0, fm);
            unpack16<BF>(rk[slot][m], kk);
            unpack16<BF>(rq[slot][m], qq);
            unpack16<BF>(rb[slot][m], bb);
            if (p.qkn) {                       // uniform
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    kk[e] *= fk[m];
                    qq[e] *= fq[m];
                }
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                if constexpr (fg2) {           // k <- sqrt(beta) k, b <- 1
                    kk[e] *= sqrt_hw(bb[e]);
                    bb[e] = 1.f;
                }
                const float d = cs[r][m][e];
                const float ef = exp2_hw(d), ei = exp2_hw(-d);
                kh[e] = bb[e] * kk[e] * ef;
                qh[e] = qq[e] * ef;
                kb[e] = kk[e] * ei;
                xx[e] = kh[e] * fm[e];
                qg[e] = qh[e] * fm[e];
            }
            const int col = CB * blk(m) + VEC * gi;    // column within the round's tiles
            *reinterpret_cast<u32x4 *>(&tkh[row * SB + col]) = pack16<BF>(kh);
            *reinterpret_cast<u32x4 *>(&tqh[row * SB + col]) = pack16<BF>(qh);
            *reinterpret_cast<u32x4 *>(&tkb[row * SB + col]) = pack16<BF>(kb);
            X[r][m] = pack16<BF>(xx);
            // gamma . q in the record's fragment order: row tile row / 16, k tile j
            if constexpr (BF) {
#pragma unroll
                for (int h4 = 0; h4 < 2; ++h4) {
                    const int q4 = 8 * gi + 4 * h4, half = q4 >= 16 ? 1 : 0, lgq = (q4 & 15) >> 2;
                    const size_t sl = ((static_cast<size_t>(row >> 4) * NKD + j) * 64 + 16 * lgq + (row & 15)) * 2 + half;
                    st_rec<NTR>(&reinterpret_cast<u32x2 *>(qgrec)[sl],
                                u32x2{pack_bf16x2(qg[4 * h4], qg[4 * h4 + 1]), pack_bf16x2(qg[4 * h4 + 2], qg[4 * h4 + 3])});
                }
            } else {
                st_rec<NTR>(&reinterpret_cast<f32x4 *>(qgrec)[((row >> 4) * NKD + j) * 64 + 16 * gi + (row & 15)],
                            f32x4{qg[0], qg[1], qg[2], qg[3]});
            }
        }
        lds_barrier();                         // round r's tiles are written
        // A^T and M^T of the block pairs (lane: A[16R + li][16I + 4 lg + ii]), one k tile
        // per block of the round
#pragma unroll
        for (int pi = 0; pi < PPW; ++pi) {
            const int idx = wave + NWV * pi;
            if (idx >= NPAIR) break;
            int R, I;
            pair_of(idx, NS, R, I);
#pragma unroll
            for (int jl = 0; jl < CPR; ++jl) {
                u32x4 kbv = *reinterpret_cast<const u32x4 *>(&tkb[(16 * I + li) * SB + CB * jl + VEC * lg]);
                if (R != I) {
                    const float *f = &s_foff[(R * (R - 1) / 2 + I) * DK + CB * (r * CPR + jl) + VEC * lg];
                    float x[VEC];
                    unpack16<BF>(kbv, x);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) x[e] *= f[e];
                    kbv = pack16<BF>(x);
                }
                const u32x4 khv = *reinterpret_cast<const u32x4 *>(&tkh[(16 * R + li) * SB + CB * jl + VEC * lg]);
                const u32x4 qhv = *reinterpret_cast<const u32x4 *>(&tqh[(16 * R + li) * SB + CB * jl + VEC * lg]);
                if constexpr (BF) {
                    accA[pi] = mma_k32(kbv, khv, accA[pi]);
                    accM[pi] = mma_k32(kbv, qhv, accM[pi]);
                } else {
                    const f32x4 a = __builtin_bit_cast(f32x4, kbv);
                    accA[pi] = mma_k16_f32(a, __builtin_bit_cast(f32x4, khv), accA[pi]);
                    accM[pi] = mma_k16_f32(a, __builtin_bit_cast(f32x4, qhv), accM[pi]);
                }
            }
        }
        // KgT fragments of this round's channel tiles: (channel tile, token k tile) blocks
        for (int f = wave; f < RCT * NKC; f += NWV) {
            const int ctl = f / NKC, kt = f - ctl * NKC;     // channel tile within the round
            const int rt = RCT * r + ctl;                    // channel tile of the record
            const int ch = 16 * rt + li;                     // this lane's channel
            float vals[Op<BF>::EPL];
            if constexpr (BF) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int k0 = kt * 32 + 16 * hh + 4 * lg;
                    const u32x2 tv = lds_tr4(&tkb[(k0 + (li >> 2)) * SB + 16 * ctl + 4 * (li & 3)]);
                    const float fkv = s_fkg[(2 * kt + hh) * DK + ch];
                    vals[4 * hh + 0] = bf16_lo(tv.x) * fkv;
                    vals[4 * hh + 1] = bf16_hi(tv.x) * fkv;
                    vals[4 * hh + 2] = bf16_lo(tv.y) * fkv;
                    vals[4 * hh + 3] = bf16_hi(tv.y) * fkv;
                }
            } else {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int tk = kt * 16 + 4 * lg + jj;
                    vals[jj] = io<T>::ld(&tkb[tk * SB + 16 * ctl + li]) * s_fkg[(tk >> 4) * DK + ch];
                }
            }
            st_rec<NTR>(&kgrec[(rt * NKC + kt) * 64 + lane], pack16<BF>(vals));
        }
    }

    // ---- w and v (issued now, consumed after the solve) ----
    u32x4 rw[NRV][IPW], rv[NRV][IPW];
#pragma unroll
    for (int r = 0; r < NRV; ++r)
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            rw[r][m] = zero4;
            rv[r][m] = zero4;
            if (row_ok(m)) {
                const size_t ov = (static_cast<size_t>(tok(m)) * p.h_v + h) * DV +
                                  CB * (r * CPR + blk(m)) + VEC * gi;
                rv[r][m] = *reinterpret_cast<const u32x4 *>(vp + ov);
                if constexpr (b_scalar) {
                    rw[r][m] = bcast(bp + static_cast<size_t>(tok(m)) * p.h_v + h);
                } else if constexpr (GM == GATES_FG2) {
                    // beta [.., d_k] indexes like w [.., d_v] (d_v = d_k)
                    rw[r][m] = *reinterpret_cast<const u32x4 *>(bp + ov);
                } else {
                    rw[r][m] = *reinterpret_cast<const u32x4 *>(wp + ov);
                }
            }
        }

    // ---- A to LDS (blocks of the lower triangle), M to the record ----
    char *mrec = rec + R_::M;
#pragma unroll
    for (int pi = 0; pi < PPW; ++pi) {
        const int idx = wave + NWV * pi;
        if (idx >= NPAIR) break;
        int R, I;
        pair_of(idx, NS, R, I);
        const bool dg = R == I;
        f32x4 a4, m4;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int il = 4 * lg + ii;
            a4[ii] = (dg && il >= li) ? 0.f : accA[pi][ii];
            m4[ii] = (dg && il > li) ? 0.f : accM[pi][ii];
        }
        *reinterpret_cast<f32x4 *>(&s_A[tri_blk(R, I) * BS + li * BSTR + 4 * lg]) = a4;
        if constexpr (BF) {
            st_rec<NTR>(&reinterpret_cast<u32x2 *>(mrec)[(((R * NKC + (I >> 1)) * 64 + lane) << 1) + (I & 1)], f4_to_b16(m4));
            if (dg && !(R & 1) && R + 1 < NS)    // the upper half of a k tile on the diagonal
                st_rec<NTR>(&reinterpret_cast<u32x2 *>(mrec)[(((R * NKC + (R >> 1)) * 64 + lane) << 1) + 1], u32x2{0u, 0u});
        } else {
            st_rec<NTR>(&reinterpret_cast<f32x4 *>(mrec)[(R * NKC + I) * 64 + lane], m4);
        }
    }
    lds_barrier();

    // ---- T = (I + A)^{-1}: diagonal blocks by forward substitution (one lane per column) ----
    if (tid < 16 * NS) {
        const int R = tid >> 4, jcol = tid & 15;
        const float *Ab = &s_A[tri_blk(R, R) * BS];
        float x[16], acc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            x[m] = m == jcol ? 1.f : (m > jcol ? -acc[m] : 0.f);
#pragma unroll
            for (int r = m + 1; r < 16; ++r) acc[r] += Ab[r * BSTR + m] * x[m];
        }
        float *Tb = &s_T[tri_blk(R, R) * BS];
#pragma unroll
        for (int r = 0; r < 16; ++r) Tb[r * BSTR + jcol] = x[r];
    }
    lds_barrier();
    // off-diagonal blocks by levels d = R - I: T_RI = -T_RR sum_{I <= m < R} A_Rm T_mI
#pragma unroll
    for (int d = 1; d < NS; ++d) {
        for (int b = wave; b < NS - d; b += NWV) {
            const int R = b + d, I = b;
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
            for (int m = I; m < R; ++m) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&s_A[tri_blk(R, m) * BS + li * BSTR + 4 * lg]);
                f32x4 bT;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) bT[s2] = s_T[tri_blk(m, I) * BS + (4 * lg + s2) * BSTR + li];
                P = mma_k16_f32(a, bT, P);
            }
            const f32x4 tRR = *reinterpret_cast<const f32x4 *>(&s_T[tri_blk(R, R) * BS + li * BSTR + 4 * lg]);
            const f32x4 Tn = mma_k16_f32(tRR, P, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) s_T[tri_blk(R, I) * BS + (4 * lg + ii) * BSTR + li] = -Tn[ii];
        }
        lds_barrier();
    }
    if constexpr (BF) {
        // bf16 copy of T, row-major [C][STB], zero above the diagonal blocks, over A
        bf16_t *s_Tb = reinterpret_cast<bf16_t *>(s_A);
        for (int idx = tid; idx < C * C / 8; idx += NT) {
            const int r = idx / (C / 8), c8 = (idx % (C / 8)) * 8;
            const int R = r >> 4, I = c8 >> 4;
            float t8[8];
            if (I <= R) {
                const float *src = &s_T[tri_blk(R, I) * BS + (r & 15) * BSTR + (c8 & 15)];
#pragma unroll
                for (int e = 0; e < 8; ++e) t8[e] = src[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) t8[e] = 0.f;
            }
            *reinterpret_cast<u32x4 *>(&s_Tb[r * STB + c8]) = pack16<true>(t8);
        }
    }

    if constexpr (TALIAS) lds_barrier();     // every read of the fp32 T is done
    if constexpr (BF) {
        if (p.tmat != nullptr) {               // T for the chunked backward
            lds_barrier();
            const bf16_t *s_Tb = reinterpret_cast<const bf16_t *>(s_A);
            bf16_t *dst = static_cast<bf16_t *>(p.tmat) + static_cast<size_t>(item) * C * C;
            for (int idx = tid; idx < C * C / 8; idx += NT) {
                const int r = idx / (C / 8), c8 = (idx % (C / 8)) * 8;
                *reinterpret_cast<u32x4 *>(&dst[r * C + c8]) =
                    *reinterpret_cast<const u32x4 *>(&s_Tb[r * STB + c8]);
            }
        }
    }

    // ---- W~^T = X^T T^T per key round, U~ = T (w.v) per value round ----
    // wave roles: channel tile ctl = wave % RCT of the round, row tiles R = wave / RCT + k
    // (NWV / RCT); with two row-tile groups the even and the odd row tiles carry equal k
    // ranges
    const int ctl = wave % RCT, rg = wave / RCT;
    constexpr int RSTEP = NWV / RCT;
    const bf16_t *s_Tb = reinterpret_cast<const bf16_t *>(s_A);
    char *wrec = rec + R_::Wn;
#pragma unroll
    for (int rnd = 0; rnd < NR + NRV; ++rnd) {
        const bool isW = rnd < NR;
        const int r = isW ? rnd : rnd - NR;
        T *xt = s_tile + (rnd & 1) * TILE;
        // this lane's rows of X (key rounds) or of w.v (value rounds)
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            if (!live(m)) continue;
            const int row = 16 * subR(m) + t;
            u32x4 v4;
            if (isW) {
                v4 = X[r < NR ? r : 0][m];
            } else {
                float ww[VEC], vv[VEC], pr[VEC];
                unpack16<BF>(rw[r < NRV ? r : 0][m], ww);
                unpack16<BF>(rv[r < NRV ? r : 0][m], vv);
#pragma unroll
                for (int e = 0; e < VEC; ++e) pr[e] = (fg2 ? sqrt_hw(ww[e]) : ww[e]) * vv[e];
                v4 = pack16<BF>(pr);
            }
            *reinterpret_cast<u32x4 *>(&xt[row * SB + CB * blk(m) + VEC * gi]) = v4;
        }
        lds_barrier();                         // this round's tile (and, first time, T) is ready
        const int ct = RCT * r + ctl;          // channel (or value column) tile of the record
        if constexpr (BF) {
            u32x4 xb[NKC];                     // k = tokens 32 kt + 8 lg + 0..7 of column 16 ctl + li
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) {
                const int k0 = kt * 32 + 8 * lg + (li >> 2);
                const u32x2 lo = lds_tr4(&xt[k0 * SB + 16 * ctl + 4 * (li & 3)]);
                const u32x2 hi = lds_tr4(&xt[(k0 + 4) * SB + 16 * ctl + 4 * (li & 3)]);
                xb[kt] = u32x4{lo.x, lo.y, hi.x, hi.y};
            }
            for (int R = rg; R < NS; R += RSTEP) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < NKC; ++kt) {
                    if (kt * 32 > 16 * R + 15) break;
                    const u32x4 tb = *reinterpret_cast<const u32x4 *>(&s_Tb[(16 * R + li) * STB + kt * 32 + 8 * lg]);
                    acc = isW ? mma_k32(xb[kt], tb, acc) : mma_k32(tb, xb[kt], acc);
                }
                if (isW) {   // lane: W~[16R + li][16 ct + 4 lg + ii] -> -W~ fragments
                    st_rec<NTR>(&reinterpret_cast<u32x2 *>(wrec)[(((R * NKD + (ct >> 1)) * 64 + lane) << 1) + (ct & 1)],
                                f4_to_b16(-acc));
                } else {     // lane: U~[16R + 4 lg + ii][16 ct + li], a D-layout tile
                    st_rec<NTR>(&reinterpret_cast<u32x2 *>(rec + R_::Ut + (static_cast<size_t>(ct) * NS + R) * R_::UT_TILE)[lane],
                                f4_to_b16(acc));
                }
            }
        } else {
            float xv[NKC][4];
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt)
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) xv[kt][s2] = io<T>::ld(&xt[(kt * 16 + 4 * lg + s2) * SB + 16 * ctl + li]);
            for (int R = rg; R < NS; R += RSTEP) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int kt = 0; kt <= R; ++kt) {
                    const f32x4 tv = *reinterpret_cast<const f32x4 *>(&s_T[tri_blk(R, kt) * BS + li * BSTR + 4 * lg]);
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2)
                        acc = isW ? __builtin_amdgcn_mfma_f32_16x16x4f32(xv[kt][s2], tv[s2], acc, 0, 0, 0)
                                  : __builtin_amdgcn_mfma_f32_16x16x4f32(tv[s2], xv[kt][s2], acc, 0, 0, 0);
                }
                if (isW) st_rec<NTR>(&reinterpret_cast<f32x4 *>(wrec)[(R * NKD + ct) * 64 + lane], -acc);
                else st_rec<NTR>(&reinterpret_cast<f32x4 *>(rec + R_::Ut + (static_cast<size_t>(ct) * NS + R) * R_::UT_TILE)[lane], acc);
            }
        }
    }
}

// Waves per workgroup and channel blocks per round: eight waves over two blocks where a
// round then gives every wave a sub-chunk (64-token chunks; the LDS of two workgroups still
// fits a CU) or two (128-token chunks of bf16 records, one workgroup per CU with the fp32 T
// over the round tiles); four waves over one block otherwise.
template <bool BF, int C, int DK, int DV> struct PrepShape {
    static constexpr int NJ = DK / (BF ? 32 : 16), NJV = DV / (BF ? 32 : 16);
    static constexpr bool WIDE = (C == 64 || (C == 128 && BF)) && NJ % 2 == 0 && NJV % 2 == 0;
    static constexpr int NWV = WIDE ? 8 : 4, CPR = WIDE ? 2 : 1;
};

// Records beyond the last-level cache (MALL, 256 MB on MI355X) are written with
// non-temporal stores (gate-mode instances keep the default stores: fewer instances).
constexpr size_t kStreamRecordBytes = static_cast<size_t>(256) << 20;

template <typename T, bool BF, int C, int DK, int DV>
hipError_t launch_prep_t(const ChunkParams &p, int64_t items, hipStream_t st) {
    if (items <= 0) return hipSuccess;
    ChunkParams q = p;
    q.xgroup = p.group > 1 && items % (8 * p.group) == 0 ? p.group : 0;
    using PS = PrepShape<BF, C, DK, DV>;
    constexpr int W = PS::NWV, R = PS::CPR;
    const dim3 g(static_cast<unsigned>(items)), b(64 * W);
    const bool ntr = static_cast<size_t>(items) * Rec<C, DK, DV, BF>::bytes > kStreamRecordBytes;
    switch (p.gmode) {
    case GATES_KDA: hipLaunchKernelGGL((prep_kernel<T, BF, C, DK, DV, GATES_KDA, W, R, false>), g, b, 0, st, q); break;
    case GATES_GDN: hipLaunchKernelGGL((prep_kernel<T, BF, C, DK, DV, GATES_GDN, W, R, false>), g, b, 0, st, q); break;
    case GATES_FG2_PLUS: hipLaunchKernelGGL((prep_kernel<T, BF, C, DK, DV, GATES_FG2_PLUS, W, R, false>), g, b, 0, st, q); break;
    case GATES_FG2:
        if constexpr (DK == DV) hipLaunchKernelGGL((prep_kernel<T, BF, C, DK, DV, GATES_FG2, W, R, false>), g, b, 0, st, q);
        else return hipErrorInvalidValue;
        break;
    default:
        if (ntr) hipLaunchKernelGGL((prep_kernel<T, BF, C, DK, DV, GATES_GDN2, W, R, true>), g, b, 0, st, q);
        else hipLaunchKernelGGL((prep_kernel<T, BF, C, DK, DV, GATES_GDN2, W, R, false>), g, b, 0, st, q);
    }
    return hipGetLastError();
}

}  // namespace gdn2

namespace gdn2 {

template <typename T, bool BF, int C>
static hipError_t launch_prep_c(const ChunkParams &p, int dk, int dv, int64_t items, hipStream_t st) {
    if (dk == 128 && dv == 128) return launch_prep_t<T, BF, C, 128, 128>(p, items, st);
    if (dk == 64 && dv == 64) return launch_prep_t<T, BF, C, 64, 64>(p, items, st);
    if (dk == 128 && dv == 64) return launch_prep_t<T, BF, C, 128, 64>(p, items, st);
    if (dk == 64 && dv == 128) return launch_prep_t<T, BF, C, 64, 128>(p, items, st);
    return hipErrorInvalidValue;
}

hipError_t launch_prep(const ChunkParams &p, int chunk, int dk, int dv, bool bf16, int64_t items,
                       hipStream_t st) {
    if (bf16) {
        if (chunk == 32) return launch_prep_c<bf16_t, true, 32>(p, dk, dv, items, st);
        if (chunk == 64) return launch_prep_c<bf16_t, true, 64>(p, dk, dv, items, st);
        if (chunk == 128) return launch_prep_c<bf16_t, true, 128>(p, dk, dv, items, st);
    } else {
        if (chunk == 32) return launch_prep_c<float, false, 32>(p, dk, dv, items, st);
        if (chunk == 64) return launch_prep_c<float, false, 64>(p, dk, dv, items, st);
        if (chunk == 128) return launch_prep_c<float, false, 128>(p, dk, dv, items, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn2
