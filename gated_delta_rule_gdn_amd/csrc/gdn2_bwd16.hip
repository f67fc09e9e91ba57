// gdn2_bwd16.hip -- chunked backward of Gated DeltaNet-2 for bf16 inputs, on bf16 matrix
// cores.
//
// The algebra is that of gdn2_bwd.hip: the chunked WY form of the burn-gdn2 docs page,
// section "Architecture" (Chunk mode), differentiated chunk by chunk. Within a chunk of
// C = 64 tokens entering with state S and leaving with S' (record operands of the chunked
// forward: Wn = -W~, Qg = gamma.q, Kg = (gamma_C / gamma).k, M, U~, gamma_C; T = (I + A)^-1;
// X = w.v, Y = gamma.b.k), given dO and dS' = dL/dS':
//   dU = M^T dO + Kg dS',   dS = gamma_C dS' + Qg^T dO + Wn^T dU     (to the chunk before)
//   U = U~ + Wn S,  dQg = dO S^T,  dW~ = -dU S^T,  dKg = U dS'^T,  dM = lower(dO U^T),
//   dX = T^T dU,  dY = T^T dW~,  dT = dU X^T + dW~ Y^T,  dA = strictly-lower(-T^T dT T^T),
// then the chain rule through the decay factors to q, k, b and log alpha.
//
// Every product here takes bf16 operands from LDS (or from the forward's records) and
// accumulates in fp32; the reverse state pass keeps dS in fp32 registers. Kernels of one call:
//   (forward re-run)    the chunked forward without o, also writing the state entering every
//                       chunk and U = U~ + Wn S of every chunk as bf16 fragments (the precision
//                       every product below takes them in) and T of every record; its state
//                       pass's output waves form the reverse pass's operands from each staged
//                       record and dO: Kg and Wn^T as matrix-core fragments, E1 = M^T dO and
//                       E2 = Qg^T dO (BwdOps)
//   bwd_rseg_kernel     (dense batches with few pairs only) per later segment of chunks:
//                       its gradient transition Q and zero-start result R, and the gradient
//                       entering the segment before the last
//   bwd_rchain_kernel   per (sequence, value head, 16 state columns[, segment]), from the
//                       last chunk: dU = E1 + Kg dS' and dS = gamma_C dS' + E2 + Wn^T dU;
//                       writes dS' and dU of every chunk (bf16) and dS0 (fp32)
//   bwd_grads16_kernel  per record, every gradient of the chunk: dQg, dW~, dKg, dM,
//                       dX (-> dv, dw), dT, dA, the decay sums, dq, dk, db and dlog_alpha
#include "gdn2_chunk.h"

namespace gdn2 {

namespace {

constexpr int C = 64;
constexpr int NKC = C / 32;        // bf16 k tiles over the chunk
constexpr int NRC = C / 16;        // 16-row tiles over the chunk

// Row strides (bf16 elements) of LDS tiles with rows of 64 or 128 elements. The 16 rows of
// a fragment read (8 bytes per lane) fall on distinct banks, and so do the four rows of a
// transposing read.
template <int K> struct Pad { static constexpr int S = K == 64 ? 72 : 152; };

// Per-record buffers (bytes).
template <int DK, int DV>
struct BL16 {
    // the forward re-run's state pass -> bwd_rchain_kernel (BwdOps, gdn2_chunk.h)
    using BO = BwdOps<DK, DV>;
    static constexpr size_t KgA = BO::KgA;                                // Kg, A fragments [C][DK]
    static constexpr size_t WnT = BO::WnT;                                // Wn^T, A fragments [DK][C]
    static constexpr size_t OPS = BO::E1;
    static constexpr size_t E1 = BO::E1;                                  // bf16 D tiles [slice][C/16]
    static constexpr size_t E2 = BO::E2;                                  // bf16 D tiles [slice][DK/16]
    static constexpr size_t CREC = BO::bytes;
    // bwd_rchain_kernel -> bwd_grads16_kernel, bf16 D tiles
    static constexpr size_t DSN = 0;                                      // dS' [slice][DK/16]
    static constexpr size_t DU = DSN + static_cast<size_t>(DK) * DV * 2;  // dU [slice][C/16]
    static constexpr size_t COUT = DU + static_cast<size_t>(C) * DV * 2;
};

struct B16Params {
    const bf16_t *q, *k, *v, *la, *b, *w, *dO;
    const float *dS_T;                 // [N][h_v][DK][DV], or NULL
    const int32_t *cu, *map;           // packed batches: offsets and chunk map, else NULL
    const char *rec;                   // records of the forward re-run
    const bf16_t *tmat;                // T per record, [C][C]
    const u32x4 *ck;                   // state entering every chunk: bf16 B fragments of the
                                       // state pass, [record][DV/16][DK/32][64 lanes]
    const u32x4 *uck;                  // U = U~ + Wn S of every chunk, the same fragments
                                       // [record][DV/16][C/32][64 lanes]
    char *crec, *cout;
    float *dq, *dk, *dv, *dw, *dla, *db, *dS0;
    // segmented reverse pass (nseg > 1): the gradient entering segment nseg-2 [pair][DK][DV],
    // transitions Q [pair][nseg-2] (SegPFrag) and zero-start results R [pair][nseg-2][DK][DV]
    float *rseg_S, *rseg_Q, *rseg_R;
    int num_seqs, seqlen, nc_dense, h_k, h_v, group, num_pairs;
    int nseg, seg_len;
};

__device__ __forceinline__ bool locate16(const B16Params &p, int chunk, int &n, int &j,
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

// Fragment (perm order, gdn2_mfma.h) whose k index runs along the columns of a row-major
// bf16 LDS tile: lane (li, lg) receives t[r0 + li][k0 + perm(lg, jj)].
__device__ __forceinline__ u32x4 row_frag(const bf16_t *t, int stride, int r0, int k0, int li, int lg) {
    const bf16_t *q = t + (r0 + li) * stride + k0 + 4 * lg;
    const u32x2 a = *reinterpret_cast<const u32x2 *>(q);
    const u32x2 b = *reinterpret_cast<const u32x2 *>(q + 16);
    return u32x4{a.x, a.y, b.x, b.y};
}
// Fragment whose k index runs along the rows: lane (li, lg) receives t[k0 + perm(lg, jj)][c0 + li]
// (two transposing reads).
__device__ __forceinline__ u32x4 col_frag(const bf16_t *t, int stride, int k0, int c0, int li, int lg) {
    const bf16_t *q = t + (k0 + 4 * lg + (li >> 2)) * stride + c0 + 4 * (li & 3);
    const u32x2 a = lds_tr4(q);
    const u32x2 b = lds_tr4(q + 16 * stride);
    return u32x4{a.x, a.y, b.x, b.y};
}
// One lane's part of a 16x16 output tile (rows r0 + 4 lg + ii, column c0 + li) into a
// row-major bf16 tile, from fp32 or from bf16 already rounded.
__device__ __forceinline__ void put_tile(bf16_t *t, int stride, int r0, int c0, f32x4 v, int li, int lg) {
    bf16_t *q = t + (r0 + 4 * lg) * stride + c0 + li;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) q[ii * stride].bits = f32_to_bf16_bits(v[ii]);
}
__device__ __forceinline__ void put_tile16(bf16_t *t, int stride, int r0, int c0, u32x2 v, int li, int lg) {
    bf16_t *q = t + (r0 + 4 * lg) * stride + c0 + li;
    q[0].bits = static_cast<uint16_t>(v.x & 0xffffu);
    q[stride].bits = static_cast<uint16_t>(v.x >> 16);
    q[2 * stride].bits = static_cast<uint16_t>(v.y & 0xffffu);
    q[3 * stride].bits = static_cast<uint16_t>(v.y >> 16);
}
__device__ __forceinline__ f32x4 b16_to_f4(u32x2 v) {
    return f32x4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
}
__device__ __forceinline__ float f32of(const bf16_t *p) { return bf16_to_f32(p->bits); }
// Four fp32 values as a bf16 operand hi = bf16(x) and its remainder lo = bf16(x - hi)
// (hi + lo keeps about 16 significant bits).
__device__ __forceinline__ void split4(const float (&x)[4], u32x2 &hi, u32x2 &lo) {
    hi.x = pack_bf16x2(x[0], x[1]);
    hi.y = pack_bf16x2(x[2], x[3]);
    lo.x = pack_bf16x2(x[0] - bf16_lo(hi.x), x[1] - bf16_hi(hi.x));
    lo.y = pack_bf16x2(x[2] - bf16_lo(hi.y), x[3] - bf16_hi(hi.y));
}

// ---------------------------------------------------------------------------------------
// bwd_rchain_kernel: the reverse state pass. A workgroup owns NWS 16-column slices of dS of
// one (sequence, value head): one chain wave per slice holds its d_k x 16 slice in fp32
// registers, and four copy waves stage each chunk's Kg and Wn^T fragments, gamma_C and the
// slices' E1 and E2 tiles in LDS NBUF - 1 chunks ahead (direct global-to-LDS loads), so that
// a chunk's staging latency overlaps several chunk steps. Each chunk step first issues all
// of its LDS operand reads, then the products. The chain waves issue no global loads and
// never wait on memory: their stores of dS' and dU stay in flight. The workgroups of one
// (sequence, head) are placed on one XCD (blocks are dispatched to the XCDs round-robin),
// where they share the records in L2.
template <int DK, int DV, int NWS>
struct RChain {
    static constexpr int NCP = 4;
    static constexpr int OPS = static_cast<int>(BL16<DK, DV>::OPS);
    static constexpr int NRT = DK / 16;
    static constexpr int EB = (C + DK) * 16 * 2;            // E1 and E2 tiles of one slice
    static constexpr int STAGE = OPS + DK * 4 + NWS * EB;
    static constexpr int NBUF = 4 * STAGE <= 160 * 1024 ? 4 : 3;
    static constexpr int LDS = NBUF * STAGE;
    static constexpr int G = DV / 16 / NWS;                 // workgroups per (sequence, head)
    // direct loads one copy wave issues per stage (copy wave 0 also loads gamma_C)
    static constexpr int per(int cw) {
        return (OPS / 1024 - cw + NCP - 1) / NCP + (cw == 0 ? 1 : 0) +
               NWS * ((EB / 1024 - cw + NCP - 1) / NCP);
    }
};

// (one workgroup per CU by its LDS: the register budget of one wave per SIMD)
template <int DK, int DV, int NWS>
__global__ __launch_bounds__(64 * (NWS + 4)) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_rchain_kernel(B16Params p) {
    using R_ = Rec<C, DK, DV, true>;
    using L_ = BL16<DK, DV>;
    using RC = RChain<DK, DV, NWS>;
    constexpr int RT = DK / 16, NKD = DK / 32, NCP = RC::NCP, OPS = RC::OPS, EB = RC::EB;
    constexpr int STAGE = RC::STAGE, G = RC::G, NBUF = RC::NBUF;
    static_assert(NCP == 4 && (NBUF - 2) * RC::per(0) < 64 && EB % 1024 == 0, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // unit = (pair, segment in reverse order rg); its G workgroups share an XCD
    const int bid = blockIdx.x, idx = bid >> 3;
    const int unit = (idx / G) * 8 + (bid & 7), part = idx - (idx / G) * G;
    if (unit >= p.num_pairs * p.nseg) return;               // uniform over the workgroup
    const int pair = unit / p.nseg, rg = unit - pair * p.nseg;
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
    // this workgroup's chunks [cb, ce), taken from ce - 1 down to cb (segment g = nseg-1-rg)
    const int g = p.nseg - 1 - rg;
    const int cb = p.nseg > 1 ? g * p.seg_len : 0;
    const int ce = p.nseg > 1 ? min(nchunks, cb + p.seg_len) : nchunks;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const bool chain = wave < NWS;
    const int cw = wave - NWS;                              // copy wave index
    const int s = part * NWS + wave;                        // value slice of a chain wave
    auto recno = [&](int c) { return static_cast<size_t>(cbase + c) * p.h_v + h; };
    auto slot = [&](int c) { return smem + (c % NBUF) * STAGE; };
    auto stage = [&](int c) {                               // copy waves: chunk c into its slot
        char *dst = slot(c);
        const char *cr = p.crec + recno(c) * L_::CREC;
        for (int blk = cw; blk < OPS / 1024; blk += NCP) dma16(cr + blk * 1024 + lane * 16, dst + blk * 1024);
        if (cw == 0 && lane < DK / 4)
            dma16(p.rec + recno(c) * R_::bytes + R_::gC + lane * 16, dst + OPS);
#pragma unroll
        for (int q = 0; q < NWS; ++q) {
            const int sl = part * NWS + q;
            const char *e1 = cr + L_::E1 + static_cast<size_t>(sl) * NRC * 512;
            const char *e2 = cr + L_::E2 + static_cast<size_t>(sl) * RT * 512;
            char *d = dst + OPS + DK * 4 + q * EB;
            for (int blk = cw; blk < EB / 1024; blk += NCP) {
                const char *src = blk < NRC / 2 ? e1 + blk * 1024 : e2 + (blk - NRC / 2) * 1024;
                dma16(src + lane * 16, d + blk * 1024);
            }
        }
    };
    // copy waves: wait until the stage of chunk c has landed, with `newer` later-issued
    // stages allowed to stay in flight
    auto wait_stage = [&](int newer) {
        if (newer <= 0) {
            wait_vmem();
            return;
        }
        const bool one = newer == 1;
        switch (cw) {          // each copy wave counts its own loads per stage
        case 0: if (one) wait_vmem_n<RC::per(0)>(); else wait_vmem_n<(NBUF - 2) * RC::per(0)>(); break;
        case 1: if (one) wait_vmem_n<RC::per(1)>(); else wait_vmem_n<(NBUF - 2) * RC::per(1)>(); break;
        case 2: if (one) wait_vmem_n<RC::per(2)>(); else wait_vmem_n<(NBUF - 2) * RC::per(2)>(); break;
        default: if (one) wait_vmem_n<RC::per(3)>(); else wait_vmem_n<(NBUF - 2) * RC::per(3)>(); break;
        }
    };

    // dS' rows 16 rt + 4 lg + ii, column 16 s + li: from dS_T for the last segment, else from
    // the gradient entering segment nseg - 2, carried over segments rg' = 1 .. rg - 1 for
    // rg >= 2 (dS <- Q dS + R, Q staged at the start of the LDS before any chunk)
    f32x4 D[RT];
    const size_t sbase = (static_cast<size_t>(n) * p.h_v + h) * DK * DV;
    if (chain) {
        const float *Din = rg == 0 ? p.dS_T : p.rseg_S;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                D[rt][ii] = Din ? Din[sbase + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + 16 * s + li] : 0.f;
    }
    {
        using PF = SegPFrag<DK, true>;
        constexpr int H = RT / 2, NBLK = static_cast<int>(PF::BYTES / 1024);
        static_assert(PF::BYTES + NWS * RT * 1024 <= static_cast<size_t>(RC::LDS), "carry fits");
        const int nq = p.nseg - 2;
        for (int hq = 1; hq < rg; ++hq) {   // rg >= 2 only; uniform over the workgroup
            if (!chain) {
                const char *Qh = reinterpret_cast<const char *>(p.rseg_Q) +
                                 (static_cast<size_t>(pair) * nq + hq - 1) * PF::BYTES;
                for (int blk = cw; blk < NBLK; blk += NCP) dma16(Qh + blk * 1024 + lane * 16, smem + blk * 1024);
                wait_vmem();
            }
            f32x4 Rl[H], Rh[H];
            if (chain) {
                const float *Rq = p.rseg_R + (static_cast<size_t>(pair) * nq + hq - 1) * DK * DV;
#pragma unroll
                for (int j = 0; j < H; ++j)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        Rl[j][ii] = Rq[static_cast<size_t>(16 * j + 4 * lg + ii) * DV + 16 * s + li];
                        Rh[j][ii] = Rq[static_cast<size_t>(16 * (H + j) + 4 * lg + ii) * DV + 16 * s + li];
                    }
            }
            raw_barrier();                  // Q staged
            if (chain) {                    // both halves from the same dS (the products pack it first)
                f32x4 A[RT], B[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) A[rt] = B[rt] = D[rt];
                f32x4 *xd = reinterpret_cast<f32x4 *>(smem + PF::BYTES) + wave * RT * 64;
                PF::template carry_half<0>(smem, Rl, A, xd);
                PF::template carry_half<H>(smem, Rh, B, xd);
#pragma unroll
                for (int j = 0; j < H; ++j) {
                    D[j] = A[j];
                    D[H + j] = B[H + j];
                }
            }
            wait_lds();
            raw_barrier();                  // every read of Q done before the LDS is restaged
        }
    }
    if (ce > cb) {
        if (!chain) {
            for (int c = ce - 1; c >= cb && c > ce - NBUF; --c) stage(c);
            wait_stage(min(ce - 1 - cb, NBUF - 2));
        }
        lds_barrier();
    }
    for (int c = ce - 1; c >= cb; --c) {
        if (!chain) {
            if (c - cb >= NBUF - 1) stage(c - (NBUF - 1));
            if (c - cb >= 1) wait_stage(min(c - cb - 1, NBUF - 2));   // chunk c - 1 has landed
        } else {
            const char *buf = slot(c);
            const u32x4 *kga = reinterpret_cast<const u32x4 *>(buf);
            const u32x4 *wnt = kga + C * DK / 8;
            const float *gam = reinterpret_cast<const float *>(buf + OPS);
            const u32x2 *e1 = reinterpret_cast<const u32x2 *>(buf + OPS + DK * 4 + wave * EB);
            const u32x2 *e2 = e1 + NRC * 64;
            // every LDS operand of the step first
            u32x4 ka[NRC][NKD], wa[RT][NKC];
            u32x2 e1v[NRC], e2v[RT];
            f32x4 g4[RT];
#pragma unroll
            for (int ut = 0; ut < NRC; ++ut) {
                e1v[ut] = e1[ut * 64 + lane];
#pragma unroll
                for (int kt = 0; kt < NKD; ++kt) ka[ut][kt] = kga[(ut * NKD + kt) * 64 + lane];
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                e2v[rt] = e2[rt * 64 + lane];
                g4[rt] = *reinterpret_cast<const f32x4 *>(&gam[16 * rt + 4 * lg]);
#pragma unroll
                for (int kt = 0; kt < NKC; ++kt) wa[rt][kt] = wnt[(rt * NKC + kt) * 64 + lane];
            }
            asm volatile("" ::: "memory");
            char *co = p.cout + recno(c) * L_::COUT;
            u32x2 *dsn = reinterpret_cast<u32x2 *>(co + L_::DSN) + s * RT * 64 + lane;
            u32x2 *du = reinterpret_cast<u32x2 *>(co + L_::DU) + s * NRC * 64 + lane;
            u32x4 Dp[NKD];
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) Dp[kt] = dpair_to_b32(D[2 * kt], D[2 * kt + 1]);
            f32x4 U[NRC];
#pragma unroll
            for (int ut = 0; ut < NRC; ++ut) {
                f32x4 acc = b16_to_f4(e1v[ut]);
#pragma unroll
                for (int kt = 0; kt < NKD; ++kt) acc = mma_k32(ka[ut][kt], Dp[kt], acc);
                U[ut] = acc;
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) dsn[rt * 64] = f4_to_b16(D[rt]);
            u32x4 Up[NKC];
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) Up[kt] = dpair_to_b32(U[2 * kt], U[2 * kt + 1]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4 acc = b16_to_f4(e2v[rt]);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) acc[ii] += g4[rt][ii] * D[rt][ii];
#pragma unroll
                for (int kt = 0; kt < NKC; ++kt) acc = mma_k32(wa[rt][kt], Up[kt], acc);
                D[rt] = acc;
            }
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) {
                du[(2 * kt) * 64] = Up[kt].xy;
                du[(2 * kt + 1) * 64] = Up[kt].zw;
            }
        }
        lds_barrier();                                      // slot(c) free; slot(c - 1) ready
    }
    if (chain && g == 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                p.dS0[sbase + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + 16 * s + li] = D[rt][ii];
    }
}

// ---------------------------------------------------------------------------------------
// Segmented reverse pass (dense batches with few (sequence, value head) pairs). The reverse
// recursion is affine in the state gradient: dS_before = (diag(gamma_C) + Wn^T Kg) dS_after
// + (E2 + Wn^T E1), so over a segment of chunks dS_in = Q dS_out + R. Segments are taken in
// reverse order, rg = nseg - 1 - g for segment g of chunks [g L, (g + 1) L):
//   bwd_rseg_kernel   rg = 0 (the last segment): the true run from dS_T, whose result is
//                     the gradient entering segment nseg - 2 from above; rg = 1 .. nseg - 2:
//                     R (from zero) and Q (the chain run on the columns of the identity
//                     without E1 and E2). Only the chain is computed.
//   bwd_rchain_kernel every segment from its own start, with outputs; segment rg >= 2 first
//                     carries the gradient entering segment nseg - 2 over rg = 1 .. rg - 1,
//                     dS <- Q dS + R.
// ---------------------------------------------------------------------------------------
constexpr int kRSegWaves = 4;    // chain waves per reverse segment-pass workgroup
constexpr int kRSegCopy = 4;
constexpr int kRSegRSlices = 2;  // R slices per workgroup (their E1 and E2 tiles are staged too)

// Q workgroups (up to kRSegWaves slices of Q) stage Kg, Wn^T and gamma_C per chunk; R
// workgroups (kRSegRSlices slices of R) also their slices' E1 and E2 tiles. Each kind takes
// as many stages (<= 4) as fit in the LDS, so that up to three chunks are in flight.
template <int DK, int DV>
struct RSegLayout {
    using L_ = BL16<DK, DV>;
    static constexpr int OPS = static_cast<int>(L_::OPS);             // Kg, Wn^T fragments
    static constexpr int EB = (C + DK) * 16 * 2;                      // E1 and E2 tiles of a slice
    static constexpr int GC = OPS;                                    // gamma_C, fp32 [DK]
    static constexpr int EO = GC + DK * 4;                            // [slice] E1, E2 tiles
    static constexpr int QBUF = EO, RBUF = EO + kRSegRSlices * EB;
    static constexpr int QN = QBUF * 4 <= 160 * 1024 ? 4 : 160 * 1024 / QBUF;
    static constexpr int RN = RBUF * 4 <= 160 * 1024 ? 4 : 160 * 1024 / RBUF;
    static constexpr int LDS = QN * QBUF > RN * RBUF ? QN * QBUF : RN * RBUF;
    static constexpr int NQ = DK / 16, NR = DV / 16;                  // Q and R column slices
    static constexpr int QG = (NQ + kRSegWaves - 1) / kRSegWaves;
    static constexpr int GROUPS = QG + (NR + kRSegRSlices - 1) / kRSegRSlices;
    static_assert(QN >= 2 && RN >= 2 && EB % 1024 == 0, "reverse segment stages");
};

// s_waitcnt vmcnt(min(n, 63)), n chosen at run time (copy waves only, off the critical path)
template <int N = 63>
__device__ __forceinline__ void wait_vmem_upto(int n) {
    if constexpr (N == 0) {
        wait_vmem_n<0>();
    } else {
        if (n >= N) wait_vmem_n<N>();
        else wait_vmem_upto<N - 1>(n);
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(64 * (kRSegWaves + kRSegCopy)) void bwd_rseg_kernel(B16Params p) {
    using R_ = Rec<C, DK, DV, true>;
    using L_ = BL16<DK, DV>;
    using SG = RSegLayout<DK, DV>;
    constexpr int RT = DK / 16, NKD = DK / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;

    const int bid = blockIdx.x, xcd = bid & 7, rest = bid >> 3;
    const int grp = rest % SG::GROUPS;
    const int unit = (rest / SG::GROUPS) * 8 + xcd;
    const int nsa = p.nseg - 1;
    if (unit >= p.num_pairs * nsa) return;
    const int pair = unit / nsa, rg = unit - pair * nsa;
    const bool qgrp = grp < SG::QG;
    if (qgrp && rg == 0) return;                  // the last segment needs no Q (uniform)
    const int n = pair / p.h_v, h = pair - n * p.h_v;
    // this workgroup's slices [v0, v1) of Q (qgrp) or of R
    const int v0 = qgrp ? grp * kRSegWaves : (grp - SG::QG) * kRSegRSlices;
    const int v1 = qgrp ? min(v0 + kRSegWaves, SG::NQ) : min(v0 + kRSegRSlices, SG::NR);
    const int nb = qgrp ? SG::QN : SG::RN, sb = qgrp ? SG::QBUF : SG::RBUF;
    const int g = p.nseg - 1 - rg;
    const int cb = g * p.seg_len;
    const int ce = min(p.nc_dense, cb + p.seg_len);
    const int nst = ce - cb;                      // chunks, taken from ce - 1 down to cb
    const int cbase = n * p.nc_dense;
    auto recno = [&](int c) { return static_cast<size_t>(cbase + c) * p.h_v + h; };
    auto slot = [&](int i) { return smem + (i % nb) * sb; };

    if (wave >= kRSegWaves) {
        // ---- copy waves: up to nb - 1 steps in flight; step i is chunk ce - 1 - i
        const int cw = wave - kRSegWaves;
        const int ner = qgrp ? 0 : v1 - v0;       // R slices whose E1, E2 are staged
        auto issue = [&](int i) {
            char *dst = slot(i);
            const int c = ce - 1 - i;
            const char *cr = p.crec + recno(c) * L_::CREC;
            for (int blk = cw; blk < SG::OPS / 1024; blk += kRSegCopy) dma16(cr + blk * 1024 + lane * 16, dst + blk * 1024);
            if (cw == kRSegCopy - 1 && lane < DK / 4)
                dma16(p.rec + recno(c) * R_::bytes + R_::gC + lane * 16, dst + SG::GC);
            for (int r = 0; r < ner; ++r) {
                const char *e1 = cr + L_::E1 + static_cast<size_t>(v0 + r) * NRC * 512;
                const char *e2 = cr + L_::E2 + static_cast<size_t>(v0 + r) * RT * 512;
                char *d = dst + SG::EO + r * SG::EB;
                for (int blk = cw; blk < SG::EB / 1024; blk += kRSegCopy) {
                    const char *src = blk < NRC / 2 ? e1 + blk * 1024 : e2 + (blk - NRC / 2) * 1024;
                    dma16(src + lane * 16, d + blk * 1024);
                }
            }
        };
        // direct loads this wave issues per step (the loops of issue())
        const int per = (SG::OPS / 1024 - cw + kRSegCopy - 1) / kRSegCopy + (cw == kRSegCopy - 1 ? 1 : 0) +
                        ner * ((SG::EB / 1024 - cw + kRSegCopy - 1) / kRSegCopy);
        int issued = 0;
        for (; issued < nst && issued < nb - 1; ++issued) issue(issued);
        for (int i = 0; i < nst; ++i) {
            wait_vmem_upto((issued - 1 - i) * per);   // step i has landed
            raw_barrier();                  // step i is staged; step i-1 fully consumed
            if (issued < nst) issue(issued++);   // into the slot of step i-1
        }
        return;
    }

    // ---- chain waves ----
    const int v = v0 + wave;
    const bool active = v < v1;                   // uniform per wave
    const int col = 16 * v + li;
    f32x4 D[RT];
    const size_t sbase = static_cast<size_t>(pair) * DK * DV;
    const bool fromT = active && !qgrp && rg == 0 && p.dS_T != nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int row = 16 * rt + 4 * lg + ii;
            D[rt][ii] = fromT ? p.dS_T[sbase + static_cast<size_t>(row) * DV + col]
                              : (qgrp && row == col ? 1.f : 0.f);
        }
    for (int i = 0; i < nst; ++i) {
        const char *buf = slot(i);
        raw_barrier();                      // step i is staged; step i-1 fully consumed
        if (!active) continue;
        const u32x4 *kga = reinterpret_cast<const u32x4 *>(buf);
        const u32x4 *wnt = kga + C * DK / 8;
        const float *gam = reinterpret_cast<const float *>(buf + SG::GC);
        const u32x2 *e1 = reinterpret_cast<const u32x2 *>(buf + SG::EO + wave * SG::EB);
        const u32x2 *e2 = e1 + NRC * 64;
        // the products' LDS operands first (no E1, E2 on Q columns)
        u32x4 ka[NRC][NKD], wa[RT][NKC];
        u32x2 e1v[NRC], e2v[RT];
#pragma unroll
        for (int ut = 0; ut < NRC; ++ut) {
            if (!qgrp) e1v[ut] = e1[ut * 64 + lane];
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) ka[ut][kt] = kga[(ut * NKD + kt) * 64 + lane];
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (!qgrp) e2v[rt] = e2[rt * 64 + lane];
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) wa[rt][kt] = wnt[(rt * NKC + kt) * 64 + lane];
        }
        u32x4 Dp[NKD];
#pragma unroll
        for (int kt = 0; kt < NKD; ++kt) Dp[kt] = dpair_to_b32(D[2 * kt], D[2 * kt + 1]);
        // dU = E1 + Kg dS'
        f32x4 U[NRC];
#pragma unroll
        for (int ut = 0; ut < NRC; ++ut) {
            f32x4 acc = qgrp ? f32x4{0.f, 0.f, 0.f, 0.f} : b16_to_f4(e1v[ut]);
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) acc = mma_k32(ka[ut][kt], Dp[kt], acc);
            U[ut] = acc;
        }
        u32x4 Up[NKC];
#pragma unroll
        for (int kt = 0; kt < NKC; ++kt) Up[kt] = dpair_to_b32(U[2 * kt], U[2 * kt + 1]);
        // dS = E2 + gamma_C dS' + Wn^T dU
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 acc = qgrp ? f32x4{0.f, 0.f, 0.f, 0.f} : b16_to_f4(e2v[rt]);
            const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&gam[16 * rt + 4 * lg]);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) acc[ii] += g4[ii] * D[rt][ii];
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) acc = mma_k32(wa[rt][kt], Up[kt], acc);
            D[rt] = acc;
        }
        wait_lds();
    }
    if (!active) return;
    if (qgrp) {
        char *dst = reinterpret_cast<char *>(p.rseg_Q) +
                    (static_cast<size_t>(pair) * (nsa - 1) + rg - 1) * SegPFrag<DK, true>::BYTES;
        SegPFrag<DK, true>::put_slice(dst, v, D);
        return;
    }
    float *dst = rg == 0 ? p.rseg_S + static_cast<size_t>(pair) * DK * DV   // entering segment nseg-2
                         : p.rseg_R + (static_cast<size_t>(pair) * (nsa - 1) + rg - 1) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            dst[static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] = D[rt][ii];
}

// ---------------------------------------------------------------------------------------
// bwd_grads16_kernel: per record, every gradient of the chunk, in two phases that share one
// LDS allocation (one workgroup of eight waves per CU by its LDS: the register budget of two
// waves per SIMD).
//
// Phase 1, the products with S, dS', dO and dU:
//   U = U~ + Wn S,  dQg = dO S^T,  dW~ = -dU S^T,  dKg = U dS'^T,  dM = lower(dO U^T),
//   dT1 = dU X^T,  dX = T^T dU (-> dv = w dX, dw = v dX),  dgamma_C = sum_col dS' . S.
// [C][DK] products are formed in (row tile B, channel tile ct) tiles t = wave + 8 j, [C][DV]
// ones in (row tile wave / 2, column tiles of half wave % 2), [C][C] ones in tiles wave and
// wave + 8; the [C][DK] and [C][C] results stay in registers for phase 2, which uses the
// same tiles. Phase 2's inputs (k, q, b, log alpha) are loaded with phase 1's and wait in
// registers.
//
// Phase 2, the products through T and the decay factors: the cumulative log decay is rebuilt
// from log alpha (log2 units, fp32); dY = T^T dW~, dT = dT1 + dW~ Y^T, dA = strictly-lower(
// -T^T dT T^T). The decay sums
//   P1[x] = sum_{i<x} dA[x,i] k_i E[x,i],   P3[x] = sum_{i<=x} dM[x,i] k_i E[x,i]
//   P2[x] = sum_{r>x} dA[r,x] bk_r E[r,x],  P4[x] = sum_{r>=x} dM[r,x] q_r E[r,x]
// (E[r,i] = exp(g_r - g_i) per channel) run on the matrix cores per 16-row block B with the
// block's middle row rho as reference, E[x,i] = exp(g_x - g_rho) exp(g_rho - g_i): every
// factor spans at most 8 tokens of decay or is <= 1. The factor operands are split into bf16
// hi and lo parts (two products each): P1 and P2 (and P3 and P4) enter dg with opposite
// signs and cancel over the chunk, and a single bf16 rounding of their operands would leave
// d log alpha about ten times less accurate than the other gradients. The wave that owns
// channel tile ct of row block B holds that tile of dQg, dKg and dY and takes the
// elementwise chain rule to dq, dk, db and the decay gradient dg there; d log alpha is the
// reverse cumulative sum of dg over the chunk plus the gamma_C terms, which reach every row.
template <int DK, int DV>
struct GLay {
    static constexpr int SV = Pad<DV>::S, SK = Pad<DK>::S, SC = Pad<C>::S;
    static constexpr int SQ = DK + 8;          // k, b, q, log alpha: rows or single elements only
    static constexpr int SG = DK + 4;          // fp32 cumulative decay
    // both phases: T [C][SC] bf16, dgamma_C [DK] fp32
    static constexpr int T_ = 0, DGL = T_ + 2 * C * SC, BASE = DGL + 4 * DK;
    // phase 1 (bf16 tiles)
    static constexpr int S_ = BASE;                       // [DK][SV]: S, then dS'
    static constexpr int O_ = S_ + 2 * DK * SV;           // [C][SV] dO
    static constexpr int DU = O_ + 2 * C * SV;            // [C][SV] dU
    static constexpr int U_ = DU + 2 * C * SV;            // [C][SV] U
    static constexpr int W_ = U_ + 2 * C * SV;            // [C][SV] w
    static constexpr int V_ = W_ + 2 * C * SV;            // [C][SV] v
    static constexpr int END1 = V_ + 2 * C * SV;
    // phase 2
    static constexpr int G_ = BASE;                       // [C][SG] fp32
    static constexpr int TOT = G_ + 4 * C * SG;           // [2][C/16][DK] fp32
    static constexpr int K_ = TOT + 4 * 2 * NRC * DK;     // [C][SQ] bf16 each: k, b, q, log alpha
    static constexpr int B_ = K_ + 2 * C * SQ, Q_ = B_ + 2 * C * SQ, LA = Q_ + 2 * C * SQ;
    static constexpr int DW = LA + 2 * C * SQ;            // [C][SK] dW~
    static constexpr int DT = DW + 2 * C * SK;            // [C][SC] dT, then Z, then dA
    static constexpr int DM = DT + 2 * C * SC;            // [C][SC] dM
    static constexpr int END2 = DM + 2 * C * SC;
    static constexpr int LDS = END1 > END2 ? END1 : END2;
    static_assert(BASE % 16 == 0 && O_ % 16 == 0 && DU % 16 == 0 && U_ % 16 == 0 && W_ % 16 == 0 &&
                      V_ % 16 == 0 && TOT % 16 == 0 && K_ % 16 == 0 && B_ % 16 == 0 && Q_ % 16 == 0 &&
                      LA % 16 == 0 && DW % 16 == 0 && DT % 16 == 0 && DM % 16 == 0,
                  "16-byte aligned regions");
};

template <int DK, int DV>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_grads16_kernel(B16Params p) {
    using L_ = BL16<DK, DV>;
    using GL = GLay<DK, DV>;
    constexpr int SV = GL::SV, SK = GL::SK, SC = GL::SC, SQ = GL::SQ, SG = GL::SG;
    constexpr int NKD = DK / 32, NKV = DV / 32, RT = DK / 16, CT = DK / 16, VT = DV / 16;
    constexpr int TPW = NRC * CT / 8, UPW = NRC * VT / 8;
    constexpr int NSF = DK * DV / 8 / 512, NUF = C * DV / 8 / 512, NOV = C * DV / 8 / 512,
                  NKV8 = C * DK / 8 / 512;
    constexpr int NUT = NRC * VT / 8, NDT = RT * VT / 8;
    constexpr int PARTS = 512 / DK, RP = C / PARTS;
    static_assert(TPW >= 1 && UPW >= 1 && NSF >= 1 && NUF >= 1 && NOV >= 1 && NUT >= 1 && NDT >= 1 && NKV8 >= 1 &&
                      PARTS * DK == 512 && 8 % RT == 0, "split");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16_t *Tl = reinterpret_cast<bf16_t *>(smem + GL::T_);
    float *dgl = reinterpret_cast<float *>(smem + GL::DGL);
    bf16_t *Sl = reinterpret_cast<bf16_t *>(smem + GL::S_);
    bf16_t *Ol = reinterpret_cast<bf16_t *>(smem + GL::O_);
    bf16_t *dUl = reinterpret_cast<bf16_t *>(smem + GL::DU);
    bf16_t *Ul = reinterpret_cast<bf16_t *>(smem + GL::U_);
    bf16_t *wl = reinterpret_cast<bf16_t *>(smem + GL::W_);
    bf16_t *vl = reinterpret_cast<bf16_t *>(smem + GL::V_);

    const int item = blockIdx.x, chunk = item / p.h_v, h = item - chunk * p.h_v;
    int n, j;
    int64_t start, end;
    if (!locate16(p, chunk, n, j, start, end)) return;
    const int64_t t0 = start + static_cast<int64_t>(j) * C;
    const int Lr = static_cast<int>(min<int64_t>(C, end - t0));
    const int hk = h / p.group;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const u32x4 *S = p.ck + static_cast<size_t>(item) * (DK * DV / 8);
    const char *co = p.cout + static_cast<size_t>(item) * L_::COUT;
    const bf16_t *Tg = p.tmat + static_cast<size_t>(item) * C * C;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    // token strides (elements) of the [.., h, d] gradient layouts
    const int tsv = p.h_v * DV, tsk = p.h_k * DK, tsg = p.h_v * DK;

    // every global load of both phases first
    u32x4 sv[NSF];
#pragma unroll
    for (int i = 0; i < NSF; ++i) sv[i] = S[tid + 512 * i];
    // row r0 + (512 / (d / 8)) i and columns c8 .. c8 + 7 of the [C][d] tiles for this thread
    const int rv0 = tid / (DV / 8), cv8 = (tid - rv0 * (DV / 8)) * 8;
    const size_t ov0 = (static_cast<size_t>(t0 + rv0) * p.h_v + h) * DV + cv8;
    u32x4 ov[NOV], wv[NOV], vv[NOV];
#pragma unroll
    for (int i = 0; i < NOV; ++i) {
        const int r = rv0 + (512 / (DV / 8)) * i;
        ov[i] = wv[i] = vv[i] = zero4;
        if (r < Lr) {
            const size_t off = ov0 + static_cast<size_t>((512 / (DV / 8)) * i) * tsv;
            ov[i] = *reinterpret_cast<const u32x4 *>(p.dO + off);
            wv[i] = *reinterpret_cast<const u32x4 *>(p.w + off);
            vv[i] = *reinterpret_cast<const u32x4 *>(p.v + off);
        }
    }
    const u32x4 tv = reinterpret_cast<const u32x4 *>(Tg)[tid];
    u32x2 duv[NUT], dsv[NDT];
#pragma unroll
    for (int i = 0; i < NUT; ++i) duv[i] = reinterpret_cast<const u32x2 *>(co + L_::DU)[(wave + 8 * i) * 64 + lane];
#pragma unroll
    for (int i = 0; i < NDT; ++i) dsv[i] = reinterpret_cast<const u32x2 *>(co + L_::DSN)[(wave + 8 * i) * 64 + lane];
    const int urt = wave >> 1, uct0 = (wave & 1) * UPW;
    u32x4 uf[NUF];                      // U of the forward's state pass
#pragma unroll
    for (int i = 0; i < NUF; ++i) uf[i] = p.uck[static_cast<size_t>(item) * (C * DV / 8) + tid + 512 * i];
    const int rk0 = tid / (DK / 8), ck8 = (tid - rk0 * (DK / 8)) * 8;
    const size_t ok0 = (static_cast<size_t>(t0 + rk0) * p.h_k + hk) * DK + ck8;
    const size_t og0 = (static_cast<size_t>(t0 + rk0) * p.h_v + h) * DK + ck8;
    u32x4 kv[NKV8], bv[NKV8], qv[NKV8], av[NKV8];
#pragma unroll
    for (int i = 0; i < NKV8; ++i) {
        const int r = rk0 + (512 / (DK / 8)) * i;
        kv[i] = bv[i] = qv[i] = av[i] = zero4;
        if (r < Lr) {
            const size_t ok = ok0 + static_cast<size_t>((512 / (DK / 8)) * i) * tsk;
            const size_t og = og0 + static_cast<size_t>((512 / (DK / 8)) * i) * tsg;
            kv[i] = *reinterpret_cast<const u32x4 *>(p.k + ok);
            qv[i] = *reinterpret_cast<const u32x4 *>(p.q + ok);
            bv[i] = *reinterpret_cast<const u32x4 *>(p.b + og);
            av[i] = *reinterpret_cast<const u32x4 *>(p.la + og);
        }
    }

    // ---- phase 1 ----
    if (tid < DK) dgl[tid] = 0.f;
#pragma unroll
    for (int i = 0; i < NSF; ++i) {          // fragment (column tile, k tile) = two D tiles
        const int f = (tid >> 6) + 8 * i, ct = f / NKD, kt = f - ct * NKD;
        put_tile16(Sl, SV, 32 * kt, 16 * ct, u32x2{sv[i].x, sv[i].y}, li, lg);
        put_tile16(Sl, SV, 32 * kt + 16, 16 * ct, u32x2{sv[i].z, sv[i].w}, li, lg);
    }
#pragma unroll
    for (int i = 0; i < NOV; ++i) {
        const int e = tid + 512 * i, r = e / (DV / 8), c8 = (e - r * (DV / 8)) * 8;
        *reinterpret_cast<u32x4 *>(&Ol[r * SV + c8]) = ov[i];
        *reinterpret_cast<u32x4 *>(&wl[r * SV + c8]) = wv[i];
        *reinterpret_cast<u32x4 *>(&vl[r * SV + c8]) = vv[i];
    }
    {
        const int r = tid / (C / 8), c8 = (tid - r * (C / 8)) * 8;
        *reinterpret_cast<u32x4 *>(&Tl[r * SC + c8]) = tv;
    }
#pragma unroll
    for (int i = 0; i < NUT; ++i) {
        const int ti = wave + 8 * i, s = ti / NRC, ut = ti - s * NRC;
        put_tile16(dUl, SV, 16 * ut, 16 * s, duv[i], li, lg);
    }
#pragma unroll
    for (int i = 0; i < NUF; ++i) {          // fragment (column tile, token k tile) = two D tiles
        const int f = (tid >> 6) + 8 * i, ct = f / NKC, kt = f - ct * NKC;
        put_tile16(Ul, SV, 32 * kt, 16 * ct, u32x2{uf[i].x, uf[i].y}, li, lg);
        put_tile16(Ul, SV, 32 * kt + 16, 16 * ct, u32x2{uf[i].z, uf[i].w}, li, lg);
    }
    lds_barrier();

    // dQg = dO S^T, dW~ = -dU S^T (kept for phase 2)
    f32x4 dqg[TPW];
    u32x2 dwv[TPW];
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
        const int t = wave + 8 * jj, B = t / CT, ct = t - B * CT;
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1;
#pragma unroll
        for (int kt = 0; kt < NKV; ++kt) {
            const u32x4 sb = row_frag(Sl, SV, 16 * ct, 32 * kt, li, lg);
            a1 = mma_k32(row_frag(Ol, SV, 16 * B, 32 * kt, li, lg), sb, a1);
            a2 = mma_k32(row_frag(dUl, SV, 16 * B, 32 * kt, li, lg), sb, a2);
        }
        dqg[jj] = a1;
        dwv[jj] = f4_to_b16(-a2);
    }
    // dgamma_C (before exp): sum over the columns of dS' . S. The wave's dS' tiles all lie in
    // row tile wave % (d_k / 16): sum over them, then over the 16 columns of a tile.
    {
        const int rt = wave % RT;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NDT; ++i) {
            const int s = (wave + 8 * i) / RT;
            const f32x4 d4 = b16_to_f4(dsv[i]);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) acc[ii] += d4[ii] * f32of(&Sl[(16 * rt + 4 * lg + ii) * SV + 16 * s + li]);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            float x = acc[ii];
            x += __shfl_xor(x, 1);
            x += __shfl_xor(x, 2);
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
            if (li == 0) atomicAdd(&dgl[16 * rt + 4 * lg + ii], x);
        }
    }
    lds_barrier();                                  // S no longer read; U written
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
        const int ti = wave + 8 * i, s = ti / RT, rt = ti - s * RT;
        put_tile16(Sl, SV, 16 * rt, 16 * s, dsv[i], li, lg);
    }
    lds_barrier();

    // dKg = U dS'^T (kept for phase 2)
    f32x4 dkg[TPW];
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
        const int t = wave + 8 * jj, B = t / CT, ct = t - B * CT;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < NKV; ++kt)
            acc = mma_k32(row_frag(Ul, SV, 16 * B, 32 * kt, li, lg), row_frag(Sl, SV, 16 * ct, 32 * kt, li, lg), acc);
        dkg[jj] = acc;
    }
    // dM = lower(dO U^T) and dT1 = dU X^T, X = w.v (kept for phase 2)
    u32x2 dmv[2];
    f32x4 dt1[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int t = wave + 8 * q, R = t >> 2, I = t & 3;
        f32x4 am = {0.f, 0.f, 0.f, 0.f}, at = am;
#pragma unroll
        for (int kt = 0; kt < NKV; ++kt) {
            if (I <= R)
                am = mma_k32(row_frag(Ol, SV, 16 * R, 32 * kt, li, lg), row_frag(Ul, SV, 16 * I, 32 * kt, li, lg), am);
            const u32x4 xw = row_frag(wl, SV, 16 * I, 32 * kt, li, lg), xv = row_frag(vl, SV, 16 * I, 32 * kt, li, lg);
            u32x4 xb;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                xb[e] = pack_bf16x2(bf16_lo(xw[e]) * bf16_lo(xv[e]), bf16_hi(xw[e]) * bf16_hi(xv[e]));
            at = mma_k32(row_frag(dUl, SV, 16 * R, 32 * kt, li, lg), xb, at);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            if (16 * I + li > 16 * R + 4 * lg + ii) am[ii] = 0.f;
        dmv[q] = f4_to_b16(am);
        dt1[q] = at;
    }
    // dX = T^T dU, then dv = w dX and dw = v dX
#pragma unroll
    for (int jj = 0; jj < UPW; ++jj) {
        const int ct = uct0 + jj;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < NKC; ++kt)
            acc = mma_k32(col_frag(Tl, SC, 32 * kt, 16 * urt, li, lg), col_frag(dUl, SV, 32 * kt, 16 * ct, li, lg), acc);
        const int x0 = 16 * urt + 4 * lg, col = 16 * ct + li;
        const size_t o0 = (static_cast<size_t>(t0 + x0) * p.h_v + h) * DV + col;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int x = x0 + ii;
            if (x < Lr) {
                const size_t off = o0 + static_cast<size_t>(ii) * tsv;
                p.dv[off] = f32of(&wl[x * SV + col]) * acc[ii];
                p.dw[off] = f32of(&vl[x * SV + col]) * acc[ii];
            }
        }
    }
    lds_barrier();                                  // phase 1's tiles are no longer read

    // ---- phase 2 ----
    float *gl = reinterpret_cast<float *>(smem + GL::G_);
    float *tot = reinterpret_cast<float *>(smem + GL::TOT);
    bf16_t *kl = reinterpret_cast<bf16_t *>(smem + GL::K_);
    bf16_t *bl = reinterpret_cast<bf16_t *>(smem + GL::B_);
    bf16_t *ql = reinterpret_cast<bf16_t *>(smem + GL::Q_);
    bf16_t *lal = reinterpret_cast<bf16_t *>(smem + GL::LA);
    bf16_t *dWl = reinterpret_cast<bf16_t *>(smem + GL::DW);
    bf16_t *dTl = reinterpret_cast<bf16_t *>(smem + GL::DT);
    bf16_t *dMl = reinterpret_cast<bf16_t *>(smem + GL::DM);
#pragma unroll
    for (int i = 0; i < NKV8; ++i) {
        const int e = tid + 512 * i, r = e / (DK / 8), c8 = (e - r * (DK / 8)) * 8;
        *reinterpret_cast<u32x4 *>(&kl[r * SQ + c8]) = kv[i];
        *reinterpret_cast<u32x4 *>(&bl[r * SQ + c8]) = bv[i];
        *reinterpret_cast<u32x4 *>(&ql[r * SQ + c8]) = qv[i];
        *reinterpret_cast<u32x4 *>(&lal[r * SQ + c8]) = av[i];
    }
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
        const int t = wave + 8 * jj, B = t / CT, ct = t - B * CT;
        put_tile16(dWl, SK, 16 * B, 16 * ct, dwv[jj], li, lg);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int t = wave + 8 * q;
        put_tile16(dMl, SC, 16 * (t >> 2), 16 * (t & 3), dmv[q], li, lg);
    }
    lds_barrier();
    {   // g: the PARTS lanes of a channel are adjacent; exclusive prefix of the part sums
        const int gc = tid / PARTS, gpart = tid - gc * PARTS;
        float la[RP];
#pragma unroll
        for (int r = 0; r < RP; ++r) la[r] = f32of(&lal[(gpart * RP + r) * SQ + gc]);
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            run += la[r] * kLog2e;
            la[r] = run;
        }
        float pre = 0.f;
#pragma unroll
        for (int q = 0; q < PARTS - 1; ++q) {
            const float o = __shfl(run, (lane & ~(PARTS - 1)) + q);
            if (q < gpart) pre += o;
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) gl[(gpart * RP + r) * SG + gc] = la[r] + pre;
    }
    // dY = T^T dW~ (own tiles)
    f32x4 dy[TPW];
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
        const int t = wave + 8 * jj, B = t / CT, ct = t - B * CT;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < NKC; ++kt)
            acc = mma_k32(col_frag(Tl, SC, 32 * kt, 16 * B, li, lg), col_frag(dWl, SK, 32 * kt, 16 * ct, li, lg), acc);
        dy[jj] = acc;
    }
    lds_barrier();                                  // g is complete
    // dT = dU X^T + dW~ Y^T, Y = gamma . b . k built per fragment
    f32x4 tt[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int t = wave + 8 * q, R = t >> 2, I = t & 3, i = 16 * I + li;
        f32x4 acc = dt1[q];
#pragma unroll
        for (int kt = 0; kt < NKD; ++kt) {
            const u32x4 kb = row_frag(kl, SQ, 16 * I, 32 * kt, li, lg), bb = row_frag(bl, SQ, 16 * I, 32 * kt, li, lg);
            const f32x4 g0 = *reinterpret_cast<const f32x4 *>(&gl[i * SG + 32 * kt + 4 * lg]);
            const f32x4 g1 = *reinterpret_cast<const f32x4 *>(&gl[i * SG + 32 * kt + 16 + 4 * lg]);
            u32x4 yb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ga = exp2_hw(e < 2 ? g0[2 * e] : g1[2 * e - 4]);
                const float gb = exp2_hw(e < 2 ? g0[2 * e + 1] : g1[2 * e - 3]);
                yb[e] = pack_bf16x2(ga * bf16_lo(bb[e]) * bf16_lo(kb[e]), gb * bf16_hi(bb[e]) * bf16_hi(kb[e]));
            }
            acc = mma_k32(row_frag(dWl, SK, 16 * R, 32 * kt, li, lg), yb, acc);
        }
        tt[q] = acc;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int t = wave + 8 * q;
        put_tile(dTl, SC, 16 * (t >> 2), 16 * (t & 3), tt[q], li, lg);
    }
    lds_barrier();
    // Z = T^T dT
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int t = wave + 8 * q, R = t >> 2, I = t & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < NKC; ++kt)
            acc = mma_k32(col_frag(Tl, SC, 32 * kt, 16 * R, li, lg), col_frag(dTl, SC, 32 * kt, 16 * I, li, lg), acc);
        tt[q] = acc;
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int t = wave + 8 * q;
        put_tile(dTl, SC, 16 * (t >> 2), 16 * (t & 3), tt[q], li, lg);
    }
    lds_barrier();
    // dA = strictly-lower(-Z T^T)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int t = wave + 8 * q, R = t >> 2, I = t & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < NKC; ++kt)
            acc = mma_k32(row_frag(dTl, SC, 16 * R, 32 * kt, li, lg), row_frag(Tl, SC, 16 * I, 32 * kt, li, lg), acc);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[ii] = 16 * I + li < 16 * R + 4 * lg + ii ? -acc[ii] : 0.f;
        tt[q] = acc;
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int t = wave + 8 * q;
        put_tile(dTl, SC, 16 * (t >> 2), 16 * (t & 3), tt[q], li, lg);
    }
    lds_barrier();

    // The decay sums of the own tiles. All of a wave's tiles lie in channel tile wave % CT
    // (8 % CT == 0), so the factor operands are formed once per 16-row block kb, relative to
    // that block's middle row: F = k 2^(g_mid(kb) - g_i) (P1, P3), G2 = bk 2^(g_r - g_mid(kb))
    // and G4 = q 2^(g_r - g_mid(kb)) (P2, P4). A tile of row block B takes block kb's products
    // scaled by 2^(g_mid(B) - g_mid(kb)) (kb < B) or 2^(g_mid(kb) - g_mid(B)) (kb > B), both
    // <= 1 and one per channel, i.e. per lane; at kb = B the factor is 1.
    const bf16_t *dAl = dTl;
    const int cw = 16 * (wave % CT) + li;
    f32x4 A1[TPW], A2[TPW], A3[TPW], A4[TPW];
    float gmB[TPW];
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
        const int B = (wave + 8 * jj) / CT;
        gmB[jj] = gl[(16 * B + 7) * SG + cw];
        A1[jj] = A2[jj] = A3[jj] = A4[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < NRC; ++kb) {
        const float gm = gl[(16 * kb + 7) * SG + cw];
        float f[4], f2[4], f4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * kb + 4 * lg + e;
            const float gi = gl[i * SG + cw], kk = f32of(&kl[i * SQ + cw]);
            const float ex = exp2_hw(gi - gm);
            f[e] = kk * exp2_hw(gm - gi);
            f2[e] = f32of(&bl[i * SQ + cw]) * kk * ex;
            f4[e] = f32of(&ql[i * SQ + cw]) * ex;
        }
        u32x2 fh, fl, h2, l2, h4, l4;
        split4(f, fh, fl);
        split4(f2, h2, l2);
        split4(f4, h4, l4);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj) {
            const int B = (wave + 8 * jj) / CT;
            if (kb <= B) {                      // P1, P3: i in block kb
                const u32x2 d1 = *reinterpret_cast<const u32x2 *>(&dAl[(16 * B + li) * SC + 16 * kb + 4 * lg]);
                const u32x2 d3 = *reinterpret_cast<const u32x2 *>(&dMl[(16 * B + li) * SC + 16 * kb + 4 * lg]);
                if (kb == B) {
                    A1[jj] = mma_k16_bf16(d1, fl, mma_k16_bf16(d1, fh, A1[jj]));
                    A3[jj] = mma_k16_bf16(d3, fl, mma_k16_bf16(d3, fh, A3[jj]));
                } else {
                    const float sc = exp2_hw(gmB[jj] - gm);
                    A1[jj] += sc * mma_k16_bf16(d1, fl, mma_k16_bf16(d1, fh, z));
                    A3[jj] += sc * mma_k16_bf16(d3, fl, mma_k16_bf16(d3, fh, z));
                }
            }
            if (kb >= B) {                      // P2, P4: r in block kb
                const int ofs = (16 * kb + 4 * lg + (li >> 2)) * SC + 16 * B + 4 * (li & 3);
                const u32x2 d2 = lds_tr4(&dAl[ofs]);
                const u32x2 d4 = lds_tr4(&dMl[ofs]);
                if (kb == B) {
                    A2[jj] = mma_k16_bf16(d2, l2, mma_k16_bf16(d2, h2, A2[jj]));
                    A4[jj] = mma_k16_bf16(d4, l4, mma_k16_bf16(d4, h4, A4[jj]));
                } else {
                    const float sc = exp2_hw(gm - gmB[jj]);
                    A2[jj] += sc * mma_k16_bf16(d2, l2, mma_k16_bf16(d2, h2, z));
                    A4[jj] += sc * mma_k16_bf16(d4, l4, mma_k16_bf16(d4, h4, z));
                }
            }
        }
    }

    // the elementwise chain rule on the own tiles
    float dgv[TPW][4], own[TPW];
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
        const int t = wave + 8 * jj, B = t / CT, ct = t - B * CT, c = 16 * ct + li;
        const float grho = gmB[jj];
        const f32x4 a1 = A1[jj], a2 = A2[jj], a3 = A3[jj], a4 = A4[jj];
        const float gL = gl[(C - 1) * SG + c];
        float sg = 0.f, sk = 0.f;
        const int x0 = 16 * B + 4 * lg;
        const size_t okx = (static_cast<size_t>(t0 + x0) * p.h_k + hk) * DK + c;
        const size_t ogx = (static_cast<size_t>(t0 + x0) * p.h_v + h) * DK + c;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int x = x0 + ii;
            const float gx = gl[x * SG + c];
            const float f0 = exp2_hw(gx - grho), f1 = exp2_hw(grho - gx);
            const float p1 = a1[ii] * f0, p3 = a3[ii] * f0, p2 = a2[ii] * f1, p4 = a4[ii] * f1;
            const float ga = exp2_hw(gx), fk = exp2_hw(gL - gx);
            const float kk = f32of(&kl[x * SQ + c]), qq = f32of(&ql[x * SQ + c]), bb = f32of(&bl[x * SQ + c]);
            const float bk = bb * kk;
            const float dyv = dy[jj][ii], dq_ = dqg[jj][ii], dk_ = dkg[jj][ii];
            const float dbk = p1 + ga * dyv;
            const float kd = fk * kk * dk_;
            const float g_ = bk * p1 - kk * p2 + qq * p3 - kk * p4 + ga * bk * dyv + ga * qq * dq_ - kd;
            dgv[jj][ii] = g_;
            sg += g_;
            sk += kd;
            if (x < Lr) {
                const size_t ok = okx + static_cast<size_t>(ii) * tsk;
                const size_t og = ogx + static_cast<size_t>(ii) * tsg;
                const float vq = p3 + ga * dq_, vk = p4 + p2 + fk * dk_ + bb * dbk;
                if (p.group == 1) {
                    p.dq[ok] = vq;
                    p.dk[ok] = vk;
                } else {
                    atomicAdd(p.dq + ok, vq);
                    atomicAdd(p.dk + ok, vk);
                }
                p.db[og] = kk * dbk;
            }
        }
        own[jj] = sg;
        sg += __shfl_xor(sg, 16);
        sg += __shfl_xor(sg, 32);
        sk += __shfl_xor(sk, 16);
        sk += __shfl_xor(sk, 32);
        if (lg == 0) {
            tot[B * DK + c] = sg;
            tot[(NRC + B) * DK + c] = sk;
        }
    }
    lds_barrier();
    // d log alpha[x] = gamma_C dgamma_C + sum_all kd + sum_{x' >= x} dg[x']
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
        const int t = wave + 8 * jj, B = t / CT, ct = t - B * CT, c = 16 * ct + li;
        float all = 0.f, later = 0.f;
#pragma unroll
        for (int b2 = 0; b2 < NRC; ++b2) {
            all += tot[(NRC + b2) * DK + c];
            if (b2 > B) later += tot[b2 * DK + c];
        }
        const float o1 = __shfl(own[jj], li + 16), o2 = __shfl(own[jj], li + 32), o3 = __shfl(own[jj], li + 48);
        const float below = (lg < 1 ? o1 : 0.f) + (lg < 2 ? o2 : 0.f) + (lg < 3 ? o3 : 0.f);
        float acc = exp2_hw(gl[(C - 1) * SG + c]) * dgl[c] + all + later + below;
        float *dla0 = p.dla + (static_cast<size_t>(t0 + 16 * B + 4 * lg) * p.h_v + h) * DK + c;
#pragma unroll
        for (int ii = 3; ii >= 0; --ii) {
            acc += dgv[jj][ii];
            if (16 * B + 4 * lg + ii < Lr) dla0[static_cast<size_t>(ii) * tsg] = acc;
        }
    }
}


__global__ void zero2_kernel(float *a, float *b, int64_t n) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        a[i] = 0.f;
        b[i] = 0.f;
    }
}

constexpr int kChainSlices = 1;     // value slices per reverse-pass workgroup
constexpr int kSegChainSlices = 2;  // the same when the reverse pass is segmented
constexpr int64_t kRSegTargetWGs = 256;

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// Segmentation of the reverse pass: dense batches whose reverse pass would leave at least
// half of the CUs idle, in at least three segments of at least four chunks, aiming at about
// kRSegTargetWGs workgroups of kSegChainSlices slices. With nseg segments the serial depth is
// about two segments plus nseg - 2 carries instead of every chunk.
struct RSegPlan {
    int nseg, seg_len;
};
static RSegPlan rseg_plan(bool packed, int64_t pairs, int nc, int d_v) {
    const RSegPlan one{1, nc};
    const int64_t g1 = d_v / 16 / kChainSlices, g2 = d_v / 16 / kSegChainSlices;
    if (packed || pairs <= 0 || nc < 12 || 2 * pairs * g1 > kRSegTargetWGs) return one;
    int64_t G = kRSegTargetWGs / (pairs * g2);
    if (G > nc / 4) G = nc / 4;
    if (G < 3) return one;
    const int L = static_cast<int>((nc + G - 1) / G);
    const RSegPlan sp{(nc + L - 1) / L, L};
    return sp.nseg >= 3 ? sp : one;
}

// Workspace of the bf16 backward: the forward's (map, records, segment buffers), then the
// state entering every chunk and U of every chunk (bf16 fragments), T per record, the
// per-record buffers of BL16 and the reverse pass's segment buffers (B16Params).
struct B16Ws {
    size_t ck, cu, tm, crec, cout, rs, rq, rr, total;
    RSegPlan sp;
};
static B16Ws bwd16_ws(int batch, int seqlen, int num_seqs, int h_v, int d_k, int d_v, bool packed) {
    const int64_t nrec = chunk_upper_bound(C, batch, seqlen, num_seqs, packed) * h_v;
    const int64_t pairs = static_cast<int64_t>(packed ? num_seqs : batch) * h_v;
    const size_t crec = 4 * static_cast<size_t>(C) * d_k + 2 * static_cast<size_t>(C) * d_v +
                        2 * static_cast<size_t>(d_k) * d_v;
    const size_t cout = 2 * static_cast<size_t>(d_k) * d_v + 2 * static_cast<size_t>(C) * d_v;
    B16Ws w;
    w.ck = al256(chunk_workspace_bytes(C, batch, seqlen, num_seqs, h_v, d_k, d_v, true, packed));
    w.cu = al256(w.ck + static_cast<size_t>(nrec) * d_k * d_v * 2);
    w.tm = al256(w.cu + static_cast<size_t>(nrec) * C * d_v * 2);
    w.crec = al256(w.tm + static_cast<size_t>(nrec) * C * C * 2);
    w.cout = al256(w.crec + static_cast<size_t>(nrec) * crec);
    w.sp = rseg_plan(packed, pairs, (seqlen + C - 1) / C, d_v);
    const size_t nPR = w.sp.nseg > 2 ? static_cast<size_t>(w.sp.nseg - 2) : 0;
    w.rs = al256(w.cout + static_cast<size_t>(nrec) * cout);
    w.rq = al256(w.rs + (w.sp.nseg > 1 ? static_cast<size_t>(pairs) * d_k * d_v * 4 : 0));
    w.rr = al256(w.rq + static_cast<size_t>(pairs) * nPR * d_k * d_k * 4);
    w.total = w.rr + static_cast<size_t>(pairs) * nPR * d_k * d_v * 4;
    return w;
}

template <typename K>
static hipError_t set_lds(K kern, int bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int DK, int DV>
hipError_t launch_bwd16_t(const BwdArgs &a, hipStream_t st) {
    using L_ = BL16<DK, DV>;
    static_assert(L_::CREC == 4 * static_cast<size_t>(C) * DK + 2 * static_cast<size_t>(C) * DV +
                                  2 * static_cast<size_t>(DK) * DV &&
                      L_::COUT == 2 * static_cast<size_t>(DK) * DV + 2 * static_cast<size_t>(C) * DV,
                  "the per-record buffers match bwd16_ws");
    using RC = RChain<DK, DV, kChainSlices>;
    using RC2 = RChain<DK, DV, kSegChainSlices>;
    using SG = RSegLayout<DK, DV>;
    static_assert(RC::LDS <= 160 * 1024 && RC2::LDS <= 160 * 1024 && GLay<DK, DV>::LDS <= 160 * 1024, "LDS");
    const bool packed = a.cu_seqlens != nullptr;
    const int N = packed ? a.num_seqs : a.batch;
    const int64_t nrec = chunk_upper_bound(C, a.batch, a.seqlen, a.num_seqs, packed) * a.h_v;
    const B16Ws ws = bwd16_ws(a.batch, a.seqlen, a.num_seqs, a.h_v, DK, DV, packed);
    char *base = a.workspace;

    ChunkArgs f;
    f.q = a.q; f.k = a.k; f.v = a.v; f.log_alpha = a.log_alpha; f.b = a.b; f.w = a.w;
    f.S0 = a.S0; f.cu_seqlens = a.cu_seqlens; f.o = nullptr; f.S_T = nullptr;   // states only
    f.workspace = base;
    f.batch = a.batch; f.seqlen = a.seqlen; f.num_seqs = a.num_seqs;
    f.h_k = a.h_k; f.h_v = a.h_v; f.d_k = DK; f.d_v = DV; f.bf16 = true;
    f.chunk = C;
    f.fu = Fusion{};
    f.fu.cks16 = base + ws.ck;
    f.fu.cku16 = base + ws.cu;
    f.fu.bops = base + ws.crec;
    f.fu.bdo = a.dO;
    f.fu.tmat = base + ws.tm;
    f.fu.ck_in = a.ck_in;
    hipError_t e = launch_chunk_fwd(f, st);
    if (e != hipSuccess) return e;

    B16Params p;
    p.q = static_cast<const bf16_t *>(a.q); p.k = static_cast<const bf16_t *>(a.k);
    p.v = static_cast<const bf16_t *>(a.v); p.la = static_cast<const bf16_t *>(a.log_alpha);
    p.b = static_cast<const bf16_t *>(a.b); p.w = static_cast<const bf16_t *>(a.w);
    p.dO = static_cast<const bf16_t *>(a.dO);
    p.dS_T = a.dS_T;
    p.cu = a.cu_seqlens;
    p.map = packed ? reinterpret_cast<const int32_t *>(base) : nullptr;
    p.rec = base + chunk_map_bytes(a.num_seqs, packed);
    p.tmat = reinterpret_cast<const bf16_t *>(base + ws.tm);
    p.ck = reinterpret_cast<const u32x4 *>(base + ws.ck);
    p.uck = reinterpret_cast<const u32x4 *>(base + ws.cu);
    p.crec = base + ws.crec;
    p.cout = base + ws.cout;
    p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dw = a.dw; p.dla = a.dla; p.db = a.db; p.dS0 = a.dS0;
    p.num_seqs = N; p.seqlen = a.seqlen;
    p.nc_dense = (a.seqlen + C - 1) / C;
    p.h_k = a.h_k; p.h_v = a.h_v; p.group = a.h_v / a.h_k;
    p.num_pairs = N * a.h_v;
    p.nseg = ws.sp.nseg;
    p.seg_len = ws.sp.seg_len;
    p.rseg_S = p.nseg > 1 ? reinterpret_cast<float *>(base + ws.rs) : nullptr;
    p.rseg_Q = p.nseg > 2 ? reinterpret_cast<float *>(base + ws.rq) : nullptr;
    p.rseg_R = p.nseg > 2 ? reinterpret_cast<float *>(base + ws.rr) : nullptr;

    const int64_t qk = static_cast<int64_t>(a.batch) * a.seqlen * a.h_k * DK;
    if (qk > 0 && p.group > 1) {
        const int64_t blocks = (qk + 255) / 256;
        hipLaunchKernelGGL(zero2_kernel, dim3(blocks < 4096 ? blocks : 4096), dim3(256), 0, st,
                           a.dq, a.dk, qk);
    }
    if ((e = set_lds(bwd_grads16_kernel<DK, DV>, GLay<DK, DV>::LDS)) != hipSuccess) return e;
    if (p.num_pairs > 0 && p.nseg > 1) {
        // the segment pass over segments rg = 0 .. nseg - 2, then every segment with its carry
        if ((e = set_lds(bwd_rseg_kernel<DK, DV>, SG::LDS)) != hipSuccess) return e;
        if ((e = set_lds(bwd_rchain_kernel<DK, DV, kSegChainSlices>, RC2::LDS)) != hipSuccess) return e;
        const int64_t su = static_cast<int64_t>(p.num_pairs) * (p.nseg - 1);
        hipLaunchKernelGGL((bwd_rseg_kernel<DK, DV>), dim3((su + 7) / 8 * 8 * SG::GROUPS),
                           dim3(64 * (kRSegWaves + kRSegCopy)), SG::LDS, st, p);
        const int64_t units = static_cast<int64_t>(p.num_pairs) * p.nseg;
        hipLaunchKernelGGL((bwd_rchain_kernel<DK, DV, kSegChainSlices>), dim3((units + 7) / 8 * 8 * RC2::G),
                           dim3(64 * (kSegChainSlices + RC2::NCP)), RC2::LDS, st, p);
    } else if (p.num_pairs > 0) {
        if ((e = set_lds(bwd_rchain_kernel<DK, DV, kChainSlices>, RC::LDS)) != hipSuccess) return e;
        const int64_t blocks = static_cast<int64_t>((p.num_pairs + 7) / 8) * 8 * RC::G;
        hipLaunchKernelGGL((bwd_rchain_kernel<DK, DV, kChainSlices>), dim3(blocks),
                           dim3(64 * (kChainSlices + RC::NCP)), RC::LDS, st, p);
    }
    if (nrec > 0) {
        constexpr int g_lds = GLay<DK, DV>::LDS;
        hipLaunchKernelGGL((bwd_grads16_kernel<DK, DV>), dim3(nrec), dim3(512), g_lds, st, p);
    }
    return hipGetLastError();
}

}  // namespace

size_t chunk_bwd16_workspace_bytes(int batch, int seqlen, int num_seqs, int h_v, int d_k, int d_v,
                                   bool packed) {
    return bwd16_ws(batch, seqlen, num_seqs, h_v, d_k, d_v, packed).total;
}

hipError_t launch_chunk_bwd16(const BwdArgs &a, hipStream_t st) {
    if (a.d_k == 128 && a.d_v == 128) return launch_bwd16_t<128, 128>(a, st);
    if (a.d_k == 64 && a.d_v == 64) return launch_bwd16_t<64, 64>(a, st);
    if (a.d_k == 128 && a.d_v == 64) return launch_bwd16_t<128, 64>(a, st);
    if (a.d_k == 64 && a.d_v == 128) return launch_bwd16_t<64, 128>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace gdn2
