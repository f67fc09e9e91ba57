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
//   K1 prep_kernel        (gdn2_prep.hip) one workgroup per (chunk, value head) record, fully
//                          parallel: the cumulative log decay, A and M on the matrix cores,
//                          T = (I + A)^{-1} by 16x16 blocks, the WY factors as tile GEMMs, and
//                          the per-chunk operands of K2, written already in matrix-core
//                          fragment order.
//   K2 chunk_state_kernel  per (sequence, value head, 16 columns of S): a chain wave that
//                          runs the recurrence over the chunks with its slice of S in fp32
//                          registers, an output wave that forms o from the operands the
//                          chain wave publishes, and loader waves that stage each chunk's
//                          operands in LDS one chunk ahead; writes o and S_T.
//
// Numerics: exp(g_r - g_i) is split into factors relative to the middle token of each
// 16-token sub-chunk (K1), so no factor spans more than 8 tokens of decay except the
// sub-chunk-to-sub-chunk factors, which are <= 1 (an underflow there means a negligible
// true product).
// Padding rows of a partial chunk are identity tokens (k = q = b = 0, w.v = 0,
// log alpha = 0), which leave the state unchanged.
#include "gdn2_chunk.h"

namespace gdn2 {

// K0: chunk offsets of a packed batch, map[n] = sum_{m<n} ceil(len_m / chunk), and the
// order in which the state pass takes the sequences: order[r] = the sequence of rank r by
// decreasing chunk count (ties by index), so that the longest chains are dispatched first
// and the short ones fill in behind them (up to kOrderSeqs sequences; more keep their own
// order). One workgroup of kMapThreads threads.
constexpr int kMapThreads = 256, kOrderSeqs = 256;
__global__ __launch_bounds__(kMapThreads) void chunk_map_kernel(const int32_t *__restrict__ cu,
                                                                int32_t *__restrict__ map,
                                                                int32_t *__restrict__ order,
                                                                int num_seqs, int chunk) {
    __shared__ int s_nc[kOrderSeqs];
    if (threadIdx.x == 0) {
        int acc = 0;
        map[0] = 0;
        for (int n = 0; n < num_seqs; ++n) {
            int len = cu[n + 1] - cu[n];
            len = len < 0 ? 0 : len;
            const int nc = (len + chunk - 1) / chunk;
            if (n < kOrderSeqs) s_nc[n] = nc;
            acc += nc;
            map[n + 1] = acc;
        }
    }
    __syncthreads();
    for (int n = threadIdx.x; n < num_seqs; n += kMapThreads) {
        int r = n;
        if (num_seqs <= kOrderSeqs) {
            const int c = s_nc[n];
            r = 0;
            for (int m = 0; m < num_seqs; ++m) r += s_nc[m] > c || (s_nc[m] == c && m < n);
        }
        order[r] = n;
    }
}

// ---------------------------------------------------------------------------------------
// K2: inter-chunk state pass. A workgroup owns NW 16-column slices of S (all d_k rows,
// fp32, in registers) of one (sequence, head, segment):
//   * per slice, a chain wave runs the recurrence U = U~ + Wn S, then
//     S = gamma_C S + KgT U. It publishes the matrix-core B operands of S (at chunk entry)
//     and of U in LDS, and sets a per-slice counter after each;
//   * per slice, an output wave computes O = Qg S + M U from those published operands as
//     they appear, off the recurrence's critical path. It turns the o tile round through
//     LDS (over the U operands it has consumed) into 16-byte rows and stores them. It
//     issues no other global access, so it never waits on those stores;
//   * copy waves load chunk c + 1's record (operands common to all columns, gamma_C, the
//     slices' U~) into the other half of a double-buffered LDS stage with direct
//     global-to-LDS loads (one wave cannot keep enough copies in flight).
// All waves meet once per chunk at a plain s_barrier (no memory fence: each wave waits for
// exactly what it produced before arriving). The workgroups of one (sequence, head,
// segment) run on one XCD, so its records are fetched into one L2. More slices per
// workgroup share one staged copy of each record: the pass is bound by how fast a CU can
// stream records into LDS.
// ---------------------------------------------------------------------------------------
template <int DK, int DV, bool BF>
struct StageLayout {
    using R_ = Rec<kChunk, DK, DV, BF>;
    static constexpr size_t E_O = BF ? 2 : 4;                // bytes per o element
    static constexpr size_t SHARED = R_::Ut;                 // Wn, Qg, KgT, M
    static constexpr size_t GCB = DK * 4;                    // gamma_C
    static constexpr size_t UTS = 4 * R_::UT_TILE;           // one slice's U~
    static constexpr size_t XS = R_::NKT_DK * 1024;          // published S operands
    static constexpr size_t XU = R_::NKT_C * 1024;           // published U operands / o tile
    static constexpr size_t XCH = XS + XU;
    static_assert(XU >= static_cast<size_t>(kChunk) * 16 * E_O, "o tile fits over U");
    __host__ __device__ static constexpr size_t buffer_bytes(int nw) {
        return SHARED + GCB + nw * UTS;
    }
    __host__ __device__ static constexpr size_t lds_bytes(int nw) {
        return 2 * buffer_bytes(nw) + nw * XCH;
    }
    static_assert(lds_bytes(1) <= 160 * 1024, "stage must fit in LDS");
};

// LDS of the segment carry in the state pass: P_g, then the exchange of the carried state
// ([slice][rt][lane] f32x4), placed after stage buffer 0 when the workgroup's LDS can grow to
// hold them there, so that the first chunk is staged into buffer 0 during the carry.
template <int DK, int DV, bool BF, int NW>
struct CarryLayout {
    using SL = StageLayout<DK, DV, BF>;
    static constexpr size_t P = SegPFrag<DK, BF>::BYTES;
    static constexpr size_t X = static_cast<size_t>(NW) * (DK / 16) * 1024;
    static constexpr bool EARLY = SL::buffer_bytes(NW) + P + X <= 159 * 1024;
    static constexpr size_t PSLOT = EARLY ? SL::buffer_bytes(NW) : 0;
    static constexpr size_t LDS = PSLOT + P + X > SL::lds_bytes(NW) ? PSLOT + P + X : SL::lds_bytes(NW);
    static_assert(LDS <= 159 * 1024, "carry fits in LDS");
};

// The backward's reverse-pass operands (BwdOps) of every chunk of a state-pass workgroup,
// formed by an output wave of the states-only pass (64-token chunks, bf16 records) from the
// staged record: E1 = M^T dO and E2 = Qg^T dO for its 16-column slice ct of dO, and its
// share of the Kg and Wn^T fragment blocks (blocks ow, ow + now, ...). The transposes come
// from transposing LDS reads of the staged fragments (frag_t); the slice of dO goes through
// the wave's own LDS area (row-major, 16 + 8 columns), prefetched a chunk ahead in registers
// (rows past the sequence as zeros). Meets the chunk barriers of the state pass.
template <int DK, int DV>
__device__ void bwd_operands(const ChunkParams &p, char *smem, size_t buf_bytes, char *own,
                             int cb, int ce, int64_t start, int64_t end, int cbase, int h, int ct,
                             int ow, int now) {
    using R_ = Rec<kChunk, DK, DV, true>;
    using BO = BwdOps<DK, DV>;
    constexpr int C = kChunk, NKD = DK / 32, NKC = C / 32, NRC = C / 16, NRK = DK / 16;
    constexpr int NF = NRC * NKD + NRK * NKC;         // Kg blocks, then Wn^T blocks
    constexpr int OS = 24;                            // row stride of the dO slice (elements)
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    bf16_t *od = reinterpret_cast<bf16_t *>(own);
    const bf16_t *dO = static_cast<const bf16_t *>(p.dO);
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    u32x4 d0 = zero4, d1 = zero4;                     // this lane's row of the next chunk's slice
    auto load = [&](int c) {
        const int64_t t0 = start + static_cast<int64_t>(c) * C;
        d0 = d1 = zero4;
        if (t0 + lane < end) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(
                dO + (static_cast<size_t>(t0 + lane) * p.h_v + h) * DV + 16 * ct);
            d0 = src[0];
            d1 = src[1];
        }
    };
    if (ce > cb) load(cb);
    for (int c = cb; c < ce; ++c) {
        const char *cur = smem + ((c - cb) & 1) * buf_bytes;
        raw_barrier();                      // chunk c is staged; chunk c-1 fully consumed
        *reinterpret_cast<u32x4 *>(&od[lane * OS]) = d0;
        *reinterpret_cast<u32x4 *>(&od[lane * OS + 8]) = d1;
        if (c + 1 < ce) load(c + 1);
        wait_lds();
        asm volatile("" ::: "memory");
        char *ob = p.bops + (static_cast<size_t>(cbase + c) * p.h_v + h) * BO::bytes;
        u32x4 db[NKC];                      // dO as B fragments: k = tokens, n = the slice
#pragma unroll
        for (int kt = 0; kt < NKC; ++kt) {
            const bf16_t *q = od + (32 * kt + 4 * lg + (li >> 2)) * OS + 4 * (li & 3);
            const u32x2 a = lds_tr4(q), b = lds_tr4(q + 16 * OS);
            db[kt] = u32x4{a.x, a.y, b.x, b.y};
        }
        u32x2 *e1 = reinterpret_cast<u32x2 *>(ob + BO::E1) + static_cast<size_t>(ct) * NRC * 64;
#pragma unroll
        for (int ut = 0; ut < NRC; ++ut) {  // E1 = M^T dO (M^T blocks of zeros skipped)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt)
                if (32 * kt + 31 >= 16 * ut) acc = mma_k32(frag_t(cur + R_::M, NKC, ut, kt, li, lg), db[kt], acc);
            e1[ut * 64 + lane] = f4_to_b16(acc);
        }
        u32x2 *e2 = reinterpret_cast<u32x2 *>(ob + BO::E2) + static_cast<size_t>(ct) * NRK * 64;
#pragma unroll
        for (int rt = 0; rt < NRK; ++rt) {  // E2 = Qg^T dO
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) acc = mma_k32(frag_t(cur + R_::Qg, NKD, rt, kt, li, lg), db[kt], acc);
            e2[rt * 64 + lane] = f4_to_b16(acc);
        }
        for (int f = ow; f < NF; f += now) {
            if (f < NRC * NKD) {            // Kg block (token tile, channel k tile)
                const int ut = f / NKD, kt = f - ut * NKD;
                reinterpret_cast<u32x4 *>(ob + BO::KgA)[f * 64 + lane] = frag_t(cur + R_::KgT, NKC, ut, kt, li, lg);
            } else {                        // Wn^T block (channel tile, token k tile)
                const int g = f - NRC * NKD, rt = g / NKC, kt = g - rt * NKC;
                reinterpret_cast<u32x4 *>(ob + BO::WnT)[g * 64 + lane] = frag_t(cur + R_::Wn, NKD, rt, kt, li, lg);
            }
        }
        wait_lds();                         // every read of chunk c's stage has completed
    }
}

// copy waves per state-pass workgroup: six, four with four slices (the register budget of
// twelve waves)
template <int NW> struct StateWaves {
    static constexpr int COPY = NW >= 4 ? 4 : 6;
    static constexpr int ALL = 2 * NW + COPY;
};

template <typename T, bool BF, int DK, int DV, int NW, bool GIVEN>
__global__ __launch_bounds__(64 * StateWaves<NW>::ALL) void chunk_state_kernel(ChunkParams p) {
    using R_ = Rec<kChunk, DK, DV, BF>;
    using SL = StageLayout<DK, DV, BF>;
    constexpr int C = kChunk, RT = DK / 16;
    constexpr int KT = Op<BF>::KT;
    constexpr int NKD = R_::NKT_DK, NKC = R_::NKT_C;
    constexpr int NCOPY = StateWaves<NW>::COPY;
    constexpr size_t BUF = SL::buffer_bytes(NW);
    static_assert(BF || NKD == RT, "fp32 operands are whole state tiles");
    static_assert(SL::lds_bytes(NW) <= 160 * 1024, "stage must fit in LDS");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    char *xch_base = smem + 2 * BUF;
    // Per-slice publication counters ([slice] S, [NW + slice] U). A static LDS array, so
    // every access is a plain LDS instruction: LDS operations of one wave complete in
    // issue order, so a counter written after the data it announces is never seen
    // ahead of that data.
    __shared__ int flags[2 * NW];

    // XCD-aware decode: the workgroups of one (pair, segment) unit share an XCD.
    const int bid = blockIdx.x, xcd = bid & 7, rest = bid >> 3;
    const int slice = rest % p.nslices;
    const int unit = (rest / p.nslices) * 8 + xcd;
    if (unit >= p.num_pairs * p.nseg) return;
    const int upair = unit / p.nseg, seg = unit - upair * p.nseg;
    // packed batches take the sequences longest first (the chunk-map kernel's order), so
    // that the short chains fill in behind the long ones
    const int pair = p.order ? p.order[upair / p.h_v] * p.h_v + upair % p.h_v : upair;
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
    // this workgroup's chunks [cb, ce) (the whole sequence when nseg == 1)
    const int cb = p.nseg > 1 ? seg * p.seg_len : 0;
    const int ce = p.nseg > 1 ? min(nchunks, cb + p.seg_len) : nchunks;
    auto record = [&](int c) {
        return p.rec + (static_cast<size_t>(cbase + c) * p.h_v + h) * R_::bytes;
    };

    const bool chain = wave < NW;
    const int sl = chain ? wave : wave - NW;             // slice within the workgroup
    const int ct = slice * NW + sl;
    const int col = 16 * ct + li;
    // copy waves (wave >= 2 NW): stage chunk c's record part into a stage buffer; chunk c
    // of the workgroup's segment uses buffer (c - cb) & 1
    const int ldr = wave - 2 * NW;
    // Without outputs (p.o == NULL: only the chunk states are wanted) Qg and M stay unstaged,
    // unless the output waves form the backward's operands (p.bops).
    const bool outputs = p.o != nullptr;
    const bool stage_qm = outputs || p.bops != nullptr;
    auto issue = [&](int c, char *dst) {
        const char *rec = record(c);
        for (int blk = ldr; blk < static_cast<int>(SL::SHARED / 1024); blk += NCOPY) {
            const size_t off = static_cast<size_t>(blk) * 1024;
            if (!stage_qm && ((off >= R_::Qg && off < R_::KgT) || off >= R_::M)) continue;
            dma16(rec + off + lane * 16, dst + off);
        }
        if (ldr == NCOPY - 1 && lane < static_cast<int>(SL::GCB / 16))
            dma16(rec + R_::gC + lane * 16, dst + SL::SHARED);
        // the slices' U~: column tiles slice*NW .. slice*NW + NW - 1 are contiguous in the
        // record, and so are their stage slots
        const char *us = rec + R_::Ut + static_cast<size_t>(slice) * NW * SL::UTS;
        char *ud = dst + SL::SHARED + SL::GCB;
        for (int b = ldr; b < static_cast<int>(NW * SL::UTS / 1024); b += NCOPY)
            dma16(us + b * 1024 + lane * 16, ud + b * 1024);
    };
    // State entering the first chunk (the chain waves hold it through the chunk loop): S0
    // (or zero) without segments; with segments, the copy of S0 (segment 0) or the state
    // entering segment 1 (copies made before this kernel, since S_T may be the S0 buffer and
    // the last segment can finish before the first one starts). Segment seg >= 2 carries
    // that state over segments 1 .. seg-1 first, S <- P_g S + R_g: the chain wave and the
    // output wave of each slice (idle until the chunk loop) form half the row tiles each and
    // swap halves through LDS, while the copy waves stage P_g and, where the LDS allows it,
    // the first chunk into buffer 0. `carry` and the step count are uniform over the
    // workgroup.
    using PF = SegPFrag<DK, BF>;
    using CL = CarryLayout<DK, DV, BF, NW>;
    constexpr int NBLK = static_cast<int>(PF::BYTES / 1024);
    constexpr int H = RT / 2;
    constexpr int CB_MIN = static_cast<int>(SL::SHARED / 1024) / NCOPY +
                           static_cast<int>(NW * SL::UTS / 1024) / NCOPY;   // see issue()
    char *pslot = smem + CL::PSLOT;
    f32x4 *xch = reinterpret_cast<f32x4 *>(pslot + PF::BYTES) + sl * RT * 64;
    // Given states (GIVEN: p.S_in, the backward's forward re-run): every chunk starts from its
    // own state, so nothing is carried and the chain waves only form U.
    constexpr bool given = GIVEN;
    const bool carry = seg >= 2 && !given;
    const bool holds = wave < 2 * NW;                     // chain and output waves
    f32x4 S[RT];
    const size_t sbase = static_cast<size_t>(pair) * DK * DV;
    auto given_state = [&](int c, f32x4 (&X)[RT]) {       // this wave's columns of S_in[chunk c]
        const float *g = p.S_in + (static_cast<size_t>(cbase + c) * p.h_v + h) * (DK * DV) + col;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) X[rt][ii] = g[static_cast<size_t>(16 * rt + 4 * lg + ii) * DV];
    };
    if (given) {
        if (chain && ce > cb) given_state(cb, S);
    } else if (carry ? holds : chain) {
        const float *Sin = p.nseg == 1 ? p.S0 : p.seg_S + (sbase << 1) + (seg > 0 ? DK * DV : 0);
        const size_t ibase = p.nseg == 1 ? sbase : 0;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                S[rt][ii] = Sin ? Sin[ibase + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col]
                                : 0.f;
    }
    auto stage_P = [&](int g) {            // copy waves
        const char *Pg = reinterpret_cast<const char *>(p.seg_P) +
                         (static_cast<size_t>(pair) * (p.nseg - 2) + g - 1) * PF::BYTES;
        for (int blk = ldr; blk < NBLK; blk += NCOPY) dma16(Pg + blk * 1024 + lane * 16, pslot + blk * 1024);
    };
    if (carry && !holds) stage_P(1);      // ahead of the first chunk, which is needed later
    if (CL::EARLY && !holds && ce > cb) issue(cb, smem);
    for (int g = 1; carry && g < seg; ++g) {
        f32x4 R[H];                         // this wave's half of R_g
        if (holds) {
            const float *Rg = p.seg_R + (static_cast<size_t>(pair) * (p.nseg - 2) + g - 1) * DK * DV;
            const int r0 = chain ? 0 : H;
#pragma unroll
            for (int j = 0; j < H; ++j)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    R[j][ii] = Rg[static_cast<size_t>(16 * (r0 + j) + 4 * lg + ii) * DV + col];
        } else if (CL::EARLY && g == 1 && ce > cb && stage_qm) {
            // P_1 has landed once no more than the first chunk's loads (issued after it; at
            // least CB_MIN per copy wave when Qg and M are staged) are outstanding
            wait_vmem_n<CB_MIN>();
        } else {
            wait_vmem();
        }
        raw_barrier();                      // P_g is staged; the last exchange has been read
        if (chain) PF::template carry_half<0>(pslot, R, S, xch);
        else if (holds) PF::template carry_half<H>(pslot, R, S, xch);
        wait_lds();
        raw_barrier();                      // every read of P_g is done; both halves written
        if (holds) {
#pragma unroll
            for (int j = 0; j < H; ++j) {   // the other wave's half
                if (chain) S[H + j] = xch[(H + j) * 64 + lane];
                else S[j] = xch[j * 64 + lane];
            }
            wait_lds();                     // read before the next step or buffer 1 refills
        } else if (g + 1 < seg) {
            stage_P(g + 1);
        }
    }

    if (wave >= 2 * NW) {
        // ---- copy waves: stage chunk c + 1 in the other buffer during chunk c
        if (!CL::EARLY && ce > cb) issue(cb, smem);
        for (int c = cb; c < ce; ++c) {
            wait_vmem();                    // this wave's copies for chunk c have landed
            raw_barrier();                  // chunk c is staged; chunk c-1 fully consumed
            if (c + 1 < ce) issue(c + 1, smem + ((c + 1 - cb) & 1) * BUF);
        }
        return;
    }

    u32x4 *xS = reinterpret_cast<u32x4 *>(xch_base + sl * SL::XCH);   // published S operands
    u32x4 *xU = xS + NKD * 64;                                         // published U operands
    lds_flag *flagS = (lds_flag *)(flags + sl);
    lds_flag *flagU = (lds_flag *)(flags + NW + sl);
    if (chain && lane == 0) {
        *flagS = 0;
        *flagU = 0;
    }
    wait_lds();

    if (chain) {
        // ---- chain wave ----
        for (int c = cb; c < ce; ++c) {
            const char *cur = smem + ((c - cb) & 1) * BUF;
            if (p.S_ck) {                   // the state entering chunk c, this wave's columns
                float *ck = p.S_ck + (static_cast<size_t>(cbase + c) * p.h_v + h) * (DK * DV);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        ck[static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] = S[rt][ii];
            }
            raw_barrier();                  // chunk c is staged; chunk c-1 fully consumed
            const u32x4 *wn = reinterpret_cast<const u32x4 *>(cur + R_::Wn);
            const u32x4 *kg = reinterpret_cast<const u32x4 *>(cur + R_::KgT);
            const float *gc = reinterpret_cast<const float *>(cur + SL::SHARED);
            const char *ut = cur + SL::SHARED + SL::GCB + sl * SL::UTS;
            // all operands of U = U~ + Wn S go in flight first
            u32x4 aw[4][NKD];
            f32x4 U[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int kt = 0; kt < NKD; ++kt) aw[rt][kt] = wn[(rt * NKD + kt) * 64 + lane];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if constexpr (BF) {
                    const u32x2 u = reinterpret_cast<const u32x2 *>(ut + rt * R_::UT_TILE)[lane];
                    U[rt] = f32x4{bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
                } else {
                    U[rt] = reinterpret_cast<const f32x4 *>(ut + rt * R_::UT_TILE)[lane];
                }
            }
            // publish S (chunk entry) as B operands, then its counter; with S_ck16 the same
            // bf16 fragments go to memory ([DV/16][DK/32][64 lanes] per record)
            u32x4 SB[NKD];
            u32x4 *ck16 = nullptr;
            if constexpr (BF) {
                if (p.S_ck16)
                    ck16 = static_cast<u32x4 *>(p.S_ck16) +
                           (static_cast<size_t>(cbase + c) * p.h_v + h) * (DK * DV / 8) +
                           static_cast<size_t>(ct) * NKD * 64;
            }
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) {
                if constexpr (BF) SB[kt] = dpair_to_b32(S[2 * kt], S[2 * kt + 1]);
                else SB[kt] = __builtin_bit_cast(u32x4, S[kt]);
                if (outputs) xS[kt * 64 + lane] = SB[kt];
                if (ck16) ck16[kt * 64 + lane] = SB[kt];
            }
            if (lane == 0) *flagS = c + 1;
            // given states: S is dead once packed; the next chunk's state is loaded into it
            // now and lands during this chunk's step
            if (given && c + 1 < ce) given_state(c + 1, S);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    if constexpr (BF) U[rt] = mma_k32(aw[rt][kt], SB[kt], U[rt]);
                    else U[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, aw[rt][kt]), S[kt], U[rt]);
                }
            __builtin_amdgcn_sched_barrier(0);
            // KgT operands and the decay of S, while the last U products drain
            u32x4 ak[RT][NKC];
            if (!given) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int kt = 0; kt < NKC; ++kt) ak[rt][kt] = kg[(rt * NKC + kt) * 64 + lane];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) S[rt] *= *reinterpret_cast<const f32x4 *>(gc + 16 * rt + 4 * lg);
            }
            // publish U as B operands, then its counter (and, with U_ck16, to memory)
            u32x4 UB[NKC];
            u32x4 *cku = nullptr;
            if constexpr (BF) {
                if (p.U_ck16)
                    cku = static_cast<u32x4 *>(p.U_ck16) +
                          (static_cast<size_t>(cbase + c) * p.h_v + h) * (C * DV / 8) +
                          static_cast<size_t>(ct) * NKC * 64;
            }
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) {
                if constexpr (BF) UB[kt] = dpair_to_b32(U[2 * kt], U[2 * kt + 1]);
                else UB[kt] = __builtin_bit_cast(u32x4, U[kt]);
                if (outputs) xU[kt * 64 + lane] = UB[kt];
                if (cku) cku[kt * 64 + lane] = UB[kt];
            }
            if (lane == 0) *flagU = c + 1;
            // S = gamma_C S + KgT U
            if (!given) {
#pragma unroll
                for (int kt = 0; kt < NKC; ++kt)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        if constexpr (BF) S[rt] = mma_k32(ak[rt][kt], UB[kt], S[rt]);
                        else S[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, ak[rt][kt]), U[kt], S[rt]);
                    }
            }
            wait_lds();                     // this chunk's LDS reads and writes are done
        }
        if (p.S_T && seg == p.nseg - 1) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    p.S_T[sbase + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] = S[rt][ii];
        }
        return;
    }

    // ---- output wave ----
    if (!outputs) {
        if constexpr (BF) {
            if (p.bops != nullptr) {
                bwd_operands<DK, DV>(p, smem, BUF, xch_base + sl * SL::XCH, cb, ce, start, end, cbase, h,
                                     ct, slice * NW + sl, p.nslices * NW);
                return;
            }
        }
        for (int c = cb; c < ce; ++c) raw_barrier();   // states only: meet the chunk barriers
        return;
    }
    for (int c = cb; c < ce; ++c) {
        const char *cur = smem + ((c - cb) & 1) * BUF;
        raw_barrier();                      // chunk c is staged; chunk c-1 fully consumed
        const u32x4 *qg = reinterpret_cast<const u32x4 *>(cur + R_::Qg);
        const u32x4 *mq = reinterpret_cast<const u32x4 *>(cur + R_::M);
        u32x4 aq[4][NKD], am[4][NKC];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) aq[rt][kt] = qg[(rt * NKD + kt) * 64 + lane];
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt)
                if (kt * KT <= 16 * rt + 15) am[rt][kt] = mq[(rt * NKC + kt) * 64 + lane];
        }
        f32x4 O[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // O = Qg S
        bool published = wait_flag(flagS, c + 1);
        u32x4 SB[NKD];
#pragma unroll
        for (int kt = 0; kt < NKD; ++kt) SB[kt] = xS[kt * 64 + lane];
#pragma unroll
        for (int kt = 0; kt < NKD; ++kt)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if constexpr (BF) O[rt] = mma_k32(aq[rt][kt], SB[kt], O[rt]);
                else O[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, aq[rt][kt]),
                                         __builtin_bit_cast(f32x4, SB[kt]), O[rt]);
            }
        // O += M U   (M is lower triangular: k tiles above the diagonal are skipped)
        published = wait_flag(flagU, c + 1) && published;
        u32x4 UB[NKC];
#pragma unroll
        for (int kt = 0; kt < NKC; ++kt) UB[kt] = xU[kt * 64 + lane];
#pragma unroll
        for (int kt = 0; kt < NKC; ++kt)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if (kt * KT > 16 * rt + 15) continue;
                if constexpr (BF) O[rt] = mma_k32(am[rt][kt], UB[kt], O[rt]);
                else O[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, am[rt][kt]),
                                         __builtin_bit_cast(f32x4, UB[kt]), O[rt]);
            }
        // o rows through LDS (over the consumed U operands, row-major [C][16]) into 16-byte
        // row pieces, stored straight to memory
        T *otile = reinterpret_cast<T *>(xU);
        if (!published) {                   // a wait ran out: NaN rows, not stale results
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) O[rt] = f32x4{NAN, NAN, NAN, NAN};
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                io<T>::st(&otile[(16 * rt + 4 * lg + ii) * 16 + li], O[rt][ii]);
        wait_lds();
        {
            constexpr int PPR = 16 * static_cast<int>(sizeof(T)) / 16;   // pieces per row
            const int64_t t0 = start + static_cast<int64_t>(c) * C;
            const int L = static_cast<int>(min<int64_t>(C, end - t0));
            T *op = static_cast<T *>(p.o);
#pragma unroll
            for (int idx = lane; idx < C * PPR; idx += 64) {
                const int row = idx / PPR, piece = idx - row * PPR;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(&otile[row * 16 + piece * (16 / sizeof(T))]);
                if (row < L)
                    *reinterpret_cast<u32x4 *>(op + (static_cast<size_t>(t0 + row) * p.h_v + h) * DV +
                                               16 * ct + piece * (16 / sizeof(T))) = v;
            }
        }
        wait_lds();                         // tile reads done before U is published again
    }
}

// ---------------------------------------------------------------------------------------
// Segmented state pass. The state recursion over chunks is affine in S:
//   S_{c+1} = (diag(gamma_C) + KgT Wn) S_c + KgT U~  =:  A_c S_c + B_c
// so over a segment of chunks S_end = P S_start + R, with P the product of the A_c and R
// the end state reached from S_start = 0. When a dense batch has too few (sequence, head)
// pairs to fill the GPU, the chunks of each pair are cut into nseg segments:
//   K2a chunk_seg_kernel   segment 0: a copy of S0 and the true end state from S0 (= state
//                          entering segment 1); segments 1 .. nseg-2: P (the chain run on the
//                          columns of the identity, without U~) and R (from zero). All
//                          segments run concurrently; only the chain is computed.
//   K2  chunk_state_kernel every segment from its start state, with outputs. The workgroups
//                          of segment g >= 2 first form S_g from the state entering segment
//                          1, S_{h+1} = P_h S_h + R_h for h = 1 .. g-1, on the matrix cores.
// ---------------------------------------------------------------------------------------
constexpr int kSegWaves = 4;   // chain waves per segment-pass workgroup
constexpr int kSegCopy = 4;    // copy waves per segment-pass workgroup

template <int DK, int DV, bool BF>
struct SegLayout {
    using R_ = Rec<kChunk, DK, DV, BF>;
    static constexpr size_t OPB = static_cast<size_t>(kChunk) * DK * Op<BF>::E;   // Wn / KgT
    static constexpr size_t KG = OPB;                       // KgT offset in a stage
    static constexpr size_t GC = 2 * OPB;                   // gamma_C
    static constexpr size_t UT = GC + DK * 4;               // U~ tiles of the R slices
    static constexpr size_t UTS = 4 * R_::UT_TILE;          // one column tile of U~
    static constexpr size_t BUF = UT + kSegWaves * UTS;
    static constexpr size_t LDS = 2 * BUF;
    static constexpr int NP = DK / 16, NR = DV / 16;        // P and R column slices
    static constexpr int NV = NP + NR;
    static constexpr int GROUPS = (NV + kSegWaves - 1) / kSegWaves;   // workgroups per unit
    static_assert(LDS <= 160 * 1024, "segment stage must fit in LDS");
    static_assert(R_::KgT - R_::Qg == OPB, "record layout");
};

template <typename T, bool BF, int DK, int DV>
__global__ __launch_bounds__(64 * (kSegWaves + kSegCopy)) void chunk_seg_kernel(ChunkParams p) {
    using R_ = Rec<kChunk, DK, DV, BF>;
    using SG = SegLayout<DK, DV, BF>;
    constexpr int RT = DK / 16;
    constexpr int NKD = R_::NKT_DK, NKC = R_::NKT_C;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;

    // unit = (pair, segment g < nseg - 1); its GROUPS workgroups share an XCD
    const int bid = blockIdx.x, xcd = bid & 7, rest = bid >> 3;
    const int grp = rest % SG::GROUPS;
    const int unit = (rest / SG::GROUPS) * 8 + xcd;
    const int nsa = p.nseg - 1;
    if (unit >= p.num_pairs * nsa) return;
    const int pair = unit / nsa, g = unit - pair * nsa;
    const int h = pair % p.h_v, n = pair / p.h_v;
    // virtual slices of this workgroup: v < NP are P columns (segments >= 1 only),
    // v >= NP are R columns
    const int v0 = grp * kSegWaves;
    const int vlo = g == 0 ? (v0 > SG::NP ? v0 : SG::NP) : v0;
    const int vhi = min(v0 + kSegWaves, SG::NV);
    if (vlo >= vhi) return;                       // uniform over the workgroup
    const int rlo = max(vlo, SG::NP) - SG::NP;     // R slices [rlo, rhi) are staged
    const int rhi = max(vhi, SG::NP) - SG::NP;

    const int cb = g * p.seg_len;
    const int ce = min(p.nc_dense, cb + p.seg_len);
    const int cbase = n * p.nc_dense;
    auto record = [&](int c) {
        return p.rec + (static_cast<size_t>(cbase + c) * p.h_v + h) * R_::bytes;
    };

    if (wave >= kSegWaves) {
        // ---- copy waves: Wn, KgT, gamma_C and the R slices' U~ of chunk c + 1
        const int ldr = wave - kSegWaves;
        auto issue = [&](int c, char *dst) {
            const char *rec = record(c);
            for (int blk = ldr; blk < static_cast<int>(SG::OPB / 1024); blk += kSegCopy) {
                dma16(rec + R_::Wn + blk * 1024 + lane * 16, dst + blk * 1024);
                dma16(rec + R_::KgT + blk * 1024 + lane * 16, dst + SG::KG + blk * 1024);
            }
            if (ldr == kSegCopy - 1 && lane < DK / 4) dma16(rec + R_::gC + lane * 16, dst + SG::GC);
            const char *us = rec + R_::Ut + static_cast<size_t>(rlo) * SG::UTS;
            for (int b = ldr; b < static_cast<int>((rhi - rlo) * SG::UTS / 1024); b += kSegCopy)
                dma16(us + b * 1024 + lane * 16, dst + SG::UT + b * 1024);
        };
        if (ce > cb) issue(cb, smem + (cb & 1) * SG::BUF);
        for (int c = cb; c < ce; ++c) {
            wait_vmem();
            raw_barrier();                  // chunk c is staged; chunk c-1 fully consumed
            if (c + 1 < ce) issue(c + 1, smem + ((c + 1) & 1) * SG::BUF);
        }
        return;
    }

    // ---- chain waves ----
    const int v = v0 + wave;
    const bool active = v >= vlo && v < vhi;
    const bool isP = v < SG::NP;
    const int col = 16 * (isP ? v : v - SG::NP) + li;
    f32x4 S[RT];
    float *segS = p.seg_S + static_cast<size_t>(pair) * 2 * DK * DV;
    const bool fromS0 = active && !isP && g == 0 && p.S0 != nullptr;   // uniform per wave
    if (fromS0) {
        const float *S0p = p.S0 + static_cast<size_t>(pair) * DK * DV + col;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                S[rt][ii] = S0p[static_cast<size_t>(16 * rt + 4 * lg + ii) * DV];
    } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                S[rt][ii] = (isP && 16 * rt + 4 * lg + ii == col) ? 1.f : 0.f;
    }
    if (active && g == 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                segS[static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] = S[rt][ii];
    }
    for (int c = cb; c < ce; ++c) {
        const char *cur = smem + (c & 1) * SG::BUF;
        raw_barrier();                      // chunk c is staged; chunk c-1 fully consumed
        if (!active) continue;
        const u32x4 *wn = reinterpret_cast<const u32x4 *>(cur);
        const u32x4 *kg = reinterpret_cast<const u32x4 *>(cur + SG::KG);
        const float *gc = reinterpret_cast<const float *>(cur + SG::GC);
        const char *ut = cur + SG::UT + (isP ? 0 : (v - SG::NP - rlo)) * SG::UTS;
        // every LDS operand of the chunk goes in flight first, in the order of use
        u32x4 aw[4][NKD], ak[RT][NKC];
        f32x4 U[4], g4[RT];
        typename Op<BF>::UTile ub[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) aw[rt][kt] = wn[(rt * NKD + kt) * 64 + lane];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)       // read for P slices too (discarded): no branch
            ub[rt] = reinterpret_cast<const typename Op<BF>::UTile *>(ut + rt * R_::UT_TILE)[lane];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kt = 0; kt < NKC; ++kt) ak[rt][kt] = kg[(rt * NKC + kt) * 64 + lane];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) g4[rt] = *reinterpret_cast<const f32x4 *>(gc + 16 * rt + 4 * lg);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 SB[NKD];
#pragma unroll
        for (int kt = 0; kt < NKD; ++kt) {
            if constexpr (BF) SB[kt] = dpair_to_b32(S[2 * kt], S[2 * kt + 1]);
            else SB[kt] = __builtin_bit_cast(u32x4, S[kt]);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if constexpr (BF) {
                U[rt] = f32x4{bf16_lo(ub[rt].x), bf16_hi(ub[rt].x), bf16_lo(ub[rt].y), bf16_hi(ub[rt].y)};
            } else {
                U[rt] = ub[rt];
            }
            if (isP) U[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kt = 0; kt < NKD; ++kt)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if constexpr (BF) U[rt] = mma_k32(aw[rt][kt], SB[kt], U[rt]);
                else U[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, aw[rt][kt]), S[kt], U[rt]);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) S[rt] *= g4[rt];
        u32x4 UB[NKC];
#pragma unroll
        for (int kt = 0; kt < NKC; ++kt) {
            if constexpr (BF) UB[kt] = dpair_to_b32(U[2 * kt], U[2 * kt + 1]);
            else UB[kt] = __builtin_bit_cast(u32x4, U[kt]);
        }
#pragma unroll
        for (int kt = 0; kt < NKC; ++kt)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if constexpr (BF) S[rt] = mma_k32(ak[rt][kt], UB[kt], S[rt]);
                else S[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, ak[rt][kt]), U[kt], S[rt]);
            }
        wait_lds();
    }
    if (!active) return;
    if (isP) {
        // P as matrix-core A operands (SegPFrag): this wave holds P[16 rt + 4 lg + ii][col]
        char *dst = reinterpret_cast<char *>(p.seg_P) +
                    (static_cast<size_t>(pair) * (nsa - 1) + g - 1) * SegPFrag<DK, BF>::BYTES;
        SegPFrag<DK, BF>::put_slice(dst, v, S);
        return;
    }
    float *dst = g == 0 ? segS + static_cast<size_t>(DK) * DV   // state entering segment 1
                        : p.seg_R + (static_cast<size_t>(pair) * (nsa - 1) + g - 1) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            dst[static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] = S[rt][ii];
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
size_t chunk_record_bytes(int chunk, int d_k, int d_v, bool bf16) {
    const size_t E = bf16 ? 2 : 4;
    const size_t C = static_cast<size_t>(chunk);
    const size_t gc = E * (3 * C * d_k + C * C + C * d_v);
    return (gc + static_cast<size_t>(d_k) * 4 + 255) / 256 * 256;
}

// ---------------------------------------------------------------------------------------
// Gated RMS norm of the outputs (burn-gdn2 "Architecture": Gated RMS Norm with a SiLU gate
// after the recurrence), in place on o after the state pass:
//     o <- o / sqrt(mean_c o_c^2 + eps) * weight * gate / (1 + exp(-gate))
// per (token, value head) row of d_v values. The state pass splits d_v over workgroups, so
// the row norm runs as its own pass: one group of DV/VEC lanes per row, 16-byte accesses.
// ---------------------------------------------------------------------------------------
template <typename T, int DV>
__global__ __launch_bounds__(256) void gated_norm_kernel(T *__restrict__ o,
                                                         const T *__restrict__ gate,
                                                         const float *__restrict__ nw, float eps,
                                                         int64_t rows) {
    constexpr int VEC = 16 / sizeof(T);    // elements per 16-byte vector
    constexpr int LPR = DV / VEC;          // lanes per row
    constexpr int RPB = 256 / LPR;         // rows per block
    static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row split");
    const int cl = threadIdx.x % LPR;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR;
    if (row >= rows) return;               // whole lane groups leave together
    const size_t off = static_cast<size_t>(row) * DV + cl * VEC;
    float x[VEC], g[VEC];
    unpack16<sizeof(T) == 2>(*reinterpret_cast<const u32x4 *>(o + off), x);
    unpack16<sizeof(T) == 2>(*reinterpret_cast<const u32x4 *>(gate + off), g);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < VEC; ++j) ss += x[j] * x[j];
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m);
    const float scale = rsqrtf(ss * (1.f / DV) + eps);
#pragma unroll
    for (int j = 0; j < VEC; ++j)
        x[j] = x[j] * scale * nw[cl * VEC + j] * (g[j] / (1.f + __expf(-g[j])));
    *reinterpret_cast<u32x4 *>(o + off) = pack16<sizeof(T) == 2>(x);
}

int64_t chunk_upper_bound(int chunk, int batch, int seqlen, int num_seqs, bool packed) {
    const int64_t per = (static_cast<int64_t>(seqlen) + chunk - 1) / chunk;
    return packed ? per + num_seqs : per * batch;
}

// chunk map [num_seqs + 1] and the state pass's sequence order [num_seqs] (chunk_map_kernel)
size_t chunk_map_bytes(int num_seqs, bool packed) {
    return packed ? (static_cast<size_t>(num_seqs + 1) * 4 + 255) / 256 * 256 +
                        (static_cast<size_t>(num_seqs) * 4 + 255) / 256 * 256
                  : 0;
}
static size_t chunk_order_offset(int num_seqs) {
    return (static_cast<size_t>(num_seqs + 1) * 4 + 255) / 256 * 256;
}

// Segmentation of the state pass: dense batches only, aiming at about kSegTargetWGs
// state-pass workgroups, with at least 4 chunks per segment.
constexpr int64_t kSegTargetWGs = 256;

struct SegPlan {
    int nseg, seg_len;
};

// 16-column slices per state-pass workgroup. Two, unless the (sequence, head) pairs alone
// give more two-slice workgroups than the target: then four, so that each staged record
// serves more columns (fp32 records leave room for one only).
static int state_slices(int d_v, bool bf16, int64_t pairs) {
    if (!bf16) return 1;
    const int ctiles = d_v / 16;
    if (ctiles % 4 == 0 && pairs * (ctiles / 2) > kSegTargetWGs) return 4;
    return ctiles % 2 == 0 ? 2 : 1;
}

// per_unit: state-pass workgroups per (sequence, head, segment) unit
static SegPlan seg_plan(bool packed, int64_t pairs, int nc, int64_t per_unit) {
    SegPlan sp{1, nc};
    if (packed || pairs <= 0 || nc < 8 || per_unit <= 0) return sp;
    int64_t G = kSegTargetWGs / (pairs * per_unit);
    if (G > nc / 4) G = nc / 4;
    if (G < 2) return sp;
    const int L = static_cast<int>((nc + G - 1) / G);
    sp.nseg = (nc + L - 1) / L;
    sp.seg_len = L;
    return sp;
}

static SegPlan chunk_seg_plan(bool packed, int64_t pairs, int nc, int d_v, bool bf16) {
    return seg_plan(packed, pairs, nc, (d_v / 16) / state_slices(d_v, bf16, pairs));
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Segment buffers: fp32 start states of segments 0 and 1 [pair][2][d_k][d_v], transitions
// [pair][nseg-2] (d_k x d_k as matrix-core fragments, 4 bytes per element) and fp32
// zero-start end states [pair][nseg-2][d_k][d_v]
static void seg_area(const SegPlan &sp, int64_t pairs, int d_k, int d_v, size_t off[3],
                     size_t *total) {
    const size_t nS = sp.nseg > 1 ? 2 : 0;
    const size_t nPR = sp.nseg > 2 ? static_cast<size_t>(sp.nseg - 2) : 0;
    off[0] = 0;
    off[1] = off[0] + align256(pairs * nS * d_k * d_v * 4);
    off[2] = off[1] + align256(pairs * nPR * d_k * d_k * 4);
    *total = off[2] + align256(pairs * nPR * d_k * d_v * 4);
}

// The 64-token path with the segmented state pass: bf16 records at any supported head dims,
// fp32 records at d_k = d_v = 64. Other chunk sizes and fp32 records at d = 128 take the
// generic path (prep kernel of gdn2_prep.hip, panel state pass of gdn2_state.hip).
static bool tuned_path(int chunk, int d_k, int d_v, bool bf16) {
    return chunk == kChunk && (bf16 || (d_k == 64 && d_v == 64));
}

// The segment plan of either path (the generic path's state pass has its own slices per
// workgroup).
static SegPlan path_seg_plan(int chunk, int d_k, int d_v, bool bf16, bool packed, int64_t pairs, int nc) {
    if (tuned_path(chunk, d_k, d_v, bf16)) return chunk_seg_plan(packed, pairs, nc, d_v, bf16);
    return seg_plan(packed, pairs, nc, (d_v / 16) / panel_slices(chunk, d_k, d_v, bf16));
}

size_t chunk_workspace_bytes(int chunk, int batch, int seqlen, int num_seqs, int h_v, int d_k,
                             int d_v, bool bf16, bool packed) {
    const int64_t nc = (static_cast<int64_t>(seqlen) + chunk - 1) / chunk;
    const int64_t pairs = static_cast<int64_t>(packed ? num_seqs : batch) * h_v;
    size_t segb = 0;
    {
        const SegPlan sp = path_seg_plan(chunk, d_k, d_v, bf16, packed, pairs, static_cast<int>(nc));
        size_t off[3];
        seg_area(sp, pairs, d_k, d_v, off, &segb);
    }
    return chunk_map_bytes(num_seqs, packed) +
           static_cast<size_t>(chunk_upper_bound(chunk, batch, seqlen, num_seqs, packed)) * h_v *
               chunk_record_bytes(chunk, d_k, d_v, bf16) +
           segb;
}

bool chunk_size_built(int chunk) { return chunk == 32 || chunk == 64 || chunk == 128; }


template <typename T, bool BF, int DK, int DV, int NW, bool GIVEN = false>
static hipError_t launch_state(ChunkParams p, int64_t units, hipStream_t st) {
    p.nslices = DV / 16 / NW;
    const size_t lds = CarryLayout<DK, DV, BF, NW>::LDS;
    auto kern = chunk_state_kernel<T, BF, DK, DV, NW, GIVEN>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const int64_t blocks = (units + 7) / 8 * 8 * p.nslices;
    if (blocks > 0)
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * StateWaves<NW>::ALL), lds, st, p);
    return hipGetLastError();
}

template <typename T, bool BF, int DK, int DV>
static hipError_t launch_chunk_t(const ChunkArgs &a, hipStream_t st) {
    static_assert(Rec<kChunk, DK, DV, BF>::bytes > 0, "");
    const bool packed = a.cu_seqlens != nullptr;
    const int N = packed ? a.num_seqs : a.batch;
    ChunkParams p{};
    p.q = a.q; p.k = a.k; p.v = a.v; p.log_alpha = a.log_alpha; p.b = a.b; p.w = a.w;
    p.S0 = a.S0; p.cu = a.cu_seqlens; p.o = a.o; p.S_T = a.S_T; p.S_ck = a.fu.cks; p.tmat = a.fu.tmat;
    p.S_ck16 = a.fu.cks16;
    p.U_ck16 = a.fu.cku16;
    p.bops = BF && a.o == nullptr ? a.fu.bops : nullptr;
    p.dO = a.fu.bdo;
    p.S_in = p.bops ? a.fu.ck_in : nullptr;
    if (a.fu.ck_in && !p.S_in) return hipErrorInvalidValue;   // given states: backward only
    const size_t mapb = chunk_map_bytes(a.num_seqs, packed);
    p.map = packed ? reinterpret_cast<const int32_t *>(a.workspace) : nullptr;
    p.order = packed ? reinterpret_cast<const int32_t *>(a.workspace + chunk_order_offset(N)) : nullptr;
    p.rec = a.workspace + mapb;
    p.seqlen = a.seqlen; p.num_seqs = N; p.h_k = a.h_k; p.h_v = a.h_v;
    p.group = a.h_v / a.h_k;
    p.nc_dense = (a.seqlen + kChunk - 1) / kChunk;
    p.num_pairs = N * a.h_v;
    p.qkn = a.fu.qk_norm ? 1 : 0;
    p.l2eps = a.fu.l2eps;
    p.gmode = a.fu.gmode;
    const int64_t nrec = chunk_upper_bound(kChunk, a.batch, a.seqlen, N, packed);
    const SegPlan sp = chunk_seg_plan(packed, p.num_pairs, p.nc_dense, DV, BF);
    p.nseg = sp.nseg;
    p.seg_len = sp.seg_len;
    {
        size_t off[3], segb;
        seg_area(sp, p.num_pairs, DK, DV, off, &segb);
        char *seg_base = p.rec + static_cast<size_t>(nrec) * a.h_v * Rec<kChunk, DK, DV, BF>::bytes;
        p.seg_S = reinterpret_cast<float *>(seg_base + off[0]);
        p.seg_P = reinterpret_cast<float *>(seg_base + off[1]);
        p.seg_R = reinterpret_cast<float *>(seg_base + off[2]);
    }
    if (packed) {
        hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(kMapThreads), 0, st, a.cu_seqlens,
                           reinterpret_cast<int32_t *>(a.workspace),
                           reinterpret_cast<int32_t *>(a.workspace + chunk_order_offset(N)), N, kChunk);
    }
    if (nrec > 0) {
        const hipError_t e = launch_prep(p, kChunk, DK, DV, BF, nrec * a.h_v, st);
        if (e != hipSuccess) return e;
    }
    const int64_t units = static_cast<int64_t>(p.num_pairs) * p.nseg;
    if (p.nseg > 1 && p.num_pairs > 0 && !p.S_in) {
        // segment pass (not needed when the state entering every chunk is given)
        using SGy = SegLayout<DK, DV, BF>;
        auto skern = chunk_seg_kernel<T, BF, DK, DV>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(skern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(SGy::LDS));
        if (e != hipSuccess) return e;
        const int64_t ua = static_cast<int64_t>(p.num_pairs) * (p.nseg - 1);
        const int64_t sblocks = (ua + 7) / 8 * 8 * SGy::GROUPS;
        hipLaunchKernelGGL(skern, dim3(sblocks), dim3(64 * (kSegWaves + kSegCopy)), SGy::LDS, st, p);
    }
    // K2: NW column slices per workgroup (each with a chain and an output wave, plus the
    // copy waves)
    hipError_t e;
    if constexpr (BF) {
        const int nw = state_slices(DV, BF, p.num_pairs);
        if (p.S_in) {
            if (nw == 4) e = launch_state<T, BF, DK, DV, 4, true>(p, units, st);
            else if (nw == 2) e = launch_state<T, BF, DK, DV, 2, true>(p, units, st);
            else e = launch_state<T, BF, DK, DV, 1, true>(p, units, st);
        } else if (nw == 4) e = launch_state<T, BF, DK, DV, 4>(p, units, st);
        else if (nw == 2) e = launch_state<T, BF, DK, DV, 2>(p, units, st);
        else e = launch_state<T, BF, DK, DV, 1>(p, units, st);
    } else {
        e = launch_state<T, BF, DK, DV, 1>(p, units, st);
    }
    if (e != hipSuccess || !a.fu.gate) return e;
    const int64_t rows = static_cast<int64_t>(a.batch) * a.seqlen * a.h_v;
    constexpr int RPB = 256 / (DV / (16 / sizeof(T)));
    if (rows > 0)
        hipLaunchKernelGGL((gated_norm_kernel<T, DV>), dim3((rows + RPB - 1) / RPB), dim3(256), 0,
                           st, static_cast<T *>(a.o), static_cast<const T *>(a.fu.gate), a.fu.nw,
                           a.fu.neps, rows);
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

// Generic path: any built chunk size, both dtypes, all head dims; the state pass walks each
// chunk in row panels and runs every (sequence, head) from its start (no segments).
static hipError_t launch_chunk_generic(const ChunkArgs &a, hipStream_t st) {
    if (a.fu.cks16 || a.fu.cku16 || a.fu.bops || a.fu.ck_in) return hipErrorInvalidValue;   // 64-token pass only
    const bool packed = a.cu_seqlens != nullptr;
    const int N = packed ? a.num_seqs : a.batch;
    const int C = a.chunk;
    ChunkParams p{};
    p.q = a.q; p.k = a.k; p.v = a.v; p.log_alpha = a.log_alpha; p.b = a.b; p.w = a.w;
    p.S0 = a.S0; p.cu = a.cu_seqlens; p.o = a.o; p.S_T = a.S_T; p.S_ck = a.fu.cks; p.tmat = a.fu.tmat;
    const size_t mapb = chunk_map_bytes(a.num_seqs, packed);
    p.map = packed ? reinterpret_cast<const int32_t *>(a.workspace) : nullptr;
    p.order = packed ? reinterpret_cast<const int32_t *>(a.workspace + chunk_order_offset(N)) : nullptr;
    p.rec = a.workspace + mapb;
    p.seqlen = a.seqlen; p.num_seqs = N; p.h_k = a.h_k; p.h_v = a.h_v;
    p.group = a.h_v / a.h_k;
    p.nc_dense = (a.seqlen + C - 1) / C;
    p.num_pairs = N * a.h_v;
    p.qkn = a.fu.qk_norm ? 1 : 0;
    p.l2eps = a.fu.l2eps;
    p.gmode = a.fu.gmode;
    const int64_t nrec = chunk_upper_bound(C, a.batch, a.seqlen, N, packed);
    const SegPlan sp = path_seg_plan(C, a.d_k, a.d_v, a.bf16, packed, p.num_pairs, p.nc_dense);
    p.nseg = sp.nseg;
    p.seg_len = sp.seg_len;
    {
        size_t off[3], segb;
        seg_area(sp, p.num_pairs, a.d_k, a.d_v, off, &segb);
        char *seg_base = p.rec + static_cast<size_t>(nrec) * a.h_v * chunk_record_bytes(C, a.d_k, a.d_v, a.bf16);
        p.seg_S = reinterpret_cast<float *>(seg_base + off[0]);
        p.seg_P = reinterpret_cast<float *>(seg_base + off[1]);
        p.seg_R = reinterpret_cast<float *>(seg_base + off[2]);
    }
    if (packed)
        hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(kMapThreads), 0, st, a.cu_seqlens,
                           reinterpret_cast<int32_t *>(a.workspace),
                           reinterpret_cast<int32_t *>(a.workspace + chunk_order_offset(N)), N, C);
    hipError_t e = launch_prep(p, C, a.d_k, a.d_v, a.bf16, nrec * a.h_v, st);
    if (e != hipSuccess) return e;
    e = launch_panel_seg(p, C, a.d_k, a.d_v, a.bf16, st);
    if (e != hipSuccess) return e;
    e = launch_panel_state(p, C, a.d_k, a.d_v, a.bf16, st);
    if (e != hipSuccess || !a.fu.gate) return e;
    const int64_t rows = static_cast<int64_t>(a.batch) * a.seqlen * a.h_v;
    if (rows <= 0) return hipSuccess;
    if (a.bf16) {
        if (a.d_v == 128) {
            constexpr int RPB = 256 / (128 / 8);
            hipLaunchKernelGGL((gated_norm_kernel<bf16_t, 128>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, st,
                               static_cast<bf16_t *>(a.o), static_cast<const bf16_t *>(a.fu.gate), a.fu.nw, a.fu.neps, rows);
        } else {
            constexpr int RPB = 256 / (64 / 8);
            hipLaunchKernelGGL((gated_norm_kernel<bf16_t, 64>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, st,
                               static_cast<bf16_t *>(a.o), static_cast<const bf16_t *>(a.fu.gate), a.fu.nw, a.fu.neps, rows);
        }
    } else {
        if (a.d_v == 128) {
            constexpr int RPB = 256 / (128 / 4);
            hipLaunchKernelGGL((gated_norm_kernel<float, 128>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, st,
                               static_cast<float *>(a.o), static_cast<const float *>(a.fu.gate), a.fu.nw, a.fu.neps, rows);
        } else {
            constexpr int RPB = 256 / (64 / 4);
            hipLaunchKernelGGL((gated_norm_kernel<float, 64>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, st,
                               static_cast<float *>(a.o), static_cast<const float *>(a.fu.gate), a.fu.nw, a.fu.neps, rows);
        }
    }
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t st) {
    if (!tuned_path(a.chunk, a.d_k, a.d_v, a.bf16)) return launch_chunk_generic(a, st);
    return a.bf16 ? launch_chunk_dt<bf16_t, true>(a, st) : launch_chunk_dt<float, false>(a, st);
}

}  // namespace gdn2
