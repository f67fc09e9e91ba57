// gdn2_state.hip -- inter-chunk state pass of the chunked WY forward for any chunk size
// (32, 64, 128) and both input dtypes at d_k, d_v in {64, 128}, on gfx950.
//
// Method: burn-gdn2 0.1.5 docs page, section "Architecture" ("Chunk WY" mode). With S the
// state entering a chunk and the chunk's record (gdn2_chunk.h):
//   U      = U~ + Wn S
//   O      = Qg S + M U
//   S_next = diag(gamma_C) S + KgT U
// The rows of U and O split into panels of PR tokens; every panel of a chunk uses the state
// entering the chunk, so
//   U_p = U~_p + Wn_p S,   O_p = Qg_p S + sum_{q <= p} M_pq U_q,   S_next = gamma_C S + sum_p KgT_p U_p
// and one panel of the record at a time is staged in LDS. This keeps the staged operands
// within LDS for 128-token chunks and for fp32 records at d = 128.
//
// A workgroup owns NW 16-column slices of S (all d_k rows, fp32 registers) of one (sequence,
// value head); per slice one chain wave runs the recurrence and one output wave forms O from
// the operands the chain wave publishes in LDS (the state's matrix-core operand once per
// chunk, each panel's U once per panel, behind LDS counters); four copy waves stage panel
// s + 1 of the record while panel s is computed (double buffering, direct global-to-LDS
// loads). All waves meet once per panel at a plain s_barrier. Dense batches with few
// (sequence, head) pairs cut every pair's chunks into segments (panel_seg_kernel below).
#include "gdn2_chunk.h"

namespace gdn2 {

template <int C, int DK, int DV, bool BF, int NW, int PR>
struct PanelLayout {
    using R_ = Rec<C, DK, DV, BF>;
    static constexpr int KT = Op<BF>::KT;
    static constexpr int NS = C / 16, P = C / PR, PRT = PR / 16;
    static constexpr int NKD = DK / KT, NKC = C / KT, NKP = PR / KT, RT = DK / 16;
    static constexpr size_t FR = 1024;                       // one fragment block
    static constexpr size_t WN = 0;                          // [PRT][NKD]
    static constexpr size_t QG = WN + PRT * NKD * FR;        // [PRT][NKD]
    static constexpr size_t KG = QG + PRT * NKD * FR;        // [RT][NKP]
    static constexpr size_t MM = KG + RT * NKP * FR;         // [PRT][NKC]
    static constexpr size_t GC = MM + PRT * NKC * FR;        // fp32 [DK]
    static constexpr size_t UT = GC + DK * 4;                // [NW][PRT] D-layout tiles of U~
    static constexpr size_t UTS = PRT * R_::UT_TILE;         // one slice's U~ tiles of a panel
    static constexpr size_t BUF = (UT + NW * UTS + 255) / 256 * 256;
    // per slice: S operands (NKD fragments), the chunk's U operands (P x NKP), the o tile
    static constexpr size_t E_O = BF ? 2 : 4;
    static constexpr size_t XS = NKD * FR, XU = P * NKP * FR, XO = PR * 16 * E_O;
    static constexpr size_t XCH = XS + XU + XO;
    static constexpr size_t LDS = 2 * BUF + NW * XCH;
    static_assert(PR % KT == 0 && C % PR == 0, "whole k tiles per panel");
};

// LDS of the segment carry: P_g and the exchange of the carried state ([slice][rt][lane]
// f32x4), after stage buffer 0 (which receives the first stage meanwhile); the workgroup's
// LDS grows to hold them where the stage buffers and exchange areas are smaller.
template <int C, int DK, int DV, bool BF, int NW, int PR>
struct PanelCarry {
    using PL = PanelLayout<C, DK, DV, BF, NW, PR>;
    static constexpr size_t P = PL::BUF;
    static constexpr size_t X = P + SegPFrag<DK, BF>::BYTES;
    static constexpr size_t END = X + static_cast<size_t>(NW) * (DK / 16) * 1024;
    static constexpr size_t LDS = END > PL::LDS ? END : PL::LDS;
    static_assert(LDS <= 160 * 1024, "carry fits in LDS");
};

template <typename T, bool BF, int C, int DK, int DV, int NW, int PR>
__global__ __launch_bounds__(64 * (2 * NW + 4)) void panel_state_kernel(ChunkParams p) {
    using R_ = Rec<C, DK, DV, BF>;
    using PL = PanelLayout<C, DK, DV, BF, NW, PR>;
    constexpr int NCOPY = 4;
    constexpr int P = PL::P, PRT = PL::PRT, NKD = PL::NKD, NKC = PL::NKC, NKP = PL::NKP,
                  RT = PL::RT, NS = PL::NS, KT = PL::KT;
    static_assert(PL::LDS <= 160 * 1024, "stage must fit in LDS");
    static_assert(BF || NKD == RT, "fp32 operands are whole state tiles");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    __shared__ int flags[2 * NW];     // per slice: chunks whose S operands are out, panels whose U are
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;

    // XCD-aware decode: the workgroups of one (sequence, head, segment) share an XCD and its
    // L2 copy of the records
    const int bid = blockIdx.x, xcd = bid & 7, rest = bid >> 3;
    const int slice = rest % p.nslices;
    const int unit = (rest / p.nslices) * 8 + xcd;
    if (unit >= p.num_pairs * p.nseg) return;
    const int upair = unit / p.nseg, seg = unit - upair * p.nseg;
    // packed batches take the sequences longest first (the chunk-map kernel's order)
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
    // this workgroup's chunks [cb, ce) (the whole sequence when nseg == 1); stage s is panel
    // s % P of chunk cb + s / P
    const int cb = p.nseg > 1 ? seg * p.seg_len : 0;
    const int ce = p.nseg > 1 ? min(nchunks, cb + p.seg_len) : nchunks;
    const int nstages = (ce - cb) * P;
    auto record = [&](int c) {
        return p.rec + (static_cast<size_t>(cbase + c) * p.h_v + h) * R_::bytes;
    };
    const bool chain = wave < NW;
    const bool holds = wave < 2 * NW;               // chain and output waves
    const int sl = chain ? wave : wave - NW;
    const int ct = slice * NW + sl;                 // this slice's 16-column tile of S
    const int col = 16 * ct + li;

    // copy waves: stage s (chunk, panel) into a stage buffer
    const int ldr = wave - 2 * NW;
    auto issue = [&](int s, char *dst) {
        const int c = cb + s / P, pn = s - (s / P) * P;
        const char *rec = record(c);
        int blk = 0;                            // running 1 KB block counter
        auto copy = [&](const char *src, char *d, size_t bytes) {
            for (size_t off = 0; off < bytes; off += 1024, ++blk) {
                if (blk % NCOPY != ldr) continue;
                const size_t rem = bytes - off;
                if (rem >= 1024 || static_cast<size_t>(lane) * 16 < rem)
                    dma16(src + off + lane * 16, d + off);
            }
        };
        copy(rec + R_::Wn + static_cast<size_t>(pn) * PRT * NKD * 1024, dst + PL::WN, PRT * NKD * 1024);
        copy(rec + R_::Qg + static_cast<size_t>(pn) * PRT * NKD * 1024, dst + PL::QG, PRT * NKD * 1024);
        for (int rt = 0; rt < RT; ++rt)
            copy(rec + R_::KgT + (static_cast<size_t>(rt) * NKC + pn * NKP) * 1024,
                 dst + PL::KG + static_cast<size_t>(rt) * NKP * 1024, NKP * 1024);
        copy(rec + R_::M + static_cast<size_t>(pn) * PRT * NKC * 1024, dst + PL::MM, PRT * NKC * 1024);
        copy(rec + R_::gC, dst + PL::GC, DK * 4);
        for (int s2 = 0; s2 < NW; ++s2)
            copy(rec + R_::Ut + (static_cast<size_t>(slice * NW + s2) * NS + pn * PRT) * R_::UT_TILE,
                 dst + PL::UT + s2 * PL::UTS, PL::UTS);
    };

    // State entering the first chunk (the chain waves hold it through the chunk loop): S0 (or
    // zero) without segments; with segments, segment 0's copy of S0 or the state entering
    // segment 1, written by panel_seg_kernel. Segment seg >= 2 carries that state over
    // segments 1 .. seg-1, S <- P_g S + R_g: the chain and the output wave of each slice form
    // half the row tiles each and swap halves through LDS, while the copy waves stage P_g
    // (after stage buffer 0, which receives the first stage meanwhile).
    using PF = SegPFrag<DK, BF>;
    using CY = PanelCarry<C, DK, DV, BF, NW, PR>;
    constexpr int H = RT / 2;
    constexpr int NBLK = static_cast<int>(PF::BYTES / 1024);
    const bool carry = p.nseg > 1 && seg >= 2;      // uniform over the workgroup
    char *pslot = smem + CY::P;
    f32x4 *xc = reinterpret_cast<f32x4 *>(smem + CY::X) + sl * RT * 64;
    const size_t sbase = static_cast<size_t>(pair) * DK * DV;
    f32x4 S[RT];
    if (carry ? holds : chain) {
        const float *Sin = p.nseg == 1 ? p.S0 : p.seg_S + (sbase << 1) + (seg > 0 ? DK * DV : 0);
        const size_t ibase = p.nseg == 1 ? sbase : 0;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                S[rt][ii] = Sin ? Sin[ibase + static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] : 0.f;
    }
    auto stage_P = [&](int g) {             // copy waves
        const char *Pg = reinterpret_cast<const char *>(p.seg_P) +
                         (static_cast<size_t>(pair) * (p.nseg - 2) + g - 1) * PF::BYTES;
        for (int blk = ldr; blk < NBLK; blk += NCOPY) dma16(Pg + blk * 1024 + lane * 16, pslot + blk * 1024);
    };
    if (!holds && nstages > 0) issue(0, smem);
    if (carry && !holds) stage_P(1);
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
        } else {
            wait_vmem();                    // P_g (and the first stage) have landed
        }
        raw_barrier();                      // P_g is staged; the last exchange has been read
        if (chain) PF::template carry_half<0>(pslot, R, S, xc);
        else if (holds) PF::template carry_half<H>(pslot, R, S, xc);
        wait_lds();
        raw_barrier();                      // every read of P_g is done; both halves written
        if (holds) {
#pragma unroll
            for (int j = 0; j < H; ++j) {   // the other wave's half
                if (chain) S[H + j] = xc[(H + j) * 64 + lane];
                else S[j] = xc[j * 64 + lane];
            }
            wait_lds();
        } else if (g + 1 < seg) {
            stage_P(g + 1);
        }
    }
    if (carry) raw_barrier();               // the exchange is read before buffer 1 and the
                                            // exchange areas below are reused

    if (wave >= 2 * NW) {
        // ---- copy waves: stage (chunk, panel) s + 1 into the other buffer during stage s ----
        for (int s = 0; s < nstages; ++s) {
            wait_vmem();                            // this wave's copies for stage s have landed
            raw_barrier();                          // stage s is staged; stage s-1 fully consumed
            if (s + 1 < nstages) issue(s + 1, smem + ((s + 1) & 1) * PL::BUF);
        }
        return;
    }

    char *xbase = smem + 2 * PL::BUF + static_cast<size_t>(sl) * PL::XCH;
    u32x4 *xS = reinterpret_cast<u32x4 *>(xbase);                 // [NKD][64]
    u32x4 *xU = reinterpret_cast<u32x4 *>(xbase + PL::XS);        // [P][NKP][64]
    T *otile = reinterpret_cast<T *>(xbase + PL::XS + PL::XU);    // [PR][16]
    lds_flag *flagS = (lds_flag *)(flags + sl);
    lds_flag *flagU = (lds_flag *)(flags + NW + sl);
    if (chain && lane == 0) {
        *flagS = 0;
        *flagU = 0;
    }
    wait_lds();

    if (chain) {
        // ---- chain wave: S (this slice's columns, all d_k rows) in D layout, fp32 ----
        u32x4 SB[NKD];
        for (int s = 0; s < nstages; ++s) {
            const int cl = s / P, c = cb + cl, pn = s - cl * P;
            const char *cur = smem + (s & 1) * PL::BUF;
            if (pn == 0 && p.S_ck) {                // the state entering chunk c, this slice
                float *ck = p.S_ck + (static_cast<size_t>(cbase + c) * p.h_v + h) * (DK * DV);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        ck[static_cast<size_t>(16 * rt + 4 * lg + ii) * DV + col] = S[rt][ii];
            }
            raw_barrier();                          // stage s is staged
            const u32x4 *wn = reinterpret_cast<const u32x4 *>(cur + PL::WN);
            const u32x4 *kg = reinterpret_cast<const u32x4 *>(cur + PL::KG);
            const char *ut = cur + PL::UT + sl * PL::UTS;
            if (pn == 0) {
                // the state entering the chunk as B operands, published for the output wave,
                // then the chunk's decay applied to the fp32 state
#pragma unroll
                for (int kt = 0; kt < NKD; ++kt) {
                    if constexpr (BF) SB[kt] = dpair_to_b32(S[2 * kt], S[2 * kt + 1]);
                    else SB[kt] = __builtin_bit_cast(u32x4, S[kt]);
                    xS[kt * 64 + lane] = SB[kt];
                }
                if (lane == 0) *flagS = cl + 1;
                const float *gc = reinterpret_cast<const float *>(cur + PL::GC);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) S[rt] *= *reinterpret_cast<const f32x4 *>(gc + 16 * rt + 4 * lg);
            }
            // U_p = U~_p + Wn_p S
            f32x4 U[PRT];
#pragma unroll
            for (int rt = 0; rt < PRT; ++rt) {
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
                for (int rt = 0; rt < PRT; ++rt) {
                    const u32x4 a = wn[(rt * NKD + kt) * 64 + lane];
                    if constexpr (BF) U[rt] = mma_k32(a, SB[kt], U[rt]);
                    else U[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a), __builtin_bit_cast(f32x4, SB[kt]), U[rt]);
                }
            // publish U_p as B operands, then S += KgT_p U_p
            u32x4 UB[NKP];
#pragma unroll
            for (int kt = 0; kt < NKP; ++kt) {
                if constexpr (BF) UB[kt] = dpair_to_b32(U[2 * kt], U[2 * kt + 1]);
                else UB[kt] = __builtin_bit_cast(u32x4, U[kt]);
                xU[(pn * NKP + kt) * 64 + lane] = UB[kt];
            }
            if (lane == 0) *flagU = s + 1;
#pragma unroll
            for (int kt = 0; kt < NKP; ++kt)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const u32x4 a = kg[(rt * NKP + kt) * 64 + lane];
                    if constexpr (BF) S[rt] = mma_k32(a, UB[kt], S[rt]);
                    else S[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a), __builtin_bit_cast(f32x4, UB[kt]), S[rt]);
                }
            wait_lds();
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
    u32x4 SB[NKD];
    bool published = true;
    T *op = static_cast<T *>(p.o);
    for (int s = 0; s < nstages; ++s) {
        const int cl = s / P, c = cb + cl, pn = s - cl * P;
        const char *cur = smem + (s & 1) * PL::BUF;
        raw_barrier();                              // stage s is staged
        const u32x4 *qg = reinterpret_cast<const u32x4 *>(cur + PL::QG);
        const u32x4 *mq = reinterpret_cast<const u32x4 *>(cur + PL::MM);
        if (pn == 0) {
            published = wait_flag(flagS, cl + 1);
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) SB[kt] = xS[kt * 64 + lane];
        }
        f32x4 O[PRT];
#pragma unroll
        for (int rt = 0; rt < PRT; ++rt) O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < NKD; ++kt)
#pragma unroll
            for (int rt = 0; rt < PRT; ++rt) {
                const u32x4 a = qg[(rt * NKD + kt) * 64 + lane];
                if constexpr (BF) O[rt] = mma_k32(a, SB[kt], O[rt]);
                else O[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a), __builtin_bit_cast(f32x4, SB[kt]), O[rt]);
            }
        // O_p += M_pq U_q over the panels q <= p (M is lower triangular: k tiles past a row
        // tile's diagonal are skipped)
        for (int q = 0; q <= pn; ++q) {
            published = wait_flag(flagU, cl * P + q + 1) && published;
#pragma unroll
            for (int ktl = 0; ktl < NKP; ++ktl) {
                const int kt = q * NKP + ktl;       // k tile of the chunk
                const u32x4 ub = xU[(q * NKP + ktl) * 64 + lane];
#pragma unroll
                for (int rt = 0; rt < PRT; ++rt) {
                    if (kt * KT > 16 * (pn * PRT + rt) + 15) continue;
                    const u32x4 a = mq[(rt * NKC + kt) * 64 + lane];
                    if constexpr (BF) O[rt] = mma_k32(a, ub, O[rt]);
                    else O[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a), __builtin_bit_cast(f32x4, ub), O[rt]);
                }
            }
        }
        if (!published) {                           // a wait ran out: NaN rows, not stale results
#pragma unroll
            for (int rt = 0; rt < PRT; ++rt) O[rt] = f32x4{NAN, NAN, NAN, NAN};
        }
        // o rows through LDS ([PR][16], row-major) into 16-byte row pieces
#pragma unroll
        for (int rt = 0; rt < PRT; ++rt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                io<T>::st(&otile[(16 * rt + 4 * lg + ii) * 16 + li], O[rt][ii]);
        wait_lds();
        {
            constexpr int PPR = 16 * static_cast<int>(sizeof(T)) / 16;   // 16-byte pieces per row
            const int64_t t0 = start + static_cast<int64_t>(c) * C + pn * PR;
            const int L = static_cast<int>(min<int64_t>(PR, end - t0));
#pragma unroll
            for (int idx = lane; idx < PR * PPR; idx += 64) {
                const int row = idx / PPR, piece = idx - row * PPR;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(&otile[row * 16 + piece * (16 / sizeof(T))]);
                if (row < L)
                    *reinterpret_cast<u32x4 *>(op + (static_cast<size_t>(t0 + row) * p.h_v + h) * DV +
                                               16 * ct + piece * (16 / sizeof(T))) = v;
            }
        }
        wait_lds();                                 // tile reads done before the next panel's stores
    }
}

// ---------------------------------------------------------------------------------------
// Segmented panel pass (dense batches with few (sequence, head) pairs), as in the 64-token
// path of gdn2_chunk.hip: the chunks of every pair are cut into nseg segments of seg_len
// chunks. panel_seg_kernel runs the chain alone for segments 0 .. nseg-2: segment 0 from
// S0 (its end state is the state entering segment 1; it also keeps a copy of S0, since
// S_T may be the S0 buffer), segments g >= 1 from zero (their end state R_g) and on the
// columns of the identity without U~ (their transition P_g, in SegPFrag form). The state
// pass then starts every segment from its own state, carrying segments g >= 2 over
// P_1 .. P_{g-1}. Both stage the records one panel at a time.
// ---------------------------------------------------------------------------------------
constexpr int kPSegWaves = 4;   // chain waves (virtual slices) per segment-pass workgroup
constexpr int kPSegCopy = 4;    // copy waves per segment-pass workgroup

template <int C, int DK, int DV, bool BF, int PR>
struct PSegLayout {
    using R_ = Rec<C, DK, DV, BF>;
    static constexpr int KT = Op<BF>::KT, NS = C / 16, P = C / PR, PRT = PR / 16;
    static constexpr int NKD = DK / KT, NKC = C / KT, NKP = PR / KT, RT = DK / 16;
    static constexpr size_t FR = 1024;
    static constexpr size_t WN = 0;                                  // [PRT][NKD] blocks
    static constexpr size_t KG = WN + PRT * NKD * FR;                // [RT][NKP] blocks
    static constexpr size_t GC = KG + RT * NKP * FR;                 // gamma_C, fp32 [DK]
    static constexpr size_t UT = GC + DK * 4;                        // [slot][PRT] U~ tiles
    static constexpr size_t UTS = PRT * R_::UT_TILE;
    static constexpr size_t BUF = (UT + kPSegWaves * UTS + 255) / 256 * 256;
    static constexpr size_t LDS = 2 * BUF;
    static constexpr int NP = DK / 16, NR = DV / 16, NV = NP + NR;   // P and R column slices
    static constexpr int GROUPS = (NV + kPSegWaves - 1) / kPSegWaves;   // workgroups per unit
    static_assert(LDS <= 160 * 1024, "segment stage must fit in LDS");
};

template <typename T, bool BF, int C, int DK, int DV, int PR>
__global__ __launch_bounds__(64 * (kPSegWaves + kPSegCopy)) void panel_seg_kernel(ChunkParams p) {
    using R_ = Rec<C, DK, DV, BF>;
    using SG = PSegLayout<C, DK, DV, BF, PR>;
    constexpr int P = SG::P, PRT = SG::PRT, NKD = SG::NKD, NKC = SG::NKC, NKP = SG::NKP,
                  RT = SG::RT, NS = SG::NS;
    static_assert(BF || NKD == RT, "fp32 operands are whole state tiles");
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
    // virtual slices of this workgroup: v < NP are P columns (segments >= 1 only), v >= NP R
    const int v0 = grp * kPSegWaves;
    const int vlo = g == 0 ? (v0 > SG::NP ? v0 : SG::NP) : v0;
    const int vhi = min(v0 + kPSegWaves, SG::NV);
    if (vlo >= vhi) return;                       // uniform over the workgroup
    const int rlo = max(vlo, SG::NP) - SG::NP;     // R slices [rlo, rhi) have their U~ staged
    const int rhi = max(vhi, SG::NP) - SG::NP;
    const int cb = g * p.seg_len;
    const int ce = min(p.nc_dense, cb + p.seg_len);
    const int nst = (ce - cb) * P;                  // panel stages
    const int cbase = n * p.nc_dense;
    auto record = [&](int c) {
        return p.rec + (static_cast<size_t>(cbase + c) * p.h_v + h) * R_::bytes;
    };

    if (wave >= kPSegWaves) {
        // ---- copy waves: stage s + 1 (panel pn of chunk c) in the other buffer during stage s
        const int ldr = wave - kPSegWaves;
        auto issue = [&](int s, char *dst) {
            const int c = cb + s / P, pn = s - (s / P) * P;
            const char *rec = record(c);
            int blk = 0;                            // running 1 KB block counter
            auto copy = [&](const char *src, char *d, size_t bytes) {
                for (size_t off = 0; off < bytes; off += 1024, ++blk) {
                    if (blk % kPSegCopy != ldr) continue;
                    const size_t rem = bytes - off;
                    if (rem >= 1024 || static_cast<size_t>(lane) * 16 < rem)
                        dma16(src + off + lane * 16, d + off);
                }
            };
            copy(rec + R_::Wn + static_cast<size_t>(pn) * PRT * NKD * 1024, dst + SG::WN, PRT * NKD * 1024);
            for (int rt = 0; rt < RT; ++rt)
                copy(rec + R_::KgT + (static_cast<size_t>(rt) * NKC + pn * NKP) * 1024,
                     dst + SG::KG + static_cast<size_t>(rt) * NKP * 1024, NKP * 1024);
            copy(rec + R_::gC, dst + SG::GC, DK * 4);
            for (int r = rlo; r < rhi; ++r)
                copy(rec + R_::Ut + (static_cast<size_t>(r) * NS + pn * PRT) * R_::UT_TILE,
                     dst + SG::UT + (r - rlo) * SG::UTS, SG::UTS);
        };
        if (nst > 0) issue(0, smem);
        for (int s = 0; s < nst; ++s) {
            wait_vmem();
            raw_barrier();                  // stage s is staged; stage s-1 fully consumed
            if (s + 1 < nst) issue(s + 1, smem + ((s + 1) & 1) * SG::BUF);
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
    u32x4 SB[NKD];
    for (int s = 0; s < nst; ++s) {
        const int pn = s - (s / P) * P;
        const char *cur = smem + (s & 1) * SG::BUF;
        raw_barrier();                      // stage s is staged; stage s-1 fully consumed
        if (!active) continue;
        const u32x4 *wn = reinterpret_cast<const u32x4 *>(cur + SG::WN);
        const u32x4 *kg = reinterpret_cast<const u32x4 *>(cur + SG::KG);
        if (pn == 0) {                      // the chunk's entry state as B operands, then its decay
#pragma unroll
            for (int kt = 0; kt < NKD; ++kt) {
                if constexpr (BF) SB[kt] = dpair_to_b32(S[2 * kt], S[2 * kt + 1]);
                else SB[kt] = __builtin_bit_cast(u32x4, S[kt]);
            }
            const float *gc = reinterpret_cast<const float *>(cur + SG::GC);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) S[rt] *= *reinterpret_cast<const f32x4 *>(gc + 16 * rt + 4 * lg);
        }
        // U_p = U~_p + Wn_p S (U~ left out for P columns)
        const char *ut = cur + SG::UT + (isP ? 0 : (v - SG::NP - rlo)) * SG::UTS;
        f32x4 U[PRT];
#pragma unroll
        for (int rt = 0; rt < PRT; ++rt) {
            if (isP) {
                U[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            } else if constexpr (BF) {
                const u32x2 u = reinterpret_cast<const u32x2 *>(ut + rt * R_::UT_TILE)[lane];
                U[rt] = f32x4{bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
            } else {
                U[rt] = reinterpret_cast<const f32x4 *>(ut + rt * R_::UT_TILE)[lane];
            }
        }
#pragma unroll
        for (int kt = 0; kt < NKD; ++kt)
#pragma unroll
            for (int rt = 0; rt < PRT; ++rt) {
                const u32x4 a = wn[(rt * NKD + kt) * 64 + lane];
                if constexpr (BF) U[rt] = mma_k32(a, SB[kt], U[rt]);
                else U[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a), __builtin_bit_cast(f32x4, SB[kt]), U[rt]);
            }
        // S += KgT_p U_p
        u32x4 UB[NKP];
#pragma unroll
        for (int kt = 0; kt < NKP; ++kt) {
            if constexpr (BF) UB[kt] = dpair_to_b32(U[2 * kt], U[2 * kt + 1]);
            else UB[kt] = __builtin_bit_cast(u32x4, U[kt]);
        }
#pragma unroll
        for (int kt = 0; kt < NKP; ++kt)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const u32x4 a = kg[(rt * NKP + kt) * 64 + lane];
                if constexpr (BF) S[rt] = mma_k32(a, UB[kt], S[rt]);
                else S[rt] = mma_k16_f32(__builtin_bit_cast(f32x4, a), __builtin_bit_cast(f32x4, UB[kt]), S[rt]);
            }
        wait_lds();
    }
    if (!active) return;
    if (isP) {
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

template <int C, int DK, int DV, bool BF> struct PanelPlan;   // slices per workgroup, panel rows
template <int C, int DK, int DV> struct PanelPlan<C, DK, DV, true> {
    static constexpr int PR = C < 64 ? C : 64;
    static constexpr int NW = PanelLayout<C, DK, DV, true, 2, PR>::LDS <= 158 * 1024 && (DV / 16) % 2 == 0 ? 2 : 1;
};
template <int C, int DK, int DV> struct PanelPlan<C, DK, DV, false> {
    static constexpr int PR = 32;
    static constexpr int NW = PanelLayout<C, DK, DV, false, 2, PR>::LDS <= 158 * 1024 && (DV / 16) % 2 == 0 ? 2 : 1;
};

template <typename T, bool BF, int C, int DK, int DV>
static hipError_t launch_panel_t(ChunkParams p, hipStream_t st) {
    constexpr int NW = PanelPlan<C, DK, DV, BF>::NW, PR = PanelPlan<C, DK, DV, BF>::PR;
    constexpr size_t LDS = PanelCarry<C, DK, DV, BF, NW, PR>::LDS;
    p.nslices = DV / 16 / NW;
    auto kern = panel_state_kernel<T, BF, C, DK, DV, NW, PR>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(LDS));
    if (e != hipSuccess) return e;
    const int64_t units = static_cast<int64_t>(p.num_pairs) * p.nseg;
    const int64_t blocks = (units + 7) / 8 * 8 * p.nslices;
    if (blocks > 0)
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * (2 * NW + 4)), LDS, st, p);
    return hipGetLastError();
}

template <typename T, bool BF, int C, int DK, int DV>
static hipError_t launch_pseg_t(const ChunkParams &p, hipStream_t st) {
    constexpr int PR = PanelPlan<C, DK, DV, BF>::PR;
    using SG = PSegLayout<C, DK, DV, BF, PR>;
    auto kern = panel_seg_kernel<T, BF, C, DK, DV, PR>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(SG::LDS));
    if (e != hipSuccess) return e;
    const int64_t ua = static_cast<int64_t>(p.num_pairs) * (p.nseg - 1);
    const int64_t blocks = (ua + 7) / 8 * 8 * SG::GROUPS;
    if (blocks > 0)
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * (kPSegWaves + kPSegCopy)), SG::LDS, st, p);
    return hipGetLastError();
}

template <typename T, bool BF, int C>
static hipError_t launch_pseg_c(const ChunkParams &p, int dk, int dv, hipStream_t st) {
    if (dk == 128 && dv == 128) return launch_pseg_t<T, BF, C, 128, 128>(p, st);
    if (dk == 64 && dv == 64) return launch_pseg_t<T, BF, C, 64, 64>(p, st);
    if (dk == 128 && dv == 64) return launch_pseg_t<T, BF, C, 128, 64>(p, st);
    if (dk == 64 && dv == 128) return launch_pseg_t<T, BF, C, 64, 128>(p, st);
    return hipErrorInvalidValue;
}

hipError_t launch_panel_seg(const ChunkParams &p, int chunk, int dk, int dv, bool bf16, hipStream_t st) {
    if (p.nseg <= 1) return hipSuccess;
    if (bf16) {
        if (chunk == 32) return launch_pseg_c<bf16_t, true, 32>(p, dk, dv, st);
        if (chunk == 64) return launch_pseg_c<bf16_t, true, 64>(p, dk, dv, st);
        if (chunk == 128) return launch_pseg_c<bf16_t, true, 128>(p, dk, dv, st);
    } else {
        if (chunk == 32) return launch_pseg_c<float, false, 32>(p, dk, dv, st);
        if (chunk == 64) return launch_pseg_c<float, false, 64>(p, dk, dv, st);
        if (chunk == 128) return launch_pseg_c<float, false, 128>(p, dk, dv, st);
    }
    return hipErrorInvalidValue;
}

template <bool BF, int C>
static int panel_nw_c(int dk, int dv) {
    if (dk == 128 && dv == 128) return PanelPlan<C, 128, 128, BF>::NW;
    if (dk == 64 && dv == 64) return PanelPlan<C, 64, 64, BF>::NW;
    if (dk == 128 && dv == 64) return PanelPlan<C, 128, 64, BF>::NW;
    return PanelPlan<C, 64, 128, BF>::NW;
}

int panel_slices(int chunk, int dk, int dv, bool bf16) {
    if (bf16) return chunk == 32 ? panel_nw_c<true, 32>(dk, dv) : chunk == 64 ? panel_nw_c<true, 64>(dk, dv)
                                                                                 : panel_nw_c<true, 128>(dk, dv);
    return chunk == 32 ? panel_nw_c<false, 32>(dk, dv) : chunk == 64 ? panel_nw_c<false, 64>(dk, dv)
                                                                       : panel_nw_c<false, 128>(dk, dv);
}

template <typename T, bool BF, int C>
static hipError_t launch_panel_c(const ChunkParams &p, int dk, int dv, hipStream_t st) {
    if (dk == 128 && dv == 128) return launch_panel_t<T, BF, C, 128, 128>(p, st);
    if (dk == 64 && dv == 64) return launch_panel_t<T, BF, C, 64, 64>(p, st);
    if (dk == 128 && dv == 64) return launch_panel_t<T, BF, C, 128, 64>(p, st);
    if (dk == 64 && dv == 128) return launch_panel_t<T, BF, C, 64, 128>(p, st);
    return hipErrorInvalidValue;
}

hipError_t launch_panel_state(const ChunkParams &p, int chunk, int dk, int dv, bool bf16,
                              hipStream_t st) {
    if (bf16) {
        if (chunk == 32) return launch_panel_c<bf16_t, true, 32>(p, dk, dv, st);
        if (chunk == 64) return launch_panel_c<bf16_t, true, 64>(p, dk, dv, st);
        if (chunk == 128) return launch_panel_c<bf16_t, true, 128>(p, dk, dv, st);
    } else {
        if (chunk == 32) return launch_panel_c<float, false, 32>(p, dk, dv, st);
        if (chunk == 64) return launch_panel_c<float, false, 64>(p, dk, dv, st);
        if (chunk == 128) return launch_panel_c<float, false, 128>(p, dk, dv, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn2
