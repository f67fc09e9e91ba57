// gdn2_chunk.h -- definitions shared by the kernels of the chunked forward: the per-chunk
// record that the prep kernel writes and the state passes read, the launch parameters, and
// small device helpers.
#pragma once
#include "gdn2_common.h"
#include "gdn2_internal.h"
#include "gdn2_mfma.h"

namespace gdn2 {

template <bool BF> struct Op;
template <> struct Op<true> {     // bf16 operands, K = 32 per fragment block
    using type = bf16_t;
    using UTile = u32x2;              // one lane's part of a D-layout tile of U~ (4 x bf16)
    static constexpr int KT = 32, EPL = 8, E = 2;
};
template <> struct Op<false> {    // fp32 operands, K = 16 per fragment block
    using type = float;
    using UTile = f32x4;
    static constexpr int KT = 16, EPL = 4, E = 4;
};

// Per (chunk, value head) workspace record of a chunk of C tokens. A-operand matrices are
// stored as 1 KB fragment blocks (64 lanes x 16 B) in (row tile, k tile) order, in perm
// order (gdn2_mfma.h):
//   Wn  = -W~          [C][DK]   (state pass: U = U~ + Wn S)
//   Qg  = gamma . q     [C][DK]   (state pass: O = Qg S + M U)
//   KgT = ((gamma_C / gamma) . k)^T  [DK][C]  (state pass: S = gamma_C S + KgT U)
//   M                   [C][C]    (blocks above the diagonal are never read, except the
//                                  upper half of a k tile that straddles the diagonal,
//                                  which holds zeros)
// U~ is stored as 16x16 output tiles (D layout), column tile major (tile ct * C/16 + rt);
// gamma_C as fp32 [DK].
template <int C, int DK, int DV, bool BF>
struct Rec {
    static constexpr size_t E = Op<BF>::E;
    static constexpr size_t Wn = 0;
    static constexpr size_t Qg = Wn + static_cast<size_t>(C) * DK * E;
    static constexpr size_t KgT = Qg + static_cast<size_t>(C) * DK * E;
    static constexpr size_t M = KgT + static_cast<size_t>(DK) * C * E;
    static constexpr size_t Ut = M + static_cast<size_t>(C) * C * E;
    static constexpr size_t gC = Ut + static_cast<size_t>(C) * DV * E;
    static constexpr size_t bytes = (gC + DK * 4 + 255) / 256 * 256;
    static constexpr int NKT_DK = DK / Op<BF>::KT;     // k tiles over d_k
    static constexpr int NKT_C = C / Op<BF>::KT;       // k tiles over the chunk
    static constexpr size_t UT_TILE = 64 * 4 * E;      // one D-layout tile
};

// Per-record operands of the chunked backward's reverse state pass (64-token chunks, bf16):
//   KgA  Kg = (KgT)^T as A fragment blocks [C/16][DK/32]
//   WnT  Wn^T as A fragment blocks         [DK/16][C/32]
//   E1   M^T dO as bf16 D tiles            [DV/16 slice][C/16]
//   E2   Qg^T dO as bf16 D tiles           [DV/16 slice][DK/16]
template <int DK, int DV>
struct BwdOps {
    static constexpr size_t KgA = 0;
    static constexpr size_t WnT = KgA + static_cast<size_t>(kChunk) * DK * 2;
    static constexpr size_t E1 = WnT + static_cast<size_t>(DK) * kChunk * 2;
    static constexpr size_t E2 = E1 + static_cast<size_t>(kChunk) * DV * 2;
    static constexpr size_t bytes = E2 + static_cast<size_t>(DK) * DV * 2;
};

struct ChunkParams {
    const void *q, *k, *v, *log_alpha, *b, *w;
    const float *S0;
    const int32_t *cu;
    const int32_t *map;
    const int32_t *order;  // packed batches, state passes: sequence of each rank (longest
                           // first, chunk_map_kernel), or NULL
    void *o;
    float *S_T;
    float *S_ck;         // state entering every chunk [chunk][h_v][DK][DV], or NULL
    const float *S_in;   // with bops: the state entering every chunk, given (the layout of
                         // S_ck); the chain then only forms U, and nothing is carried
    void *S_ck16;        // the same states as bf16 B fragments, [chunk][h_v][DV/16][DK/32][64]
                         // x 16 B (64-token path, bf16 records only), or NULL
    void *U_ck16;        // U = U~ + Wn S of every chunk as bf16 B fragments, [chunk][h_v]
                         // [DV/16][C/32][64] x 16 B (same paths), or NULL
    char *bops;          // with o == NULL: the chunked backward's per-record reverse-pass
                         // operands (BwdOps), formed by the output waves, or NULL
    const void *dO;      // gradient of o, [.., h_v, DV] (with bops)
    char *rec;           // first per-(chunk, head) record
    void *tmat;          // bf16 inputs: T = (I + A)^-1 per record, [C][C] row-major, or NULL
    // Segmented state pass (dense batches with few (sequence, head) pairs): the chunks of
    // every pair are split into nseg segments of seg_len chunks that run concurrently.
    float *seg_S;        // [pair][2][DK][DV]       states entering segments 0 (copy of S0) and 1
    float *seg_P;        // [pair][nseg-2] SegPFrag transition of segments 1 .. nseg-2
    float *seg_R;        // [pair][nseg-2][DK][DV]  end state of segments 1 .. nseg-2 from 0
    int seqlen, num_seqs, h_k, h_v, group, nc_dense, num_pairs, nslices;
    int nseg, seg_len;
    int qkn;             // nonzero: q and k rows are L2-normalised in K1
    float l2eps;
    int gmode;           // GateMode: how b (and w, log_alpha) carry the gates
    int xgroup;          // prep kernel: the value heads per key head when block b maps to the
                         // record that puts a key head's G value heads on one XCD back to
                         // back (items a multiple of 8 G), else 0 (record b)
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

template <bool BF>
__device__ __forceinline__ void unpack16(u32x4 v, float *out) {
    if constexpr (BF) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            out[2 * q] = bf16_lo(v[q]);
            out[2 * q + 1] = bf16_hi(v[q]);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = __uint_as_float(v[q]);
    }
}

constexpr float kLog2e = 1.4426950408889634f;

// LDS transpose read (ds_read_b64_tr_b16). Within each 16-lane group, lane j names an 8-byte
// chunk; lane i receives element i % 4 of the chunks of lanes 4a + i / 4, a = 0..3. With
// lane j pointing at row k0 + j / 4, columns c0 + 4 (j % 4) .. + 3 of a row-major 16-bit
// tile, lane i therefore receives rows k0 .. k0 + 3 of column c0 + i: four consecutive k of
// a matrix-core operand, read from a tile stored with k as its row index.
typedef short s16x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_tr4(const void *p) {
    const s16x4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4v *)(p));
    return __builtin_bit_cast(u32x2, r);
}
// A fragment of X^T read from X stored as A fragment blocks (the record layout above; X has
// nkx k tiles): the block of X^T at row tile ry and k tile ky, i.e. lane (li, lg) receives
// X[32 ky + perm(lg, jj)][16 ry + li]. Each lane names the 8-byte run of four consecutive
// columns of X that the transposing read distributes (see lds_tr4).
__device__ __forceinline__ u32x4 frag_t(const char *x, int nkx, int ry, int ky, int li, int lg) {
    const int r = 32 * ky + 4 * lg + (li >> 2), c = 16 * ry + 4 * (li & 3);
    const int off = ((((r >> 4) * nkx + (c >> 5)) * 64 + ((c & 15) >> 2) * 16 + (r & 15)) << 4) +
                    ((c & 31) >> 4) * 8;
    const u32x2 lo = lds_tr4(x + off);
    const u32x2 hi = lds_tr4(x + off + nkx * 1024);   // rows r + 16: the next row tile of X
    return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// 2^x on the transcendental unit (the prep kernel keeps its cumulative decay in log2 units)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Record stores: non-temporal when the records cannot stay in the last-level cache until
// the state pass reads them.
template <bool NT, typename V>
__device__ __forceinline__ void st_rec(V *p, V v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// s_waitcnt with lgkmcnt(0) only
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier without a memory fence (so it never waits for outstanding loads). The
// empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Barrier for data exchanged through LDS only: this wave's LDS accesses complete, then the
// workgroup meets. Unlike __syncthreads() it does not wait for outstanding global loads and
// stores (on gfx9 a workgroup fence waits for every vector memory operation in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    wait_lds();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS (lds_dst: the wave's base address,
// lane l writes lds_dst + 16 l)
__device__ __forceinline__ void dma16(const void *src, void *lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16, 0, 0);
}

// s_waitcnt with vmcnt(0) only (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt with vmcnt(N) only: at most N vector memory loads of this wave outstanding
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

// An int in LDS, accessed with plain LDS instructions (no generic-pointer path).
typedef __attribute__((address_space(3))) volatile int lds_flag;

// Spin (bounded) until an LDS flag written by another wave of the workgroup reaches `want`.
// The writer is always able to progress, so the bound is never reached in a correct run; it
// guarantees that every wave exits. Returns false if the bound was reached: the caller then
// writes NaN in place of the outputs that depended on the flag, so a missed publication
// shows up in the results instead of passing stale operands on silently.
__device__ __forceinline__ bool wait_flag(lds_flag *flag, int want) {
    bool ok = false;
    for (int spin = 0; spin < (1 << 22); ++spin) {
        if (*flag >= want) {
            ok = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    return ok;
}

// Segment transitions P (d_k x d_k; the segmented state passes of gdn2_chunk.hip and gdn2_state.hip) as the segment pass
// writes them and the state pass reads them: matrix-core A operands, so that the product
// P S needs no transposition. Fragment (rt, kt) covers rows 16 rt .. 16 rt + 15 and one k
// tile of columns; lane li + 16 lg holds row 16 rt + li at the k slots of group lg (the perm
// order of mma_k32 for bf16 records, k = 4 lg + s for fp32 ones).
//   bf16 records: two planes hi = bf16(P) and lo = bf16(P - hi), each [RT][DK/32][64][8]
//                 bf16; P S is formed as hi S_hi + hi S_lo + lo S_hi, which keeps about 16
//                 significant bits of the fp32 operands;
//   fp32 records: one plane [RT][RT][64][4] fp32.
template <int DK, bool BF>
struct SegPFrag {
    static constexpr int RT = DK / 16, NK = BF ? DK / 32 : DK / 16;
    static constexpr size_t PLANE = static_cast<size_t>(RT) * NK * 64 * 16;   // bytes
    static constexpr size_t BYTES = BF ? 2 * PLANE : PLANE;
    static_assert(BYTES == static_cast<size_t>(DK) * DK * 4, "the size of an fp32 P");
    // stores element P[r][c]
    __device__ static void put(char *base, int r, int c, float x) {
        const int rt = r >> 4, lane = (r & 15) + 16 * ((c & 15) >> 2);
        if constexpr (BF) {
            const int kt = c >> 5, slot = 4 * ((c >> 4) & 1) + (c & 3);
            const size_t off = ((static_cast<size_t>(rt) * NK + kt) * 64 + lane) * 16 + slot * 2;
            const __bf16 hi = static_cast<__bf16>(x);
            const __bf16 lo = static_cast<__bf16>(x - static_cast<float>(hi));
            *reinterpret_cast<__bf16 *>(base + off) = hi;
            *reinterpret_cast<__bf16 *>(base + PLANE + off) = lo;
        } else {
            const int kt = c >> 4, slot = c & 3;
            const size_t off = ((static_cast<size_t>(rt) * NK + kt) * 64 + lane) * 16 + slot * 4;
            *reinterpret_cast<float *>(base + off) = x;
        }
    }
    // Stores the 16 columns 16 v .. 16 v + 15 of P that a wave holds in D layout (lane
    // (li, lg): rows 16 rt + 4 lg + ii of column 16 v + li, in S[rt][ii]). Each group of four
    // lanes transposes its 4 x 4 blocks with lane shuffles, so that every lane then holds
    // four consecutive columns of one row: one 8-byte piece per bf16 plane (or one 16-byte
    // fp32 piece) instead of four 2-byte (4-byte) element stores. Whole wave.
    __device__ static void put_slice(char *base, int v, const f32x4 (&S)[RT]) {
        const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
        const int q = li & 3, m = li >> 2;
        const int lanep = 4 * lg + q + 16 * m;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            // round d: send row (q + d) & 3, receive from lane (q - d) & 3 of the group its
            // row q, i.e. column 4 m + ((q - d) & 3) of row 4 lg + q
            float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int si = (q + d) & 3, pi = (q - d) & 3;
                const float send = si == 0 ? S[rt][0] : si == 1 ? S[rt][1] : si == 2 ? S[rt][2] : S[rt][3];
                const float recv = __shfl(send, (lane & ~3) | pi);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = pi == e ? recv : o[e];
            }
            if constexpr (BF) {
                const size_t off = ((static_cast<size_t>(rt) * NK + (v >> 1)) * 64 + lanep) * 16 + 8 * (v & 1);
                u32x2 hi, lo;
                hi.x = pack_bf16x2(o[0], o[1]);
                hi.y = pack_bf16x2(o[2], o[3]);
                lo.x = pack_bf16x2(o[0] - bf16_lo(hi.x), o[1] - bf16_hi(hi.x));
                lo.y = pack_bf16x2(o[2] - bf16_lo(hi.y), o[3] - bf16_hi(hi.y));
                *reinterpret_cast<u32x2 *>(base + off) = hi;
                *reinterpret_cast<u32x2 *>(base + PLANE + off) = lo;
            } else {
                const size_t off = ((static_cast<size_t>(rt) * NK + v) * 64 + lanep) * 16;
                *reinterpret_cast<f32x4 *>(base + off) = f32x4{o[0], o[1], o[2], o[3]};
            }
        }
    }
    // Row tiles R0 .. R0 + RT/2 - 1 of P S + R, for the 16 columns of S a wave holds in D
    // layout (lane: rows 16 rt + 4 lg + ii of its column), written over those tiles of S and
    // into the exchange `xch` ([rt][lane]); P staged in LDS at `pl`, R (these tiles) in D
    // layout. The fragments of the next row tile are read while the products of one run.
    template <int R0>
    __device__ static void carry_half(const char *pl, const f32x4 (&R)[RT / 2], f32x4 (&S)[RT],
                                      f32x4 *xch) {
        constexpr int H = RT / 2;
        const int lane = threadIdx.x & 63;
        // this lane's LDS address in the staged P, kept opaque so that the compiler folds only
        // the fragment offsets (< 64 KB) into the LDS instructions instead of keeping one
        // address register per fragment
        uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                            (__attribute__((address_space(3))) const char *)pl)) + lane * 16;
        asm volatile("" : "+v"(base));
        auto frag = [&](uint32_t off) {
            return *(__attribute__((address_space(3))) const u32x4 *)(static_cast<uintptr_t>(base + off));
        };
        f32x4 acc[H];
#pragma unroll
        for (int j = 0; j < H; ++j) acc[j] = R[j];
        if constexpr (BF) {
            u32x4 sh[NK], sl[NK];
#pragma unroll
            for (int kt = 0; kt < NK; ++kt) {
                const f32x4 a = S[2 * kt], b = S[2 * kt + 1];
                sh[kt] = dpair_to_b32(a, b);
                const f32x4 ar = {bf16_lo(sh[kt].x), bf16_hi(sh[kt].x), bf16_lo(sh[kt].y), bf16_hi(sh[kt].y)};
                const f32x4 br = {bf16_lo(sh[kt].z), bf16_hi(sh[kt].z), bf16_lo(sh[kt].w), bf16_hi(sh[kt].w)};
                sl[kt] = dpair_to_b32(a - ar, b - br);
            }
            u32x4 fh[2][NK], fl[2][NK];
#pragma unroll
            for (int kt = 0; kt < NK; ++kt) {
                fh[0][kt] = frag((R0 * NK + kt) * 1024);
                fl[0][kt] = frag(PLANE + (R0 * NK + kt) * 1024);
            }
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const int cb = j & 1, nb = cb ^ 1;
                if (j + 1 < H) {
#pragma unroll
                    for (int kt = 0; kt < NK; ++kt) {
                        fh[nb][kt] = frag(((R0 + j + 1) * NK + kt) * 1024);
                        fl[nb][kt] = frag(PLANE + ((R0 + j + 1) * NK + kt) * 1024);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kt = 0; kt < NK; ++kt) {
                    acc[j] = mma_k32(fh[cb][kt], sh[kt], acc[j]);
                    acc[j] = mma_k32(fh[cb][kt], sl[kt], acc[j]);
                    acc[j] = mma_k32(fl[cb][kt], sh[kt], acc[j]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            f32x4 f[2][NK];
#pragma unroll
            for (int kt = 0; kt < NK; ++kt) f[0][kt] = __builtin_bit_cast(f32x4, frag((R0 * NK + kt) * 1024));
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const int cb = j & 1, nb = cb ^ 1;
                if (j + 1 < H) {
#pragma unroll
                    for (int kt = 0; kt < NK; ++kt)
                        f[nb][kt] = __builtin_bit_cast(f32x4, frag(((R0 + j + 1) * NK + kt) * 1024));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kt = 0; kt < NK; ++kt) acc[j] = mma_k16_f32(f[cb][kt], S[kt], acc[j]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int j = 0; j < H; ++j) {
            S[R0 + j] = acc[j];
            xch[(R0 + j) * 64 + lane] = acc[j];
        }
    }
};

// The intra-chunk pass (gdn2_prep.hip): one record per (chunk, value head) item, for the
// chunk sizes and dims it is built for.
hipError_t launch_prep(const ChunkParams &p, int chunk, int dk, int dv, bool bf16, int64_t items,
                       hipStream_t st);
// The panel state pass (gdn2_state.hip) over the records of launch_prep, its segment pass
// (nothing to do when p.nseg == 1) and the 16-column slices per state-pass workgroup.
hipError_t launch_panel_state(const ChunkParams &p, int chunk, int dk, int dv, bool bf16,
                              hipStream_t st);
hipError_t launch_panel_seg(const ChunkParams &p, int chunk, int dk, int dv, bool bf16, hipStream_t st);
int panel_slices(int chunk, int dk, int dv, bool bf16);

}  // namespace gdn2
