// gdn2_decode.hip -- fused recurrent forward of Gated DeltaNet-2: T tokens per sequence
// against a persistent per-(sequence, head) state, read and written once per call.
//
// Method: burn-gdn2 0.1.5 docs page, section "Architecture" (per-token recurrence, the
// "FusedRecurrent" mode). The state update is evaluated in its rank-1 form, which is the
// definition with the erase matrix never formed:
//     S'  = diag(alpha) S                      (alpha = exp(log_alpha), key axis = rows)
//     y   = S'^T (b . k),   z = S'^T q          (two column reductions over d_k)
//     u   = w . v - y
//     S   = S' + k u^T                          (= (I - k (b.k)^T) S' + k (w.v)^T)
//     o   = S^T q = z + (k . q) u
// The llama.cpp decode notes (LocalAI mirror, section 2) describe the same fused
// read-update-write of a persistent state, with the state held in registers across the
// tokens of one call; section 4 notes that the step is bound by the traffic of the fp32
// state and names a bf16 state as a way to cut it. This kernel therefore moves each state
// through HBM exactly once per call, whatever T is, and can keep the state in bf16 (half
// the bytes).
//
// State cache: the states live in a pool of slots; sequence n uses slot idx[n] (or n when
// no index is given). A slot outside [0, num_slots) marks a padding entry: the state is not
// touched and the sequence's o rows are zero.
//
// Design for gfx950: one 256-thread workgroup per (sequence, value head) state. Thread t
// owns one 16-byte vector of adjacent columns (4 fp32 or 8 bf16) of DK / RG rows, so each
// wave instruction reads or writes whole contiguous rows. All state loads are issued
// before any arithmetic. The state stays in fp32 registers across the T tokens; the token
// vectors are staged in LDS eight tokens at a time. The column reductions run as a wave
// shuffle across row groups and then a sum over the four waves through LDS.
#include "gdn2_common.h"
#include "gdn2_internal.h"
#include "gdn2_mfma.h"

namespace gdn2 {

constexpr int kDecodeThreads = 256;   // threads per (sequence, head) state
constexpr int kTokBlock = 8;          // tokens staged in LDS at a time

// States larger than the last-level cache (MALL, 256 MB on MI355X) are written back with
// non-temporal stores: no step can find them cached, and streaming them past the cache
// measured 24 % faster for a 403 MB state. Smaller states keep ordinary stores, so that the
// next step reads them from the cache.
constexpr size_t kStreamStateBytes = static_cast<size_t>(256) << 20;

// 16-byte state vectors: 4 fp32 or 8 bf16 columns, widened to fp32 in registers.
template <typename ST> struct svec;
template <> struct svec<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void ld(const float *p, float *x) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
    template <bool NTS>
    static __device__ __forceinline__ void st(float *p, const float *x) {
        const f32x4 v = {x[0], x[1], x[2], x[3]};
        if constexpr (NTS) __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
        else *reinterpret_cast<f32x4 *>(p) = v;
    }
};
template <> struct svec<bf16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void ld(const bf16_t *p, float *x) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(v[i]);
            x[2 * i + 1] = bf16_hi(v[i]);
        }
    }
    template <bool NTS>
    static __device__ __forceinline__ void st(bf16_t *p, const float *x) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);   // RNE
        if constexpr (NTS) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
        else *reinterpret_cast<u32x4 *>(p) = v;
    }
};

template <typename T, typename ST, int DK, int DV, bool NTS>
__global__ __launch_bounds__(kDecodeThreads) void recurrent_fwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ log_alpha, const T *__restrict__ b, const T *__restrict__ w,
    ST *__restrict__ S, const int32_t *__restrict__ idx, T *__restrict__ o, int ntok,
    int num_slots, int h_k, int h_v, int group) {
    constexpr int NT = kDecodeThreads, NW = NT / 64;
    constexpr int VN = svec<ST>::N;   // columns per thread
    constexpr int CG = DV / VN;       // column groups per row
    constexpr int RG = NT / CG;       // row groups
    constexpr int RPT = DK / RG;      // rows per thread
    constexpr int TB = kTokBlock;
    static_assert(RPT >= 1 && RG * RPT == DK, "tile shape");
    static_assert(CG <= 64 && 64 % CG == 0, "a wave must hold whole row groups");

    // staged token vectors: decay, b.k, k, q (key axis) and w.v (value axis)
    __shared__ float s_a[TB][DK], s_bk[TB][DK], s_k[TB][DK], s_q[TB][DK], s_wv[TB][DV];
    __shared__ float s_red[2][NW][2 * DV + 4];

    const int pair = blockIdx.x;
    const int n = pair / h_v;
    const int h = pair - n * h_v;
    const int hk = h / group;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int wave = tid >> 6, lane = tid & 63;

    const int slot = idx ? idx[n] : n;
    if (slot < 0 || slot >= num_slots) {     // padding entry: zero o rows, state untouched
        for (int i = tid; i < ntok * DV; i += NT) {
            const int t = i / DV, c = i - t * DV;
            io<T>::st(o + ((static_cast<size_t>(n) * ntok + t) * h_v + h) * DV + c, 0.f);
        }
        return;
    }

    ST *Sp = S + (static_cast<size_t>(slot) * h_v + h) * DK * DV;
    float s[RPT][VN];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        svec<ST>::ld(Sp + static_cast<size_t>(rg + RG * i) * DV + VN * cg, s[i]);

    for (int t0 = 0; t0 < ntok; t0 += TB) {
        const int nb = min(TB, ntok - t0);
        if (t0 > 0) __syncthreads();         // the previous block's vectors are consumed
        // Token vectors of this block, widened to fp32 and staged in LDS.
        for (int i = tid; i < nb * (DK + DV); i += NT) {
            const int tt = i / (DK + DV), c = i - tt * (DK + DV);
            const size_t tok = static_cast<size_t>(n) * ntok + t0 + tt;
            if (c < DK) {
                const size_t kq_off = (tok * h_k + hk) * DK + c;
                const size_t g_off = (tok * h_v + h) * DK + c;
                const float kk = io<T>::ld(k + kq_off);
                s_k[tt][c] = kk;
                s_q[tt][c] = io<T>::ld(q + kq_off);
                s_bk[tt][c] = io<T>::ld(b + g_off) * kk;
                s_a[tt][c] = __expf(io<T>::ld(log_alpha + g_off));
            } else {
                const size_t off = (tok * h_v + h) * DV + (c - DK);
                s_wv[tt][c - DK] = io<T>::ld(w + off) * io<T>::ld(v + off);
            }
        }
        __syncthreads();

        for (int tt = 0; tt < nb; ++tt) {
            const int buf = tt & 1;
            float y[VN], z[VN];
#pragma unroll
            for (int j = 0; j < VN; ++j) y[j] = z[j] = 0.f;
            float kq = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rg + RG * i;
                const float a = s_a[tt][r], bk = s_bk[tt][r], qq = s_q[tt][r];
#pragma unroll
                for (int j = 0; j < VN; ++j) {
                    s[i][j] *= a;
                    y[j] += bk * s[i][j];
                    z[j] += qq * s[i][j];
                }
                kq += s_k[tt][r] * qq;
            }
            // Sum over the row groups held by this wave (lanes that differ by multiples of CG).
#pragma unroll
            for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
                for (int j = 0; j < VN; ++j) {
                    y[j] += __shfl_xor(y[j], off);
                    z[j] += __shfl_xor(z[j], off);
                }
                kq += __shfl_xor(kq, off);
            }
            if (lane < CG) {
#pragma unroll
                for (int j = 0; j < VN; j += 4) {
                    *reinterpret_cast<f32x4 *>(&s_red[buf][wave][VN * cg + j]) =
                        f32x4{y[j], y[j + 1], y[j + 2], y[j + 3]};
                    *reinterpret_cast<f32x4 *>(&s_red[buf][wave][DV + VN * cg + j]) =
                        f32x4{z[j], z[j + 1], z[j + 2], z[j + 3]};
                }
                if (lane == 0) s_red[buf][wave][2 * DV] = kq;
            }
            // One barrier per token: s_red is double-buffered, and a thread that writes
            // buffer buf again (two tokens later) has passed the next token's barrier, which
            // every thread reaches only after reading this token's sums.
            __syncthreads();
            float Y[VN], Z[VN];
#pragma unroll
            for (int j = 0; j < VN; ++j) Y[j] = Z[j] = 0.f;
            float KQ = 0.f;
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
#pragma unroll
                for (int j = 0; j < VN; j += 4) {
                    const f32x4 yy = *reinterpret_cast<const f32x4 *>(&s_red[buf][wv][VN * cg + j]);
                    const f32x4 zz = *reinterpret_cast<const f32x4 *>(&s_red[buf][wv][DV + VN * cg + j]);
                    Y[j] += yy.x; Y[j + 1] += yy.y; Y[j + 2] += yy.z; Y[j + 3] += yy.w;
                    Z[j] += zz.x; Z[j + 1] += zz.y; Z[j + 2] += zz.z; Z[j + 3] += zz.w;
                }
                KQ += s_red[buf][wv][2 * DV];
            }
            float u[VN];
#pragma unroll
            for (int j = 0; j < VN; ++j) u[j] = s_wv[tt][VN * cg + j] - Y[j];
            if (rg == 0) {
                T *op = o + ((static_cast<size_t>(n) * ntok + t0 + tt) * h_v + h) * DV + VN * cg;
#pragma unroll
                for (int j = 0; j < VN; j += 4)
                    io<T>::st4(op + j, f32x4{Z[j] + KQ * u[j], Z[j + 1] + KQ * u[j + 1],
                                             Z[j + 2] + KQ * u[j + 2], Z[j + 3] + KQ * u[j + 3]});
            }
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const float kk = s_k[tt][rg + RG * i];
#pragma unroll
                for (int j = 0; j < VN; ++j) s[i][j] += kk * u[j];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        svec<ST>::template st<NTS>(Sp + static_cast<size_t>(rg + RG * i) * DV + VN * cg, s[i]);
}

template <typename T, typename ST, int DK, int DV>
static hipError_t launch_recurrent_t(const DecodeArgs &a, hipStream_t st) {
    const int pairs = a.num_seqs * a.h_v;
    const size_t state_bytes = static_cast<size_t>(pairs) * DK * DV * sizeof(ST);
    auto kern = state_bytes > kStreamStateBytes ? recurrent_fwd_kernel<T, ST, DK, DV, true>
                                                : recurrent_fwd_kernel<T, ST, DK, DV, false>;
    hipLaunchKernelGGL(kern, dim3(pairs), dim3(kDecodeThreads), 0, st,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), static_cast<const T *>(a.log_alpha),
                       static_cast<const T *>(a.b), static_cast<const T *>(a.w),
                       static_cast<ST *>(a.S), a.idx, static_cast<T *>(a.o), a.ntok,
                       a.num_slots, a.h_k, a.h_v, a.h_v / a.h_k);
    return hipGetLastError();
}

template <typename T, typename ST>
static hipError_t launch_recurrent_dt(const DecodeArgs &a, hipStream_t st) {
    if (a.d_k == 128 && a.d_v == 128) return launch_recurrent_t<T, ST, 128, 128>(a, st);
    if (a.d_k == 64 && a.d_v == 64) return launch_recurrent_t<T, ST, 64, 64>(a, st);
    if (a.d_k == 128 && a.d_v == 64) return launch_recurrent_t<T, ST, 128, 64>(a, st);
    return launch_recurrent_t<T, ST, 64, 128>(a, st);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
    if (a.num_seqs == 0 || a.h_v == 0 || a.ntok == 0) return hipSuccess;
    if (a.bf16)
        return a.state_bf16 ? launch_recurrent_dt<bf16_t, bf16_t>(a, st)
                            : launch_recurrent_dt<bf16_t, float>(a, st);
    return a.state_bf16 ? launch_recurrent_dt<float, bf16_t>(a, st)
                        : launch_recurrent_dt<float, float>(a, st);
}

}  // namespace gdn2
