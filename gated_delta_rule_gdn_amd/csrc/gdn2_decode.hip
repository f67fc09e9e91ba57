// gdn2_decode.hip -- fused recurrent step of Gated DeltaNet-2 (one token per sequence).
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
// read-update-write of a persistent state and note that the step is bound by the traffic
// of the fp32 state; this kernel therefore moves each state through HBM exactly once.
//
// Design for gfx950: one 256-thread workgroup per (sequence, value head) state. Thread t
// owns 4 adjacent columns (one 16-byte vector) of DK / RG rows, so each wave instruction
// reads or writes whole contiguous rows (2 rows of 512 B at d_v = 128). All state loads are
// issued before any arithmetic to keep 256 B per thread in flight. The column reductions
// run as a wave shuffle across row groups and then a 4-way sum through LDS.
#include "gdn2_common.h"
#include "gdn2_internal.h"

namespace gdn2 {

constexpr int kDecodeThreads = 256;   // threads per (sequence, head) state

// States larger than the last-level cache (MALL, 256 MB on MI355X) are written back with
// non-temporal stores: no step can find them cached, and streaming them past the cache
// measured 24 % faster for a 403 MB state. Smaller states keep ordinary stores, so that the
// next step reads them from the cache.
constexpr size_t kStreamStateBytes = static_cast<size_t>(256) << 20;

template <typename T, int DK, int DV, bool NTS>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ log_alpha, const T *__restrict__ b, const T *__restrict__ w,
    float *__restrict__ S, T *__restrict__ o, int h_k, int h_v, int group) {
    constexpr int NT = kDecodeThreads, NW = NT / 64;
    constexpr int C4 = DV / 4;        // 16-byte column groups per row
    constexpr int RG = NT / C4;       // row groups
    constexpr int RPT = DK / RG;      // rows per thread
    static_assert(RPT >= 1 && RG * RPT == DK, "tile shape");
    static_assert(C4 <= 64 && 64 % C4 == 0, "a wave must hold whole row groups");

    __shared__ float s_a[DK], s_bk[DK], s_k[DK], s_q[DK], s_wv[DV];
    __shared__ float s_red[NW][2 * DV + 4];

    const int pair = blockIdx.x;
    const int n = pair / h_v;
    const int h = pair - n * h_v;
    const int hk = h / group;
    const int tid = threadIdx.x;
    const int cg = tid % C4;
    const int rg = tid / C4;

    float *Sp = S + static_cast<size_t>(pair) * DK * DV;
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = io<float>::ld4(Sp + static_cast<size_t>(rg + RG * i) * DV + 4 * cg);

    // Token vectors of this (sequence, head), widened to fp32 and staged in LDS.
    // (key-axis vectors on the first DK threads, w.v on the next DV, wrapping round)
    for (int i = tid; i < DK + DV; i += NT) {
        if (i < DK) {
            const size_t kq_off = (static_cast<size_t>(n) * h_k + hk) * DK + i;
            const size_t g_off = (static_cast<size_t>(n) * h_v + h) * DK + i;
            const float kk = io<T>::ld(k + kq_off);
            s_k[i] = kk;
            s_q[i] = io<T>::ld(q + kq_off);
            s_bk[i] = io<T>::ld(b + g_off) * kk;
            s_a[i] = __expf(io<T>::ld(log_alpha + g_off));
        } else {
            const size_t off = (static_cast<size_t>(n) * h_v + h) * DV + (i - DK);
            s_wv[i - DK] = io<T>::ld(w + off) * io<T>::ld(v + off);
        }
    }
    __syncthreads();

    f32x4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
    float kr[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float a = s_a[r], bk = s_bk[r], qq = s_q[r];
        kr[i] = s_k[r];
        s[i] *= a;
        y += bk * s[i];
        z += qq * s[i];
        kq += kr[i] * qq;
    }
    // Sum over the row groups held by this wave (lanes that differ by multiples of C4).
#pragma unroll
    for (int off = C4; off < 64; off <<= 1) {
        y.x += __shfl_xor(y.x, off); y.y += __shfl_xor(y.y, off);
        y.z += __shfl_xor(y.z, off); y.w += __shfl_xor(y.w, off);
        z.x += __shfl_xor(z.x, off); z.y += __shfl_xor(z.y, off);
        z.z += __shfl_xor(z.z, off); z.w += __shfl_xor(z.w, off);
        kq += __shfl_xor(kq, off);
    }
    const int wave = tid >> 6, lane = tid & 63;
    if (lane < C4) {
        *reinterpret_cast<f32x4 *>(&s_red[wave][4 * cg]) = y;
        *reinterpret_cast<f32x4 *>(&s_red[wave][DV + 4 * cg]) = z;
        if (lane == 0) s_red[wave][2 * DV] = kq;
    }
    __syncthreads();
    f32x4 Y = {0.f, 0.f, 0.f, 0.f}, Z = {0.f, 0.f, 0.f, 0.f};
    float KQ = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
        Y += *reinterpret_cast<const f32x4 *>(&s_red[wv][4 * cg]);
        Z += *reinterpret_cast<const f32x4 *>(&s_red[wv][DV + 4 * cg]);
        KQ += s_red[wv][2 * DV];
    }
    const f32x4 wv4 = *reinterpret_cast<const f32x4 *>(&s_wv[4 * cg]);
    const f32x4 u = wv4 - Y;
    if (rg == 0) {
        const f32x4 ov = Z + KQ * u;
        io<T>::st4(o + (static_cast<size_t>(n) * h_v + h) * DV + 4 * cg, ov);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        s[i] += kr[i] * u;
        f32x4 *dst = reinterpret_cast<f32x4 *>(Sp + static_cast<size_t>(rg + RG * i) * DV + 4 * cg);
        if constexpr (NTS) __builtin_nontemporal_store(s[i], dst);
        else *dst = s[i];
    }
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t st) {
    const int pairs = a.num_seqs * a.h_v;
    const size_t state_bytes = static_cast<size_t>(pairs) * DK * DV * 4;
    auto kern = state_bytes > kStreamStateBytes ? decode_step_kernel<T, DK, DV, true>
                                                : decode_step_kernel<T, DK, DV, false>;
    hipLaunchKernelGGL(kern, dim3(pairs), dim3(kDecodeThreads), 0, st,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), static_cast<const T *>(a.log_alpha),
                       static_cast<const T *>(a.b), static_cast<const T *>(a.w), a.S,
                       static_cast<T *>(a.o), a.h_k, a.h_v, a.h_v / a.h_k);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_dt(const DecodeArgs &a, hipStream_t st) {
    if (a.d_k == 128 && a.d_v == 128) return launch_decode_t<T, 128, 128>(a, st);
    if (a.d_k == 64 && a.d_v == 64) return launch_decode_t<T, 64, 64>(a, st);
    if (a.d_k == 128 && a.d_v == 64) return launch_decode_t<T, 128, 64>(a, st);
    return launch_decode_t<T, 64, 128>(a, st);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
    if (a.num_seqs == 0 || a.h_v == 0) return hipSuccess;
    return a.bf16 ? launch_decode_dt<bf16_t>(a, st) : launch_decode_dt<float>(a, st);
}

}  // namespace gdn2
