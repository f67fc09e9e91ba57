// gdn2_gates.hip -- input mappings of other gated delta-rule variants onto the GDN-2 form.
//
// The GDN-2 update (burn-gdn2 docs page, "Architecture") is
//     S_t = (I - k_t (b_t . k_t)^T) diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T,
// and the page says its channel-wise gates b_t and w_t replace the scalar gate of Kimi
// Delta Attention. The variants below are therefore GDN-2 with particular inputs:
//   KDA       scalar beta_t per (token, head):         b_t = w_t = beta_t 1
//   GDN       scalar decay and scalar beta_t:           log alpha_t broadcast over d_k,
//                                                       b_t = w_t = beta_t 1
//   FG2-GDN   vector beta_t in R^{d_k} (FG2-GDN page, section 2A): the update uses
//             k~ = sqrt(beta) . k and v~ = sqrt(beta) . v, S_t = (I - k~ k~^T) D S + k~ v~^T,
//             i.e. GDN-2 with k' = k~, v' = v~ (d_v = d_k), b = w = 1
//   FG2-GDN+  beta^k in R^{d_k} and beta^v in R^{d_v} (FG2-GDN page, section 2B: erase
//             strength through beta^k, write strength through beta^v): k' = sqrt(beta^k) . k,
//             b = 1, v' = v, w = sqrt(beta^v)
// One elementwise pass writes the GDN-2 inputs that change; the caller then runs the
// regular GDN-2 calls on them. The backward of a mapping is its chain rule, again
// elementwise: gradients of b and w (and of a broadcast log alpha) sum over the channels;
// d sqrt(beta) / d beta = 1 / (2 sqrt(beta)). Because k' depends on the value head in the FG2 modes, those
// modes write k' (and q, when value heads share key heads) per value head.
#include "gdn2_common.h"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
    static constexpr int N = 4;
    __device__ static void load(const float *p, float (&x)[4]) {
        const float4 v = *reinterpret_cast<const float4 *>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
    __device__ static void store(float *p, const float (&x)[4]) {
        *reinterpret_cast<float4 *>(p) = float4{x[0], x[1], x[2], x[3]};
    }
};
template <>
struct Vec16<bf16_t> {
    static constexpr int N = 8;
    __device__ static void load(const bf16_t *p, float (&x)[8]) {
        const uint4 v = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static void store(bf16_t *p, const float (&x)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = static_cast<uint32_t>(f32_to_bf16_bits(x[2 * i])) |
                   (static_cast<uint32_t>(f32_to_bf16_bits(x[2 * i + 1])) << 16);
        }
        *reinterpret_cast<uint4 *>(p) = uint4{w[0], w[1], w[2], w[3]};
    }
};

template <typename T>
__device__ __forceinline__ float scalar_at(const T *p, size_t i) { return io<T>::ld(p + i); }

// One thread per 16 bytes of one output row piece. Index space: key-axis pieces
// (rows x h_v x d_k / N) first, then value-axis pieces (rows x h_v x d_v / N).
template <typename T, int MODE>
__global__ __launch_bounds__(256) void map_gates_kernel(GateArgs a) {
    constexpr int N = Vec16<T>::N;
    const T *q = static_cast<const T *>(a.q), *k = static_cast<const T *>(a.k);
    const T *v = static_cast<const T *>(a.v), *la = static_cast<const T *>(a.log_alpha);
    const T *beta = static_cast<const T *>(a.beta), *beta_v = static_cast<const T *>(a.beta_v);
    const int64_t pk = static_cast<int64_t>(a.rows) * a.h_v * (a.d_k / N);
    const int64_t pv = static_cast<int64_t>(a.rows) * a.h_v * (a.d_v / N);
    const int G = a.h_v / a.h_k;
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < pk + pv;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const bool key_axis = i < pk;
        const int64_t j = key_axis ? i : i - pk;
        const int d = key_axis ? a.d_k : a.d_v;
        const int cp = d / N;
        const int64_t rh = j / cp;                      // row * h_v + h
        const int c0 = static_cast<int>(j - rh * cp) * N;
        const int64_t row = rh / a.h_v;
        const int h = static_cast<int>(rh - row * a.h_v);
        const size_t o = static_cast<size_t>(rh) * d + c0;   // [rows][h_v][d] offset
        float x[N];
        if constexpr (MODE == GATES_KDA || MODE == GATES_GDN) {
            const float bt = scalar_at(beta, static_cast<size_t>(rh));
#pragma unroll
            for (int e = 0; e < N; ++e) x[e] = bt;
            if (key_axis) {
                Vec16<T>::store(static_cast<T *>(a.b_out) + o, x);
                if constexpr (MODE == GATES_GDN) {
                    const float lt = scalar_at(la, static_cast<size_t>(rh));
#pragma unroll
                    for (int e = 0; e < N; ++e) x[e] = lt;
                    Vec16<T>::store(static_cast<T *>(a.log_alpha_out) + o, x);
                }
            } else {
                Vec16<T>::store(static_cast<T *>(a.w_out) + o, x);
            }
        } else {                                        // GATES_FG2, GATES_FG2_PLUS
            if (key_axis) {
                const size_t ok = (static_cast<size_t>(row) * a.h_k + h / G) * a.d_k + c0;
                float bk[N], kk[N];
                Vec16<T>::load(beta + o, bk);
                Vec16<T>::load(k + ok, kk);
#pragma unroll
                for (int e = 0; e < N; ++e) x[e] = sqrt_hw(bk[e]) * kk[e];
                Vec16<T>::store(static_cast<T *>(a.k_out) + o, x);
#pragma unroll
                for (int e = 0; e < N; ++e) x[e] = 1.f;
                Vec16<T>::store(static_cast<T *>(a.b_out) + o, x);
                if (a.q_out) {
                    Vec16<T>::load(q + ok, x);
                    Vec16<T>::store(static_cast<T *>(a.q_out) + o, x);
                }
            } else if constexpr (MODE == GATES_FG2) {   // d_v == d_k: beta indexes alike
                float bk[N], vv[N];
                Vec16<T>::load(beta + o, bk);
                Vec16<T>::load(v + o, vv);
#pragma unroll
                for (int e = 0; e < N; ++e) x[e] = sqrt_hw(bk[e]) * vv[e];
                Vec16<T>::store(static_cast<T *>(a.v_out) + o, x);
#pragma unroll
                for (int e = 0; e < N; ++e) x[e] = 1.f;
                Vec16<T>::store(static_cast<T *>(a.w_out) + o, x);
            } else {
                float bv[N];
                Vec16<T>::load(beta_v + o, bv);
#pragma unroll
                for (int e = 0; e < N; ++e) x[e] = sqrt_hw(bv[e]);
                Vec16<T>::store(static_cast<T *>(a.w_out) + o, x);
            }
        }
    }
}

template <typename T, int MODE>
hipError_t launch_t(const GateArgs &a, hipStream_t st) {
    constexpr int N = Vec16<T>::N;
    const int64_t pieces = static_cast<int64_t>(a.rows) * a.h_v * ((a.d_k + a.d_v) / N);
    if (pieces <= 0) return hipSuccess;
    const int64_t blocks = (pieces + 255) / 256;
    const int grid = static_cast<int>(blocks < 8192 ? blocks : 8192);
    hipLaunchKernelGGL((map_gates_kernel<T, MODE>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_mode(const GateArgs &a, hipStream_t st) {
    switch (a.mode) {
    case GATES_KDA: return launch_t<T, GATES_KDA>(a, st);
    case GATES_GDN: return launch_t<T, GATES_GDN>(a, st);
    case GATES_FG2: return launch_t<T, GATES_FG2>(a, st);
    default: return launch_t<T, GATES_FG2_PLUS>(a, st);
    }
}

// ---- the chain rule back through the mappings --------------------------------------------

// Four consecutive elements of an input-dtype tensor (8- or 16-byte aligned) as floats.
template <typename T>
__device__ __forceinline__ void ld4(const T *p, float (&x)[4]) {
    if constexpr (sizeof(T) == 4) {
        const float4 v = *reinterpret_cast<const float4 *>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        x[0] = __uint_as_float(v.x << 16);
        x[1] = __uint_as_float(v.x & 0xffff0000u);
        x[2] = __uint_as_float(v.y << 16);
        x[3] = __uint_as_float(v.y & 0xffff0000u);
    }
}
__device__ __forceinline__ float4 ldf4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void stf4(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<float4 *>(p) = float4{a, b, c, d};
}

// KDA and GDN: b = w = beta (and log alpha, GDN) broadcast over the channels, so their
// gradients sum over the channels. Sixteen lanes per (row, value head), four floats per
// lane per step, then a sum over the sixteen lanes.
template <int MODE>
__global__ __launch_bounds__(256) void map_gates_bwd_scalar_kernel(GateBwdArgs a) {
    const int64_t units = a.rows * a.h_v;
    const int sub = threadIdx.x & 15;
    for (int64_t u = (blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x) >> 4; u < units;
         u += (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 4) {   // uniform per 16 lanes
        const float *db = a.db_m + u * a.d_k, *dw = a.dw_m + u * a.d_v;
        float sb = 0.f, sl = 0.f;
        for (int c = 4 * sub; c < a.d_k; c += 64) {
            const float4 x = ldf4(db + c);
            sb += (x.x + x.y) + (x.z + x.w);
            if constexpr (MODE == GATES_GDN) {
                const float4 y = ldf4(a.dla_m + u * a.d_k + c);
                sl += (y.x + y.y) + (y.z + y.w);
            }
        }
        for (int c = 4 * sub; c < a.d_v; c += 64) {
            const float4 x = ldf4(dw + c);
            sb += (x.x + x.y) + (x.z + x.w);
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
            sb += __shfl_xor(sb, m);
            if constexpr (MODE == GATES_GDN) sl += __shfl_xor(sl, m);
        }
        if (sub == 0) {
            a.dbeta[u] = sb;
            if constexpr (MODE == GATES_GDN) a.dla[u] = sl;
        }
    }
}

// FG2 and FG2+: one thread per four channels. Index space, in order: (row, value head, four
// key channels) for dbeta (and dv, FG2, whose d_v = d_k); (row, value head, four value
// channels) for dbeta_v (FG2+); (row, key head, four key channels) for dk and, when value
// heads share key heads, dq (sums over the key head's value heads).
template <typename T, int MODE>
__global__ __launch_bounds__(256) void map_gates_bwd_fg2_kernel(GateBwdArgs a) {
    const T *k = static_cast<const T *>(a.k), *v = static_cast<const T *>(a.v);
    const T *beta = static_cast<const T *>(a.beta), *beta_v = static_cast<const T *>(a.beta_v);
    const int G = a.h_v / a.h_k;
    const int64_t nA = a.rows * a.h_v * (a.d_k / 4);
    const int64_t nB = MODE == GATES_FG2_PLUS ? a.rows * a.h_v * (a.d_v / 4) : 0;
    const int64_t nC = a.rows * a.h_k * (a.d_k / 4);
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < nA + nB + nC;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        if (i < nA) {                                   // (row, h, c..c+3) on the key axis
            const int64_t rh = i / (a.d_k / 4);
            const int c = static_cast<int>(i - rh * (a.d_k / 4)) * 4;
            const int64_t row = rh / a.h_v;
            const int h = static_cast<int>(rh - row * a.h_v);
            const size_t o = static_cast<size_t>(rh) * a.d_k + c;
            float bt[4], kk[4];
            ld4(beta + o, bt);
            ld4(k + (static_cast<size_t>(row) * a.h_k + h / G) * a.d_k + c, kk);
            const float4 gk = ldf4(a.dk_m + o);
            const float gka[4] = {gk.x, gk.y, gk.z, gk.w};
            float db[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) db[e] = gka[e] * kk[e];
            if constexpr (MODE == GATES_FG2) {          // v' = sqrt(beta) v, d_v = d_k
                float vv[4];
                ld4(v + o, vv);
                const float4 gv = ldf4(a.dv_m + o);
                const float gva[4] = {gv.x, gv.y, gv.z, gv.w};
                float dvo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float sb = sqrt_hw(bt[e]);
                    db[e] += gva[e] * vv[e];
                    dvo[e] = sb * gva[e];
                }
                stf4(a.dv + o, dvo[0], dvo[1], dvo[2], dvo[3]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) db[e] = db[e] / (2.f * sqrt_hw(bt[e]));
            stf4(a.dbeta + o, db[0], db[1], db[2], db[3]);
        } else if (i < nA + nB) {                       // (row, h, j..j+3) on the value axis
            const int64_t j = i - nA;
            const int64_t rh = j / (a.d_v / 4);
            const size_t o = static_cast<size_t>(rh) * a.d_v + static_cast<int>(j - rh * (a.d_v / 4)) * 4;
            float bv[4];
            ld4(beta_v + o, bv);
            const float4 gw = ldf4(a.dw_m + o);
            stf4(a.dbeta_v + o, gw.x / (2.f * sqrt_hw(bv[0])), gw.y / (2.f * sqrt_hw(bv[1])),
                 gw.z / (2.f * sqrt_hw(bv[2])), gw.w / (2.f * sqrt_hw(bv[3])));
        } else {                                        // (row, key head, c..c+3)
            const int64_t j = i - nA - nB;
            const int64_t rk = j / (a.d_k / 4);
            const int c = static_cast<int>(j - rk * (a.d_k / 4)) * 4;
            const int64_t row = rk / a.h_k;
            const int hk = static_cast<int>(rk - row * a.h_k);
            float sk[4] = {0.f, 0.f, 0.f, 0.f}, sq[4] = {0.f, 0.f, 0.f, 0.f};
            for (int g = 0; g < G; ++g) {
                const size_t o = (static_cast<size_t>(row) * a.h_v + hk * G + g) * a.d_k + c;
                float bt[4];
                ld4(beta + o, bt);
                const float4 gk = ldf4(a.dk_m + o);
                sk[0] += sqrt_hw(bt[0]) * gk.x;
                sk[1] += sqrt_hw(bt[1]) * gk.y;
                sk[2] += sqrt_hw(bt[2]) * gk.z;
                sk[3] += sqrt_hw(bt[3]) * gk.w;
                if (G > 1) {
                    const float4 gq = ldf4(a.dq_m + o);
                    sq[0] += gq.x; sq[1] += gq.y; sq[2] += gq.z; sq[3] += gq.w;
                }
            }
            const size_t ok = static_cast<size_t>(rk) * a.d_k + c;
            stf4(a.dk + ok, sk[0], sk[1], sk[2], sk[3]);
            if (G > 1) stf4(a.dq + ok, sq[0], sq[1], sq[2], sq[3]);
        }
    }
}

template <typename T>
hipError_t launch_bwd_fg2(const GateBwdArgs &a, hipStream_t st) {
    const int64_t n = a.rows * (a.h_v * (a.d_k / 4) + (a.mode == GATES_FG2_PLUS ? a.h_v * (a.d_v / 4) : 0) +
                                a.h_k * (a.d_k / 4));
    const int64_t blocks = (n + 255) / 256;
    const int grid = static_cast<int>(blocks < 8192 ? blocks : 8192);
    if (a.mode == GATES_FG2)
        hipLaunchKernelGGL((map_gates_bwd_fg2_kernel<T, GATES_FG2>), dim3(grid), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((map_gates_bwd_fg2_kernel<T, GATES_FG2_PLUS>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_map_gates(const GateArgs &a, hipStream_t st) {
    return a.bf16 ? launch_mode<bf16_t>(a, st) : launch_mode<float>(a, st);
}

hipError_t launch_map_gates_bwd(const GateBwdArgs &a, hipStream_t st) {
    if (a.rows <= 0) return hipSuccess;
    if (a.mode == GATES_KDA || a.mode == GATES_GDN) {
        const int64_t blocks = (a.rows * a.h_v * 16 + 255) / 256;
        const int grid = static_cast<int>(blocks < 8192 ? blocks : 8192);
        if (a.mode == GATES_KDA)
            hipLaunchKernelGGL(map_gates_bwd_scalar_kernel<GATES_KDA>, dim3(grid), dim3(256), 0, st, a);
        else
            hipLaunchKernelGGL(map_gates_bwd_scalar_kernel<GATES_GDN>, dim3(grid), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    return a.bf16 ? launch_bwd_fg2<bf16_t>(a, st) : launch_bwd_fg2<float>(a, st);
}

}  // namespace gdn2
