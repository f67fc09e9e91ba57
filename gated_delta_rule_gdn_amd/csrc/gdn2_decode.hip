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
// The GDN decode verify page (LocalAI mirror), section 2, describes the same fused
// read-update-write of a persistent state, with the state held in registers across the
// tokens of one call; section 4 notes that the step is bound by the traffic of the fp32
// state and names a bf16 state as a way to cut it. This kernel therefore moves each state
// through HBM exactly once per call, whatever T is, and can keep the state in bf16 (half
// the bytes).
//
// Optional fusions (burn-gdn2 "Architecture": ShortConv and L2-Norm before the recurrence,
// Gated RMS Norm with a SiLU gate after it): a causal depthwise convolution of width 4 over
// q, k and v with its three-input state in the cache (GDN decode verify page, sections 1
// and 2), q and k divided by their L2 norms, and each output row replaced by
// o / sqrt(mean o^2 + eps) * weight * silu(gate).
//
// State cache: the states live in a pool of slots; sequence n uses slot idx[n] (or n when
// no index is given). A slot outside [0, num_slots) marks a padding entry: the state is not
// touched and the sequence's o rows are zero.
//
// Design for gfx950: one 256-thread workgroup per (sequence, value head) state, one 16-byte
// vector (4 fp32 or 8 bf16 columns) per lane per row (lane geometry below). All state
// loads are issued before any arithmetic, and the state stays in fp32 registers across the
// T tokens. The token vectors are staged in LDS eight tokens at a time; the two reductions
// over d_k run inside each wave on DPP row rotations and the gfx950 row-swap instructions
// (VALU work, no LDS traffic).
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

// State vectors: 4 fp32 or 8 bf16 columns (16 bytes), or 4 bf16 columns (8 bytes), widened
// to fp32 in registers.
template <typename ST, int N = 16 / static_cast<int>(sizeof(ST))> struct svec;
template <> struct svec<float, 4> {
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
template <> struct svec<bf16_t, 8> {
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
template <> struct svec<bf16_t, 4> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void ld(const bf16_t *p, float *x) {
        const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
        x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
        x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    }
    template <bool NTS>
    static __device__ __forceinline__ void st(bf16_t *p, const float *x) {
        const u32x2 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};   // RNE
        if constexpr (NTS) __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
        else *reinterpret_cast<u32x2 *>(p) = v;
    }
};

// Sum of x over the lanes of a wave that share lane % CGW (CGW a power of two < 64): row
// rotations within 16-lane rows (DPP row_ror:1/2/4/8) for strides below 16, then the gfx950 row-swap
// instructions for 16 and 32. Every lane ends with the full sum. All of it is VALU work.
template <int CGW>
__device__ __forceinline__ float lane_group_sum(float x) {
    if constexpr (CGW <= 1) x += __builtin_amdgcn_update_dpp(0.f, x, 0x121, 0xF, 0xF, false);
    if constexpr (CGW <= 2) x += __builtin_amdgcn_update_dpp(0.f, x, 0x122, 0xF, 0xF, false);
    if constexpr (CGW <= 4) x += __builtin_amdgcn_update_dpp(0.f, x, 0x124, 0xF, 0xF, false);
    if constexpr (CGW <= 8) x += __builtin_amdgcn_update_dpp(0.f, x, 0x128, 0xF, 0xF, false);
    if constexpr (CGW <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);                       // + lane ^ 16
    }
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);                        // + lane ^ 32
}

// Lane geometry of one state. The workgroup's four waves split the state either by rows
// (COLW = false: each wave holds whole rows, so every wave instruction reads whole rows,
// the best pattern for streaming; the d_k reductions then finish across the waves through
// LDS, one barrier per token) or by columns (COLW = true: each wave holds a quarter of the
// columns of every row, 128-byte pieces of rows; the reductions stay inside the wave, so
// tokens need no barrier). Single-token calls are bound by the state traffic and take the
// row split; multi-token calls are bound by the per-token dependency chain and take the
// column split.
template <int DK, int DV, int VN, bool COLW>
struct Geom {
    static constexpr int NW = kDecodeThreads / 64;
    static constexpr int WC = COLW ? DV / NW : DV;    // columns a wave spans
    static constexpr int CG = WC / VN;                // column groups a wave spans
    static constexpr int RGW = 64 / CG;               // row groups in one wave
    static constexpr int RG = COLW ? RGW : RGW * NW;  // row groups of the workgroup
    static constexpr int RPT = DK / RG;               // rows per lane
    static_assert(CG >= 1 && CG <= 64 && (CG & (CG - 1)) == 0, "lane layout");
    static_assert(RPT >= 1 && RG * RPT == DK, "tile shape");
};

// CV: with the short causal convolution of q, k and v. Every workgroup convolves its q and
// k (those of its key head) from the conv state, which it only reads there: the G value
// heads of a key head all need the old q/k state, so conv_qk_state_kernel rewrites it
// after this kernel. The v channels belong to one value head, so the workgroup rewrites
// their state itself.
template <typename T, typename ST, int DK, int DV, bool NTS, bool COLW, bool FU, bool CV>
__global__ __launch_bounds__(kDecodeThreads) void recurrent_fwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ log_alpha, const T *__restrict__ b, const T *__restrict__ w,
    ST *__restrict__ S, const int32_t *__restrict__ idx, T *__restrict__ o, int ntok,
    int num_slots, int h_k, int h_v, int group, int qkn, float l2eps,
    const T *__restrict__ gate, const float *__restrict__ nw, float neps,
    const float *__restrict__ cw, float *__restrict__ cst, int csilu, int gmode) {
    constexpr int NT = kDecodeThreads, NW = NT / 64;
    // columns per lane: one 16-byte vector; four columns for a bf16 state in multi-token
    // calls, whose per-token reductions then run over fewer values and lanes
    constexpr int VN = COLW ? 4 : svec<ST>::N;
    using SV = svec<ST, VN>;
    using Gm = Geom<DK, DV, VN, COLW>;
    constexpr int CG = Gm::CG, RG = Gm::RG, RPT = Gm::RPT;
    // The row split serves single-token calls only (the launch picks it for T = 1), so its
    // token loop is resolved at compile time.
    constexpr int TB = COLW ? kTokBlock : 1;
    const int nt = COLW ? ntok : 1;
    // the fusions are compiled only into the FU instantiations
    const bool do_qkn = FU && qkn != 0;
    const bool do_gate = FU && gate != nullptr;

    // staged token vectors: (decay, b.k, q, k) per key-axis row, and w.v per column
    __shared__ f32x4 s_tok[TB][DK];
    __shared__ float s_wv[TB][DV];
    // per-wave partial sums (row split only): y, z, then k.q, |q|^2, |k|^2
    __shared__ float s_red[COLW ? 1 : NW][COLW ? 1 : 2 * DV + 4];
    // outputs of the block's tokens, for the gated norm over d_v
    __shared__ float s_o[TB][DV];

    const int pair = blockIdx.x;
    const int n = pair / h_v;
    const int h = pair - n * h_v;
    const int hk = h / group;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int cg = lane % CG;
    const int rg = COLW ? lane / CG : tid / CG;       // row group: rows rg + RG i
    const int c0 = (COLW ? wave * Gm::WC : 0) + cg * VN;   // first column of this lane

    const int slot = idx ? idx[n] : n;
    if (slot < 0 || slot >= num_slots) {     // padding entry: zero o rows, state untouched
        for (int i = tid; i < nt * DV; i += NT) {
            const int t = i / DV, c = i - t * DV;
            io<T>::st(o + ((static_cast<size_t>(n) * nt + t) * h_v + h) * DV + c, 0.f);
        }
        return;
    }

    // short convolution: channel ch at token tg of this call; raw(t') reads the call's own
    // inputs, earlier tokens come from the conv state (the last three inputs, oldest first)
    const int C = 2 * h_k * DK + h_v * DV;
    float *cs = CV ? cst + static_cast<size_t>(slot) * 3 * C : nullptr;
    // (Both candidate inputs of a tap are loaded and one is selected, so that all loads of a
    // channel issue together instead of one round trip per tap.)
    auto conv_at = [&](int ch, int tg, auto raw) -> float {
        const f32x4 wt = *reinterpret_cast<const f32x4 *>(cw + static_cast<size_t>(ch) * 4);
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tp = tg - 3 + j;
            const float a = raw(tp < 0 ? 0 : tp);
            const float b = cs[(tp < 0 ? 3 + tp : 0) * C + ch];
            x[j] = tp >= 0 ? a : b;
        }
        const float acc = wt.x * x[0] + wt.y * x[1] + wt.z * x[2] + wt.w * x[3];
        return csilu ? acc / (1.f + __expf(-acc)) : acc;
    };

    // new conv state of this head's v channels (their last three inputs), loaded now and
    // stored once the first block's staging has read the old state. Channel cvc belongs to
    // thread tid (column split) or to the thread that stages v column cvc (row split).
    float cv_new[CV ? 3 : 1];
    const int cvc = COLW ? tid : tid - DK;
    const bool cvown = cvc >= 0 && cvc < DV;
    if constexpr (CV && COLW) {
        if (cvown) {
            const int ch = 2 * h_k * DK + h * DV + tid;
#pragma unroll
            for (int e = 0; e < 3; ++e) {
                const int tp = nt - 3 + e;
                const float a = io<T>::ld(v + ((static_cast<size_t>(n) * nt + (tp < 0 ? 0 : tp)) * h_v + h) * DV + tid);
                const float b = cs[(tp < 0 ? 3 + tp : 0) * C + ch];
                cv_new[e] = tp >= 0 ? a : b;
            }
        }
    }

    ST *Sp = S + (static_cast<size_t>(slot) * h_v + h) * DK * DV;
    float s[RPT][VN];
    // Single-token calls with the convolution stage their one token before the state loads
    // (EARLY); every other instance loads the state first.
    // Gate modes (GateMode): KDA and GDN read one b per (token, value head) from b, which
    // also serves as w, GDN one decay per (token, value head); FG2 reads beta [..][DK] from b
    // (k <- sqrt(beta) k, b <- 1, w <- sqrt(beta), d_v = d_k), FG2+ beta_v from w
    // (w <- sqrt(beta_v)). `tok` is the token row of the call's [N][T] layout.
    const bool b_scalar = gmode == GATES_KDA || gmode == GATES_GDN;
    const bool la_scalar = gmode == GATES_GDN;
    const bool fg2 = gmode == GATES_FG2 || gmode == GATES_FG2_PLUS;
    auto gate_la = [&](size_t tok, int r) {
        const size_t rh = tok * h_v + h;
        return io<T>::ld(log_alpha + (la_scalar ? rh : rh * DK + r));
    };
    auto gate_b = [&](size_t tok, int r) {
        const size_t rh = tok * h_v + h;
        return io<T>::ld(b + (b_scalar ? rh : rh * DK + r));
    };
    auto gate_w = [&](size_t tok, int c) {
        const size_t rh = tok * h_v + h;
        if (b_scalar) return io<T>::ld(b + rh);
        if (gmode == GATES_FG2) return sqrt_hw(io<T>::ld(b + rh * DK + c));
        const float x = io<T>::ld(w + rh * DV + c);
        return gmode == GATES_FG2_PLUS ? sqrt_hw(x) : x;
    };
    // staged key row: (decay, b . k, q, k), with FG2's key scaling
    auto stage_key = [&](float la, float bv, float qq, float kk) {
        const float kx = fg2 ? sqrt_hw(bv) * kk : kk;
        return f32x4{__expf(la), (fg2 ? 1.f : bv) * kx, qq, kx};
    };
    constexpr bool EARLY = CV && !COLW;
    if constexpr (EARLY) {
        // One token, one staging entry per thread (key row tid, or v column tid - DK). Its
        // loads are issued before the state loads: vector memory returns in issue order, so
        // the convolution arithmetic then waits only for its own inputs and overlaps the
        // state stream instead of following it (measured: 72.8 -> 69.0 us per step for the
        // decode workload; without the convolution this order measured slower).
        const bool krow = tid < DK, vcol = tid >= DK && tid < DK + DV;
        const int r = krow ? tid : 0, c = vcol ? tid - DK : 0;
        const size_t kq_off = (static_cast<size_t>(n) * h_k + hk) * DK + r;
        const size_t v_off = (static_cast<size_t>(n) * h_v + h) * DV + c;
        float xk = 0.f, xq = 0.f, xla = 0.f, xb = 0.f, xw = 0.f, xv = 0.f;
        f32x4 wk4 = {}, wq4 = {}, wv4 = {};
        float ck[3] = {}, cq[3] = {}, cvv[3] = {};
        const int chq = hk * DK + r, chk = h_k * DK + hk * DK + r, chv = 2 * h_k * DK + h * DV + c;
        if (krow) {
            xk = io<T>::ld(k + kq_off);
            xq = io<T>::ld(q + kq_off);
            xla = gate_la(n, r);
            xb = gate_b(n, r);
            if constexpr (CV) {
                wk4 = *reinterpret_cast<const f32x4 *>(cw + static_cast<size_t>(chk) * 4);
                wq4 = *reinterpret_cast<const f32x4 *>(cw + static_cast<size_t>(chq) * 4);
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    ck[j] = cs[j * C + chk];
                    cq[j] = cs[j * C + chq];
                }
            }
        }
        if (vcol) {
            xw = gate_w(n, c);
            xv = io<T>::ld(v + v_off);
            if constexpr (CV) {
                wv4 = *reinterpret_cast<const f32x4 *>(cw + static_cast<size_t>(chv) * 4);
#pragma unroll
                for (int j = 0; j < 3; ++j) cvv[j] = cs[j * C + chv];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            SV::ld(Sp + static_cast<size_t>(rg + RG * i) * DV + c0, s[i]);
        __builtin_amdgcn_sched_barrier(0);
        // one token: taps 0-2 read the conv state, tap 3 the token itself
        auto conv1 = [&](f32x4 wt, const float *old, float x) {
            const float acc = wt.x * old[0] + wt.y * old[1] + wt.z * old[2] + wt.w * x;
            return csilu ? acc / (1.f + __expf(-acc)) : acc;
        };
        if (krow) {
            const float kk = CV ? conv1(wk4, ck, xk) : xk;
            const float qq = CV ? conv1(wq4, cq, xq) : xq;
            s_tok[0][r] = stage_key(xla, xb, qq, kk);
        }
        if (vcol) {
            s_wv[0][c] = xw * (CV ? conv1(wv4, cvv, xv) : xv);
            if constexpr (CV) {
                cv_new[0] = cvv[1];
                cv_new[1] = cvv[2];
                cv_new[2] = xv;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            SV::ld(Sp + static_cast<size_t>(rg + RG * i) * DV + c0, s[i]);
    }

    for (int t0 = 0; t0 < nt; t0 += TB) {
        const int nb = min(TB, nt - t0);
        if (t0 > 0) __syncthreads();         // the previous block's vectors are consumed
        // one pass over the block's nb (DK + DV) entries, spread over all threads (the EARLY
        // instance staged its single token above)
        for (int i = tid; !EARLY && i < nb * (DK + DV); i += NT) {
            if (i < nb * DK) {
                const int tt = i / DK, r = i - tt * DK;
                const size_t tok = static_cast<size_t>(n) * nt + t0 + tt;
                const size_t kq_off = (tok * h_k + hk) * DK + r;
                float kk, qq;
                if constexpr (CV) {
                    const size_t base = static_cast<size_t>(n) * nt;
                    kk = conv_at(h_k * DK + hk * DK + r, t0 + tt, [&](int tp) {
                        return io<T>::ld(k + ((base + tp) * h_k + hk) * DK + r); });
                    qq = conv_at(hk * DK + r, t0 + tt, [&](int tp) {
                        return io<T>::ld(q + ((base + tp) * h_k + hk) * DK + r); });
                } else {
                    kk = io<T>::ld(k + kq_off);
                    qq = io<T>::ld(q + kq_off);
                }
                s_tok[tt][r] = stage_key(gate_la(tok, r), gate_b(tok, r), qq, kk);
            } else {
                const int iv = i - nb * DK, tt = iv / DV, c = iv - tt * DV;
                const size_t off = ((static_cast<size_t>(n) * nt + t0 + tt) * h_v + h) * DV + c;
                float vv;
                if constexpr (CV) {
                    const size_t base = static_cast<size_t>(n) * nt;
                    vv = conv_at(2 * h_k * DK + h * DV + c, t0 + tt, [&](int tp) {
                        return io<T>::ld(v + ((base + tp) * h_v + h) * DV + c); });
                } else {
                    vv = io<T>::ld(v + off);
                }
                s_wv[tt][c] = gate_w(static_cast<size_t>(n) * nt + t0 + tt, c) * vv;
            }
        }
        __syncthreads();
        if constexpr (CV) {
            // the old state is read only by the first three tokens, all in the first block
            if (t0 == 0 && cvown) {
#pragma unroll
                for (int e = 0; e < 3; ++e) cs[e * C + 2 * h_k * DK + h * DV + cvc] = cv_new[e];
            }
        }

        for (int tt = 0; tt < nb; ++tt) {
            float y[VN], z[VN];
#pragma unroll
            for (int j = 0; j < VN; ++j) y[j] = z[j] = 0.f;
            float kq = 0.f, qsq = 0.f, ksq = 0.f;
            float kr[COLW ? 1 : RPT];             // the row split keeps k in registers
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const f32x4 g = s_tok[tt][rg + RG * i];     // decay, b.k, q, k
                if constexpr (!COLW) kr[i] = g.w;
#pragma unroll
                for (int j = 0; j < VN; ++j) {
                    s[i][j] *= g.x;
                    y[j] += g.y * s[i][j];
                    z[j] += g.z * s[i][j];
                }
                kq += g.w * g.z;
                qsq += g.z * g.z;
                ksq += g.w * g.w;
            }
            // sum over the row groups of this wave (lanes that share lane % CG)
#pragma unroll
            for (int j = 0; j < VN; ++j) {
                y[j] = lane_group_sum<CG>(y[j]);
                z[j] = lane_group_sum<CG>(z[j]);
            }
            kq = lane_group_sum<CG>(kq);
            if (do_qkn) {
                qsq = lane_group_sum<CG>(qsq);
                ksq = lane_group_sum<CG>(ksq);
            }
            if constexpr (!COLW) {
                // and over the waves, through LDS (one token per call: one barrier)
                if (lane < CG) {
#pragma unroll
                    for (int j = 0; j < VN; j += 4) {
                        *reinterpret_cast<f32x4 *>(&s_red[wave][c0 + j]) =
                            f32x4{y[j], y[j + 1], y[j + 2], y[j + 3]};
                        *reinterpret_cast<f32x4 *>(&s_red[wave][DV + c0 + j]) =
                            f32x4{z[j], z[j + 1], z[j + 2], z[j + 3]};
                    }
                    if (lane == 0) {
                        s_red[wave][2 * DV] = kq;
                        s_red[wave][2 * DV + 1] = qsq;
                        s_red[wave][2 * DV + 2] = ksq;
                    }
                }
                __syncthreads();
#pragma unroll
                for (int j = 0; j < VN; ++j) y[j] = z[j] = 0.f;
                kq = qsq = ksq = 0.f;
#pragma unroll
                for (int wv = 0; wv < NW; ++wv) {
#pragma unroll
                    for (int j = 0; j < VN; j += 4) {
                        const f32x4 yy = *reinterpret_cast<const f32x4 *>(&s_red[wv][c0 + j]);
                        const f32x4 zz = *reinterpret_cast<const f32x4 *>(&s_red[wv][DV + c0 + j]);
                        y[j] += yy.x; y[j + 1] += yy.y; y[j + 2] += yy.z; y[j + 3] += yy.w;
                        z[j] += zz.x; z[j + 1] += zz.y; z[j + 2] += zz.z; z[j + 3] += zz.w;
                    }
                    kq += s_red[wv][2 * DV];
                    qsq += s_red[wv][2 * DV + 1];
                    ksq += s_red[wv][2 * DV + 2];
                }
            }
            // q/k L2-norm: the products are linear in q and in k, so the raw vectors are
            // used and the sums scaled: y by 1/|k|, z by 1/|q|, k.q by both, k u^T by 1/|k|
            float nk = 1.f;
            if (do_qkn) {
                const float nq = rsqrtf(qsq + l2eps);
                nk = rsqrtf(ksq + l2eps);
#pragma unroll
                for (int j = 0; j < VN; ++j) {
                    y[j] *= nk;
                    z[j] *= nq;
                }
                kq *= nq * nk;
            }
            float u[VN];
#pragma unroll
            for (int j = 0; j < VN; ++j) u[j] = s_wv[tt][c0 + j] - y[j];
            if (rg == 0) {
                if (do_gate) {
#pragma unroll
                    for (int j = 0; j < VN; ++j) s_o[tt][c0 + j] = z[j] + kq * u[j];
                } else {
                    T *op = o + ((static_cast<size_t>(n) * nt + t0 + tt) * h_v + h) * DV + c0;
#pragma unroll
                    for (int j = 0; j < VN; j += 4)
                        io<T>::st4(op + j, f32x4{z[j] + kq * u[j], z[j + 1] + kq * u[j + 1],
                                                 z[j + 2] + kq * u[j + 2],
                                                 z[j + 3] + kq * u[j + 3]});
                }
            }
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                float kk;
                if constexpr (COLW) kk = s_tok[tt][rg + RG * i].w * nk;
                else kk = kr[i] * nk;
#pragma unroll
                for (int j = 0; j < VN; ++j) s[i][j] += kk * u[j];
            }
        }
        if (do_gate) {
            // gated RMS norm of each output row over d_v, one wave per token
            __syncthreads();
            constexpr int PL = DV / 64;           // values per lane
            for (int tt = wave; tt < nb; tt += NW) {
                float ov[PL], ss = 0.f;
#pragma unroll
                for (int j = 0; j < PL; ++j) {
                    ov[j] = s_o[tt][lane * PL + j];
                    ss += ov[j] * ov[j];
                }
                ss = lane_group_sum<1>(ss);
                const float scale = rsqrtf(ss * (1.f / DV) + neps);
                const size_t row = ((static_cast<size_t>(n) * nt + t0 + tt) * h_v + h) * DV;
#pragma unroll
                for (int j = 0; j < PL; ++j) {
                    const int c = lane * PL + j;
                    const float gv = io<T>::ld(gate + row + c);
                    io<T>::st(o + row + c, ov[j] * scale * nw[c] * (gv / (1.f + __expf(-gv))));
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        SV::template st<NTS>(Sp + static_cast<size_t>(rg + RG * i) * DV + c0, s[i]);

}

// The new conv state of the q and k channels, after recurrent_fwd_kernel has convolved them
// from the old one: the last three inputs of each channel (older state entries shift down
// when the call had fewer than three tokens). One thread per channel of one sequence.
template <typename T, int DK>
__global__ __launch_bounds__(256) void conv_qk_state_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const int32_t *__restrict__ idx,
    float *__restrict__ cst, int num_seqs, int ntok, int num_slots, int h_k, int C) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int per = 2 * h_k * DK;                 // q and k channels of one sequence
    if (i >= static_cast<int64_t>(num_seqs) * per) return;
    const int n = static_cast<int>(i / per), ch = static_cast<int>(i % per);
    const int slot = idx ? idx[n] : n;
    if (slot < 0 || slot >= num_slots) return;
    const T *src = ch < h_k * DK ? q : k;
    const int r = ch % (h_k * DK);                // key head * DK + row
    float *cs = cst + static_cast<size_t>(slot) * 3 * C;
    float nv[3];
#pragma unroll
    for (int e = 0; e < 3; ++e) {            // both candidates loaded: one round trip
        const int tp = ntok - 3 + e;
        const float a = io<T>::ld(src + (static_cast<size_t>(n) * ntok + (tp < 0 ? 0 : tp)) * h_k * DK + r);
        const float b = cs[(tp < 0 ? 3 + tp : 0) * C + ch];
        nv[e] = tp >= 0 ? a : b;
    }
#pragma unroll
    for (int e = 0; e < 3; ++e) cs[e * C + ch] = nv[e];
}

template <typename T, typename ST, int DK, int DV, bool FU, bool CV>
static hipError_t launch_recurrent_f(const DecodeArgs &a, hipStream_t st) {
    const int pairs = a.num_seqs * a.h_v;
    const size_t state_bytes = static_cast<size_t>(pairs) * DK * DV * sizeof(ST);
    const bool nts = state_bytes > kStreamStateBytes, colw = a.ntok > 1;
    auto kern = colw ? (nts ? recurrent_fwd_kernel<T, ST, DK, DV, true, true, FU, CV>
                            : recurrent_fwd_kernel<T, ST, DK, DV, false, true, FU, CV>)
                     : (nts ? recurrent_fwd_kernel<T, ST, DK, DV, true, false, FU, CV>
                            : recurrent_fwd_kernel<T, ST, DK, DV, false, false, FU, CV>);
    hipLaunchKernelGGL(kern, dim3(pairs), dim3(kDecodeThreads), 0, st,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), static_cast<const T *>(a.log_alpha),
                       static_cast<const T *>(a.b), static_cast<const T *>(a.w),
                       static_cast<ST *>(a.S), a.idx, static_cast<T *>(a.o), a.ntok,
                       a.num_slots, a.h_k, a.h_v, a.h_v / a.h_k, a.fu.qk_norm ? 1 : 0,
                       a.fu.l2eps, static_cast<const T *>(a.fu.gate), a.fu.nw, a.fu.neps,
                       a.fu.cw, a.fu.cst, a.fu.csilu ? 1 : 0, a.fu.gmode);
    if constexpr (CV) {
        const int64_t threads = static_cast<int64_t>(a.num_seqs) * 2 * a.h_k * DK;
        const int C = 2 * a.h_k * DK + a.h_v * DV;
        hipLaunchKernelGGL((conv_qk_state_kernel<T, DK>), dim3((threads + 255) / 256), dim3(256),
                           0, st, static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                           a.idx, a.fu.cst, a.num_seqs, a.ntok, a.num_slots, a.h_k, C);
    }
    return hipGetLastError();
}

template <typename T, typename ST, int DK, int DV>
static hipError_t launch_recurrent_t(const DecodeArgs &a, hipStream_t st) {
    if (a.fu.cw) return launch_recurrent_f<T, ST, DK, DV, true, true>(a, st);
    if (a.fu.qk_norm || a.fu.gate) return launch_recurrent_f<T, ST, DK, DV, true, false>(a, st);
    return launch_recurrent_f<T, ST, DK, DV, false, false>(a, st);
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
