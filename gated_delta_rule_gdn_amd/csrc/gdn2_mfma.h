// gdn2_mfma.h -- CDNA4 (gfx950) matrix-core helpers and the fragment layouts they assume.
//
// All products are 16x16 output tiles D (16 x 16 fp32) += A (16 x K) * B (K x 16) on one
// 64-lane wave. With lane l = 16 * lg + li (li = l % 16, lg = l / 16):
//   output D      lane l holds D[4 lg + ii][li], ii = 0..3             (f32x4)
//   A operand     lane l holds row li of A; B operand lane l holds column li of B
//   k slots       the lanes of group lg hold the same k slots of A and of B; the
//                 instruction sums over all (lg, slot) pairs, so any one-to-one map from
//                 (lg, slot) to the true k index works as long as A and B use the same one.
// Instructions used:
//   v_mfma_f32_16x16x32_bf16   8 bf16 slots per lane  (K = 32 per instruction)
//   v_mfma_f32_16x16x16_bf16   4 bf16 slots per lane  (K = 16)
//   v_mfma_f32_16x16x4_f32     1 fp32 slot per lane   (K = 4)
//
// "D-layout chaining": a product whose B operand is a previous output D (rows = k) needs no
// data movement. For K = 16 fp32 (four x4 steps) step s takes slot s of each D row group,
// i.e. k = 4 lg + s; for K = 32 bf16 two D tiles give slots 0-3 (k = 4 lg + jj) and
// slots 4-7 (k = 16 + 4 lg + jj - 4). The A operand is then stored with the same k map
// ("perm order" below) so that each lane reads its 16 bytes contiguously.
#pragma once
#include "gdn2_common.h"

namespace gdn2 {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// D += A * B, K = 32, bf16 operands packed 8 per lane (4 dwords).
__device__ __forceinline__ f32x4 mma_k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D += A * B, K = 16, bf16 operands packed 4 per lane (2 dwords).
__device__ __forceinline__ f32x4 mma_k16_bf16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// D += A * B, K = 16 in fp32 as four K = 4 steps; step s uses slot s of a and b.
__device__ __forceinline__ f32x4 mma_k16_f32(f32x4 a, f32x4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
    return c;
}

// Two D tiles (k rows 0-15 and 16-31) -> one bf16 B operand for mma_k32 (perm order).
__device__ __forceinline__ u32x4 dpair_to_b32(f32x4 lo, f32x4 hi) {
    u32x4 r;
    r.x = pack_bf16x2(lo.x, lo.y);
    r.y = pack_bf16x2(lo.z, lo.w);
    r.z = pack_bf16x2(hi.x, hi.y);
    r.w = pack_bf16x2(hi.z, hi.w);
    return r;
}

__device__ __forceinline__ u32x2 f4_to_b16(f32x4 x) {
    u32x2 r;
    r.x = pack_bf16x2(x.x, x.y);
    r.y = pack_bf16x2(x.z, x.w);
    return r;
}

// k index of slot jj of lane group lg in a perm-order A block (see above).
template <bool BF>
__device__ __forceinline__ int perm_k(int lg, int jj) {
    if constexpr (BF) return jj < 4 ? 4 * lg + jj : 16 + 4 * lg + (jj - 4);
    else return 4 * lg + jj;
}

}  // namespace gdn2
