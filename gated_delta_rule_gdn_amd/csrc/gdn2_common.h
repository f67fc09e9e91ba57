// gdn2_common.h -- device helpers shared by the gfx950 kernels of libgdn2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

// Raw bf16 storage (the ABI's bf16 tensors are plain 16-bit words).
struct bf16_t { uint16_t bits; };

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Square root on the transcendental unit (within 1 ulp): the gate scales of the FG2 modes.
// sqrtf's correctly rounded sequence adds a compare-and-select rescaling per value.
__device__ __forceinline__ float sqrt_hw(float x) { return __builtin_amdgcn_sqrtf(x); }

// Element loads/stores of the input dtype, widened to fp32.
template <typename T> struct io;

template <> struct io<float> {
    static __device__ __forceinline__ float val(float x) { return x; }
    static __device__ __forceinline__ float ld(const float *p) { return *p; }
    static __device__ __forceinline__ void st(float *p, float x) { *p = x; }
    static __device__ __forceinline__ f32x4 ld4(const float *p) {
        return *reinterpret_cast<const f32x4 *>(p);
    }
    static __device__ __forceinline__ void st4(float *p, f32x4 x) {
        *reinterpret_cast<f32x4 *>(p) = x;
    }
};

template <> struct io<bf16_t> {
    static __device__ __forceinline__ float val(bf16_t x) { return bf16_to_f32(x.bits); }
    static __device__ __forceinline__ float ld(const bf16_t *p) { return bf16_to_f32(p->bits); }
    static __device__ __forceinline__ void st(bf16_t *p, float x) { p->bits = f32_to_bf16_bits(x); }
    static __device__ __forceinline__ f32x4 ld4(const bf16_t *p) {
        uint2 u = *reinterpret_cast<const uint2 *>(p);
        f32x4 r;
        r.x = __uint_as_float(u.x << 16);
        r.y = __uint_as_float(u.x & 0xffff0000u);
        r.z = __uint_as_float(u.y << 16);
        r.w = __uint_as_float(u.y & 0xffff0000u);
        return r;
    }
    static __device__ __forceinline__ void st4(bf16_t *p, f32x4 x) {
        uint2 u;
        u.x = static_cast<uint32_t>(f32_to_bf16_bits(x.x)) |
              (static_cast<uint32_t>(f32_to_bf16_bits(x.y)) << 16);
        u.y = static_cast<uint32_t>(f32_to_bf16_bits(x.z)) |
              (static_cast<uint32_t>(f32_to_bf16_bits(x.w)) << 16);
        *reinterpret_cast<uint2 *>(p) = u;
    }
};

}  // namespace gdn2
