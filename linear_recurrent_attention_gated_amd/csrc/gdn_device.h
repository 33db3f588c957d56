// gdn_device.h -- device-side building blocks shared by the gated-delta-rule kernels:
// element types, round-to-nearest-even bf16 conversion, and the gfx950 MFMA tile
// operations the blockwise prefill is written in.
//
// MFMA tiles (CDNA4 matrix cores, wave64).  Every contraction here is a 16x16 output
// tile with fp32 accumulation:
//   bf16: v_mfma_f32_16x16x32_bf16  -- 32 k-values per instruction, 8 per lane
//   fp32: v_mfma_f32_16x16x4_f32    --  4 k-values per instruction, 1 per lane
// Operand placement for lane l (0..63), with KPL = k-values per lane:
//   A (16 x K): row  l % 16, k = (l / 16) * KPL + [0, KPL)
//   B (K x 16): col  l % 16, k = (l / 16) * KPL + [0, KPL)
//   D (16 x 16): col l % 16, rows (l / 16) * 4 + [0, 4)
// All operands are read from memory laid out contiguous along k, so a bf16 fragment is
// one 16-byte load and an fp32 fragment one 4-byte load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef uint16_t bf16_t;  // bfloat16 storage (upper half of an fp32)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN (quiet).
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Element-type traits: load/store of q, k, v, o and the bf16/fp32 MFMA tile op.
template <typename E> struct Elem;

template <> struct Elem<bf16_t> {
    static constexpr int KB = 32;   // k per MFMA
    static constexpr int KPL = 8;   // k per lane
    typedef bf16x8 frag;
    __device__ static __forceinline__ float to_f(bf16_t x) { return bf2f(x); }
    __device__ static __forceinline__ bf16_t from_f(float x) { return f2bf(x); }
    // fragment at p[0..7] (16-byte aligned)
    __device__ static __forceinline__ frag ld(const bf16_t* p) {
        u16x8 u = *reinterpret_cast<const u16x8*>(p);
        return __builtin_bit_cast(frag, u);
    }
    // fragment from 8 consecutive floats, rounded to bf16
    __device__ static __forceinline__ frag ld_f(const float* p) {
        u16x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = f2bf(p[e]);
        return __builtin_bit_cast(frag, u);
    }
    __device__ static __forceinline__ frag zero() {
        u16x8 u = {0, 0, 0, 0, 0, 0, 0, 0};
        return __builtin_bit_cast(frag, u);
    }
    __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Elem<float> {
    static constexpr int KB = 4;
    static constexpr int KPL = 1;
    typedef float frag;
    __device__ static __forceinline__ float to_f(float x) { return x; }
    __device__ static __forceinline__ float from_f(float x) { return x; }
    __device__ static __forceinline__ frag ld(const float* p) { return *p; }
    __device__ static __forceinline__ frag ld_f(const float* p) { return *p; }
    __device__ static __forceinline__ frag zero() { return 0.0f; }
    __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

}  // namespace gdn
