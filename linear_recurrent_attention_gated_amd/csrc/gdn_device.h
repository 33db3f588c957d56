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
// Operands read from memory laid out contiguous along k are one 16-byte load per bf16
// fragment and per four fp32 fragments (Elem::GRP).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef uint16_t bf16_t;  // bfloat16 storage (upper half of an fp32)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32: round to nearest even,
// NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
    f32x2 x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Element-type traits: load/store of q, k, v, o and the bf16/fp32 MFMA tile op.

// Operand fragments read straight from accumulator tiles use a permuted k order: for k-block
// kb and lane group g (= lane / 16), fragment element e holds k = kperm(kb, g, e).  With it a
// 16x16 accumulator tile (lane: column l % 16, rows 4 g + [0, 4)) supplies KPL k-values per lane
// without any lane exchange: bf16 blocks of 32 take rows 4g..4g+3 of tiles 2kb and 2kb+1;
// fp32 blocks of 4 take row 4g + (kb & 3) of tile kb / 4.  Since a contraction sums over k,
// any order works as long as both operands use the same one.
template <typename E> struct Elem;

template <> struct Elem<bf16_t> {
    static constexpr int KB = 32;   // k per MFMA
    static constexpr int KPL = 8;   // k per lane
    typedef bf16x8 frag;
    __device__ static __forceinline__ int kperm(int kb, int g, int e) {
        return 32 * kb + 16 * (e >> 2) + 4 * g + (e & 3);
    }
    // offset of element 0 of the permuted fragment (kb, g) in a k-contiguous row
    __device__ static __forceinline__ int poff(int kb, int g) { return 32 * kb + 4 * g; }
    // permuted fragment k-block kb from two accumulator tiles: lo = k-tile 2 kb, hi = 2 kb + 1
    __device__ static __forceinline__ frag pack(f32x4 lo, f32x4 hi) {
        uint4 u;
        u.x = f2bf2(lo[0], lo[1]);
        u.y = f2bf2(lo[2], lo[3]);
        u.z = f2bf2(hi[0], hi[1]);
        u.w = f2bf2(hi[2], hi[3]);
        return __builtin_bit_cast(frag, u);
    }
    __device__ static __forceinline__ float to_f(bf16_t x) { return bf2f(x); }
    __device__ static __forceinline__ bf16_t from_f(float x) { return f2bf(x); }
    // fragment at p[0..7] (16-byte aligned)
    __device__ static __forceinline__ frag ld(const bf16_t* p) {
        u16x8 u = *reinterpret_cast<const u16x8*>(p);
        return __builtin_bit_cast(frag, u);
    }
    // permuted-order fragment of k-block kb from a k-contiguous row: row[kb * 32 + 4 g + 0..3]
    // and row[kb * 32 + 16 + 4 g + 0..3]   (p = row + kb * 32 + 4 g, 8-byte aligned)
    __device__ static __forceinline__ frag ld_perm(const bf16_t* p) {
        uint2 a = *reinterpret_cast<const uint2*>(p);
        uint2 b = *reinterpret_cast<const uint2*>(p + 16);
        uint4 u = {a.x, a.y, b.x, b.y};
        return __builtin_bit_cast(frag, u);
    }
    // fragment from 8 consecutive floats, rounded to bf16
    __device__ static __forceinline__ frag ld_f(const float* p) {
        uint4 u;
        u.x = f2bf2(p[0], p[1]);
        u.y = f2bf2(p[2], p[3]);
        u.z = f2bf2(p[4], p[5]);
        u.w = f2bf2(p[6], p[7]);
        return __builtin_bit_cast(frag, u);
    }
    // the fragment, or zeros where `keep` is false (branch-free)
    __device__ static __forceinline__ frag keep_if(frag a, bool keep) {
        uint4 u = __builtin_bit_cast(uint4, a);
        const uint32_t m = keep ? 0xffffffffu : 0u;
        u.x &= m; u.y &= m; u.z &= m; u.w &= m;
        return __builtin_bit_cast(frag, u);
    }
    __device__ static __forceinline__ frag zero() {
        u16x8 u = {0, 0, 0, 0, 0, 0, 0, 0};
        return __builtin_bit_cast(frag, u);
    }
    __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // Fragments in 16-byte lane groups (see the fp32 traits): a bf16 fragment is one group.
    static constexpr int GRP = 1;
    __device__ static __forceinline__ int doff(int kb, int g) { return kb * 32 + g * 8; }
    __device__ static __forceinline__ int foff(int kb, int lane) { return (kb * 64 + lane) * 8; }
    __device__ static __forceinline__ void ld_grp(const bf16_t* p, frag* f) { f[0] = ld(p); }
    __device__ static __forceinline__ void st_grp(bf16_t* p, const frag* f) {
        *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, f[0]);
    }
};

template <> struct Elem<float> {
    static constexpr int KB = 4;
    static constexpr int KPL = 1;
    __device__ static __forceinline__ int kperm(int kb, int g, int) {
        return 16 * (kb >> 2) + 4 * g + (kb & 3);
    }
    __device__ static __forceinline__ int poff(int kb, int g) { return kperm(kb, g, 0); }
    typedef float frag;
    __device__ static __forceinline__ float to_f(float x) { return x; }
    __device__ static __forceinline__ float from_f(float x) { return x; }
    __device__ static __forceinline__ frag ld(const float* p) { return *p; }
    __device__ static __forceinline__ frag ld_perm(const float* p) { return *p; }
    __device__ static __forceinline__ frag ld_f(const float* p) { return *p; }
    __device__ static __forceinline__ frag zero() { return 0.0f; }
    __device__ static __forceinline__ frag keep_if(frag a, bool keep) { return keep ? a : 0.0f; }
    __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    // An fp32 fragment is 4 bytes per lane, so operands are moved four fragments at a time:
    //   doff(kb, g)    offset in a row contiguous along k of fragment kb's element for lane
    //                  group g.  Products over dk use the permuted order here too, so that
    //                  fragments 4j..4j+3 of a lane are 4 consecutive row elements;
    //   foff(kb, lane) offset of fragment kb's lane element in an array of stored fragments:
    //                  fragments 4j..4j+3 of a lane are adjacent (one 16-byte piece per lane).
    static constexpr int GRP = 4;
    __device__ static __forceinline__ int doff(int kb, int g) { return poff(kb, g); }
    __device__ static __forceinline__ int foff(int kb, int lane) {
        return ((kb >> 2) * 64 + lane) * 4 + (kb & 3);
    }
    __device__ static __forceinline__ void ld_grp(const float* p, frag* f) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
    }
    __device__ static __forceinline__ void st_grp(float* p, const frag* f) {
        *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    }
};

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// Makes a register value opaque to the compiler at this point (an empty asm that "modifies"
// it): nothing derived from it can be computed earlier, and a load that produced it is waited
// for here at the latest.
template <typename T>
__device__ __forceinline__ void reg_fence(T& x) {
    static_assert(sizeof(T) == 16 || sizeof(T) == 4, "16- or 4-byte values");
    if constexpr (sizeof(T) == 16) {
        uint4 u = __builtin_bit_cast(uint4, x);
        asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
        x = __builtin_bit_cast(T, u);
    } else {
        uint32_t u = __builtin_bit_cast(uint32_t, x);
        asm volatile("" : "+v"(u));
        x = __builtin_bit_cast(T, u);
    }
}

// Streaming (nontemporal) 16-byte global accesses, for data a launch touches once: they carry
// the nontemporal cache hint, under which HBM reads and writes stream faster than with the
// default policy (a plain device copy on MI355X: ~6.2 TB/s with the hint, ~4.9 without).
__device__ __forceinline__ float4 ld_stream4(const float* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_stream4(float* p, float4 v) {
    const f32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

// element e of an operand fragment, as stored
__device__ __forceinline__ bf16_t frag_elem(bf16x8 f, int e) { return __builtin_bit_cast(u16x8, f)[e]; }
__device__ __forceinline__ float frag_elem(float f, int) { return f; }

// L2 normalisation of q and k, x / sqrt(|x|^2 + eps): eps keeps a zero vector finite
constexpr float kNormEps = 1e-6f;

// Sum over each aligned group of L lanes (L = 4, 8, 16 or 32), returned to every lane of the
// group: two quad permutations, the half-row and row mirrors (DPP, on the VALU), and for 32
// the gfx950 row swap.  Every lane adds the same two partial sums (in either order), so all
// lanes of a group hold the bitwise-same result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave (lane l gets x_0 + ... + x_l), on the VALU:
// shifts by 1, 2, 4 and 8 lanes inside each row of 16 (DPP row_shr; a lane without a source
// adds 0), then the last lane of rows 0 and 2 added into rows 1 and 3 (row_bcast:15) and the
// last lane of row 1 into rows 2 and 3 (row_bcast:31).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or_zero(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_or_zero<0x111, 0xf>(x);   // row_shr:1
    x += dpp_or_zero<0x112, 0xf>(x);   // row_shr:2
    x += dpp_or_zero<0x114, 0xf>(x);   // row_shr:4
    x += dpp_or_zero<0x118, 0xf>(x);   // row_shr:8
    x += dpp_or_zero<0x142, 0xa>(x);   // row_bcast:15, rows 1 and 3
    x += dpp_or_zero<0x143, 0xc>(x);   // row_bcast:31, rows 2 and 3
    return x;
}

template <int L>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(L == 4 || L == 8 || L == 16 || L == 32, "group size");
    x += dpp_f<0xB1>(x);    // quad_perm [1,0,3,2]: partner lane ^ 1
    x += dpp_f<0x4E>(x);    // quad_perm [2,3,0,1]: partner lane ^ 2
    if constexpr (L >= 8) x += dpp_f<0x141>(x);   // row_half_mirror: the other quad of each 8
    if constexpr (L >= 16) x += dpp_f<0x140>(x);   // row_mirror: the other half of each 16
    if constexpr (L >= 32) {
        // swap odd rows of one copy with even rows of the other: the pair of results holds,
        // in every lane, its own row's value and its partner row's (rows of 16 lanes)
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return x;
}

// group_sum of two and of three independent values, one reduction step of each in turn (the
// DPP reads of one hide the wait states after the adds of the others)
template <int L>
__device__ __forceinline__ void group_sum2(float& x, float& y) {
    static_assert(L == 4 || L == 8 || L == 16 || L == 32, "group size");
    x += dpp_f<0xB1>(x); y += dpp_f<0xB1>(y);
    x += dpp_f<0x4E>(x); y += dpp_f<0x4E>(y);
    if constexpr (L >= 8) { x += dpp_f<0x141>(x); y += dpp_f<0x141>(y); }
    if constexpr (L >= 16) { x += dpp_f<0x140>(x); y += dpp_f<0x140>(y); }
    if constexpr (L >= 32) {
        const auto rx = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        const auto ry = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
        x = __uint_as_float(rx[0]) + __uint_as_float(rx[1]);
        y = __uint_as_float(ry[0]) + __uint_as_float(ry[1]);
    }
}
template <int L>
__device__ __forceinline__ void group_sum3(float& x, float& y, float& z) {
    static_assert(L == 4 || L == 8 || L == 16 || L == 32, "group size");
    x += dpp_f<0xB1>(x); y += dpp_f<0xB1>(y); z += dpp_f<0xB1>(z);
    x += dpp_f<0x4E>(x); y += dpp_f<0x4E>(y); z += dpp_f<0x4E>(z);
    if constexpr (L >= 8) { x += dpp_f<0x141>(x); y += dpp_f<0x141>(y); z += dpp_f<0x141>(z); }
    if constexpr (L >= 16) { x += dpp_f<0x140>(x); y += dpp_f<0x140>(y); z += dpp_f<0x140>(z); }
    if constexpr (L >= 32) {
        const auto rx = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        const auto ry = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
        const auto rz = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
        x = __uint_as_float(rx[0]) + __uint_as_float(rx[1]);
        y = __uint_as_float(ry[0]) + __uint_as_float(ry[1]);
        z = __uint_as_float(rz[0]) + __uint_as_float(rz[1]);
    }
}

// Launches kernel<<<grid, block, 0, s>>>(args...) and returns the status of that launch
// alone.  hipLaunchKernel reports its own failure directly, so an error left pending by
// earlier, unrelated HIP work on the calling thread is neither consumed nor reported as this
// launch's.
template <typename... A>
inline hipError_t launch_kernel(void (*kernel)(A...), dim3 grid, dim3 block, hipStream_t s,
                                A... args) {
    void* argv[sizeof...(A) > 0 ? sizeof...(A) : 1] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s);
}

// Workgroup barrier for LDS traffic: wait until this wave's LDS reads and writes have
// completed, then synchronise the waves.  Unlike __syncthreads() it does not wait for
// outstanding global loads or stores, so prefetches and output stores stay in flight across
// it.  The kernels here exchange data between waves only through LDS.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// fp32 16x16 output tile on the fp32 matrix cores: D = A(16 x K) B(K x 16) + D, with A and B
// read from row-major fp32 LDS blocks (A rows lda apart, B rows ldb apart).  K % 4 == 0.
__device__ __forceinline__ f32x4 mma_tile_f32(const float* A, int lda, const float* B, int ldb,
                                              int K, f32x4 acc, int lane) {
    const int r = lane & 15, kk = lane >> 4;
    for (int k0 = 0; k0 < K; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + k0 + kk], B[(k0 + kk) * ldb + r], acc, 0, 0, 0);
    return acc;
}

}  // namespace gdn
