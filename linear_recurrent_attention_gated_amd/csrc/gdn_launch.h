// gdn_launch.h -- internal dispatch from run-time sizes to the compiled kernel variants.
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_decode.h"
#include "gdn_prefill.h"

namespace gdn {

// One entry per (element type, chunk); each switches on (dk, dv).  `stages`: bit 1 runs the
// intra-chunk kernel, bit 2 the inter-chunk kernel.  Return hipErrorInvalidValue
// for a (dk, dv) pair that was not compiled (the API validates before calling).
hipError_t prefill_bf16_c16(int dk, int dv, const PrefillParams& p, int stages, hipStream_t s);
hipError_t prefill_bf16_c32(int dk, int dv, const PrefillParams& p, int stages, hipStream_t s);
hipError_t prefill_bf16_c64(int dk, int dv, const PrefillParams& p, int stages, hipStream_t s);
hipError_t prefill_f32_c16(int dk, int dv, const PrefillParams& p, int stages, hipStream_t s);
hipError_t prefill_f32_c32(int dk, int dv, const PrefillParams& p, int stages, hipStream_t s);
hipError_t prefill_f32_c64(int dk, int dv, const PrefillParams& p, int stages, hipStream_t s);

// Token-sequential prefill (gdn_sequential.h); uses the q, k, v, g, beta, state, o, size,
// Ts / t0 and qk_norm fields of p, no workspace.
hipError_t sequential_bf16(int dk, int dv, const PrefillParams& p, hipStream_t s);
hipError_t sequential_f32(int dk, int dv, const PrefillParams& p, hipStream_t s);

hipError_t decode_bf16(int dk, int dv, const DecodeParams& p, hipStream_t s);
hipError_t decode_f32(int dk, int dv, const DecodeParams& p, hipStream_t s);

// One launch over up to kDecodeLayersPerLaunch layers (gdn_decode.h).
hipError_t decode_layers_bf16(int dk, int dv, const DecodeTable& t, hipStream_t s);
hipError_t decode_layers_f32(int dk, int dv, const DecodeTable& t, hipStream_t s);

// T == 0: state_out <- state_in (or zeros).
hipError_t copy_state(const float* in, float* out, size_t n, hipStream_t s);

}  // namespace gdn

// Expands to a switch over the supported head dimensions calling FN<DK, DV>(args...).
#define GDN_SWITCH_DIMS(dk, dv, FN, ...)                                        \
    switch ((dk) * 1000 + (dv)) {                                               \
        case 32032: return FN<32, 32>(__VA_ARGS__);                             \
        case 32064: return FN<32, 64>(__VA_ARGS__);                             \
        case 32128: return FN<32, 128>(__VA_ARGS__);                            \
        case 64032: return FN<64, 32>(__VA_ARGS__);                             \
        case 64064: return FN<64, 64>(__VA_ARGS__);                             \
        case 64128: return FN<64, 128>(__VA_ARGS__);                            \
        case 128032: return FN<128, 32>(__VA_ARGS__);                           \
        case 128064: return FN<128, 64>(__VA_ARGS__);                           \
        case 128128: return FN<128, 128>(__VA_ARGS__);                          \
        default: return hipErrorInvalidValue;                                   \
    }
