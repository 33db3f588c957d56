// gdn_decode.hip -- decode-step variants and the T == 0 state copy.
#include "gdn_launch.h"

namespace gdn {

template <int DK, int DV>
static hipError_t run_bf16(const DecodeParams& p, hipStream_t s) { return launch_decode<bf16_t, DK, DV>(p, s); }
template <int DK, int DV>
static hipError_t run_f32(const DecodeParams& p, hipStream_t s) { return launch_decode<float, DK, DV>(p, s); }

hipError_t decode_bf16(int dk, int dv, const DecodeParams& p, hipStream_t s) { GDN_SWITCH_DIMS(dk, dv, run_bf16, p, s) }
hipError_t decode_f32(int dk, int dv, const DecodeParams& p, hipStream_t s) { GDN_SWITCH_DIMS(dk, dv, run_f32, p, s) }

template <int DK, int DV>
static hipError_t run_layers_bf16(const DecodeTable& t, hipStream_t s) { return launch_decode_layers<bf16_t, DK, DV>(t, s); }
template <int DK, int DV>
static hipError_t run_layers_f32(const DecodeTable& t, hipStream_t s) { return launch_decode_layers<float, DK, DV>(t, s); }

hipError_t decode_layers_bf16(int dk, int dv, const DecodeTable& t, hipStream_t s) { GDN_SWITCH_DIMS(dk, dv, run_layers_bf16, t, s) }
hipError_t decode_layers_f32(int dk, int dv, const DecodeTable& t, hipStream_t s) { GDN_SWITCH_DIMS(dk, dv, run_layers_f32, t, s) }

// Grid-stride copy (or zero fill when in == nullptr) of n floats.
__global__ __launch_bounds__(256) void copy_state_kernel(const float* in, float* out, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        out[i] = in ? in[i] : 0.f;
}

hipError_t copy_state(const float* in, float* out, size_t n, hipStream_t s) {
    if (n == 0 || in == out) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    return launch_kernel(copy_state_kernel, dim3((unsigned)blocks), dim3(256), s, in, out, n);
}

}  // namespace gdn
