// gdn_sequential.hip -- token-sequential prefill variants (see gdn_sequential.h).
#include "gdn_launch.h"
#include "gdn_sequential.h"

namespace gdn {

template <int DK, int DV>
static hipError_t run_bf16(const PrefillParams& p, hipStream_t s) { return launch_sequential<bf16_t, DK, DV>(p, s); }
template <int DK, int DV>
static hipError_t run_f32(const PrefillParams& p, hipStream_t s) { return launch_sequential<float, DK, DV>(p, s); }

hipError_t sequential_bf16(int dk, int dv, const PrefillParams& p, hipStream_t s) { GDN_SWITCH_DIMS(dk, dv, run_bf16, p, s) }
hipError_t sequential_f32(int dk, int dv, const PrefillParams& p, hipStream_t s) { GDN_SWITCH_DIMS(dk, dv, run_f32, p, s) }

}  // namespace gdn
