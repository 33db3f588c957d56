// gdn_prefill_inst.hip -- compiled once per (element type, chunk) pair:
//   -DGDN_ELEM_BF16=1|0  -DGDN_CHUNK=16|32|64
// so the variants build in parallel; each object defines one dispatch entry of
// gdn_launch.h.
#include "gdn_launch.h"

#if GDN_ELEM_BF16
#define GDN_E bf16_t
#define GDN_TAG bf16
#else
#define GDN_E float
#define GDN_TAG f32
#endif
#define GDN_FN_(t, c) prefill_##t##_c##c
#define GDN_FN(t, c) GDN_FN_(t, c)

namespace gdn {

template <int DK, int DV>
static hipError_t run(const PrefillParams& p, int stages, hipStream_t s) {
    return launch_prefill<GDN_E, DK, DV, GDN_CHUNK>(p, stages, s);
}

hipError_t GDN_FN(GDN_TAG, GDN_CHUNK)(int dk, int dv, const PrefillParams& p, int stages,
                                     hipStream_t s) {
    GDN_SWITCH_DIMS(dk, dv, run, p, stages, s)
}

}  // namespace gdn
