// Prefill kernels instantiated for fp32 inputs (fp32 MFMA).
#include "la_launch.h"
#include "la_prefill_launch.inl"

namespace la {
hipError_t launch_prefill_fp32(const PrefillParams& p, int D, int B, int W, int variant, hipStream_t st, hipEvent_t e0,
                               hipEvent_t e1) {
    return dispatch_prefill<float>(p, D, B, W, variant, st, e0, e1);
}
}  // namespace la
