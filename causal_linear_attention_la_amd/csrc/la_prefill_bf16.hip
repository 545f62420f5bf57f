// Prefill kernels instantiated for bf16 inputs (bf16 MFMA, fp32 accumulation).
#include "la_launch.h"
#include "la_prefill_launch.inl"

namespace la {
hipError_t launch_prefill_bf16(const PrefillParams& p, int D, int B, int W, hipStream_t st, hipEvent_t e0,
                               hipEvent_t e1) {
    return dispatch_prefill<bf16_t>(p, D, B, W, st, e0, e1);
}
}  // namespace la
