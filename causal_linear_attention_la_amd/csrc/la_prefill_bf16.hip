// Prefill kernels instantiated for bf16 inputs (bf16 MFMA, fp32 accumulation).
#include "la_launch.h"
#include "la_prefill_launch.inl"

namespace la {
// Explicit instantiations: the host pass otherwise calls, but does not emit,
// the launch stubs of the transpose-read kernels.
template __global__ void v2::la_prefill_main_v2<128, 64, 128, 2>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<128, 64, 128, 3>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<128, 64, 64, 2>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<128, 64, 64, 3>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<64, 64, 64, 2>(PrefillParams);
template __global__ void v2::la_segment_state_v2<128, 64, 128>(PrefillParams);
template __global__ void v2::la_segment_state_v2<128, 64, 64>(PrefillParams);
template __global__ void v2::la_segment_state_v2<64, 64, 64>(PrefillParams);

hipError_t launch_prefill_bf16(const PrefillParams& p, int D, int B, int W, int variant, hipStream_t st, hipEvent_t e0,
                               hipEvent_t e1) {
    return dispatch_prefill<bf16_t>(p, D, B, W, variant, st, e0, e1);
}
}  // namespace la
