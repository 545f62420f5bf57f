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
template __global__ void v2::la_ws_transpose_v2<128, 128>(float*, int64_t);
template __global__ void v2::la_ws_transpose_v2<128, 64>(float*, int64_t);
template __global__ void v2::la_ws_transpose_v2<64, 64>(float*, int64_t);

hipError_t launch_ws_transpose(float* ws, int64_t states, int D, int W, hipStream_t st) {
    if (states <= 0) return hipSuccess;
    const dim3 grid((unsigned)states), block(kThreads);
    if (D == 128 && W == 128) return launch_kernel(v2::la_ws_transpose_v2<128, 128>, grid, block, st, ws, states);
    if (D == 128 && W == 64) return launch_kernel(v2::la_ws_transpose_v2<128, 64>, grid, block, st, ws, states);
    if (D == 64 && W == 64) return launch_kernel(v2::la_ws_transpose_v2<64, 64>, grid, block, st, ws, states);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16(const PrefillParams& p, int D, int B, int W, int variant, hipStream_t st, hipEvent_t e0,
                               hipEvent_t e1) {
    return dispatch_prefill<bf16_t>(p, D, B, W, variant, st, e0, e1);
}
}  // namespace la
