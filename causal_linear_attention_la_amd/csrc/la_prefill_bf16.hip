// Prefill kernels instantiated for bf16 inputs (bf16 MFMA, fp32 accumulation).
#include "la_launch.h"
#include "la_prefill_launch.inl"

namespace la {
// Explicit instantiations: the host pass otherwise calls, but does not emit,
// the launch stubs of the transpose-read kernels.
template __global__ void v2::la_prefill_main_v2<128, 64, 128, 2, false>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<128, 64, 128, 3, false>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<128, 64, 64, 2, false>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<128, 64, 64, 3, false>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<64, 64, 64, 2, false>(PrefillParams);
template __global__ void v2::la_segment_state_v2<128, 64, 128, false>(PrefillParams);
template __global__ void v2::la_segment_state_v2<128, 64, 64, false>(PrefillParams);
template __global__ void v2::la_segment_state_v2<64, 64, 64, false>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<128, 64, 128, 2, true>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<128, 64, 64, 2, true>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<128, 64, 64, 3, true>(PrefillParams);
template __global__ void v2::la_prefill_main_v2<64, 64, 64, 2, true>(PrefillParams);
template __global__ void v2::la_segment_state_v2<128, 64, 128, true>(PrefillParams);
template __global__ void v2::la_segment_state_v2<128, 64, 64, true>(PrefillParams);
template __global__ void v2::la_segment_state_v2<64, 64, 64, true>(PrefillParams);
template __global__ void v2::la_prefill_main_v2_b128<128, 128>(PrefillParams);
template __global__ void v2::la_prefill_main_v2_b128<128, 64>(PrefillParams);
template __global__ void v2::la_prefill_main_v2_b128<64, 64>(PrefillParams);
template __global__ void v2::la_prefill_pair_v2<128, 64, 128, 2>(PrefillParams, PrefillParams);
template __global__ void v2::la_prefill_pair_v2<128, 64, 128, 3>(PrefillParams, PrefillParams);
template __global__ void v2::la_prefill_pair_v2<128, 64, 64, 2>(PrefillParams, PrefillParams);
template __global__ void v2::la_prefill_pair_v2<128, 64, 64, 3>(PrefillParams, PrefillParams);
template __global__ void v2::la_prefill_pair_v2<64, 64, 64, 2>(PrefillParams, PrefillParams);
template __global__ void v2::la_ws_transpose_v2<128, 128>(const float*, float*, int64_t, const int32_t*);
template __global__ void v2::la_ws_transpose_v2<128, 64>(const float*, float*, int64_t, const int32_t*);
template __global__ void v2::la_ws_transpose_v2<64, 64>(const float*, float*, int64_t, const int32_t*);

hipError_t launch_ws_transpose(const float* src, float* dst, int64_t states, int D, int W, const int32_t* reuse,
                               hipStream_t st) {
    if (states <= 0) return hipSuccess;
    const dim3 grid((unsigned)states), block(kThreads);
    if (D == 128 && W == 128)
        return launch_kernel(v2::la_ws_transpose_v2<128, 128>, grid, block, st, src, dst, states, reuse);
    if (D == 128 && W == 64)
        return launch_kernel(v2::la_ws_transpose_v2<128, 64>, grid, block, st, src, dst, states, reuse);
    if (D == 64 && W == 64) return launch_kernel(v2::la_ws_transpose_v2<64, 64>, grid, block, st, src, dst, states, reuse);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_pair(const PrefillParams& p0, const PrefillParams& p1, int D, int W, int slots,
                               hipStream_t st) {
    // twice the single pass's grid, a multiple of 16 (see la_prefill_pair_v2)
    const dim3 grid((unsigned)(16 * ((p0.units + 7) / 8))), block(kThreads);
    if (D == 128 && W == 128 && slots == 3)
        return launch_kernel(v2::la_prefill_pair_v2<128, 64, 128, 3>, grid, block, st, p0, p1);
    if (D == 128 && W == 128 && slots == 2)
        return launch_kernel(v2::la_prefill_pair_v2<128, 64, 128, 2>, grid, block, st, p0, p1);
    if (D == 128 && W == 64 && slots == 3)
        return launch_kernel(v2::la_prefill_pair_v2<128, 64, 64, 3>, grid, block, st, p0, p1);
    if (D == 128 && W == 64 && slots == 2)
        return launch_kernel(v2::la_prefill_pair_v2<128, 64, 64, 2>, grid, block, st, p0, p1);
    if (D == 64 && W == 64 && slots == 2)
        return launch_kernel(v2::la_prefill_pair_v2<64, 64, 64, 2>, grid, block, st, p0, p1);
    return hipErrorInvalidValue;
}

hipError_t launch_ws_claim(uint64_t* marker, uint64_t key, int32_t* decision, hipStream_t st) {
    return launch_kernel(la_ws_claim_kernel<64>, dim3(1), dim3(64), st, marker, key, decision);
}

hipError_t launch_prefill_bf16(const PrefillParams& p, int D, int B, int W, int variant, hipStream_t st, hipEvent_t e0,
                               hipEvent_t e1) {
    return dispatch_prefill<bf16_t>(p, D, B, W, variant, st, e0, e1);
}
}  // namespace la
