// Internal launch entry points (one translation unit per dtype / kernel family).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "la_decode_kernels.h"
#include "la_prefill_kernels.h"
#include "la_prefill_v2.h"

namespace la {

template <class T>
struct nodeduce {
    using type = T;
};

// Launches `kernel` and returns the status of this launch alone.  (After a
// `<<<...>>>` launch the only check is hipGetLastError, which also reports
// errors that earlier calls on the thread left behind -- another library's
// failed query, say -- and would make a good launch look failed.)
template <typename... KArgs>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                                typename nodeduce<KArgs>::type... args) {
    void* ptrs[] = {static_cast<void*>(&args)..., nullptr};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, st);
}

// Enqueues the prefill kernels for one plan: segment states (nseg > 1), prefix
// scan (scan != 0), then the block loop bracketed by the optional events.
// variant: 0 = automatic, 1 = reference block loop, 2 = transpose-read block
// loop (bf16, d >= 64, block 64, slices >= 64 columns only).
hipError_t launch_prefill_bf16(const PrefillParams& p, int D, int B, int W, int variant, hipStream_t st,
                               hipEvent_t ev_begin, hipEvent_t ev_end);
hipError_t launch_prefill_fp32(const PrefillParams& p, int D, int B, int W, int variant, hipStream_t st,
                               hipEvent_t ev_begin, hipEvent_t ev_end);
hipError_t launch_decode(const DecodeParams& p, int D, int dtype, hipStream_t st);
// Transposes the first `states` segment states of a transpose-read plan's
// workspace from src into dst, which may be src itself (la_ws_transpose_v2);
// D, W as in that plan.  With `reuse` non-null, only if *reuse is 1 when the
// kernel runs.
hipError_t launch_ws_transpose(const float* src, float* dst, int64_t states, int D, int W, const int32_t* reuse,
                               hipStream_t st);
// The block loops of two transpose-read passes with the same plan (bf16,
// block 64; W and slots as in that plan) in one launch (la_prefill_pair_v2).
hipError_t launch_prefill_pair(const PrefillParams& p0, const PrefillParams& p1, int D, int W, int slots,
                               hipStream_t st);
// Compares the workspace's stamped key with `key`, writes the result (1 or 0)
// to *decision and clears the stamp (la_ws_claim_kernel).
hipError_t launch_ws_claim(uint64_t* marker, uint64_t key, int32_t* decision, hipStream_t st);

}  // namespace la
