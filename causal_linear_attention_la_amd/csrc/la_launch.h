// Internal launch entry points (one translation unit per dtype / kernel family).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "la_decode_kernels.h"
#include "la_prefill_kernels.h"
#include "la_prefill_v2.h"

namespace la {

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
// workspace in place (la_ws_transpose_v2); D, W as in that plan.
hipError_t launch_ws_transpose(float* ws, int64_t states, int D, int W, hipStream_t st);

}  // namespace la
