// Internal launch entry points (one translation unit per dtype / kernel family).
#pragma once
#include <hip/hip_runtime.h>

#include "la_decode_kernels.h"
#include "la_prefill_kernels.h"

namespace la {

// Enqueues the prefill kernels for one plan: segment states (nseg > 1), prefix
// scan (scan != 0), then the block loop bracketed by the optional events.
hipError_t launch_prefill_bf16(const PrefillParams& p, int D, int B, int W, hipStream_t st, hipEvent_t ev_begin,
                               hipEvent_t ev_end);
hipError_t launch_prefill_fp32(const PrefillParams& p, int D, int B, int W, hipStream_t st, hipEvent_t ev_begin,
                               hipEvent_t ev_end);
hipError_t launch_decode(const DecodeParams& p, int D, int dtype, hipStream_t st);

}  // namespace la
