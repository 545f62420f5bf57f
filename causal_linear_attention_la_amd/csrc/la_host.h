// Host-only argument validation and work planning for the C ABI.  Pure C++
// (no HIP): built into the library and, separately, into a sanitizer-checked
// host test.
#pragma once
#include <cstddef>
#include <cstdint>

#include "../../include/la.h"

namespace la {

struct Plan {
    int32_t L = 0;      // segment length
    int32_t S = 1;      // value slices
    int32_t W = 0;      // value-slice width d / S
    int32_t nseg = 1;
    int32_t scan = 0;   // run the prefix-scan kernel
    int32_t variant = 1;  // block loop: 1 generic, 2 transpose-read
    int32_t slots = 2;    // tile slots of the transpose-read loop
    int64_t units = 0;  // nseg * H * S
    size_t ws_bytes = 0;
    size_t ws_states_off = 0;
    size_t ws_flags_off = 0;
};

// Element size of a dtype (0 if unknown).
size_t elem_size(int dtype);

// Planning from shapes only; LA_OK or the status la_prefill would return for
// these shapes.
la_status make_plan(int64_t T, int32_t num_seqs, int32_t H, int32_t d, int32_t block, int dtype,
                    const la_prefill_opts* opts, Plan* out);

// Full prefill validation (shapes, plan, pointers, alignment, overlap, workspace).
la_status validate_prefill(const void* q, const void* k, const void* v, const void* o, const int32_t* cu, int32_t H,
                           int32_t d, int32_t block, const float* kv_in, const float* kv_out, int32_t num_seqs,
                           int64_t T, int dtype, const void* ws, size_t ws_bytes, const la_prefill_opts* opts,
                           Plan* plan);

// Backward: outputs (dq, dk, dv, dkv_in) overlap neither an input nor each other.
la_status validate_backward_outputs(const void* q, const void* k, const void* v, const void* dout, const float* kv_in,
                                    const float* dkv_out, const void* dq, const void* dk, const void* dv,
                                    const float* dkv_in, int32_t num_seqs, int32_t H, int32_t d, int64_t T, int dtype);

la_status validate_decode(const void* q, const void* k, const void* v, const float* S, const void* o,
                          int32_t num_seqs, int32_t H, int32_t d, int dtype);

}  // namespace la
