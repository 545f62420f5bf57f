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
    int64_t units = 0;  // block-loop workgroups: nseg * H * S, or max_pieces * H * S (packed)
    // Document pieces instead of fixed segments: every document is cut into
    // pieces of at most L tokens, laid out longest first by a planning kernel
    // (the host cannot see the document lengths), one workgroup per (piece,
    // head, slice).  Only documents longer than L need segment states.
    int32_t packed = 0;
    int32_t max_pieces = 0;   // bound on the pieces: num_seqs + floor(T / L)
    int32_t state_slots = 0;  // bound on the segment states of the pieces: floor(T / L)
    size_t ws_bytes = 0;
    size_t ws_states_off = 0;
    size_t ws_flags_off = 0;
    size_t ws_pieces_off = 0;  // packed: piece table, 4 int32 per piece
    size_t ws_slots_off = 0;   // packed: state-slot table, 2 int32 per slot
    size_t ws_marker_off = 0;  // header at offset 0 of every workspace: 64-bit key of the forward call
                               // whose states the workspace holds (+0), a backward's reuse decision (+64)
    // The backward runs its two reverse passes in one launch (la_prefill_pair_v2)
    // when the workspace also holds, after ws_bytes, a transposed copy of the
    // segment states (the second pass's): bwd_ws_bytes in all, which is
    // ws_bytes when the plan has no segment states or no transpose-read loop.
    size_t ws_tstates_off = 0;
    size_t bwd_ws_bytes = 0;
    // segment states per head held in the workspace
    int64_t states() const { return packed ? state_slots : nseg - 1; }
};

// Element size of a dtype (0 if unknown).
size_t elem_size(int dtype);

// Planning from shapes only; LA_OK or the status la_prefill would return for
// these shapes.
la_status make_plan(int64_t T, int32_t num_seqs, int32_t H, int32_t d, int32_t block, int dtype,
                    const la_prefill_opts* opts, Plan* out, bool decay = false);

// Full prefill validation (shapes, plan, pointers, alignment, overlap, workspace).
la_status validate_prefill(const void* q, const void* k, const void* v, const void* o, const int32_t* cu, int32_t H,
                           int32_t d, int32_t block, const float* kv_in, const float* kv_out, int32_t num_seqs,
                           int64_t T, int dtype, const void* ws, size_t ws_bytes, const la_prefill_opts* opts,
                           Plan* plan, bool decay = false);

// Backward: outputs (dq, dk, dv, dkv_in) overlap neither an input nor each other.
la_status validate_backward_outputs(const void* q, const void* k, const void* v, const void* dout, const float* kv_in,
                                    const float* dkv_out, const void* dq, const void* dk, const void* dv,
                                    const float* dkv_in, int32_t num_seqs, int32_t H, int32_t d, int64_t T, int dtype);

// [a, a + na) and [b, b + nb) overlap (empty ranges or null pointers never do).
bool overlaps_range(const void* a, size_t na, const void* b, size_t nb);
// A read-only buffer [a, a + na) overlaps one of a prefill's outputs: o, the
// final states (when given) or the plan's workspace.
bool overlaps_outputs(const void* a, size_t na, const void* o, const float* kv_out, const void* ws, const Plan& plan,
                      int64_t T, int32_t num_seqs, int32_t H, int32_t d, int dtype);

la_status validate_decode(const void* q, const void* k, const void* v, const float* S, const void* o,
                          int32_t num_seqs, int32_t H, int32_t d, int dtype);

}  // namespace la
