// Host-only validation and planning (see la_host.h).
#include "la_host.h"

#include <algorithm>
#include <climits>

#include "la_tiles.h"

namespace la {

namespace {

constexpr int kNumCUs = 256;      // MI355X compute units
// A dispatch's grid is at most 2^32 - 1 work-items per dimension; the block
// loop and the segment-state kernel launch 8 * ceil(units / 8) workgroups of
// 256 lanes, so a plan may hold at most this many units.
constexpr int64_t kMaxUnits = 8 * (((int64_t)1 << 32) - 1) / (8 * 256);
// The transpose-read kernels address a 64-token block of one head through a
// buffer descriptor: row offsets up to 64 rows of H * d * 2 bytes must fit the
// descriptor's 32-bit range.
constexpr int64_t kMaxBlockBytes = ((int64_t)1 << 32) - 1;
constexpr int kUnitsTarget = 256; // block-loop workgroups to aim for (one per CU)
constexpr int kMinSegment = 256;  // shorter segments spend more on state traffic than they gain
constexpr int kMaxLookback = 16;  // a unit sums at most this many segment states
// The transpose-read loop takes three tile slots (loads two blocks ahead) on
// segments of at least this many blocks; shorter ones start faster with two.
constexpr int kThreeSlotMinBlocks = 16;
constexpr int kShortSegmentBlocks = 12;
// The full-width transpose-read loop sums at most this many on segments of
// more than kThreeSlotMinBlocks blocks.
constexpr int kMaxLookbackWideLong = 8;
// Document pieces are chosen when there are at least as many documents as
// segments per head (the mean document fits one segment, so most documents
// need no segment state), the units stay within a few per CU (each unit pays
// a pipeline start), and no document can need more than kMaxLookback states.
constexpr int kMaxPackedUnitsPerCU = 8;
constexpr int kMaxPackedDocs = 4096;  // the planning kernel: 1024 lanes x 4 documents

bool is_pow2_in(int32_t x, int32_t lo, int32_t hi) {
    if (x < lo || x > hi) return false;
    return (x & (x - 1)) == 0;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [a, a+na) and [b, b+nb) overlap (empty ranges never overlap)
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool mul_ok(int64_t a, int64_t b, int64_t& out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    out = a * b;
    return true;
}

}  // namespace

size_t elem_size(int dtype) { return dtype == LA_BF16 ? 2 : dtype == LA_FP32 ? 4 : 0; }

la_status make_plan(int64_t T, int32_t num_seqs, int32_t H, int32_t d, int32_t block, int dtype,
                    const la_prefill_opts* opts, Plan* out, bool decay) {
    if (H < 1 || num_seqs < 1 || T < 0 || T > INT32_MAX) return LA_ERR_INVALID_ARG;
    const size_t es = elem_size(dtype);
    if (es == 0) return LA_ERR_UNSUPPORTED;
    if (!(d == 16 || d == 32 || d == 64 || d == 128)) return LA_ERR_UNSUPPORTED;
    if (!(block == 32 || block == 64 || block == 128)) return LA_ERR_UNSUPPORTED;

    auto slice_ok = [&](int32_t S) {
        if (S < 1 || d % S != 0) return false;
        return main_fits((int)es, d, block, d / S);
    };
    // the transpose-read block loops: bf16, d >= 64, slices >= 64 columns, 64-token blocks or
    // (plain variant) 128-token blocks, and 64 rows of H * d bf16 (a tile) addressable with
    // 32-bit offsets
    auto v2_ok = [&](int32_t S) {
        if (dtype != LA_BF16 || d < 64 || S < 1 || d % S != 0 || (int64_t)H * d * 2 * 64 > kMaxBlockBytes)
            return false;
        return d / S >= 64 && (block == 64 || (block == 128 && !decay));
    };
    const int32_t variant = opts ? opts->variant : 0;
    if (variant < 0 || variant > 2) return LA_ERR_UNSUPPORTED;

    Plan p;
    const int64_t work = T * (int64_t)H;
    if (opts && opts->value_slices != 0) {
        if (!is_pow2_in(opts->value_slices, 1, 4) ||
            !(slice_ok(opts->value_slices) || (variant != 1 && v2_ok(opts->value_slices))))
            return LA_ERR_UNSUPPORTED;
        p.S = opts->value_slices;
    } else if (block == 128 && variant != 1 && v2_ok(1)) {
        // the 128-token transpose-read loop at full width (faster than 64-column
        // slices: long_1m 2.64 against 3.08 ms per call)
        p.S = 1;
    } else {
        int32_t chosen = 0;
        const bool want_v2 = variant != 1 && v2_ok(1);
        for (int32_t S = 1; S <= 4; S *= 2) {
            if (!slice_ok(S)) continue;
            if (want_v2 && !v2_ok(S)) break;  // keep the faster loop rather than split further
            chosen = S;
            if (work * S / kUnitsTarget >= kMinSegment) break;
        }
        if (chosen == 0) return LA_ERR_UNSUPPORTED;
        p.S = chosen;
    }
    p.W = d / p.S;
    if (variant == 2 && !v2_ok(p.S)) return LA_ERR_UNSUPPORTED;
    p.variant = (variant == 0 ? v2_ok(p.S) : variant == 2) ? 2 : 1;  // the loop that will run

    // Look-back or scan for segments of length L.  Without the scan a unit
    // that starts inside a document sums the states of that document's
    // earlier segments in its prologue, on its own critical path; the
    // segments of one head run on one XCD, so after the first unit those
    // states come from that XCD's L2.  Measured against the scan's extra
    // launch: the look-back wins up to 15 predecessors on both block loops
    // (3-16 %) and loses slightly (1-4 %) at 31; on the full-width loop with
    // long segments it still wins at 7 (5 %) but not at 15 (16 x 65536
    // tokens: 2.5 % slower).  The longest document is estimated from the
    // mean length.
    auto needs_scan = [&](int64_t L, int32_t W) {
        const int64_t ns = T == 0 ? 1 : (T + L - 1) / L;
        if (ns <= 1) return false;
        const int64_t mean_len = (T + num_seqs - 1) / num_seqs;
        const int64_t span = std::min<int64_t>(ns, num_seqs == 1 ? ns : (mean_len + L - 1) / L + 1);
        const bool wide_long = p.variant == 2 && W >= 128 && L / block > kThreeSlotMinBlocks;
        return ns - 1 > kMaxLookback || span - 1 > (wide_long ? kMaxLookbackWideLong : kMaxLookback);
    };

    if (opts && opts->seg_len != 0) {
        if (opts->seg_len < block || opts->seg_len % block != 0) return LA_ERR_UNSUPPORTED;
        p.L = opts->seg_len;
    } else {
        int64_t L = work * p.S / kUnitsTarget;
        L = (L / block) * block;
        int64_t floor_len = T < kMinSegment ? T : kMinSegment;
        floor_len = ((floor_len + block - 1) / block) * block;
        if (L < floor_len) L = floor_len;
        if (L < block) L = block;
        if (L > INT32_MAX / 2) L = (INT32_MAX / 2 / block) * block;
        // Segments of at most kShortSegmentBlocks blocks: two value slices with
        // twice the segment length keep the unit count and halve the segments
        // per document, which is faster while segments are this short (the
        // 64-column loop is the quicker one per block, and it needs no scan
        // where the full width would): 8192 tokens x 8 heads 44.9 -> 34.6 us
        // per call, 2048 x 32 36.6 -> 31.1, 16384 x 8 62.3 -> 56.7, 24576 x 8
        // (12 blocks) 80.9 -> 75.8; at 16 blocks it loses (32768 x 8: 101.8
        // -> 103.2).
        const bool auto_s = !(opts && opts->value_slices != 0);
        if (auto_s && !(opts && opts->force_scan) && p.variant == 2 && L / block <= kShortSegmentBlocks &&
            slice_ok(2 * p.S) && v2_ok(2 * p.S) && 2 * L <= INT32_MAX / 2 && !needs_scan(2 * L, d / (2 * p.S))) {
            p.S *= 2;
            p.W = d / p.S;
            L *= 2;
        }
        p.L = (int32_t)L;
    }
    const int64_t nseg = T == 0 ? 1 : (T + p.L - 1) / p.L;
    if (nseg > INT32_MAX) return LA_ERR_UNSUPPORTED;
    p.nseg = (int32_t)nseg;
    p.units = nseg * (int64_t)H * p.S;
    const int32_t work_list = opts ? opts->work_list : 0;
    if (work_list < 0 || work_list > 2) return LA_ERR_UNSUPPORTED;
    {
        const int64_t pieces = (int64_t)num_seqs + T / p.L;
        const bool fits = T > 0 && num_seqs <= kMaxPackedDocs && nseg - 1 <= kMaxLookback &&
                          pieces * H * p.S <= kMaxUnits && !(opts && opts->force_scan);
        const bool want = num_seqs > 1 && num_seqs >= nseg && pieces * H * p.S <= (int64_t)kMaxPackedUnitsPerCU * kNumCUs;
        if (work_list == 2 && !fits) return LA_ERR_UNSUPPORTED;
        if (fits && (work_list == 2 || (work_list == 0 && want))) {
            p.packed = 1;
            p.max_pieces = (int32_t)pieces;
            p.state_slots = (int32_t)(T / p.L);
            p.units = pieces * H * p.S;
        }
    }
    if (p.units > kMaxUnits) return LA_ERR_UNSUPPORTED;
    p.scan = !p.packed && p.nseg > 1 && ((opts && opts->force_scan) || needs_scan(p.L, p.W)) ? 1 : 0;
    // the scan kernel runs one lane per 4 state entries of a segment (H * d * d entries)
    if (p.scan && (int64_t)H * d * d / 4 > (((int64_t)1 << 32) - 1)) return LA_ERR_UNSUPPORTED;
    const int32_t slots = opts ? opts->slots : 0;
    if (!(slots == 0 || slots == 2 || slots == 3)) return LA_ERR_UNSUPPORTED;
    if (p.variant == 2 && block == 128) {
        // the 128-token loop always runs three slots (one block's two halves and the next block's first)
        if (slots == 2) return LA_ERR_UNSUPPORTED;
        p.slots = 3;
    } else {
        // (the decayed full-width loop has no registers for a third slot)
        const bool three_ok = p.variant == 2 && d == 128 && !(decay && p.W == 128);
        if (slots == 3 && !three_ok) return LA_ERR_UNSUPPORTED;
        if (slots != 0) p.slots = slots;
        else p.slots = three_ok && p.L / block >= kThreeSlotMinBlocks ? 3 : 2;
        if (p.variant != 2) p.slots = 2;  // (the generic loop has no slot choice)
    }

    // Workspace: a 256-byte header at offset 0 whatever the plan (the stamp of
    // the forward call whose segment states it holds, and a backward's reuse
    // decision), then the states and the plan's tables.
    auto round256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    constexpr size_t kHeader = 256;
    if (p.packed) {
        int64_t states;
        if (!mul_ok(std::max<int64_t>(p.state_slots, 1), (int64_t)H * d * d, states) || !mul_ok(states, 4, states))
            return LA_ERR_UNSUPPORTED;
        p.ws_states_off = kHeader;
        p.ws_flags_off = kHeader + round256((size_t)states);
        p.ws_pieces_off = p.ws_flags_off + 256;
        p.ws_slots_off = p.ws_pieces_off + round256((size_t)p.max_pieces * 16);
        p.ws_bytes = p.ws_slots_off + round256((size_t)std::max(p.state_slots, 1) * 8);
    } else if (p.nseg > 1) {
        int64_t states;
        if (!mul_ok(nseg, (int64_t)H * d * d, states) || !mul_ok(states, 4, states)) return LA_ERR_UNSUPPORTED;
        p.ws_states_off = kHeader;
        p.ws_flags_off = kHeader + round256((size_t)states);
        p.ws_bytes = p.ws_flags_off + round256((size_t)nseg * 4);
    }
    p.ws_marker_off = 0;
    p.bwd_ws_bytes = p.ws_bytes;
    if (p.variant == 2 && p.states() > 0) {
        int64_t states;
        if (!mul_ok(p.states(), (int64_t)H * d * d, states) || !mul_ok(states, 4, states)) return LA_ERR_UNSUPPORTED;
        p.ws_tstates_off = round256(p.ws_bytes);
        p.bwd_ws_bytes = p.ws_tstates_off + round256((size_t)states);
    }
    *out = p;
    return LA_OK;
}

la_status validate_prefill(const void* q, const void* k, const void* v, const void* o, const int32_t* cu, int32_t H,
                           int32_t d, int32_t block, const float* kv_in, const float* kv_out, int32_t num_seqs,
                           int64_t T, int dtype, const void* ws, size_t ws_bytes, const la_prefill_opts* opts,
                           Plan* plan, bool decay) {
    if (!q || !k || !v || !o || !cu) return LA_ERR_INVALID_ARG;
    la_status st = make_plan(T, num_seqs, H, d, block, dtype, opts, plan, decay);
    if (st != LA_OK) return st;
    const size_t es = elem_size(dtype);
    int64_t n;
    if (!mul_ok(T, (int64_t)H * d, n) || !mul_ok(n, (int64_t)es, n)) return LA_ERR_INVALID_ARG;
    const size_t tensor = (size_t)n;
    int64_t ns;
    if (!mul_ok(num_seqs, (int64_t)H * d * d, ns) || !mul_ok(ns, 4, ns)) return LA_ERR_INVALID_ARG;
    const size_t state = (size_t)ns;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(cu, 4))
        return LA_ERR_INVALID_ARG;
    if (kv_out && !aligned(kv_out, 16)) return LA_ERR_INVALID_ARG;
    if (kv_in && !aligned(kv_in, 16)) return LA_ERR_INVALID_ARG;
    // the incoming states are read while outputs are written: no overlap with any output
    if (kv_in && (overlap(kv_in, state, o, tensor) || overlap(kv_in, state, kv_out, state)))
        return LA_ERR_INVALID_ARG;
    if (overlap(o, tensor, q, tensor) || overlap(o, tensor, k, tensor) || overlap(o, tensor, v, tensor))
        return LA_ERR_INVALID_ARG;
    if (kv_out && (overlap(kv_out, state, q, tensor) || overlap(kv_out, state, k, tensor) ||
                   overlap(kv_out, state, v, tensor) || overlap(kv_out, state, o, tensor)))
        return LA_ERR_INVALID_ARG;
    if (plan->ws_bytes > 0) {
        if (!ws || ws_bytes < plan->ws_bytes) return LA_ERR_WORKSPACE;
        if (!aligned(ws, 256)) return LA_ERR_INVALID_ARG;
        const size_t wn = plan->ws_bytes;
        if (overlap(ws, wn, q, tensor) || overlap(ws, wn, k, tensor) || overlap(ws, wn, v, tensor) ||
            overlap(ws, wn, o, tensor) || (kv_out && overlap(ws, wn, kv_out, state)) ||
            (kv_in && overlap(ws, wn, kv_in, state)))
            return LA_ERR_INVALID_ARG;
    }
    return LA_OK;
}

la_status validate_backward_outputs(const void* q, const void* k, const void* v, const void* dout, const float* kv_in,
                                    const float* dkv_out, const void* dq, const void* dk, const void* dv,
                                    const float* dkv_in, int32_t num_seqs, int32_t H, int32_t d, int64_t T, int dtype) {
    int64_t n, ns;
    if (!mul_ok(T, (int64_t)H * d, n) || !mul_ok(n, (int64_t)elem_size(dtype), n)) return LA_ERR_INVALID_ARG;
    if (!mul_ok(num_seqs, (int64_t)H * d * d, ns) || !mul_ok(ns, 4, ns)) return LA_ERR_INVALID_ARG;
    const size_t tn = (size_t)n, sn = (size_t)ns;
    const void* ins[6] = {q, k, v, dout, kv_in, dkv_out};
    const size_t in_sz[6] = {tn, tn, tn, tn, sn, sn};
    const void* outs[4] = {dq, dk, dv, dkv_in};
    const size_t out_sz[4] = {tn, tn, tn, sn};
    for (int a = 0; a < 4; ++a) {
        for (int b = 0; b < 6; ++b)
            if (overlap(outs[a], out_sz[a], ins[b], in_sz[b])) return LA_ERR_INVALID_ARG;
        for (int b = a + 1; b < 4; ++b)
            if (overlap(outs[a], out_sz[a], outs[b], out_sz[b])) return LA_ERR_INVALID_ARG;
    }
    if (dkv_in && !aligned(dkv_in, 16)) return LA_ERR_INVALID_ARG;
    return LA_OK;
}

bool overlaps_range(const void* a, size_t na, const void* b, size_t nb) { return overlap(a, na, b, nb); }

bool overlaps_outputs(const void* a, size_t na, const void* o, const float* kv_out, const void* ws, const Plan& plan,
                      int64_t T, int32_t num_seqs, int32_t H, int32_t d, int dtype) {
    const size_t tensor = (size_t)T * H * d * elem_size(dtype);
    const size_t state = (size_t)num_seqs * H * d * d * 4;
    return overlap(a, na, o, tensor) || overlap(a, na, kv_out, state) || overlap(a, na, ws, plan.ws_bytes);
}

la_status validate_decode(const void* q, const void* k, const void* v, const float* S, const void* o,
                          int32_t num_seqs, int32_t H, int32_t d, int dtype) {
    if (!q || !k || !v || !S || !o) return LA_ERR_INVALID_ARG;
    if (num_seqs < 1 || H < 1) return LA_ERR_INVALID_ARG;
    const size_t es = elem_size(dtype);
    if (es == 0) return LA_ERR_UNSUPPORTED;
    if (!(d == 16 || d == 32 || d == 64 || d == 128)) return LA_ERR_UNSUPPORTED;
    int64_t pairs, n, ns;
    if (!mul_ok(num_seqs, H, pairs) || !mul_ok(pairs, (int64_t)d * es, n) || !mul_ok(pairs, (int64_t)d * d * 4, ns))
        return LA_ERR_INVALID_ARG;
    // one 256-lane workgroup per (sequence, head): the grid's work-items must fit 32 bits
    if (pairs * 256 > (((int64_t)1 << 32) - 1)) return LA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(S, 16) || !aligned(o, 16))
        return LA_ERR_INVALID_ARG;
    const size_t tn = (size_t)n, sn = (size_t)ns;
    if (overlap(o, tn, q, tn) || overlap(o, tn, k, tn) || overlap(o, tn, v, tn) || overlap(o, tn, S, sn) ||
        overlap(S, sn, q, tn) || overlap(S, sn, k, tn) || overlap(S, sn, v, tn))
        return LA_ERR_INVALID_ARG;
    return LA_OK;
}

}  // namespace la
