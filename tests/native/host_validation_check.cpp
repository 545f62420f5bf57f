// Host-only checks of argument validation and planning, built with
// -fsanitize=address,undefined by tests/test_abi.py (no GPU, no HIP).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <climits>
#include <initializer_list>

#include "../../causal_linear_attention_la_amd/csrc/la_host.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                \
        }                                                              \
    } while (0)

static void* P(uintptr_t x) { return reinterpret_cast<void*>(x); }

int main() {
    using namespace la;
    Plan p;
    const uintptr_t G = 1ull << 40;  // fake, never dereferenced
    void *q = P(G), *k = P(2 * G), *v = P(3 * G), *o = P(4 * G);
    const int32_t* cu = static_cast<const int32_t*>(P(5 * G));
    float* kv = static_cast<float*>(P(6 * G));
    void* ws = P(7 * G);

    // plans for the standard shapes
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK);
    EXPECT(p.L % 64 == 0 && p.units == (int64_t)p.nseg * 8 * p.S && p.W * p.S == 128);
    EXPECT(make_plan(256, 1, 2, 16, 32, LA_FP32, nullptr, &p) == LA_OK && p.nseg == 1 && p.ws_bytes == 0);
    // 128-token blocks: the transpose-read loop at full width with three slots; the generic loop
    // (32-column slices, the widest whose tiles fit) when asked for, or for the decayed variant
    EXPECT(make_plan(1048576, 1, 8, 128, 128, LA_BF16, nullptr, &p) == LA_OK && p.W == 128 && p.variant == 2 &&
           p.slots == 3 && p.L % 128 == 0);
    {
        la_prefill_opts o1{};
        o1.variant = 1;
        EXPECT(make_plan(1048576, 1, 8, 128, 128, LA_BF16, &o1, &p) == LA_OK && p.W == 32 && p.variant == 1);
        EXPECT(make_plan(1048576, 1, 8, 128, 128, LA_BF16, nullptr, &p, true) == LA_OK && p.variant == 1);
        la_prefill_opts o2{};
        o2.slots = 2;
        EXPECT(make_plan(1048576, 1, 8, 128, 128, LA_BF16, &o2, &p) == LA_ERR_UNSUPPORTED);
        la_prefill_opts o3{};
        o3.value_slices = 1;  // full width: the transpose-read loop only (the generic loop's tiles do not fit)
        EXPECT(make_plan(8192, 1, 8, 128, 128, LA_BF16, &o3, &p) == LA_OK && p.W == 128 && p.variant == 2 &&
               p.slots == 3);
        o3.variant = 1;
        EXPECT(make_plan(8192, 1, 8, 128, 128, LA_BF16, &o3, &p) == LA_ERR_UNSUPPORTED);
        EXPECT(make_plan(8192, 1, 8, 64, 128, LA_BF16, nullptr, &p) == LA_OK && p.W == 64 && p.variant == 2);
        la_prefill_opts o4{};
        o4.value_slices = 2;
        EXPECT(make_plan(8192, 1, 8, 128, 128, LA_BF16, &o4, &p) == LA_OK && p.W == 64 && p.variant == 2);
        o4.variant = 1;
        EXPECT(make_plan(8192, 1, 8, 128, 128, LA_BF16, &o4, &p) == LA_ERR_UNSUPPORTED);
    }
    EXPECT(make_plan(0, 3, 4, 64, 64, LA_BF16, nullptr, &p) == LA_OK && p.nseg == 1 && p.units == 4 * p.S);
    // every (d, block, dtype) combination has some plan
    for (int d : {16, 32, 64, 128})
        for (int b : {32, 64, 128})
            for (int dt : {0, 1}) {
                la_status st = make_plan(5000, 3, 4, d, b, dt, nullptr, &p);
                bool fp32_big = (dt == 1 && d >= 64 && b == 128);
                EXPECT(fp32_big ? st == LA_ERR_UNSUPPORTED : st == LA_OK);
            }
    // explicit knobs
    la_prefill_opts o1{};
    o1.seg_len = 64;
    o1.value_slices = 4;
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, &o1, &p) == LA_OK && p.L == 64 && p.S == 4 && p.nseg == 128 && p.scan == 1);
    o1.seg_len = 96;
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, &o1, &p) == LA_ERR_UNSUPPORTED);
    o1.seg_len = 0;
    o1.value_slices = 3;
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, &o1, &p) == LA_ERR_UNSUPPORTED);
    o1.value_slices = 8;
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, &o1, &p) == LA_ERR_UNSUPPORTED);
    // segments of up to 12 blocks go to two slices of twice the length
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.S == 2 && p.L == 512 && p.nseg == 16 &&
           p.scan == 0 && p.units == 256);
    EXPECT(make_plan(16384, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.S == 2 && p.L == 1024 && p.scan == 0);
    EXPECT(make_plan(24576, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.S == 2 && p.L == 1536 && p.scan == 0);
    EXPECT(make_plan(32768, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.S == 1 && p.L == 1024 && p.scan == 1);
    EXPECT(make_plan(4096, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.S == 2 && p.L == 256 && p.scan == 0);
    EXPECT(make_plan(12288, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.S == 2 && p.L == 768 && p.scan == 0);
    // look-back up to 16 predecessors (8 on the full-width loop with long segments), the scan beyond
    EXPECT(make_plan(4096, 1, 32, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.W == 64 && p.nseg == 4 && p.scan == 0);
    EXPECT(make_plan(8192, 1, 16, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.W == 64 && p.nseg == 8 && p.scan == 0);
    EXPECT(make_plan(8192, 1, 32, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.W == 128 && p.nseg == 8 && p.scan == 0);
    la_prefill_opts o5{};
    o5.seg_len = 512;
    o5.value_slices = 1;
    EXPECT(make_plan(8704, 1, 16, 128, 64, LA_BF16, &o5, &p) == LA_OK && p.W == 128 && p.nseg == 17 && p.scan == 0);
    EXPECT(make_plan(9216, 1, 16, 128, 64, LA_BF16, &o5, &p) == LA_OK && p.W == 128 && p.nseg == 18 && p.scan == 1);
    o5.value_slices = 2;
    EXPECT(make_plan(8704, 1, 16, 128, 64, LA_BF16, &o5, &p) == LA_OK && p.W == 64 && p.nseg == 17 && p.scan == 0);
    EXPECT(make_plan(9216, 1, 16, 128, 64, LA_BF16, &o5, &p) == LA_OK && p.W == 64 && p.nseg == 18 && p.scan == 1);
    EXPECT(make_plan(2048, 1, 32, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.S == 2 && p.L == 512 && p.scan == 0);
    EXPECT(make_plan(4096, 1, 16, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.S == 2 && p.L == 512 && p.scan == 0);
    EXPECT(make_plan(4096, 1, 64, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.W == 128 && p.nseg == 4 && p.scan == 0);
    EXPECT(make_plan(65536, 64, 16, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.nseg == 16 && p.scan == 0);
    EXPECT(make_plan(65536, 1, 16, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.nseg == 16 && p.scan == 1);
    EXPECT(make_plan(16384, 1, 16, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.L == 1024 && p.scan == 0);
    EXPECT(make_plan(16384, 1, 32, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.L == 2048 && p.nseg == 8 && p.scan == 0);
    la_prefill_opts o4{};
    o4.force_scan = 1;
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, &o4, &p) == LA_OK && p.S == 1 && p.L == 256 && p.scan == 1);
    o4.force_scan = 0;
    o4.variant = 1;
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, &o4, &p) == LA_OK && p.S == 1 && p.L == 256);
    // tile slots: three on long segments of the d = 128 transpose-read loop, two otherwise
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.slots == 2);
    EXPECT(make_plan(1048576, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.slots == 3);
    EXPECT(make_plan(1048576, 1, 8, 64, 64, LA_BF16, nullptr, &p) == LA_OK && p.slots == 2);
    EXPECT(make_plan(1048576, 1, 8, 128, 64, LA_FP32, nullptr, &p) == LA_OK && p.slots == 2);
    la_prefill_opts o3{};
    o3.slots = 3;
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, &o3, &p) == LA_OK && p.slots == 3);
    EXPECT(make_plan(8192, 1, 8, 64, 64, LA_BF16, &o3, &p) == LA_ERR_UNSUPPORTED);
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_FP32, &o3, &p) == LA_ERR_UNSUPPORTED);
    o3.variant = 1;
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, &o3, &p) == LA_ERR_UNSUPPORTED);
    o3.variant = 0;
    o3.slots = 2;
    EXPECT(make_plan(1048576, 1, 8, 128, 64, LA_BF16, &o3, &p) == LA_OK && p.slots == 2);
    o3.slots = 1;
    EXPECT(make_plan(8192, 1, 8, 128, 64, LA_BF16, &o3, &p) == LA_ERR_UNSUPPORTED);

    // shape errors
    EXPECT(make_plan(-1, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(make_plan(10, 0, 8, 128, 64, LA_BF16, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(make_plan(10, 1, 0, 128, 64, LA_BF16, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(make_plan(10, 1, 8, 96, 64, LA_BF16, nullptr, &p) == LA_ERR_UNSUPPORTED);
    EXPECT(make_plan(10, 1, 8, 128, 48, LA_BF16, nullptr, &p) == LA_ERR_UNSUPPORTED);
    EXPECT(make_plan(10, 1, 8, 128, 64, 7, nullptr, &p) == LA_ERR_UNSUPPORTED);
    EXPECT(make_plan((int64_t)1 << 33, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_ERR_INVALID_ARG);

    // document pieces: chosen when the documents outnumber the segments per head and the units stay few
    EXPECT(make_plan(131072, 20, 64, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.packed == 1 && p.max_pieces == 24 &&
           p.state_slots == 4 && p.units == 24 * 64 && p.scan == 0 && p.ws_pieces_off >= p.ws_flags_off &&
           p.ws_slots_off >= p.ws_pieces_off + 24 * 16 && p.ws_bytes >= p.ws_slots_off + 4 * 8 && p.states() == 4);
    EXPECT(make_plan(131072, 300, 64, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.packed == 0);  // too many units
    EXPECT(make_plan(8192, 2, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.packed == 0);  // fewer documents than segments
    la_prefill_opts o8{};
    o8.work_list = 2;
    EXPECT(make_plan(8192, 2, 8, 128, 64, LA_BF16, &o8, &p) == LA_OK && p.packed == 1 && p.max_pieces == 18);
    o8.seg_len = 64;  // a document could need 127 earlier pieces
    EXPECT(make_plan(8192, 2, 8, 128, 64, LA_BF16, &o8, &p) == LA_ERR_UNSUPPORTED);
    o8.seg_len = 0;
    o8.force_scan = 1;
    EXPECT(make_plan(8192, 2, 8, 128, 64, LA_BF16, &o8, &p) == LA_ERR_UNSUPPORTED);
    o8.force_scan = 0;
    EXPECT(make_plan(100000, 5000, 8, 128, 64, LA_BF16, &o8, &p) == LA_ERR_UNSUPPORTED);  // over 4096 documents
    EXPECT(make_plan(0, 3, 8, 128, 64, LA_BF16, &o8, &p) == LA_ERR_UNSUPPORTED);          // no tokens
    o8.work_list = 1;
    EXPECT(make_plan(131072, 20, 64, 128, 64, LA_BF16, &o8, &p) == LA_OK && p.packed == 0);
    o8.work_list = 3;
    EXPECT(make_plan(131072, 20, 64, 128, 64, LA_BF16, &o8, &p) == LA_ERR_UNSUPPORTED);

    // dispatch limits: a plan whose grid would not fit one dispatch is refused
    // before anything is enqueued (at most 2^32 - 1 work-items: 16,777,208 units)
    la_prefill_opts o6{};
    o6.seg_len = 64;
    o6.value_slices = 1;
    o6.variant = 1;
    EXPECT(make_plan((int64_t)64 * 262143, 1, 64, 16, 64, LA_BF16, &o6, &p) == LA_OK && p.units == 16777152);
    EXPECT(make_plan((int64_t)64 * 262144, 1, 64, 16, 64, LA_BF16, &o6, &p) == LA_ERR_UNSUPPORTED);
    EXPECT(make_plan(INT32_MAX, 1, 8, 128, 64, LA_BF16, &o6, &p) == LA_ERR_UNSUPPORTED);
    // the transpose-read loop needs 64 rows of H * d bf16 within 32-bit offsets
    EXPECT(make_plan(1024, 1, 262143, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.variant == 2);
    EXPECT(make_plan(1024, 1, 262144, 128, 64, LA_BF16, nullptr, &p) == LA_OK && p.variant == 1);
    la_prefill_opts o7{};
    o7.variant = 2;
    EXPECT(make_plan(1024, 1, 262144, 128, 64, LA_BF16, &o7, &p) == LA_ERR_UNSUPPORTED);
    EXPECT(make_plan(1024, 1, 524287, 64, 64, LA_BF16, &o7, &p) == LA_OK && p.variant == 2);
    EXPECT(make_plan(1024, 1, 524288, 64, 64, LA_BF16, &o7, &p) == LA_ERR_UNSUPPORTED);

    // pointer errors
    const int64_t T = 8192;
    EXPECT(make_plan(T, 1, 8, 128, 64, LA_BF16, nullptr, &p) == LA_OK);
    const size_t need = p.ws_bytes;
    EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, nullptr, kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_OK);
    EXPECT(validate_prefill(nullptr, k, v, o, cu, 8, 128, 64, nullptr, kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(validate_prefill(q, k, v, nullptr, cu, 8, 128, 64, nullptr, kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(validate_prefill(q, k, v, o, nullptr, 8, 128, 64, nullptr, kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(validate_prefill(P(G + 8), k, v, o, cu, 8, 128, 64, nullptr, kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(validate_prefill(q, k, v, P(G + 4096), cu, 8, 128, 64, nullptr, kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, nullptr, static_cast<float*>(P(4 * G + 64)), 1, T, LA_BF16, ws, need, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, nullptr, kv, 1, T, LA_BF16, nullptr, need, nullptr, &p) == (need ? LA_ERR_WORKSPACE : LA_OK));
    if (need) {
        EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, nullptr, kv, 1, T, LA_BF16, ws, need - 1, nullptr, &p) == LA_ERR_WORKSPACE);
        EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, nullptr, kv, 1, T, LA_BF16, P(7 * G + 16), need, nullptr, &p) == LA_ERR_INVALID_ARG);
        EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, nullptr, kv, 1, T, LA_BF16, P(G), need, nullptr, &p) == LA_ERR_INVALID_ARG);
    }
    EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, nullptr, nullptr, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_OK);
    // incoming states: aligned, and overlapping no output
    float* kin = static_cast<float*>(P(8 * G));
    EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, kin, kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_OK);
    EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, static_cast<float*>(P(8 * G + 4)), kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, kv, kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_ERR_INVALID_ARG);
    EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, static_cast<float*>(P(4 * G + 256)), kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_ERR_INVALID_ARG);
    if (need) EXPECT(validate_prefill(q, k, v, o, cu, 8, 128, 64, static_cast<float*>(ws), kv, 1, T, LA_BF16, ws, need, nullptr, &p) == LA_ERR_INVALID_ARG);

    // decode
    EXPECT(validate_decode(q, k, v, kv, o, 256, 64, 128, LA_BF16) == LA_OK);
    EXPECT(validate_decode(q, k, v, kv, o, 0, 64, 128, LA_BF16) == LA_ERR_INVALID_ARG);
    EXPECT(validate_decode(q, k, v, kv, o, 256, 64, 100, LA_BF16) == LA_ERR_UNSUPPORTED);
    EXPECT(validate_decode(q, k, v, kv, q, 256, 64, 128, LA_BF16) == LA_ERR_INVALID_ARG);
    EXPECT(validate_decode(q, k, v, static_cast<float*>(P(G + 16)), o, 256, 64, 128, LA_BF16) == LA_ERR_INVALID_ARG);
    EXPECT(validate_decode(q, k, v, static_cast<float*>(P(6 * G + 4)), o, 256, 64, 128, LA_BF16) == LA_ERR_INVALID_ARG);
    EXPECT(validate_decode(q, k, v, kv, o, 256, 64, 128, 5) == LA_ERR_UNSUPPORTED);
    // one workgroup of 256 lanes per pair: at most 16,777,215 pairs in a grid
    EXPECT(validate_decode(q, k, v, kv, o, 65535, 256, 16, LA_BF16) == LA_OK);
    EXPECT(validate_decode(q, k, v, kv, o, 65536, 256, 16, LA_BF16) == LA_ERR_UNSUPPORTED);

    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("host validation checks passed\n");
    return 0;
}
