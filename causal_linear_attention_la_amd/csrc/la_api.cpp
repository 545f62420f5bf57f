// C ABI (include/la.h): validate on the host, plan, enqueue.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/la.h"
#include "la_host.h"
#include "la_launch.h"

using la::Plan;

// Workspace of la_prefill_noalloc: one copy per GPU, in device memory for as
// long as the process runs.  On the host this name is only a handle for
// hipGetSymbolAddress, never an address a kernel may use.
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device: looked up once per
// device (with that device current) and kept.
la_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LA_ERR_HIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LA_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LA_OK;
}

// Key of a forward call's segment states: its inputs' addresses, shapes and
// plan (FNV-1a over them; never 0).  A backward handed the workspace with
// forward_states reuses the states only if the key stamped there is its own.
uint64_t states_key(const Plan& plan, const void* q, const void* k, const void* v, const int32_t* cu, int32_t H,
                    int32_t d, int32_t block, int32_t num_seqs, int64_t T, la_dtype dtype,
                    const float* decay = nullptr) {
    const uint64_t parts[] = {(uint64_t)(uintptr_t)decay, (uint64_t)(uintptr_t)q, (uint64_t)(uintptr_t)k,
                              (uint64_t)(uintptr_t)v,
                              (uint64_t)(uintptr_t)cu, (uint64_t)H, (uint64_t)d, (uint64_t)block,
                              (uint64_t)num_seqs, (uint64_t)T, (uint64_t)dtype, (uint64_t)plan.L, (uint64_t)plan.S,
                              (uint64_t)plan.nseg, (uint64_t)plan.scan, (uint64_t)plan.packed,
                              (uint64_t)plan.variant, (uint64_t)plan.slots};
    uint64_t h = 1469598103934665603ull;
    for (uint64_t x : parts)
        for (int b = 0; b < 8; ++b) {
            h ^= (x >> (8 * b)) & 0xff;
            h *= 1099511628211ull;
        }
    return h ? h : 1;
}

char* ws_at(void* workspace, size_t off) { return static_cast<char*>(workspace) + off; }

// Fills the launch parameters of one validated prefill pass and enqueues it.
// Every pass with a workspace has its block loop write the workspace's stamp:
// a forward call (stamp) its key when it leaves segment states there, anything
// else 0, so a stamp is only ever found next to the states it names.
// reuse: a backward's decision word (the state and scan kernels then do
// nothing when it reads 1).
// The kernel parameters of one prefill pass.
la::PrefillParams make_params(const Plan& plan, const void* q, const void* k, const void* v, void* o,
                              const int32_t* cu, int32_t H, int32_t d, int32_t block, const float* kv_in, int kv_in_t,
                              float* kv_out, int rev, int32_t num_seqs, int64_t T, la_dtype dtype, void* workspace,
                              int skip_prefix, bool stamp, const int32_t* reuse, const float* decay) {
    la::PrefillParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.cu = cu;
    p.kv_in = kv_in;
    p.kv_out = kv_out;
    p.ws = plan.ws_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ws_states_off) : nullptr;
    p.flags = plan.ws_bytes ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.ws_flags_off) : nullptr;
    p.packed = plan.packed;
    p.max_pieces = plan.max_pieces;
    p.state_slots = plan.state_slots;
    p.pieces = plan.packed ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.ws_pieces_off) : nullptr;
    p.slot_tab = plan.packed ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.ws_slots_off) : nullptr;
    p.T = (int32_t)T;
    p.num_seqs = num_seqs;
    p.H = H;
    p.L = plan.L;
    p.nseg = plan.nseg;
    p.S = plan.S;
    p.scan = plan.scan;
    p.rev = rev;
    p.kv_in_t = kv_in_t;
    p.slots = plan.slots;
    p.skip_prefix = skip_prefix;
    if (plan.ws_bytes > 0) {
        p.marker = reinterpret_cast<uint64_t*>(ws_at(workspace, plan.ws_marker_off));
        p.key = stamp && plan.states() > 0 ? states_key(plan, q, k, v, cu, H, d, block, num_seqs, T, dtype, decay)
                                           : 0;
    }
    p.reuse = reuse;
    p.decay = decay;
    p.units = plan.units;
    p.per_xcd = (plan.units + 7) / 8;
    return p;
}

la_status launch(const la::PrefillParams& p, const Plan& plan, int32_t d, int32_t block, la_dtype dtype, void* stream,
                 hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = dtype == LA_BF16 ? la::launch_prefill_bf16(p, d, block, plan.W, plan.variant, s, e0, e1)
                                    : la::launch_prefill_fp32(p, d, block, plan.W, plan.variant, s, e0, e1);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status enqueue_prefill(const Plan& plan, const void* q, const void* k, const void* v, void* o, const int32_t* cu,
                          int32_t H, int32_t d, int32_t block, const float* kv_in, int kv_in_t, float* kv_out,
                          int rev, int32_t num_seqs, int64_t T, la_dtype dtype, void* workspace, void* stream,
                          hipEvent_t e0, hipEvent_t e1, int skip_prefix = 0, bool stamp = false,
                          const int32_t* reuse = nullptr, const float* decay = nullptr) {
    const la::PrefillParams p = make_params(plan, q, k, v, o, cu, H, d, block, kv_in, kv_in_t, kv_out, rev, num_seqs,
                                            T, dtype, workspace, skip_prefix, stamp, reuse, decay);
    return launch(p, plan, d, block, dtype, stream, e0, e1);
}

// Two plans that decompose the work identically (the backward's two reverse passes).
bool same_plan(const Plan& a, const Plan& b) {
    return a.L == b.L && a.S == b.S && a.W == b.W && a.nseg == b.nseg && a.scan == b.scan && a.variant == b.variant &&
           a.slots == b.slots && a.units == b.units && a.packed == b.packed && a.max_pieces == b.max_pieces &&
           a.state_slots == b.state_slots && a.ws_bytes == b.ws_bytes;
}

}  // namespace

extern "C" {

const char* la_status_string(la_status s) {
    switch (s) {
        case LA_OK: return "LA_OK";
        case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG";
        case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
        case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE";
        case LA_ERR_HIP: return "LA_ERR_HIP";
        default: return "LA_ERR_UNKNOWN";
    }
}

la_status la_prefill_plan(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t d, int32_t block,
                          la_dtype dtype, const la_prefill_opts* opts, la_prefill_plan_info* out) {
    Plan p;
    la_status st = la::make_plan(total_tokens, num_seqs, H, d, block, (int)dtype, opts, &p);
    if (st != LA_OK) return st;
    if (out) {
        out->seg_len = p.L;
        out->value_slices = p.S;
        out->num_segments = p.nseg;
        out->scan = p.scan;
        out->units = p.units;
        out->workspace_bytes = p.ws_bytes;
        out->variant = p.variant;
        out->slots = p.slots;
        out->packed = p.packed;
    }
    return LA_OK;
}

size_t la_prefill_workspace_size_ex(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t d, int32_t block,
                                    la_dtype dtype, const la_prefill_opts* opts) {
    Plan p;
    if (la::make_plan(total_tokens, num_seqs, H, d, block, (int)dtype, opts, &p) != LA_OK) return 0;
    return p.ws_bytes;
}

size_t la_prefill_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t d, int32_t block,
                                 la_dtype dtype) {
    return la_prefill_workspace_size_ex(total_tokens, num_seqs, H, d, block, dtype, nullptr);
}

size_t la_prefill_backward_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t d, int32_t block,
                                          la_dtype dtype, const la_prefill_opts* opts) {
    Plan p;
    if (la::make_plan(total_tokens, num_seqs, H, d, block, (int)dtype, opts, &p) != LA_OK) return 0;
    return p.bwd_ws_bytes;
}

la_status la_prefill_resume(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens,
                            int32_t H, int32_t d, int32_t block, const float* kv_state_in, float* kv_state_out,
                            int32_t num_seqs, int64_t total_tokens, la_dtype dtype, void* workspace,
                            size_t workspace_bytes, void* stream, const la_prefill_opts* opts) {
    Plan plan;
    la_status st = la::validate_prefill(q, k, v, o, cu_seqlens, H, d, block, kv_state_in, kv_state_out, num_seqs,
                                        total_tokens, (int)dtype, workspace, workspace_bytes, opts, &plan);
    if (st != LA_OK) return st;
    hipEvent_t e0 = opts ? static_cast<hipEvent_t>(opts->main_begin_event) : nullptr;
    hipEvent_t e1 = opts ? static_cast<hipEvent_t>(opts->main_end_event) : nullptr;
    return enqueue_prefill(plan, q, k, v, o, cu_seqlens, H, d, block, kv_state_in, 0, kv_state_out, 0, num_seqs,
                           total_tokens, dtype, workspace, stream, e0, e1, 0, true);
}

la_status la_prefill_decay(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens,
                           int32_t H, int32_t d, int32_t block, const float* decay, const float* kv_state_in,
                           float* kv_state_out, int32_t num_seqs, int64_t total_tokens, la_dtype dtype,
                           void* workspace, size_t workspace_bytes, void* stream, const la_prefill_opts* opts) {
    if (!decay || reinterpret_cast<uintptr_t>(decay) % 4 != 0) return LA_ERR_INVALID_ARG;
    Plan plan;
    la_status st = la::validate_prefill(q, k, v, o, cu_seqlens, H, d, block, kv_state_in, kv_state_out, num_seqs,
                                        total_tokens, (int)dtype, workspace, workspace_bytes, opts, &plan, true);
    if (st != LA_OK) return st;
    // the factors are read while the outputs are written: no overlap with any output
    if (la::overlaps_outputs(decay, (size_t)H * 4, o, kv_state_out, workspace, plan, total_tokens, num_seqs, H, d,
                             (int)dtype))
        return LA_ERR_INVALID_ARG;
    hipEvent_t e0 = opts ? static_cast<hipEvent_t>(opts->main_begin_event) : nullptr;
    hipEvent_t e1 = opts ? static_cast<hipEvent_t>(opts->main_end_event) : nullptr;
    return enqueue_prefill(plan, q, k, v, o, cu_seqlens, H, d, block, kv_state_in, 0, kv_state_out, 0, num_seqs,
                           total_tokens, dtype, workspace, stream, e0, e1, 0, true, nullptr, decay);
}

la_status la_prefill_backward(const void* q, const void* k, const void* v, const void* dout,
                              const int32_t* cu_seqlens, int32_t H, int32_t d, int32_t block,
                              const float* kv_state_in, const float* dkv_state_out, void* dq, void* dk, void* dv,
                              float* dkv_state_in, int32_t num_seqs, int64_t total_tokens, la_dtype dtype,
                              void* workspace, size_t workspace_bytes, void* stream, const la_prefill_opts* opts) {
    if (!dout || !dq || !dk || !dv) return LA_ERR_INVALID_ARG;
    // every pass is a prefill with other operand roles; all are validated before any is enqueued
    Plan p1, p2, p3;
    la_status st = la::validate_prefill(dout, v, k, dq, cu_seqlens, H, d, block, kv_state_in, nullptr, num_seqs,
                                        total_tokens, (int)dtype, workspace, workspace_bytes, opts, &p1);
    if (st != LA_OK) return st;
    st = la::validate_prefill(v, dout, q, dk, cu_seqlens, H, d, block, dkv_state_out, nullptr, num_seqs, total_tokens,
                              (int)dtype, workspace, workspace_bytes, opts, &p2);
    if (st != LA_OK) return st;
    st = la::validate_prefill(k, q, dout, dv, cu_seqlens, H, d, block, dkv_state_out, dkv_state_in, num_seqs,
                              total_tokens, (int)dtype, workspace, workspace_bytes, opts, &p3);
    if (st != LA_OK) return st;
    st = la::validate_backward_outputs(q, k, v, dout, kv_state_in, dkv_state_out, dq, dk, dv, dkv_state_in, num_seqs,
                                       H, d, total_tokens, (int)dtype);
    if (st != LA_OK) return st;
    // dQ: forward pass with query dO, key V, value K, from KV_in^T.  Its
    // segment states (sums of v^T k) are the transposes of the forward's
    // (sums of k^T v): when the caller hands back the forward's workspace, they
    // are transposed in place instead of computed again.
    // The workspace holds the forward's states only if the key the forward
    // stamped there is this call's: a claim kernel compares the two, writes
    // its decision to the workspace and clears the stamp (the passes below
    // overwrite the states).  The transpose runs only on a match; otherwise
    // the state and scan kernels compute the states as usual.
    const int32_t* decision = nullptr;
    if (opts && opts->forward_states && p1.variant == 2 && p1.states() > 0) {
        hipStream_t hs = static_cast<hipStream_t>(stream);
        uint64_t* marker = reinterpret_cast<uint64_t*>(ws_at(workspace, p1.ws_marker_off));
        int32_t* dec = reinterpret_cast<int32_t*>(ws_at(workspace, p1.ws_marker_off + 64));
        const uint64_t key = states_key(p1, q, k, v, cu_seqlens, H, d, block, num_seqs, total_tokens, dtype);
        if (la::launch_ws_claim(marker, key, dec, hs) != hipSuccess) return LA_ERR_HIP;
        float* ws = reinterpret_cast<float*>(ws_at(workspace, p1.ws_states_off));
        if (la::launch_ws_transpose(ws, ws, p1.states() * H, d, p1.W, dec, hs) != hipSuccess) return LA_ERR_HIP;
        decision = dec;
    }
    st = enqueue_prefill(p1, dout, v, k, dq, cu_seqlens, H, d, block, kv_state_in, 1, nullptr, 0, num_seqs,
                         total_tokens, dtype, workspace, stream, nullptr, nullptr, 0, false, decision);
    if (st != LA_OK) return st;
    // dV (and dKV_in, the reverse state after each document's first token):
    // reverse pass with query K, key Q, value dO, from dKV_out.
    // dK: reverse pass with query V, key dO, value Q, from dKV_out^T.  Its
    // segment states (sums of dO^T q) are the transposes of the dV pass's
    // (sums of q^T dO) over the same segments, so they are transposed rather
    // than computed again from Q and dO.  The two passes read the same Q and
    // dO tiles in the same order: on the transpose-read loop, with room in the
    // workspace for the transposed copy, their block loops run in one launch,
    // each unit's two workgroups side by side on one XCD (la_prefill_pair_v2),
    // and the tiles one of them loads come from L2 for the other.
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (dtype == LA_BF16 && block == 64 && p2.variant == 2 && same_plan(p2, p3) &&
        (p3.states() == 0 || workspace_bytes >= p3.bwd_ws_bytes)) {
        la::PrefillParams pv = make_params(p3, k, q, dout, dv, cu_seqlens, H, d, block, dkv_state_out, 0,
                                           dkv_state_in, 1, num_seqs, total_tokens, dtype, workspace, 0, false,
                                           nullptr, nullptr);
        la::PrefillParams pk = make_params(p2, v, dout, q, dk, cu_seqlens, H, d, block, dkv_state_out, 1, nullptr, 1,
                                           num_seqs, total_tokens, dtype, workspace, 1, false, nullptr, nullptr);
        pv.prefix_only = 1;  // the dV pass's planning, state and scan kernels
        st = launch(pv, p3, d, block, dtype, stream);
        if (st != LA_OK) return st;
        pv.prefix_only = 0;
        if (p3.states() > 0) {
            float* tstates = reinterpret_cast<float*>(ws_at(workspace, p3.ws_tstates_off));
            if (la::launch_ws_transpose(pv.ws, tstates, p3.states() * H, d, p3.W, nullptr, hs) != hipSuccess)
                return LA_ERR_HIP;
            pk.ws = tstates;
        }
        return la::launch_prefill_pair(pv, pk, d, p3.W, p3.slots, hs) == hipSuccess ? LA_OK : LA_ERR_HIP;
    }
    st = enqueue_prefill(p3, k, q, dout, dv, cu_seqlens, H, d, block, dkv_state_out, 0, dkv_state_in, 1, num_seqs,
                         total_tokens, dtype, workspace, stream, nullptr, nullptr);
    if (st != LA_OK) return st;
    // (otherwise one after the other: the dK pass takes the dV pass's states
    // transposed in place)
    int reuse = 0;
    if (p2.variant == 2 && p2.states() > 0 && same_plan(p2, p3)) {
        float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + p3.ws_states_off);
        if (la::launch_ws_transpose(ws, ws, p3.states() * H, d, p3.W, nullptr, hs) != hipSuccess) return LA_ERR_HIP;
        reuse = 1;
    }
    return enqueue_prefill(p2, v, dout, q, dk, cu_seqlens, H, d, block, dkv_state_out, 1, nullptr, 1, num_seqs,
                           total_tokens, dtype, workspace, stream, nullptr, nullptr, reuse);
}

la_status la_prefill_ex(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens, int32_t H,
                        int32_t d, int32_t block, float* kv_state_out, int32_t num_seqs, int64_t total_tokens,
                        la_dtype dtype, void* workspace, size_t workspace_bytes, void* stream,
                        const la_prefill_opts* opts) {
    return la_prefill_resume(q, k, v, o, cu_seqlens, H, d, block, nullptr, kv_state_out, num_seqs, total_tokens,
                             dtype, workspace, workspace_bytes, stream, opts);
}

la_status la_prefill(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens, int32_t H,
                     int32_t d, int32_t block, float* kv_state_out, int32_t num_seqs, int64_t total_tokens,
                     la_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return la_prefill_ex(q, k, v, o, cu_seqlens, H, d, block, kv_state_out, num_seqs, total_tokens, dtype, workspace,
                         workspace_bytes, stream, nullptr);
}

la_status la_prefill_noalloc(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens,
                             int32_t H, int32_t d, int32_t block, float* kv_state_out, int32_t num_seqs,
                             int64_t total_tokens, la_dtype dtype, void* stream) {
    // the plan alone gives the workspace size: reject before touching the device
    Plan plan;
    la_status st = la::make_plan(total_tokens, num_seqs, H, d, block, (int)dtype, nullptr, &plan);
    if (st != LA_OK) return st;
    if (plan.ws_bytes > (size_t)LA_NOALLOC_SCRATCH_BYTES) return LA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (plan.ws_bytes > 0) {
        st = scratch_on_current_device(&ws);
        if (st != LA_OK) return st;
    }
    st = la::validate_prefill(q, k, v, o, cu_seqlens, H, d, block, nullptr, kv_state_out, num_seqs, total_tokens,
                              (int)dtype, ws, plan.ws_bytes, nullptr, &plan);
    if (st != LA_OK) return st;
    return enqueue_prefill(plan, q, k, v, o, cu_seqlens, H, d, block, nullptr, 0, kv_state_out, 0, num_seqs,
                           total_tokens, dtype, ws, stream, nullptr, nullptr, 0, true);
}

static la_status decode_impl(const void* q, const void* k, const void* v, const float* decay, float* kv_state_inout,
                             void* o, int32_t num_seqs, int32_t H, int32_t d, la_dtype dtype, void* stream) {
    la_status st = la::validate_decode(q, k, v, kv_state_inout, o, num_seqs, H, d, (int)dtype);
    if (st != LA_OK) return st;
    la::DecodeParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.S = kv_state_inout;
    p.o = o;
    p.pairs = (int64_t)num_seqs * H;
    p.decay = decay;
    p.H = H;
    p.unit = 1.0f;
    hipError_t e = la::launch_decode(p, d, (int)dtype, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status la_decode(const void* q, const void* k, const void* v, float* kv_state_inout, void* o, int32_t num_seqs,
                    int32_t H, int32_t d, la_dtype dtype, void* stream) {
    return decode_impl(q, k, v, nullptr, kv_state_inout, o, num_seqs, H, d, dtype, stream);
}

la_status la_decode_decay(const void* q, const void* k, const void* v, const float* decay, float* kv_state_inout,
                          void* o, int32_t num_seqs, int32_t H, int32_t d, la_dtype dtype, void* stream) {
    if (!decay || reinterpret_cast<uintptr_t>(decay) % 4 != 0) return LA_ERR_INVALID_ARG;
    if (la::overlaps_range(decay, (size_t)H * 4, kv_state_inout, (size_t)num_seqs * H * d * d * 4) ||
        la::overlaps_range(decay, (size_t)H * 4, o, (size_t)num_seqs * H * d * la::elem_size((int)dtype)))
        return LA_ERR_INVALID_ARG;
    return decode_impl(q, k, v, decay, kv_state_inout, o, num_seqs, H, d, dtype, stream);
}

}  // extern "C"
