// C ABI (include/la.h): validate on the host, plan, enqueue.
#include <hip/hip_runtime.h>

#include "../../include/la.h"
#include "la_host.h"
#include "la_launch.h"

using la::Plan;

namespace {

// Fills the launch parameters of one validated prefill pass and enqueues it.
la_status enqueue_prefill(const Plan& plan, const void* q, const void* k, const void* v, void* o, const int32_t* cu,
                          int32_t H, int32_t d, int32_t block, const float* kv_in, int kv_in_t, float* kv_out,
                          int rev, int32_t num_seqs, int64_t T, la_dtype dtype, void* workspace, void* stream,
                          hipEvent_t e0, hipEvent_t e1, int skip_prefix = 0) {
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
    p.units = plan.units;
    p.per_xcd = (plan.units + 7) / 8;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = dtype == LA_BF16 ? la::launch_prefill_bf16(p, d, block, plan.W, plan.variant, s, e0, e1)
                                    : la::launch_prefill_fp32(p, d, block, plan.W, plan.variant, s, e0, e1);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
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
                           total_tokens, dtype, workspace, stream, e0, e1);
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
    int reuse_fwd = 0;
    if (opts && opts->forward_states && p1.variant == 2 && p1.nseg > 1) {
        float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + p1.ws_states_off);
        if (la::launch_ws_transpose(ws, (int64_t)(p1.nseg - 1) * H, d, p1.W, static_cast<hipStream_t>(stream)) !=
            hipSuccess)
            return LA_ERR_HIP;
        reuse_fwd = 1;
    }
    st = enqueue_prefill(p1, dout, v, k, dq, cu_seqlens, H, d, block, kv_state_in, 1, nullptr, 0, num_seqs,
                         total_tokens, dtype, workspace, stream, nullptr, nullptr, reuse_fwd);
    if (st != LA_OK) return st;
    // dV (and dKV_in, the reverse state after each document's first token):
    // reverse pass with query K, key Q, value dO, from dKV_out
    st = enqueue_prefill(p3, k, q, dout, dv, cu_seqlens, H, d, block, dkv_state_out, 0, dkv_state_in, 1, num_seqs,
                         total_tokens, dtype, workspace, stream, nullptr, nullptr);
    if (st != LA_OK) return st;
    // dK: reverse pass with query V, key dO, value Q, from dKV_out^T.  Its
    // segment states (sums of dO^T q) are the transposes of the dV pass's
    // (sums of q^T dO) over the same segments: on the transpose-read loop they
    // are transposed in place rather than computed again from Q and dO.
    int reuse = 0;
    if (p2.variant == 2 && p2.nseg > 1 && p2.L == p3.L && p2.S == p3.S && p2.nseg == p3.nseg && p2.scan == p3.scan) {
        float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + p3.ws_states_off);
        if (la::launch_ws_transpose(ws, (int64_t)(p3.nseg - 1) * H, d, p3.W, static_cast<hipStream_t>(stream)) !=
            hipSuccess)
            return LA_ERR_HIP;
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

la_status la_decode(const void* q, const void* k, const void* v, float* kv_state_inout, void* o, int32_t num_seqs,
                    int32_t H, int32_t d, la_dtype dtype, void* stream) {
    la_status st = la::validate_decode(q, k, v, kv_state_inout, o, num_seqs, H, d, (int)dtype);
    if (st != LA_OK) return st;
    la::DecodeParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.S = kv_state_inout;
    p.o = o;
    p.pairs = (int64_t)num_seqs * H;
    if (p.pairs > INT32_MAX) return LA_ERR_UNSUPPORTED;
    hipError_t e = la::launch_decode(p, d, (int)dtype, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // extern "C"
