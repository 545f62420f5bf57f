/*
 * la.h -- C ABI of the causal linear attention library for AMD MI355X (gfx950).
 *
 * The operation, per document and head (tokens of that document only):
 *     KV_t = sum_{s <= t} k_s^T v_s        (d x d, row i = key dim, column j = value dim)
 *     o_t  = q_t . KV_t = sum_{s <= t} (q_t . k_s) v_s
 * i.e. linear attention without softmax, computed as on the MiniMax-01 pages:
 * "MiniMax-01技术报告解读（一）模型架构" (CSDN) and "MiniMax-01技术报告解读"
 * (qingkelab), §2.2 线性注意力 -- the right-product trick with a recursively
 * updated key-value product; Q, K, V are tiled along the sequence into blocks,
 * with a left product inside each block and a right product across blocks.
 * There is no scale, feature map or normaliser (the pages define none); the
 * causal mask includes the current token.  A decay is named on the pages but
 * not defined: la_prefill_decay / la_decode_decay take one reading of it.
 *
 * Layouts
 *   q, k, v, o : token-major packed [T, H, d]; element (t, h, i) at (t*H + h)*d + i.
 *   states     : fp32 [num_seqs, H, d, d]; element (i = key, j = value) at i*d + j,
 *                so that o = q . KV.
 *   cu_seqlens : int32 [num_seqs + 1] in DEVICE memory, 0 = c_0 <= c_1 <= ... <= c_D = T.
 *                Documents may be empty.  Monotonicity and c_D = T are preconditions
 *                (the values live on the device and are not checked).
 *
 * Ownership and execution
 *   Every pointer is caller-owned device memory.  The library allocates, frees
 *   and synchronises nothing and, apart from la_prefill_noalloc's static
 *   device array (see there), keeps no mutable global state, so calls are
 *   reentrant and thread-safe.  Work is enqueued on `stream` (a hipStream_t;
 *   NULL = the null stream) and the call returns after enqueueing.
 *
 * Errors
 *   Arguments are validated on the host before anything is enqueued; a rejected
 *   call returns a status and enqueues nothing.  A failed kernel launch returns
 *   LA_ERR_HIP (kernels enqueued before it in the same call stay enqueued).
 *   Only the call's own launches are checked: an error that earlier HIP calls
 *   left in the thread's last-error slot is neither reported nor cleared.
 *   Asynchronous device faults surface on the stream as usual.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARG = 1, /* null / misaligned / overlapping pointer, H < 1, num_seqs < 1, T < 0 */
    LA_ERR_UNSUPPORTED = 2, /* d, block, dtype or tuning value outside the supported set */
    LA_ERR_WORKSPACE = 3,   /* workspace_bytes below la_prefill_workspace_size() or NULL workspace */
    LA_ERR_HIP = 4          /* a HIP launch failed */
} la_status;

typedef enum { LA_BF16 = 0, LA_FP32 = 1 } la_dtype;

/* Bytes of device workspace la_prefill needs for this shape (0 if none).
 * Depends only on the arguments.  Returns 0 for arguments la_prefill rejects. */
size_t la_prefill_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t d, int32_t block,
                                 la_dtype dtype);

/* Prefill: causal linear attention over packed variable-length documents,
 * Lightning-style (blocks of `block` tokens: masked left product inside a
 * block, right product against the running d x d state across blocks, state
 * update KV += K^T V after each block).  The state restarts at zero at every
 * document start: packed samples are independent ("MiniMax-01技术报告解读",
 * §3.2 item 1 数据打包, item 4 变长特征支持).  Block sizes 32/64/128 follow the
 * segment options of §3.3 item 3 (多级填充); document tails are predicated,
 * not padded in memory.
 *
 *   q, k, v      [T, H, d] dtype, device, 16-byte aligned, read only.
 *   o            [T, H, d] dtype, device, 16-byte aligned, fully overwritten;
 *                must not overlap q, k, v.
 *   cu_seqlens   [num_seqs + 1] int32, device.
 *   H            heads, >= 1.
 *   d            head dim: 16, 32, 64 or 128.
 *   block        32, 64 or 128 (fp32 with d >= 64: 32 or 64).
 *   kv_state_out [num_seqs, H, d, d] fp32, device, 16-byte aligned, or NULL.
 *                Row (doc, h) receives KV after the document's last token (zero
 *                for an empty document).  Must not overlap q, k, v, o.
 *   num_seqs     documents, >= 1.
 *   total_tokens T = cu_seqlens[num_seqs], >= 0.
 *   dtype        LA_BF16 (bf16 MFMA, fp32 accumulation, fp32 state, bf16 output
 *                rounded to nearest even) or LA_FP32 (fp32 throughout).
 *   workspace    device scratch of at least la_prefill_workspace_size() bytes,
 *                256-byte aligned (NULL allowed when that size is 0).  Its
 *                contents on entry are ignored; it must not be shared by calls
 *                in flight at the same time.
 *   stream       hipStream_t or NULL.
 */
la_status la_prefill(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens, int32_t H,
                     int32_t d, int32_t block, float* kv_state_out, int32_t num_seqs, int64_t total_tokens,
                     la_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Decode: one length-1 step for num_seqs independent sequences, each with H
 * heads ("MiniMax-01技术报告解读", §3.3 item 2 分离预填充和解码执行: length-1
 * tokens get their own kernel; item 1: the step fuses the KV computation with
 * the prefix KV-cache update).  Per (seq, head):
 *     KV <- KV + k^T v ;   o = q . KV        (update first: s <= t includes t)
 *
 *   q, k, v        [num_seqs, H, d] dtype, device, 16-byte aligned.
 *   kv_state_inout [num_seqs, H, d, d] fp32, device, 16-byte aligned, updated in place.
 *   o              [num_seqs, H, d] dtype, device, 16-byte aligned; no overlap with
 *                  the other arguments.
 *   d              16, 32, 64 or 128.
 */
la_status la_decode(const void* q, const void* k, const void* v, float* kv_state_inout, void* o, int32_t num_seqs,
                    int32_t H, int32_t d, la_dtype dtype, void* stream);

/* Prefill that allocates nothing and takes no workspace argument: the same
 * operation, arguments and results as la_prefill (the same kernels and plan,
 * so bit-identical outputs), for callers that cannot allocate device memory
 * around a call -- code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The segment states that la_prefill keeps in the
 * caller's workspace go instead to a static device array inside the library,
 * LA_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held by each GPU the library runs
 * on until the process ends.  Its address is looked up once per device, on the
 * first call with that device current.
 *
 *   Returns LA_ERR_WORKSPACE, with nothing enqueued, when the call's plan needs
 *   more than LA_NOALLOC_SCRATCH_BYTES of workspace (la_prefill_workspace_size()
 *   gives that figure); shapes of up to 256 x 64 KiB segment states fit.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (two streams, two threads) race and give wrong results; calls
 *   ordered on one stream are safe.  No content needs clearing between calls.
 *   Other arguments, errors and ownership as in la_prefill.
 */
#define LA_NOALLOC_SCRATCH_BYTES (32u << 20)
la_status la_prefill_noalloc(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens,
                             int32_t H, int32_t d, int32_t block, float* kv_state_out, int32_t num_seqs,
                             int64_t total_tokens, la_dtype dtype, void* stream);

/* Human-readable status name (static string). */
const char* la_status_string(la_status s);

/* ------------------------------------------------------------------------
 * Tuned prefill: the same operation as la_prefill (identical results up to
 * floating-point summation order) with explicit work decomposition and
 * optional timing events.
 *
 * The packed token range is cut into segments of seg_len tokens; a workgroup
 * handles one (segment, head, value-column slice).  When a document spans
 * several segments, each segment first reduces its K^T V (a segment state),
 * the states are prefix-summed per document, and each segment then runs the
 * block loop from its prefix -- the single-GPU form of the LASP+ scheme of
 * "MiniMax-01技术报告解读", §3.2 item 3 (local prefix states, one exchange,
 * global prefix).
 */
typedef struct {
    int32_t seg_len;        /* tokens per segment, a multiple of block; 0 = automatic */
    int32_t value_slices;   /* 1, 2 or 4 value-column slices per head; 0 = automatic */
    int32_t force_scan;     /* 1 = always run the separate prefix-scan kernel */
    int32_t variant;        /* block-loop kernel: 0 = automatic, 1 = the generic loop
                               (every dtype/d/block), 2 = the transpose-read loops
                               (bf16, d >= 64: block 64 with slices of >= 64 columns,
                               or block 128 with slices of 64 or 128 columns, plain
                               variant only; automatic picks them whenever they apply,
                               at block 128 with one slice);
                               an unavailable choice returns LA_ERR_UNSUPPORTED */
    void* main_begin_event; /* hipEvent_t stamped when the block-loop kernel starts
                               executing, or NULL (the kernel is then launched with
                               hipExtLaunchKernel, which records both events) */
    void* main_end_event;   /* hipEvent_t stamped when it completes, or NULL */
    int32_t slots;          /* tile slots of the transpose-read loop: 0 = automatic
                               (3 on segments of 16 blocks or more), 2, or 3 (loads
                               two blocks ahead; d = 128 only).  The 128-token loop
                               always runs 3 (2 returns LA_ERR_UNSUPPORTED) */
    int32_t forward_states; /* la_prefill_backward only (the forward entry points
                               ignore it): 1 = `workspace` may hold the segment states
                               of a forward call (la_prefill / _ex / _resume) on the
                               same q, k, v, cu_seqlens, shapes, dtype and plan; the dq
                               pass then takes them (transposed) instead of computing
                               them again.  Every forward call stamps its workspace
                               with a key of those pointers, shapes and plan (or clears
                               the stamp when it leaves no states); the backward
                               compares the stamp with its own key on the device and
                               reuses the states only on a match, else computes them;
                               either way it consumes the stamp, so a second backward
                               on the same workspace computes its own, and a backward
                               without forward_states clears it.  What cannot be
                               checked: the contents of q, k, v and cu_seqlens must be
                               those the stamping forward read. */
    int32_t work_list;      /* 0 = automatic, 1 = fixed segments of seg_len tokens,
                               2 = document pieces: each document cut into pieces of
                               at most seg_len tokens, ordered longest first on the
                               device (LA_ERR_UNSUPPORTED where the plan cannot take
                               them: more than 4096 documents, a document that could
                               need more than 16 earlier pieces, or force_scan) */
} la_prefill_opts;

/* The decomposition a prefill call will use (for reports and tests). */
typedef struct {
    int32_t seg_len;
    int32_t value_slices;
    int32_t num_segments;
    int32_t scan;          /* 1 if the prefix-scan kernel runs */
    int64_t units;         /* workgroups of the block-loop kernel */
    size_t workspace_bytes;
    int32_t variant;       /* the block-loop kernel that runs: 1 = generic, 2 = transpose-read */
    int32_t slots;         /* tile slots of the transpose-read loop (2 or 3) */
    int32_t packed;        /* 1 if the work list is document pieces (units is then
                              an upper bound: workgroups past the last piece exit) */
} la_prefill_plan_info;

la_status la_prefill_plan(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t d, int32_t block,
                          la_dtype dtype, const la_prefill_opts* opts, la_prefill_plan_info* out);

size_t la_prefill_workspace_size_ex(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t d, int32_t block,
                                    la_dtype dtype, const la_prefill_opts* opts);

la_status la_prefill_ex(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens, int32_t H,
                        int32_t d, int32_t block, float* kv_state_out, int32_t num_seqs, int64_t total_tokens,
                        la_dtype dtype, void* workspace, size_t workspace_bytes, void* stream,
                        const la_prefill_opts* opts);

/* Prefill that resumes from given states (chunked prefill, prefix-cache
 * resume): identical to la_prefill_ex except that document delta starts from
 * kv_state_in[delta, h] instead of zero, i.e. for t in the document
 *     KV_t = kv_state_in + sum_{s <= t, s in the document} k_s^T v_s ,  o_t = q_t . KV_t .
 * This is the recurrence continued across a cut ("MiniMax-01技术报告解读",
 * §3.3 item 1: prefix KV cache; §3.2 item 3: a sequence piece starts from the
 * state its predecessors leave).  A sequence prefilled in chunks, each chunk
 * resuming from the previous chunk's kv_state_out, gives the single-call
 * result up to floating-point summation order.
 *
 *   kv_state_in  [num_seqs, H, d, d] fp32, device, 16-byte aligned, read only,
 *                or NULL (then exactly la_prefill_ex).  An empty document's
 *                kv_state_out is its kv_state_in.  Must not overlap o,
 *                kv_state_out or the workspace (so the state cannot be
 *                updated in place: use two buffers and swap).
 *   Everything else as in la_prefill / la_prefill_ex (opts may be NULL).
 */
la_status la_prefill_resume(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens,
                            int32_t H, int32_t d, int32_t block, const float* kv_state_in, float* kv_state_out,
                            int32_t num_seqs, int64_t total_tokens, la_dtype dtype, void* workspace,
                            size_t workspace_bytes, void* stream, const la_prefill_opts* opts);

/* Backward of la_prefill_resume: the gradients of a loss L with respect to
 * q, k, v and kv_state_in, given dL/do (dout) and dL/dkv_state_out.  The
 * pages give no backward (they train at long context with LASP+,
 * "MiniMax-01技术报告解读" §3.2 item 3); it is the chain rule applied to the
 * definition, per document and head, with S_t = KV_in + sum_{s <= t} k_s^T v_s:
 *     dq_t   = S_t dO_t                                  (a forward pass)
 *     G_s    = dKV_out + sum_{t >= s} q_t^T dO_t         (a reverse state)
 *     dk_s   = G_s v_s ,   dv_s = k_s G_s ,   dKV_in = G at the first token
 * computed as three passes of the prefill kernels: dq forward with query dO,
 * key v, value k, starting from KV_in^T; dv and dk with every document read
 * from its last token to its first (query k / key q / value dO from dKV_out,
 * then query v / key dO / value q from dKV_out^T).  The dk pass's segment
 * states are the transposes of the dv pass's; on the transpose-read loop they
 * are transposed in the workspace instead of being computed again, and, when
 * the workspace also has room for that transposed copy
 * (la_prefill_backward_workspace_size), the dv and dk block loops run in one
 * launch, where the two workgroups of each unit share the Q and dO tiles
 * through L2.  The results are the same either way, bit for bit.
 *
 *   q, k, v, dout      [T, H, d] dtype, device, 16-byte aligned, read only.
 *   kv_state_in        the forward's incoming states or NULL (zero).
 *   dkv_state_out      [num_seqs, H, d, d] fp32 gradient of the final states, or NULL (zero).
 *   dq, dk, dv         [T, H, d] dtype, device, 16-byte aligned, fully overwritten.
 *   dkv_state_in       [num_seqs, H, d, d] fp32 or NULL: gradient of kv_state_in.
 *   Outputs overlap neither an input nor each other.  The workspace is at
 *   least that of la_prefill_workspace_size_ex for the same shapes and opts
 *   (one buffer serves the passes, which run in order on `stream`);
 *   la_prefill_backward_workspace_size bytes let the two reverse passes share
 *   a launch.  Shapes, dtypes, blocks and tuning options as in la_prefill_ex;
 *   opts' events are ignored.
 */
la_status la_prefill_backward(const void* q, const void* k, const void* v, const void* dout,
                              const int32_t* cu_seqlens, int32_t H, int32_t d, int32_t block,
                              const float* kv_state_in, const float* dkv_state_out, void* dq, void* dk, void* dv,
                              float* dkv_state_in, int32_t num_seqs, int64_t total_tokens, la_dtype dtype,
                              void* workspace, size_t workspace_bytes, void* stream, const la_prefill_opts* opts);

/* Workspace bytes with which la_prefill_backward runs its dv and dk passes in
 * one launch: la_prefill_workspace_size_ex's bytes plus a transposed copy of
 * the segment states (the same when the plan has no segment states or does not
 * use the transpose-read loop).  The forward's layout is a prefix of it, so one
 * buffer of this size serves a forward call and the backward that reuses its
 * states (forward_states).  0 for unsupported shapes. */
size_t la_prefill_backward_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t d,
                                          int32_t block, la_dtype dtype, const la_prefill_opts* opts);

/* Decayed variant: the same prefill with each head's state fading by a factor
 * lambda_h before every token's update.  "MiniMax-01技术报告解读" §3.3 item 1
 * (批处理内核融合) lists a decay-value computation (衰减值计算) among the fused
 * prefill steps but never defines it; the reading taken here keeps the
 * recurrence, per document and head h:
 *     S_t = lambda_h S_{t-1} + k_t^T v_t ,   o_t = q_t . S_t
 *     i.e. o_t = sum_{s <= t} lambda_h^(t - s) (q_t . k_s) v_s  (+ lambda_h^(t+1-t0) q_t . kv_in)
 * with S = kv_state_in (or zero) before the document's first token t0;
 * lambda_h = 1 is la_prefill_resume's operation.  Blockwise: the intra-block
 * scores carry lambda^(query - key), the inter-block product lambda^(row + 1),
 * and KV <- lambda^nb KV + sum_c lambda^(nb - 1 - c) k_c^T v_c (the weights on
 * a bf16 copy of V for bf16 inputs); segment states are faded across the
 * segments between them.
 *
 *   decay       fp32 [H] in DEVICE memory, 4-byte aligned: lambda_h in [0, 1]
 *               (a precondition: the values are not checked).  Must not overlap
 *               o, kv_state_out or the workspace.  NULL: LA_ERR_INVALID_ARG.
 *   Everything else as in la_prefill_resume (opts may be NULL; its
 *   forward_states is ignored).  The workspace size is
 *   la_prefill_workspace_size_ex's for the same shapes and opts; on the
 *   full-width d = 128 loop the decayed call uses two tile slots (an explicit
 *   slots = 3 there returns LA_ERR_UNSUPPORTED).  There is no decayed backward.
 */
la_status la_prefill_decay(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens,
                           int32_t H, int32_t d, int32_t block, const float* decay, const float* kv_state_in,
                           float* kv_state_out, int32_t num_seqs, int64_t total_tokens, la_dtype dtype,
                           void* workspace, size_t workspace_bytes, void* stream, const la_prefill_opts* opts);

/* Decayed decode step (the reading above), per (seq, head):
 *     KV <- lambda_h KV + k^T v ;   o = q . KV
 * decay: fp32 [H], device, 4-byte aligned, lambda_h in [0, 1], overlapping
 * neither kv_state_inout nor o.  Otherwise as la_decode. */
la_status la_decode_decay(const void* q, const void* k, const void* v, const float* decay, float* kv_state_inout,
                          void* o, int32_t num_seqs, int32_t H, int32_t d, la_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LA_H */
