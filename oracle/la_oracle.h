/*
 * fp64 CPU oracle for causal linear attention (TEST INFRASTRUCTURE ONLY).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * call this library.  It shares no code or header with the HIP library.
 *
 * What it computes (per document and head, tokens t of that document only):
 *     KV_t = sum_{s <= t} k_s^T v_s            (d x d, key index i, value index j)
 *     o_t  = q_t . KV_t = sum_{s <= t} (q_t . k_s) v_s
 * Linear attention without softmax, written with the "right product" and a
 * recursively updated key-value product: "MiniMax-01技术报告解读（一）模型架构"
 * (CSDN) and "MiniMax-01技术报告解读" (qingkelab), section 2.2 线性注意力.
 * The state starts from kv_in (or zero) at every document start: packed
 * samples are independent ("MiniMax-01技术报告解读", §3.2 item 1 数据打包 and
 * item 4 变长特征支持).
 *
 * Input dtype codes: 0 = bf16 bit patterns (uint16), 1 = fp32, 2 = fp64.
 * Layouts: q, k, v, o token-major [T, H, d]; states [num_seqs, H, d, d] with
 * element (i = key, j = value) at i * d + j.  Return 0 on success, -1 on
 * invalid arguments.
 */
#ifndef LA_ORACLE_H
#define LA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Form (b): token-by-token recurrent right product, heads [h0, h1).
 * o (may be NULL): fp64 [T, h1 - h0, d].  kv_in / kv_out (may be NULL):
 * fp64 [num_seqs, H, d, d] (only heads h0..h1-1 are read / written).
 * nthreads <= 0 uses every online core. */
int ora_recurrent(const void* q, const void* k, const void* v, int dtype, const int32_t* cu_seqlens,
                  int32_t num_seqs, int32_t H, int32_t d, int32_t h0, int32_t h1, const double* kv_in,
                  double* o, double* kv_out, int nthreads);

/* Form (a): quadratic masked left product, every head, one thread.  For tiny
 * inputs only: O(n^2 d) per document and head. */
int ora_quadratic(const void* q, const void* k, const void* v, int dtype, const int32_t* cu_seqlens,
                  int32_t num_seqs, int32_t H, int32_t d, const double* kv_in, double* o, double* kv_out);

/* One decode step for npairs independent (sequence, head) pairs:
 *     S <- S + k^T v ;  o = q . S      (update first, then read)
 * q, k, v [npairs, d] (dtype code), S fp64 [npairs, d, d] in place, o fp64
 * [npairs, d] (may be NULL). */
int ora_decode_step(const void* q, const void* k, const void* v, int dtype, int64_t npairs, int32_t d,
                    double* S, double* o, int nthreads);

/* Backward of the prefill (not on the pages; the chain rule applied to the
 * definition above).  Given dO (dout, [T, H, d], same dtype code as q) and
 * optionally dKV_out (fp64 [num_seqs, H, d, d], the gradient of a loss with
 * respect to kv_out), writes fp64 dq, dk, dv [T, H, d] and, if dkv_in is not
 * NULL, the gradient with respect to kv_in (fp64 [num_seqs, H, d, d]):
 *   dq_t = S_t dO_t,  G_s = dKV_out + sum_{t >= s} q_t^T dO_t,
 *   dk_s = G_s v_s,   dv_s = k_s G_s,  dKV_in = G at the document's first token,
 * with S_t = kv_in + sum_{s <= t} k_s^T v_s. */
int ora_backward(const void* q, const void* k, const void* v, const void* dout, int dtype, const int32_t* cu_seqlens,
                 int32_t num_seqs, int32_t H, int32_t d, const double* kv_in, const double* dkv_out, double* dq,
                 double* dk, double* dv, double* dkv_in, int nthreads);

/* The decayed variant (a reading: the pages name a decay among the fused
 * prefill steps, "MiniMax-01技术报告解读" §3.3 item 1, but never define it):
 * per head h a factor lambda_h = decay[h] in [0, 1] (fp64 [H]) fades the state
 * before each token's update,
 *     S_t = lambda_h S_{t-1} + k_t^T v_t ,   o_t = q_t . S_t ,
 * starting from S = kv_in (or zero) before the document's first token.
 * Form (b) and form (a) (o_r = sum_{c <= r} lambda^(r-c) (q_r . k_c) v_c +
 * lambda^(r+1) q_r . kv_in), and the decode step with a factor per pair
 * (decay fp64 [npairs]): S <- lambda S + k^T v ; o = q . S.  Arguments
 * otherwise as in the undecayed functions; a factor outside [0, 1] returns -1. */
int ora_recurrent_decay(const void* q, const void* k, const void* v, int dtype, const int32_t* cu_seqlens,
                        int32_t num_seqs, int32_t H, int32_t d, int32_t h0, int32_t h1, const double* decay,
                        const double* kv_in, double* o, double* kv_out, int nthreads);
int ora_quadratic_decay(const void* q, const void* k, const void* v, int dtype, const int32_t* cu_seqlens,
                        int32_t num_seqs, int32_t H, int32_t d, const double* decay, const double* kv_in, double* o,
                        double* kv_out);
int ora_decode_step_decay(const void* q, const void* k, const void* v, int dtype, int64_t npairs, int32_t d,
                          const double* decay, double* S, double* o, int nthreads);

/* Threads the last call used (for reporting). */
int ora_last_threads(void);

#ifdef __cplusplus
}
#endif
#endif
