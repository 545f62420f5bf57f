// Decode kernel: one length-1 step per (sequence, head) pair
// ("MiniMax-01技术报告解读", §3.3 item 2 分离预填充和解码执行: length-1 tokens
// run in their own kernel; item 1: the KV computation is fused with the
// prefix-cache update).
//     KV <- KV + k^T v ;  o = q . KV   (update first, then read)
// The step streams the d x d fp32 state once (read + write) and does
// 4 d^2 flops on it: 0.5 flop/byte, so it is HBM bound and runs on the vector
// ALUs; MFMA has nothing to contract.
#pragma once
#include "la_device.h"
#include "la_tiles.h"

namespace la {

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    float* S;
    void* o;
    int64_t pairs;
    const float* decay;  // decayed variant: per-head lambda (device, [H]), or null
    int32_t H;
    float unit;          // 1.0f: the plain step's factor (see the kernel)
};

// One workgroup per pair.  Thread t owns 4 consecutive value columns
// (one float4) of D/(256/(D/4)) state rows: rows rg, rg + RG, ... with
// rg = t / (D/4).  Each state row is read and written once as coalesced
// float4s; the partial dot products of q with the updated columns are reduced
// across row groups through LDS in a fixed order (deterministic).
// Decayed variant (DK): KV <- lambda KV + k^T v with the pair's head's lambda.
template <typename TIn, int D, bool DK = false>
__global__ __launch_bounds__(kThreads) void la_decode_kernel(DecodeParams p) {
    constexpr int LPR = D / 4;                      // threads per state row
    constexpr int RG = kThreads / LPR;              // row groups
    constexpr int RPT = (D + RG - 1) / RG;          // rows per thread
    __shared__ float qs[D], ks[D];
    __shared__ float red[RG][D];

    const int64_t pair = blockIdx.x;
    if (pair >= p.pairs) return;
    const int tid = threadIdx.x;
    const int cq = tid % LPR, rg = tid / LPR;
    const TIn* qg = static_cast<const TIn*>(p.q) + pair * D;
    const TIn* kg = static_cast<const TIn*>(p.k) + pair * D;
    const TIn* vg = static_cast<const TIn*>(p.v) + pair * D;
    if (tid < D) {
        qs[tid] = to_f32(qg[tid]);
        ks[tid] = to_f32(kg[tid]);
    }
    const float v0 = to_f32(vg[4 * cq + 0]), v1 = to_f32(vg[4 * cq + 1]);
    const float v2 = to_f32(vg[4 * cq + 2]), v3 = to_f32(vg[4 * cq + 3]);
    f32x4_t* S = reinterpret_cast<f32x4_t*>(p.S + pair * (int64_t)D * D);
    // The plain step scales the state by p.unit = 1 (exact): it then has the
    // decayed step's instruction schedule, which keeps more of the state's
    // loads in flight behind its stores -- measured 0.368 against 0.383 ms per
    // 256 x 64 x 128 step with the multiply left out.
    const float lam = DK ? p.decay[pair % p.H] : p.unit;

    f32x4_t st[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int i = rg + r * RG;
        if (i < D) st[r] = __builtin_nontemporal_load(S + i * LPR + cq);
    }
    __syncthreads();
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int i = rg + r * RG;
        if (i < D) {
            const float ki = ks[i], qi = qs[i];
            f32x4_t x = st[r];
            x *= lam;
            x[0] = fmaf(ki, v0, x[0]);
            x[1] = fmaf(ki, v1, x[1]);
            x[2] = fmaf(ki, v2, x[2]);
            x[3] = fmaf(ki, v3, x[3]);
            __builtin_nontemporal_store(x, S + i * LPR + cq);
            o0 = fmaf(qi, x[0], o0);
            o1 = fmaf(qi, x[1], o1);
            o2 = fmaf(qi, x[2], o2);
            o3 = fmaf(qi, x[3], o3);
        }
    }
    if (rg < RG) {
        red[rg][4 * cq + 0] = o0;
        red[rg][4 * cq + 1] = o1;
        red[rg][4 * cq + 2] = o2;
        red[rg][4 * cq + 3] = o3;
    }
    __syncthreads();
    if (tid < D) {
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) acc += red[r][tid];
        from_f32(static_cast<TIn*>(p.o) + pair * D + tid, acc);
    }
}

}  // namespace la
