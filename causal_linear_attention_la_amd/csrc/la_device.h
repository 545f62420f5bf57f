// Device helpers for the gfx950 kernels: MFMA fragments, bf16 conversion,
// 16-byte vector moves.
//
// MFMA fragment convention used throughout.  A 16x16 output tile is computed
// from 32-wide chunks of the contraction dimension.  Lane l belongs to row
// (or column) l % 16 and to group g = l / 16; within a 32-chunk, group g
// holds the 8 contraction indices
//     kset(g) = {4g, 4g+1, 4g+2, 4g+3, 16+4g, 16+4g+1, 16+4g+2, 16+4g+3}.
// A and B fragments use the same kset, so the MFMA sums every index once
// whatever order the hardware assigns to the 8 elements.  The point of this
// kset: the fp32 accumulator of a 16x16 tile gives lane (column l%16, group g)
// rows 4g..4g+3, so two stacked accumulator tiles hold exactly kset(g) of a
// 32-chunk -- results can be written to LDS as 4-element runs and read back as
// operands with two 4-element reads.
//   bf16: one v_mfma_f32_16x16x32_bf16 per chunk.
//   fp32: eight v_mfma_f32_16x16x4_f32, element e of every group per step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

typedef uint16_t bf16_t;  // bf16 stored as raw bits

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// two fp32 -> packed bf16x2 (low half = a), one conversion instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T>
struct Frag;

template <>
struct Frag<bf16_t> {
    uint2 lo, hi;  // 4 + 4 bf16
};

template <>
struct Frag<float> {
    float4 lo, hi;
};

// Loads the kset(g) fragment of the 32-chunk starting at `chunk` (LDS).
__device__ __forceinline__ void load_frag(Frag<bf16_t>& f, const bf16_t* chunk, int g) {
    f.lo = *reinterpret_cast<const uint2*>(chunk + 4 * g);
    f.hi = *reinterpret_cast<const uint2*>(chunk + 16 + 4 * g);
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* chunk, int g) {
    f.lo = *reinterpret_cast<const float4*>(chunk + 4 * g);
    f.hi = *reinterpret_cast<const float4*>(chunk + 16 + 4 * g);
}

__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
    uint4 av = make_uint4(a.lo.x, a.lo.y, a.hi.x, a.hi.y);
    uint4 bv = make_uint4(b.lo.x, b.lo.y, b.hi.x, b.hi.y);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                  acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<float>& a, const Frag<float>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// Stores 4 fp32 values as 4 consecutive elements of type T (LDS or global).
__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4_zero(bf16_t* p) { *reinterpret_cast<uint2*>(p) = make_uint2(0, 0); }
__device__ __forceinline__ void store4_zero(float* p) { *reinterpret_cast<float4*>(p) = make_float4(0, 0, 0, 0); }

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Decayed variant: lambda^m for m >= 0 from l2 = log2(lambda), as exp2(m l2);
// lambda^0 = 1 also for lambda = 0 (l2 = -inf).
__device__ __forceinline__ float decay_pow(float l2, int m) { return m <= 0 ? 1.f : exp2f(l2 * (float)m); }
// The same divided by 2^lc (lc: log2 of a state's scale, finite).
__device__ __forceinline__ float decay_pow(float l2, int m, float lc) {
    return m <= 0 ? exp2f(-lc) : exp2f(l2 * (float)m - lc);
}

// A bf16 fragment (8 elements) scaled element by element, rounded to nearest
// even; element e of lo.x, lo.y, hi.x, hi.y is (e % 2 == 0 ? low : high) half.
__device__ __forceinline__ Frag<bf16_t> scale_frag(const Frag<bf16_t>& f, const float (&w)[8]) {
    const uint32_t in[4] = {f.lo.x, f.lo.y, f.hi.x, f.hi.y};
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = __uint_as_float(in[i] << 16) * w[2 * i];
        const float b = __uint_as_float(in[i] & 0xffff0000u) * w[2 * i + 1];
        out[i] = pack_bf16x2(a, b);
    }
    Frag<bf16_t> r;
    r.lo = make_uint2(out[0], out[1]);
    r.hi = make_uint2(out[2], out[3]);
    return r;
}

// Element e (0..7 for bf16, 0..3 for fp32) of a 16-byte vector.
__device__ __forceinline__ uint32_t lane16(const uint4& v, int e) {
    uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}
__device__ __forceinline__ uint32_t lane32(const uint4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

// Writes element e of four row vectors r[0..3] (4 consecutive tokens) as one
// 4-element run at p: the transpose step of the tile loads.
__device__ __forceinline__ void store_col4(bf16_t* p, const uint4 (&r)[4], int e) {
    uint2 v;
    v.x = lane16(r[0], e) | (lane16(r[1], e) << 16);
    v.y = lane16(r[2], e) | (lane16(r[3], e) << 16);
    *reinterpret_cast<uint2*>(p) = v;
}
__device__ __forceinline__ void store_col4(float* p, const uint4 (&r)[4], int e) {
    *reinterpret_cast<uint4*>(p) = make_uint4(lane32(r[0], e), lane32(r[1], e), lane32(r[2], e), lane32(r[3], e));
}

__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ void from_f32(bf16_t* p, float x) { *p = f32_to_bf16(x); }
__device__ __forceinline__ void from_f32(float* p, float x) { *p = x; }

}  // namespace la
