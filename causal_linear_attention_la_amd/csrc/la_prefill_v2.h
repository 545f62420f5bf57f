// Prefill kernels for bf16 with d in {64, 128}, 64-token blocks and
// value-column slices of at least 64 columns (the d = 128 hot path).
//
// Same work decomposition and results contract as la_prefill_kernels.h; the
// block loop is organised for gfx950:
//  * Q, K, V tiles go from HBM straight into LDS with buffer loads in LDS-DMA
//    mode (no staging registers), three blocks deep: the loads of block j+2
//    are issued when block j starts, so two iterations hide each load.  Rows
//    past the end of a partial block lie outside the buffer range and arrive
//    as zeros.
//  * Tiles are row-major with 128- or 256-byte rows and no padding; the
//    8-byte units of row r are permuted by XOR with an even mask, so 16-byte
//    DMA slots stay whole.  The masks make the two read patterns conflict
//    free: 16 rows at one column (row fragments) and 8 rows x 4 units
//    (transpose reads), 32 lanes per LDS cycle.
//  * Operands that contract over tokens (K^T and V^T fragments) are read with
//    ds_read_b64_tr_b16, which hands each lane 4 consecutive rows of one
//    column: one half of the kset fragment used by the MFMA helpers.
//  * Wave w owns value columns [w W/4, (w+1) W/4) of the state for all d
//    rows.  The fp32 state tiles stay in registers; for the inter product
//    O^T += KV^T Q^T two vertically adjacent state tiles are, lane for lane,
//    the A operand of one 32-wide chunk, so the state never goes through LDS.
//  * The intra product of block j (it needs the scores P of block j) runs in
//    iteration j+1 between its two barriers, where no tile buffer is being
//    written; its output rows are stored with buffer stores (rows past a
//    partial block are dropped by the range check).
#pragma once
#include "la_prefill_kernels.h"

namespace la {
namespace v2 {

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Word 3 of a raw buffer resource on gfx9: 32-bit data format, offsets in bytes.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Workgroup barrier for LDS hand-offs: waits for this wave's outstanding LDS
// operations, then s_barrier.  Outstanding vector-memory operations are
// accounted for explicitly with vm_wait.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations
// (loads, LDS-DMA loads, stores; they retire in issue order) stay in flight.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Unit permutation masks (8-byte units, even: 16-byte chunks stay whole).
template <int PITCH>
__device__ __forceinline__ int hmask(int r) {
    if constexpr (PITCH == 128) return 4 * (r & 7) + 2 * ((r >> 3) & 1);   // 256-byte rows
    else return 4 * ((r >> 1) & 3) + 2 * ((r >> 3) & 1);                   // 128-byte rows: two per 64 banks
}

// Element offset of the unit holding logical columns [col, col + 4) of `row`.
template <int PITCH>
__device__ __forceinline__ int soff(int row, int col) {
    return row * PITCH + ((((col >> 2) ^ hmask<PITCH>(row))) << 2);
}

// kset fragment of a row: lane (row, g) receives T[row][k0 + kset(g)].
template <int PITCH>
__device__ __forceinline__ void load_frag_sw(Frag<bf16_t>& f, const bf16_t* tile, int row, int k0, int g) {
    f.lo = *reinterpret_cast<const uint2*>(tile + soff<PITCH>(row, k0 + 4 * g));
    f.hi = *reinterpret_cast<const uint2*>(tile + soff<PITCH>(row, k0 + 16 + 4 * g));
}

// kset fragment of a column: lane (s = lane % 16, g) receives
// T[t0 + kset(g)][n0 + s] (rows t0 + 4g..+3 and t0 + 16 + 4g..+3), through
// ds_read_b64_tr_b16: within each 16-lane group, lane s names row
// (first + s / 4) at columns n0 + 4 (s % 4)..+3 and receives column n0 + s
// of those 4 rows.
template <int PITCH>
__device__ __forceinline__ void load_frag_tr(Frag<bf16_t>& f, const bf16_t* tile, int t0, int n0, int lane) {
    const int s = lane & 15, g = lane >> 4;
    const int r = t0 + 4 * g + (s >> 2), c = n0 + 4 * (s & 3);
    s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + soff<PITCH>(r, c)));
    s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + soff<PITCH>(r + 16, c)));
    f.lo = __builtin_bit_cast(uint2, lo);
    f.hi = __builtin_bit_cast(uint2, hi);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }

// A 64 x COLS bf16 tile moved HBM -> LDS by LDS-DMA buffer loads.  Wave w
// moves rows [16w, 16w + 16); each instruction fills RPI whole rows: lane L
// lands in 16-byte slot L, so it fetches the logical chunk that the row's
// mask puts there.
template <int COLS>
struct DmaTile {
    static constexpr int ROWB = COLS * 2;
    static constexpr int CPR = ROWB / 16;  // chunks per row
    static constexpr int RPI = 64 / CPR;   // rows per instruction
    static constexpr int NI = 16 / RPI;    // instructions per wave and block
    uint32_t voff[NI];
    int row0;

    __device__ __forceinline__ void init(int wave, int lane, uint32_t row_bytes) {
        row0 = 16 * wave;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = row0 + RPI * i + lane / CPR;
            const int chunk = (lane % CPR) ^ (hmask<COLS>(row) >> 1);
            voff[i] = (uint32_t)row * row_bytes + (uint32_t)chunk * 16u;
        }
    }
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, bf16_t* tile) const {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(tile + (row0 + RPI * i) * COLS), 16, voff[i],
                                                     0, 0, 0);
    }
};

template <int D, int B, int W>
struct Geo {
    static constexpr int NQT = B / 16;
    static constexpr int NDT = D / 16;
    static constexpr int CW = W / 4;   // value columns per wave
    static constexpr int NCW = CW / 16;
    static constexpr int LOADS = DmaTile<D>::NI * 2 + DmaTile<W>::NI;  // VMEM loads per wave and block
    static constexpr int STORES = NQT * NCW;                          // VMEM stores per wave and block
    static_assert(B == 64, "one 16-row band per wave");
    static_assert(CW % 16 == 0, "each wave owns whole 16-column tiles");
    static_assert(D == 64 || D == 128, "row widths");
    static_assert(W == 64 || W == 128, "row widths");
};

// KV[:, own cols] += K^T V over one block; keeps the V^T fragments (A operands
// of the intra product).
template <int D, int B, int W, int NA, int NC, int NK>
__device__ __forceinline__ void state_update(f32x4_t (&kv)[NA][NC], Frag<bf16_t> (&vfr)[NC][NK], const bf16_t* Ks,
                                             const bf16_t* Vs, int col0, int lane) {
    using G = Geo<D, B, W>;
    static_assert(NA == G::NDT && NC == G::NCW && NK == B / 32, "tile counts");
#pragma unroll
    for (int kc = 0; kc < B / 32; ++kc) {
#pragma unroll
        for (int c = 0; c < G::NCW; ++c) load_frag_tr<W>(vfr[c][kc], Vs, 32 * kc, col0 + 16 * c, lane);
#pragma unroll
        for (int a = 0; a < G::NDT; ++a) {
            Frag<bf16_t> kf;
            load_frag_tr<D>(kf, Ks, 32 * kc, 16 * a, lane);
#pragma unroll
            for (int c = 0; c < G::NCW; ++c) mma(kv[a][c], kf, vfr[c][kc]);
        }
    }
}

template <int D, int B, int W, int NA, int NC>
__device__ __forceinline__ void load_prefix(f32x4_t (&kv)[NA][NC], const float* src, int g, int li) {
    using G = Geo<D, B, W>;
    static_assert(NA == G::NDT && NC == G::NCW, "tile counts");
#pragma unroll
    for (int a = 0; a < G::NDT; ++a)
#pragma unroll
        for (int c = 0; c < G::NCW; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) kv[a][c][r] += src[(int64_t)(16 * a + 4 * g + r) * D + 16 * c + li];
}

template <int D, int B, int W, int NA, int NC>
__device__ __forceinline__ void store_state(const f32x4_t (&kv)[NA][NC], float* dst, int g, int li) {
    using G = Geo<D, B, W>;
    static_assert(NA == G::NDT && NC == G::NCW, "tile counts");
#pragma unroll
    for (int a = 0; a < G::NDT; ++a)
#pragma unroll
        for (int c = 0; c < G::NCW; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(int64_t)(16 * a + 4 * g + r) * D + 16 * c + li] = kv[a][c][r];
}

// ---------------------------------------------------------------------------
// Segment states (see la_segment_state_kernel): K^T V of each segment's last
// document piece when that document continues into the next segment.
template <int D, int B, int W>
__global__ __launch_bounds__(kThreads, 1) void la_segment_state_v2(PrefillParams p) {
    using G = Geo<D, B, W>;
    constexpr int NBUF = 3;
    constexpr int LOADS = DmaTile<D>::NI + DmaTile<W>::NI;
    __shared__ __align__(16) bf16_t Kb[NBUF][B * D];
    __shared__ __align__(16) bf16_t Vb[NBUF][B * W];
    int u, h, s;
    if (!unit_of(p, u, h, s)) return;
    if (u >= p.nseg - 1) return;
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t_beg = u * p.L, t_end = (u + 1) * p.L;
    const int de = doc_at(p.cu, p.num_seqs, t_end - 1);
    const int dstart = p.cu[de];
    const bool needs = p.cu[de + 1] > t_end;
    const bool chain = dstart < t_beg;
    if (h == 0 && s == 0 && tid == 0) p.flags[u] = (needs ? 1 : 0) | (chain ? 2 : 0);
    if (!needs) return;

    const bf16_t* kg = static_cast<const bf16_t*>(p.k);
    const bf16_t* vg = static_cast<const bf16_t*>(p.v);
    const uint32_t row_bytes = (uint32_t)(p.H * D * 2);
    const int col0 = wave * G::CW;
    DmaTile<D> dk;
    DmaTile<W> dv;
    dk.init(wave, lane, row_bytes);
    dv.init(wave, lane, row_bytes);
    f32x4_t kv[G::NDT][G::NCW];
#pragma unroll
    for (int a = 0; a < G::NDT; ++a)
#pragma unroll
        for (int c = 0; c < G::NCW; ++c) kv[a][c] = zero4();
    Frag<bf16_t> vfr[G::NCW][B / 32];

    const int first = max(t_beg, dstart);
    const int nblk = (t_end - first + B - 1) / B;
    auto issue = [&](int j) {
        const int b0 = first + j * B, nb = min(B, t_end - b0);
        const int64_t e0 = ((int64_t)b0 * p.H + h) * D;
        dk.issue(make_rsrc(kg + e0, (uint32_t)nb * row_bytes), Kb[j % NBUF]);
        dv.issue(make_rsrc(vg + e0 + s * W, (uint32_t)nb * row_bytes), Vb[j % NBUF]);
    };
    issue(0);
    if (nblk > 1) issue(1);
    for (int j = 0; j < nblk; ++j) {
        if (j + 1 < nblk) vm_wait<LOADS>(); else vm_wait<0>();
        lds_barrier();  // block j in LDS; block j-1 no longer read
        if (j + 2 < nblk) issue(j + 2);
        state_update<D, B, W>(kv, vfr, Kb[j % NBUF], Vb[j % NBUF], col0, lane);
    }
    store_state<D, B, W>(kv, p.ws + (((int64_t)u * p.H + h) * D) * D + s * W + col0, g, li);
}

// ---------------------------------------------------------------------------
// The block loop.
template <int D, int B, int W>
__global__ __launch_bounds__(kThreads, 1) void la_prefill_main_v2(PrefillParams p) {
    using G = Geo<D, B, W>;
    constexpr int NQT = G::NQT, NCW = G::NCW, NDT = G::NDT;
    constexpr int NTRI = NQT * (NQT + 1) / 2, NZT = NQT / 2;
    constexpr int NBUF = 3;
    constexpr int PP = B;  // P[query][key] rows: 128 bytes
    __shared__ __align__(16) bf16_t Qb[NBUF][B * D];
    __shared__ __align__(16) bf16_t Kb[NBUF][B * D];
    __shared__ __align__(16) bf16_t Vb[NBUF][B * W];
    __shared__ __align__(16) bf16_t Ps[B * PP];

    int u, h, s;
    if (!unit_of(p, u, h, s)) return;
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: descriptors in SGPRs
    const int col0 = wave * G::CW;
    const int t0 = u * p.L, t1 = min(p.T, t0 + p.L);
    const bf16_t* qg = static_cast<const bf16_t*>(p.q);
    const bf16_t* kg = static_cast<const bf16_t*>(p.k);
    const bf16_t* vg = static_cast<const bf16_t*>(p.v);
    bf16_t* og = static_cast<bf16_t*>(p.o);
    const uint32_t row_bytes = (uint32_t)(p.H * D * 2);

    DmaTile<D> dq;
    DmaTile<W> dv;
    dq.init(wave, lane, row_bytes);
    dv.init(wave, lane, row_bytes);

    Cursor c0;
    cursor_first(c0, p.cu, p.num_seqs, t0, t1, B);

    f32x4_t kv[NDT][NCW];
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int c = 0; c < NCW; ++c) kv[a][c] = zero4();
    if (c0.nb > 0 && !c0.first_of_doc) {
        const int u_first = p.scan ? u - 1 : p.cu[c0.doc] / p.L;
        for (int uu = u_first; uu < u; ++uu)
            load_prefix<D, B, W>(kv, p.ws + (((int64_t)uu * p.H + h) * D) * D + s * W + col0, g, li);
    }
    f32x4_t oacc[NQT][NCW];
#pragma unroll
    for (int b = 0; b < NQT; ++b)
#pragma unroll
        for (int c = 0; c < NCW; ++c) oacc[b][c] = zero4();
    Frag<bf16_t> vfr[NCW][B / 32];

    auto issue = [&](const Cursor& c, int buf) {
        const int64_t e0 = ((int64_t)c.b0 * p.H + h) * D;
        const uint32_t bytes = (uint32_t)c.nb * row_bytes;
        dq.issue(make_rsrc(qg + e0, bytes), Qb[buf]);
        dq.issue(make_rsrc(kg + e0, bytes), Kb[buf]);
        dv.issue(make_rsrc(vg + e0 + s * W, bytes), Vb[buf]);
    };
    // O^T += V^T P^T for the previous block, then its rows are stored.
    auto finish = [&](int pb0, int pnb) {
#pragma unroll
        for (int b = 0; b < NQT; ++b) {
#pragma unroll
            for (int kc = 0; kc <= b / 2; ++kc) {
                Frag<bf16_t> pf;
                load_frag_sw<PP>(pf, Ps, 16 * b + li, 32 * kc, g);
#pragma unroll
                for (int c = 0; c < NCW; ++c) mma(oacc[b][c], vfr[c][kc], pf);
            }
        }
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(og + ((int64_t)pb0 * p.H + h) * D + s * W + col0, (uint32_t)pnb * row_bytes);
#pragma unroll
        for (int b = 0; b < NQT; ++b)
#pragma unroll
            for (int c = 0; c < NCW; ++c) {
                u32x2_t v;
                v.x = pack2(oacc[b][c][0], oacc[b][c][1]);
                v.y = pack2(oacc[b][c][2], oacc[b][c][3]);
                __builtin_amdgcn_raw_buffer_store_b64(v, ro, (16 * b + li) * row_bytes + (16 * c + 4 * g) * 2, 0, 0);
                oacc[b][c] = zero4();
            }
    };

    Cursor c1 = c0;
    if (c1.nb > 0) cursor_next(c1, p.cu, p.num_seqs, t1, B);
    if (c0.nb > 0) issue(c0, 0);
    if (c1.nb > 0) issue(c1, 1);
    int pb0 = 0, pnb = 0;
    bool have_prev = false;
    int j = 0;
    while (c0.nb > 0) {
        Cursor c2 = c1;
        if (c2.nb > 0) cursor_next(c2, p.cu, p.num_seqs, t1, B);
        // Loads of block j are done once at most the younger operations are
        // in flight: loads of block j+1 and the stores of block j-2 (the
        // stores of block j-3 sit between them and are waited for too).
        if (c1.nb > 0) {
            if (j >= 2) vm_wait<G::LOADS + G::STORES>();
            else vm_wait<G::LOADS>();
        } else {
            vm_wait<0>();
        }
        lds_barrier();  // (A) block j visible; block j-1's tiles no longer read
        if (c2.nb > 0) issue(c2, (j + 2) % NBUF);
        if (have_prev) finish(pb0, pnb);
        lds_barrier();  // (B) scores of block j-1 consumed

        const bf16_t* Qs = Qb[j % NBUF];
        const bf16_t* Ks = Kb[j % NBUF];
        const bf16_t* Vs = Vb[j % NBUF];
        // inter: O^T += KV^T Q^T with the state before this block
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
            Frag<bf16_t> kvf[NCW];
#pragma unroll
            for (int c = 0; c < NCW; ++c) {
                kvf[c].lo = make_uint2(pack2(kv[2 * m][c][0], kv[2 * m][c][1]), pack2(kv[2 * m][c][2], kv[2 * m][c][3]));
                kvf[c].hi = make_uint2(pack2(kv[2 * m + 1][c][0], kv[2 * m + 1][c][1]),
                                       pack2(kv[2 * m + 1][c][2], kv[2 * m + 1][c][3]));
            }
#pragma unroll
            for (int b = 0; b < NQT; ++b) {
                Frag<bf16_t> qf;
                load_frag_sw<D>(qf, Qs, 16 * b + li, 32 * m, g);
#pragma unroll
                for (int c = 0; c < NCW; ++c) mma(oacc[b][c], kvf[c], qf);
            }
        }
        // state: KV += K^T V (after the inter product read it)
        state_update<D, B, W>(kv, vfr, Ks, Vs, col0, lane);

        // scores, transposed, lower-triangular tiles; P[query][key] to LDS
        for (int t = wave; t < NTRI + NZT; t += kWaves) {
            int a, b;
            if (t < NTRI) {
                b = 0;
                while ((b + 1) * (b + 2) / 2 <= t) ++b;
                a = t - b * (b + 1) / 2;
            } else {
                b = 2 * (t - NTRI);
                a = b + 1;
            }
            bf16_t* prow = Ps + soff<PP>(16 * b + li, 16 * a + 4 * g);
            if (t >= NTRI) {
                store4_zero(prow);
                continue;
            }
            f32x4_t acc = zero4();
#pragma unroll
            for (int m = 0; m < D / 32; ++m) {
                Frag<bf16_t> fa, fb;
                load_frag_sw<D>(fa, Ks, 16 * a + li, 32 * m, g);
                load_frag_sw<D>(fb, Qs, 16 * b + li, 32 * m, g);
                mma(acc, fa, fb);
            }
            if (a == b) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g + r > li) acc[r] = 0.f;
            }
            store4(prow, acc[0], acc[1], acc[2], acc[3]);
        }

        if (c0.b0 + c0.nb == c0.doc_end) {  // the document ends with this block
            if (p.kv_out)
                store_state<D, B, W>(kv, p.kv_out + (((int64_t)c0.doc * p.H + h) * D) * D + s * W + col0, g, li);
#pragma unroll
            for (int a = 0; a < NDT; ++a)
#pragma unroll
                for (int c = 0; c < NCW; ++c) kv[a][c] = zero4();
        }
        pb0 = c0.b0;
        pnb = c0.nb;
        have_prev = true;
        c0 = c1;
        c1 = c2;
        ++j;
    }
    if (have_prev) {
        lds_barrier();  // scores of the last block visible
        finish(pb0, pnb);
    }

    if (p.kv_out) {
        const int lo = doc_lower(p.cu, p.num_seqs, t0);
        const int hi = (u == p.nseg - 1) ? p.num_seqs : doc_lower(p.cu, p.num_seqs, t1);
        for (int d = lo; d < hi; ++d) {
            if (p.cu[d + 1] != p.cu[d]) continue;
            float* dst = p.kv_out + (((int64_t)d * p.H + h) * D) * D + s * W;
            for (int i = tid; i < D * W; i += kThreads) dst[(int64_t)(i / W) * D + (i % W)] = 0.f;
        }
    }
}

}  // namespace v2
}  // namespace la
