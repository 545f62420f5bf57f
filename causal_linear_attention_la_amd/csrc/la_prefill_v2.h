// Prefill kernels for bf16 with d in {64, 128}: 64-token blocks with
// value-column slices of at least 64 columns (the d = 128 hot path), and
// 128-token blocks with 64-column slices (main_v2_b128, run as two 64-row
// halves per block on the same tiles); the backward's two reverse passes can
// share one launch (la_prefill_pair_v2).
//
// Same work decomposition and results contract as la_prefill_kernels.h; the
// block loop is organised for gfx950:
//  * Q, K, V tiles go from HBM straight into LDS with buffer loads in LDS-DMA
//    mode (no staging registers), into two or three tile slots: the loads of
//    block j+1 (or j+2) are issued during iteration j, so each load has one
//    (or two) iterations to arrive.  Rows past the end of a partial block
//    lie outside the buffer range and arrive as zeros.  In reverse mode (the
//    backward's passes) the same loads mirror the rows of each block.
//  * Tiles are row-major with 128- or 256-byte rows and no padding; the
//    8-byte units of row r are permuted by XOR with an even mask, so 16-byte
//    DMA slots stay whole.  The masks make every read pattern conflict free
//    within 16 lanes: 16 rows at one 16-byte chunk (row fragments), and 4
//    rows x 4 units with unit stride 1 or 2 (transpose reads).
//  * MFMA fragments here use a contiguous contraction set: within each
//    32-wide chunk, lane group g = lane / 16 holds indices 8g..8g+7.  A row
//    fragment (Q, K, P: contraction along the row) is then one 16-byte LDS
//    read.  Operands that contract over tokens (K^T and V^T fragments) are
//    read with ds_read_b64_tr_b16, which hands each lane 4 consecutive rows of
//    one column: two such reads (rows 8g..8g+3 and 8g+4..8g+7) make a fragment.
//  * Wave w owns value columns [w W/4, (w+1) W/4) of the state for all d
//    rows.  The fp32 state tiles stay in registers.  State tile 2m + p holds,
//    in its accumulator row 4g + r, key dimension 32m + 8g + 4p + r, so the
//    tile pair (2m, 2m+1) is, lane for lane, the A operand of chunk m of the
//    inter product O^T += KV^T Q^T: the state never goes through LDS.
//  * LDS reads are the scarce resource next to the tile DMA (they delay the
//    DMA's writes into LDS), so the loop reads each operand as few times as
//    it can: the scores P^T = mask(K Q^T) are computed inside the inter
//    product's loop, from the same Q fragments, with wave w taking key band
//    w against every query band (masked tiles come out as the zeros the
//    intra product needs).
//  * The intra product of block j (it needs the scores P of block j) runs in
//    iteration j+1 between its two barriers, where no tile buffer is being
//    written; its output rows are stored with buffer stores (rows past a
//    partial block are dropped by the range check).  Except on the full-width
//    loop with three slots, the rows are packed into registers and stored
//    after the iteration's tile loads: the next iteration's wait for those
//    loads then leaves the stores in flight (stores issued between the loads
//    held every iteration up for their write latency).
//  * With one 16-column tile per wave (64-column slices) the loop has the
//    registers to issue a group's fragment reads before the products that use
//    them, paying one LDS latency per group; the full-width loop has not.
#pragma once
#include "la_prefill_kernels.h"

namespace la {
namespace v2 {

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Word 3 of a raw buffer resource on gfx9: 32-bit data format, offsets in bytes.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy bit of a buffer access on gfx950: non-temporal (streaming).
// The segment-state kernel, a pure read stream, is faster with it (long
// inputs: 0.74 -> 0.67 ms for 4.2 GB); the block loop is slower with it on
// its loads or its stores, so it keeps the default policy.
constexpr int kNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// The waits and the barrier go through builtins (not inline asm), so the
// compiler's own wait insertion knows what they cover; the empty asm
// statements keep it from moving memory accesses across them.
//
// Workgroup barrier for LDS hand-offs: waits for this wave's outstanding LDS
// operations (lgkmcnt(0); expcnt and vmcnt at their maximum, i.e. no wait),
// then s_barrier.  Outstanding vector-memory operations are accounted for
// explicitly with vm_wait.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations
// (loads, LDS-DMA loads, stores; they retire in issue order) stay in flight.
// gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}

// Unit permutation masks (8-byte units, even: 16-byte chunks stay whole).
template <int PITCH>
__device__ __forceinline__ int hmask(int r) {
    if constexpr (PITCH == 128)  // 256-byte rows
        return (8 * (r & 1)) ^ (16 * ((r >> 1) & 1)) ^ (2 * ((r >> 2) & 1)) ^ (4 * ((r >> 3) & 1));
    else  // 128-byte rows: two per 64 banks (row bit 0 picks the half)
        return (8 * ((r >> 1) & 1)) ^ (2 * ((r >> 2) & 1)) ^ (4 * ((r >> 3) & 1));
}

// Element offset of the unit holding logical columns [col, col + 4) of `row`.
template <int PITCH>
__device__ __forceinline__ int soff(int row, int col) {
    return row * PITCH + ((((col >> 2) ^ hmask<PITCH>(row))) << 2);
}

// Row fragment: lane (row, g) receives T[row][k0 + 8g .. k0 + 8g + 7], one
// 16-byte read (the even unit masks keep 16-byte chunks whole and aligned).
template <int PITCH>
__device__ __forceinline__ void load_row(Frag<bf16_t>& f, const bf16_t* tile, int row, int k0, int g) {
    const uint4 v = *reinterpret_cast<const uint4*>(tile + soff<PITCH>(row, k0 + 8 * g));
    f.lo = make_uint2(v.x, v.y);
    f.hi = make_uint2(v.z, v.w);
}

// Column fragment over tokens: lane (s = lane % 16, g) receives
// T[t0 + 8g .. t0 + 8g + 7][col(s)] through two ds_read_b64_tr_b16.  Within
// each 16-lane group, lane s names row (first + s / 4) and the 4-column unit
// starting at n0 + STRIDE (s % 4) + off, and receives element s % 4 of the
// unit named by lane 4i + s / 4 for rows first + i.  So
//   STRIDE 4, off 0: col(s) = n0 + s                          (16 columns)
//   STRIDE 8, off 4p: col(s) = n0 + 8 (s / 4) + 4p + s % 4    (a state tile's key dims)
template <int PITCH, int STRIDE>
__device__ __forceinline__ void load_tr(Frag<bf16_t>& f, const bf16_t* tile, int t0, int n0, int off, int lane) {
    const int s = lane & 15, g = lane >> 4;
    const int r = t0 + 8 * g + (s >> 2), c = n0 + STRIDE * (s & 3) + off;
    s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + soff<PITCH>(r, c)));
    s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + soff<PITCH>(r + 4, c)));
    f.lo = __builtin_bit_cast(uint2, lo);
    f.hi = __builtin_bit_cast(uint2, hi);
}

// Key dimension held by accumulator row 4g + r of state tile a.
__device__ __forceinline__ int state_row(int a, int g, int r) { return 32 * (a >> 1) + 8 * g + 4 * (a & 1) + r; }

// Value column (relative to the wave's first column) held by lane column s of
// state tile c.  A wave with two tile columns interleaves them in runs of 4,
// so that lane group g of the output accumulators of tiles 0 and 1 holds 8
// consecutive columns 8g..8g+7: one 16-byte store per row.
template <int NCW>
__device__ __forceinline__ int state_col(int c, int s) {
    if constexpr (NCW == 2) return 8 * (s >> 2) + 4 * c + (s & 3);
    else return 16 * c + s;
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
    uint32_t voff[NI];   // row * row_bytes + chunk * 16
    uint32_t coff2[NI];  // 2 * chunk * 16
    int row0;

    __device__ __forceinline__ void init(int wave, int lane, uint32_t row_bytes) {
        row0 = 16 * wave;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = row0 + RPI * i + lane / CPR;
            const int chunk = (lane % CPR) ^ (hmask<COLS>(row) >> 1);
            voff[i] = (uint32_t)row * row_bytes + (uint32_t)chunk * 16u;
            coff2[i] = (uint32_t)chunk * 32u;
        }
    }
    // Tile row r takes the buffer's row r, or, in reverse mode, its row
    // nb - 1 - r (the descriptor then starts at the block's lowest physical
    // row): rows past nb wrap to huge offsets and read as zeros either way.
    // last_row_off = (nb - 1) * row_bytes.
    // CPOL: the loads' cache policy (0 default, kNonTemporal).
    template <int CPOL = 0>
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, bf16_t* tile, bool rev = false,
                                          uint32_t last_row_off = 0) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t off = rev ? last_row_off + coff2[i] - voff[i] : voff[i];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(tile + (row0 + RPI * i) * COLS), 16, off, 0,
                                                     0, CPOL);
        }
    }
};

template <int N>
struct Slot {
    static constexpr int value = N;
};

template <int D, int B, int W>
struct Geo {
    static constexpr int NQT = B / 16;
    static constexpr int NDT = D / 16;
    static constexpr int CW = W / 4;   // value columns per wave
    static constexpr int NCW = CW / 16;
    static constexpr int LOADS = DmaTile<D>::NI * 2 + DmaTile<W>::NI;  // VMEM loads per wave and block
    static constexpr int STORES = NCW == 2 ? NQT : NQT * NCW;         // VMEM stores per wave and block
    static_assert(B == 64, "one 16-row band per wave");
    static_assert(CW % 16 == 0, "each wave owns whole 16-column tiles");
    static_assert(D == 64 || D == 128, "row widths");
    static_assert(W == 64 || W == 128, "row widths");
};

// The token part of a full block's decay weights for state_update: lane
// group g holds tokens 32 kc + 8 g + e, and lambda^(31 - 8 g - e) is the
// weight of that token within its 32-token chunk.
__device__ __forceinline__ void full_weights(float (&wfull)[8], float l2, int lane) {
#pragma unroll
    for (int e = 0; e < 8; ++e) wfull[e] = decay_pow(l2, 31 - 8 * (lane >> 4) - e);
}

// KV[:, own cols] += K^T V over one block; keeps the V^T fragments (A operands
// of the intra product).  Decayed variant (DK, l2 = log2 lambda, nb tokens in
// the block): the state is kept scaled, KV = 2^lc U, so that the fade
// lambda^nb of each block changes only the scale (the caller's lc, see
// fade_scale) and this update adds sum_c lambda^(nb - 1 - c) 2^-lc k_c^T v_c to
// U, the weights applied to a bf16 copy of the V^T fragments (lane group g
// holds tokens 32 kc + 8 g + e of each chunk); the kept fragments stay
// unscaled.  wfull (optional): the lane's lambda^(31 - 8 g - e) (full_weights),
// so that a full block's weights take one power per chunk instead of one per
// token: lambda^(B - 1 - tok) 2^-lc = wfull[e] lambda^(32 (B/32 - 1 - kc)) 2^-lc.
template <int D, int B, int W, bool DK = false, int NA, int NC, int NK>
__device__ __forceinline__ void state_update(f32x4_t (&kv)[NA][NC], Frag<bf16_t> (&vfr)[NC][NK], const bf16_t* Ks,
                                             const bf16_t* Vs, int col0, int lane, float l2 = 0.f, int nb = B,
                                             float lc = 0.f, const float* wfull = nullptr) {
    using G = Geo<D, B, W>;
    static_assert(NA == G::NDT && NC == G::NCW && NK == B / 32, "tile counts");
#pragma unroll
    for (int kc = 0; kc < B / 32; ++kc) {
#pragma unroll
        for (int c = 0; c < G::NCW; ++c) {
            if constexpr (G::NCW == 2) load_tr<W, 8>(vfr[c][kc], Vs, 32 * kc, col0, 4 * c, lane);
            else load_tr<W, 4>(vfr[c][kc], Vs, 32 * kc, col0 + 16 * c, 0, lane);
        }
        Frag<bf16_t> vs[G::NCW];
        if constexpr (DK) {
            float w[8];
            if (wfull && nb == B) {
                const float sc = decay_pow(l2, 32 * (B / 32 - 1 - kc), lc);
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = wfull[e] * sc;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int tok = 32 * kc + 8 * (lane >> 4) + e;
                    w[e] = tok < nb ? decay_pow(l2, nb - 1 - tok, lc) : 0.f;
                }
            }
#pragma unroll
            for (int c = 0; c < G::NCW; ++c) vs[c] = scale_frag(vfr[c][kc], w);
        } else {
#pragma unroll
            for (int c = 0; c < G::NCW; ++c) vs[c] = vfr[c][kc];
        }
#pragma unroll
        for (int a = 0; a < G::NDT; ++a) {
            Frag<bf16_t> kf;
            load_tr<D, 8>(kf, Ks, 32 * kc, 32 * (a >> 1), 4 * (a & 1), lane);
#pragma unroll
            for (int c = 0; c < G::NCW; ++c) mma(kv[a][c], kf, vs[c]);
        }
    }
}

// Decayed variant: the fade of a block of nb tokens on a state kept as
// KV = 2^lc U.  It lowers lc by nb log2(1/lambda); only when the scale would
// fall below 2^-kRescale (every few blocks for lambda near 1, every block for
// small lambda, lambda = 0 included) is it applied to U, which then holds the
// state itself again (lc = 0).  The weights of the block's own tokens are then
// taken relative to the new scale (state_update's lc), so U never grows past
// 2^kRescale times the state.
constexpr float kRescale = 24.f;
template <int NA, int NC>
__device__ __forceinline__ void fade_scale(f32x4_t (&kv)[NA][NC], float& lc, float l2, int nb) {
    const float next = lc + l2 * (float)nb;  // -inf for lambda = 0
    if (next >= -kRescale) {
        lc = next;
    } else {
        const float f = exp2f(next);
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int c = 0; c < NC; ++c) kv[a][c] *= f;
        lc = 0.f;
    }
}

// Segment states in the workspace are private to these kernels, so they are
// kept in register order: the (D x W) state of one (segment, head, slice) is
// 4 consecutive wave blocks of D * W / 4 floats, each [tile a][tile c][lane]
// of 4-float runs -- 16-byte, fully coalesced loads and stores.  (The scan
// kernel adds states entry by entry and does not care about the order.)
template <int D, int B, int W, bool DK = false, int NA, int NC>
__device__ __forceinline__ void load_ws(f32x4_t (&kv)[NA][NC], const float* src, int lane, float f = 1.f) {
    using G = Geo<D, B, W>;
    static_assert(NA == G::NDT && NC == G::NCW, "tile counts");
    const f32x4_t* s4 = reinterpret_cast<const f32x4_t*>(src);
#pragma unroll
    for (int a = 0; a < G::NDT; ++a)
#pragma unroll
        for (int c = 0; c < G::NCW; ++c) {
            if constexpr (DK) kv[a][c] += f * s4[(a * G::NCW + c) * 64 + lane];
            else kv[a][c] += s4[(a * G::NCW + c) * 64 + lane];
        }
}

template <int D, int B, int W, bool DK = false, int NA, int NC>
__device__ __forceinline__ void store_ws(const f32x4_t (&kv)[NA][NC], float* dst, int lane, float f = 1.f) {
    using G = Geo<D, B, W>;
    static_assert(NA == G::NDT && NC == G::NCW, "tile counts");
    f32x4_t* d4 = reinterpret_cast<f32x4_t*>(dst);
#pragma unroll
    for (int a = 0; a < G::NDT; ++a)
#pragma unroll
        for (int c = 0; c < G::NCW; ++c) {
            if constexpr (DK) d4[(a * G::NCW + c) * 64 + lane] = f * kv[a][c];
            else d4[(a * G::NCW + c) * 64 + lane] = kv[a][c];
        }
}

// A wave's block of the workspace state of unit (u, h, s).
template <int D, int W>
__device__ __forceinline__ int64_t ws_offset(const PrefillParams& p, int u, int h, int s, int wave) {
    return (((int64_t)u * p.H + h) * D) * D + (int64_t)s * D * W + (int64_t)wave * (D * W / 4);
}

// Adds a state stored in the documented [key][value] layout (kv_in) -- or,
// with `transposed`, stored [value][key].  base = the (document, head)
// matrix, col0 = the first value column this wave owns.
template <int D, int B, int W, int NA, int NC>
__device__ __forceinline__ void add_state(f32x4_t (&kv)[NA][NC], const float* base, int col0, int transposed, int g,
                                          int li, float f = 1.f) {
    using G = Geo<D, B, W>;
    static_assert(NA == G::NDT && NC == G::NCW, "tile counts");
#pragma unroll
    for (int a = 0; a < G::NDT; ++a)
#pragma unroll
        for (int c = 0; c < G::NCW; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t i = state_row(a, g, r), j = col0 + state_col<NC>(c, li);
                kv[a][c][r] += f * (transposed ? base[j * D + i] : base[i * D + j]);
            }
}

template <int D, int B, int W, bool DK = false, int NA, int NC>
__device__ __forceinline__ void store_state(const f32x4_t (&kv)[NA][NC], float* dst, int g, int li, float f = 1.f) {
    using G = Geo<D, B, W>;
    static_assert(NA == G::NDT && NC == G::NCW, "tile counts");
#pragma unroll
    for (int a = 0; a < G::NDT; ++a)
#pragma unroll
        for (int c = 0; c < G::NCW; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = DK ? f * kv[a][c][r] : kv[a][c][r];
                dst[(int64_t)state_row(a, g, r) * D + state_col<NC>(c, li)] = x;
            }
}

// ---------------------------------------------------------------------------
// Segment states (see la_segment_state_kernel): K^T V of each segment's last
// document piece when that document continues into the next segment.
template <int D, int B, int W, bool DK = false>
__global__ __launch_bounds__(kThreads, 1) void la_segment_state_v2(PrefillParams p) {
    using G = Geo<D, B, W>;
    // Two slots of two blocks each, one LDS variable per tile; the loads of
    // blocks 2i+2, 2i+3 are issued when blocks 2i, 2i+1 start.
    __shared__ __align__(16) bf16_t Kb0[2 * B * D], Kb1[2 * B * D];
    __shared__ __align__(16) bf16_t Vb0[2 * B * W], Vb1[2 * B * W];
    auto kbuf = [&](auto slot) -> bf16_t* { if constexpr (decltype(slot)::value == 0) return Kb0; else return Kb1; };
    auto vbuf = [&](auto slot) -> bf16_t* { if constexpr (decltype(slot)::value == 0) return Vb0; else return Vb1; };
    if (states_reused(p)) return;
    int u, h, s, first, t_end;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (p.packed) {  // state slot u: a whole piece [first, t_end) of one document
        int len;
        if (!slot_of(p, u, first, len, h, s)) return;
        t_end = first + len;
    } else {
        if (!unit_of(p, u, h, s)) return;
        if (u >= p.nseg - 1) return;
        const int t_beg = u * p.L;
        t_end = (u + 1) * p.L;
        // values loaded from cu are the same in every lane: readfirstlane makes
        // that visible to the compiler, which then keeps the buffer descriptors
        // built from them in scalar registers (no per-lane waterfall loops)
        const CuView cu = cu_view(p);
        const int de = __builtin_amdgcn_readfirstlane(doc_at(cu, p.num_seqs, t_end - 1));
        const int dstart = __builtin_amdgcn_readfirstlane(cu[de]);
        const bool needs = __builtin_amdgcn_readfirstlane(cu[de + 1]) > t_end;
        const bool chain = dstart < t_beg;
        if (h == 0 && s == 0 && tid == 0) p.flags[u] = (needs ? 1 : 0) | (chain ? 2 : 0);
        if (!needs) return;
        first = max(t_beg, dstart);
    }

    const bf16_t* kg = static_cast<const bf16_t*>(p.k);
    const bf16_t* vg = static_cast<const bf16_t*>(p.v);
    const uint32_t row_bytes = (uint32_t)(p.H * D * 2);
    const int col0 = wave * G::CW;
    // decayed variant: the state is faded to the end of the piece
    const float l2 = DK ? log2f(p.decay[h]) : 0.f;
    float lc = 0.f;  // decayed: the state is 2^lc kv (fade_scale)
    float wfull[8];
    if constexpr (DK) full_weights(wfull, l2, lane);
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

    const int nblk = (t_end - first + B - 1) / B;
    // Pair jj = blocks 2jj and 2jj+1.  Blocks past the last one are issued
    // with an empty range: nothing is read, their rows arrive as zeros and
    // add nothing to the state.
    auto issue = [&](int jj, auto slot) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int b0 = first + (2 * jj + half) * B;
            // (clamp kept scalar: the descriptor built from it must live in
            // scalar registers)
            const int nb = __builtin_amdgcn_readfirstlane(max(0, min(B, t_end - b0)));
            const int64_t e0 = ((int64_t)phys_block(p, min(b0, t_end), nb) * p.H + h) * D;
            const uint32_t last = (uint32_t)(nb - 1) * row_bytes;
            dk.template issue<kNonTemporal>(make_rsrc(kg + e0, (uint32_t)nb * row_bytes), kbuf(slot) + half * B * D,
                                            p.rev, last);
            dv.template issue<kNonTemporal>(make_rsrc(vg + e0 + s * W, (uint32_t)nb * row_bytes),
                                            vbuf(slot) + half * B * W, p.rev, last);
        }
    };
    const int npairs = (nblk + 1) / 2;
    // Step i fills slot i % 2 with pair i, then reads pair i - 1 from the
    // other slot while pair i is in flight: the first two pairs go out back to
    // back, so a segment of up to four blocks waits for memory once.  (The
    // first fill is issued from the loop, not ahead of it, which keeps the
    // compiler's record of the slot each DMA in flight writes exact.)
    constexpr int LP = 2 * (DmaTile<D>::NI + DmaTile<W>::NI);  // loads per wave and pair
    int i = 0;
    auto step = [&](auto slot) {
        constexpr int SLOT = decltype(slot)::value;
        lds_barrier();  // pair i - 2 (read at step i - 1) is done with this slot
        issue(i, slot);
        if (i > 0) {
            vm_wait<LP>();  // pair i - 1 is in (pair i may still be in flight) ...
            lds_barrier();  // ... for every wave
            // tokens in the two blocks of pair i - 1 (0 past the end)
            const int b0 = first + 2 * (i - 1) * B;
            const int nb0 = max(0, min(B, t_end - b0)), nb1 = max(0, min(B, t_end - b0 - B));
            if constexpr (DK) {
                if (nb0 > 0) fade_scale(kv, lc, l2, nb0);
            }
            state_update<D, B, W, DK>(kv, vfr, kbuf(Slot<1 - SLOT>{}), vbuf(Slot<1 - SLOT>{}), col0, lane, l2, nb0,
                                      lc, DK ? wfull : nullptr);
            if constexpr (DK) {
                if (nb1 > 0) fade_scale(kv, lc, l2, nb1);
            }
            state_update<D, B, W, DK>(kv, vfr, kbuf(Slot<1 - SLOT>{}) + B * D, vbuf(Slot<1 - SLOT>{}) + B * W, col0,
                                      lane, l2, nb1, lc, DK ? wfull : nullptr);
        }
        ++i;
    };
    while (true) {
        step(Slot<0>{});
        if (i > npairs) break;
        step(Slot<1>{});
        if (i > npairs) break;
    }
    store_ws<D, B, W, DK>(kv, p.ws + ws_offset<D, W>(p, u, h, s, wave), lane, DK ? exp2f(lc) : 1.f);
    vm_wait<0>();  // no tile load may still be writing into this workgroup's LDS when it ends
}

// ---------------------------------------------------------------------------
// Transposes the first `states` segment states of src into dst (the same
// place, or another area of the workspace) while keeping the block loop's
// register order: where a (segment, head) entry of src holds the state X, the
// entry of dst then holds X^T, laid out as the block loop with the same (D, W)
// expects a state.  (Each workgroup reads its whole entry before it writes.)  The two reverse passes of the backward
// sum transposed states over the same segments (q^T dO and dO^T q), so one
// pass's prefix states serve the other.  One workgroup per entry: the D x D
// state goes through LDS as a plain matrix (rows padded by 4 floats, so the
// 16-byte column reads are conflict free).
template <int D, int W>
__global__ __launch_bounds__(kThreads) void la_ws_transpose_v2(const float* src, float* dst, int64_t states,
                                                                const int32_t* reuse) {
    constexpr int NCW = W / 64;  // 16-column tiles per block-loop wave (W / 4 columns)
    constexpr int PITCH = D + 4;
    constexpr int PER_WAVE = D * W / 16, PER_SLICE = D * W / 4;  // 16-byte entries
    __shared__ __align__(16) float M[D * PITCH];
    if ((int64_t)blockIdx.x >= states) return;
    if (reuse && !*reuse) return;  // the states were not the forward's: they are computed instead
    const f32x4_t* base = reinterpret_cast<const f32x4_t*>(src + (int64_t)blockIdx.x * D * D);
    f32x4_t* out = reinterpret_cast<f32x4_t*>(dst + (int64_t)blockIdx.x * D * D);
    // entry e holds rows i0 .. i0 + 3 of column j (store_ws's order)
    auto place = [](int e, int& i0, int& j) {
        const int s = e / PER_SLICE, w = (e % PER_SLICE) / PER_WAVE, q = e % PER_WAVE;
        const int a = (q / 64) / NCW, c = (q / 64) % NCW, lane = q % 64;
        i0 = state_row(a, lane >> 4, 0);
        j = s * W + w * (W / 4) + state_col<NCW>(c, lane & 15);
    };
    // every load of the entry is issued before the first LDS write, so the
    // workgroup waits for memory once rather than once per 16-byte run
    constexpr int PER_T = D * D / 4 / kThreads;
    static_assert(PER_T * kThreads == D * D / 4, "whole runs per thread");
    f32x4_t x[PER_T];
#pragma unroll
    for (int k = 0; k < PER_T; ++k) x[k] = base[threadIdx.x + k * kThreads];
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
        int i0, j;
        place(threadIdx.x + k * kThreads, i0, j);
#pragma unroll
        for (int r = 0; r < 4; ++r) M[(i0 + r) * PITCH + j] = x[k][r];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
        const int e = threadIdx.x + k * kThreads;
        int i0, j;
        place(e, i0, j);
        out[e] = *reinterpret_cast<const f32x4_t*>(M + j * PITCH + i0);  // (X^T)[i0 + r][j] = X[j][i0 + r]
    }
}

// ---------------------------------------------------------------------------
// The block loop.  NS tile slots: with two, block j + 1's tiles are loaded
// during iteration j; with three (long segments), block j + 2's are, so each
// load has a whole iteration more to arrive and twice the bytes are in flight
// per CU -- what a 4-wave workgroup needs to keep HBM busy.  (On short
// segments the deeper start costs more than it hides.)
//
// The body runs the unit of pass-local workgroup index wg (blockIdx.x, except
// in la_prefill_pair_v2 below).
template <int D, int B, int W, int NS, bool DK = false>
__device__ __forceinline__ void main_v2(const PrefillParams& p, const int64_t wg) {
    using G = Geo<D, B, W>;
    constexpr int NQT = G::NQT, NCW = G::NCW, NDT = G::NDT;
    static_assert(NQT == kWaves, "wave w takes key band w");
    static_assert(NS == 2 || NS == 3, "two or three tile slots");
    constexpr int PP = B;  // P[query][key] rows: 128 bytes
    // Each tile of each slot is its own LDS variable: with the loop unrolled
    // by the slot count, every LDS access names its slot at compile time, so
    // the compiler sees that reads of one slot do not alias the DMA writes in
    // flight to the others and adds no waits of its own.
    constexpr int QN = B * D, VN = B * W, X3 = NS == 3 ? 1 : 0;
    __shared__ __align__(16) bf16_t Q0[QN], Q1[QN], Q2[X3 ? QN : 8];
    __shared__ __align__(16) bf16_t K0[QN], K1[QN], K2[X3 ? QN : 8];
    __shared__ __align__(16) bf16_t V0[VN], V1[VN], V2[X3 ? VN : 8];
    __shared__ __align__(16) bf16_t Ps[B * PP];
    // Late output stores: the intra product packs block j-1's rows into
    // registers and they are stored after the iteration's tile loads, so that
    // the next iteration's wait for its tiles leaves them in flight.  (The
    // full-width loop with three slots has no registers to spare; it stores
    // at once and its wait covers one iteration's loads and stores anyway.)
    constexpr bool LATE = NCW == 1 || NS == 2;
    constexpr int NST = G::STORES;  // VMEM stores per wave and block
    auto qbuf = [&](auto slot) -> bf16_t* {
        constexpr int X = decltype(slot)::value;
        if constexpr (X == 0) return Q0;
        else if constexpr (X == 1) return Q1;
        else return Q2;
    };
    auto kbuf = [&](auto slot) -> bf16_t* {
        constexpr int X = decltype(slot)::value;
        if constexpr (X == 0) return K0;
        else if constexpr (X == 1) return K1;
        else return K2;
    };
    auto vbuf = [&](auto slot) -> bf16_t* {
        constexpr int X = decltype(slot)::value;
        if constexpr (X == 0) return V0;
        else if constexpr (X == 1) return V1;
        else return V2;
    };

    stamp_key(p, wg);
    int u = 0, h, s, t0, t1;
    int lb0 = 0, lb1 = 0;  // packed: state slots of the document's earlier pieces
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: descriptors in SGPRs
    if (p.packed) {
        Piece pc;
        if (!piece_of(p, wg, pc, h, s)) return;
        if (pc.len == 0) {  // an empty document: only its final state
            if (p.kv_out) one_empty_doc_state<D, W>(p, pc.doc, h, s, tid);
            return;
        }
        t0 = pc.t0;
        t1 = pc.t0 + pc.len;
        lb0 = pc.base;
        lb1 = pc.base + (t0 - cu_view(p)[pc.doc]) / p.L;
    } else {
        if (!unit_of(p, wg, u, h, s)) return;
        t0 = u * p.L;
        t1 = min(p.T, t0 + p.L);
    }
    const int col0 = wave * G::CW;
    const bf16_t* qg = static_cast<const bf16_t*>(p.q);
    const bf16_t* kg = static_cast<const bf16_t*>(p.k);
    const bf16_t* vg = static_cast<const bf16_t*>(p.v);
    bf16_t* og = static_cast<bf16_t*>(p.o);
    const uint32_t row_bytes = (uint32_t)(p.H * D * 2);

    DmaTile<D> dq;
    DmaTile<W> dv;
    dq.init(wave, lane, row_bytes);
    dv.init(wave, lane, row_bytes);

    const CuView cuv = cu_view(p);
    Cursor c0;
    cursor_first(c0, cuv, p.num_seqs, t0, t1, B);

    // Decayed variant: this head's log2 lambda and the per-lane factors that
    // do not change from block to block: lambda^(query - key) on the scores
    // (0 above the diagonal: the causal mask), lambda^(query + 1) on the inter
    // product of query row 16 b + li.
    float l2 = 0.f, sfac[DK ? NQT : 1][4], ifac[DK ? NQT : 1], wfull[8];
    float lc = 0.f;  // decayed: the state is 2^lc kv (fade_scale)
    if constexpr (DK) {
        l2 = log2f(p.decay[h]);
        full_weights(wfull, l2, lane);
#pragma unroll
        for (int b = 0; b < NQT; ++b) {
            ifac[b] = decay_pow(l2, 16 * b + li + 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = (16 * b + li) - (16 * wave + 4 * g + r);
                sfac[b][r] = m >= 0 ? decay_pow(l2, m) : 0.f;
            }
        }
    }

    f32x4_t kv[NDT][NCW];
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int c = 0; c < NCW; ++c) kv[a][c] = zero4();
    f32x4_t oacc[NQT][NCW];
#pragma unroll
    for (int b = 0; b < NQT; ++b)
#pragma unroll
        for (int c = 0; c < NCW; ++c) oacc[b][c] = zero4();
    Frag<bf16_t> vfr[NCW][B / 32];
    u32x4_t opk[NQT];  // packed output rows of the previous block (late stores: lanes as oacc)

    // A cursor past the end (nb = 0) still issues its loads, with an empty
    // buffer range: nothing is read, zeros land in the unused slot, and every
    // path through the loop issues the same vector-memory operations (the
    // compiler's wait bookkeeping then stays exact instead of conservative).
    // The three tiles of a block (TILE 0 = Q, 1 = K, 2 = V) can be issued at
    // different points of an iteration, so the address unit works through
    // them while the wave computes instead of stalling every wave at once.
    auto issue_tile = [&](const Cursor& c, auto slot, auto tile) {
        constexpr int TILE = decltype(tile)::value;
        const int nb = max(c.nb, 0);
        const int64_t e0 = ((int64_t)(nb > 0 ? phys_block(p, c.b0, nb) : 0) * p.H + h) * D;
        const uint32_t bytes = (uint32_t)nb * row_bytes;
        const uint32_t last = (uint32_t)(nb - 1) * row_bytes;
        if constexpr (TILE == 0) dq.issue(make_rsrc(qg + e0, bytes), qbuf(slot), p.rev, last);
        else if constexpr (TILE == 1) dq.issue(make_rsrc(kg + e0, bytes), kbuf(slot), p.rev, last);
        else dv.issue(make_rsrc(vg + e0 + s * W, bytes), vbuf(slot), p.rev, last);
    };
    auto issue = [&](const Cursor& c, auto slot) {
        issue_tile(c, slot, Slot<0>{});
        issue_tile(c, slot, Slot<1>{});
        issue_tile(c, slot, Slot<2>{});
    };
    // O^T += V^T P^T for the previous block, then its rows are stored.
    auto finish = [&](int pb0, int pnb) {
        // With one tile column per wave there are registers to fetch every P
        // fragment before the first product, so the LDS latency is paid once
        // (the full-width loop has none to spare and reads them one by one).
        if constexpr (NCW == 1) {
            Frag<bf16_t> pfs[6];  // (band, chunk) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
#pragma unroll
            for (int b = 0, n = 0; b < NQT; ++b)
#pragma unroll
                for (int kc = 0; kc <= b / 2; ++kc, ++n) load_row<PP>(pfs[n], Ps, 16 * b + li, 32 * kc, g);
#pragma unroll
            for (int b = 0, n = 0; b < NQT; ++b)
#pragma unroll
                for (int kc = 0; kc <= b / 2; ++kc, ++n) mma(oacc[b][0], vfr[0][kc], pfs[n]);
        } else {
#pragma unroll
            for (int b = 0; b < NQT; ++b) {
#pragma unroll
                for (int kc = 0; kc <= b / 2; ++kc) {
                    Frag<bf16_t> pf;
                    load_row<PP>(pf, Ps, 16 * b + li, 32 * kc, g);
#pragma unroll
                    for (int c = 0; c < NCW; ++c) mma(oacc[b][c], vfr[c][kc], pf);
                }
            }
        }
        if constexpr (LATE) {
#pragma unroll
            for (int b = 0; b < NQT; ++b) {
                opk[b].x = pack2(oacc[b][0][0], oacc[b][0][1]);
                opk[b].y = pack2(oacc[b][0][2], oacc[b][0][3]);
                if constexpr (NCW == 2) {
                    opk[b].z = pack2(oacc[b][1][0], oacc[b][1][1]);
                    opk[b].w = pack2(oacc[b][1][2], oacc[b][1][3]);
                }
#pragma unroll
                for (int c = 0; c < NCW; ++c) oacc[b][c] = zero4();
            }
            return;
        }
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(og + ((int64_t)phys_block(p, pb0, pnb) * p.H + h) * D + s * W + col0, (uint32_t)pnb * row_bytes);
        // output row 16b + li of the block; in reverse mode its mirror pnb - 1 - (16b + li)
        // (negative -> a huge unsigned offset -> dropped by the range check)
        auto orow = [&](int b) -> uint32_t {
            const int r = 16 * b + li;
            return (uint32_t)(p.rev ? pnb - 1 - r : r) * row_bytes;
        };
#pragma unroll
        for (int b = 0; b < NQT; ++b) {
            if constexpr (NCW == 2) {  // columns 8g..8g+7 of row 16b + li: one 16-byte store
                u32x4_t v;
                v.x = pack2(oacc[b][0][0], oacc[b][0][1]);
                v.y = pack2(oacc[b][0][2], oacc[b][0][3]);
                v.z = pack2(oacc[b][1][0], oacc[b][1][1]);
                v.w = pack2(oacc[b][1][2], oacc[b][1][3]);
                __builtin_amdgcn_raw_buffer_store_b128(v, ro, orow(b) + (8 * g) * 2, 0, 0);
            } else {
#pragma unroll
                for (int c = 0; c < NCW; ++c) {
                    u32x2_t v;
                    v.x = pack2(oacc[b][c][0], oacc[b][c][1]);
                    v.y = pack2(oacc[b][c][2], oacc[b][c][3]);
                    __builtin_amdgcn_raw_buffer_store_b64(v, ro, orow(b) + (16 * c + 4 * g) * 2, 0, 0);
                }
            }
#pragma unroll
            for (int c = 0; c < NCW; ++c) oacc[b][c] = zero4();
        }
    };

    auto finish_store = [&](int pb0, int pnb) {
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(og + ((int64_t)phys_block(p, pb0, pnb) * p.H + h) * D + s * W + col0, (uint32_t)pnb * row_bytes);
#pragma unroll
        for (int b = 0; b < NQT; ++b) {
            const int r = 16 * b + li;
            const uint32_t off = (uint32_t)(p.rev ? pnb - 1 - r : r) * row_bytes;
            if constexpr (NCW == 2) __builtin_amdgcn_raw_buffer_store_b128(opk[b], ro, off + (8 * g) * 2, 0, 0);
            else {
                u32x2_t v;
                v.x = opk[b].x;
                v.y = opk[b].y;
                __builtin_amdgcn_raw_buffer_store_b64(v, ro, off + (4 * g) * 2, 0, 0);
            }
        }
    };

    // the block after c0 (kept from step to step with three slots)
    Cursor c1 = c0;
    if constexpr (NS == 3) {
        if (c0.nb > 0) cursor_next(c1, cuv, p.num_seqs, t1, B);
    }
    if (c0.nb > 0) {  // before the prefix loads, so the two overlap
        issue(c0, Slot<0>{});
        if constexpr (NS == 3) issue(c1, Slot<1>{});
    }
    if (c0.nb > 0 && !c0.first_of_doc) {
        const int u_first = p.packed ? lb0 : p.scan ? u - 1 : cuv[c0.doc] / p.L;
        const int u_end = p.packed ? lb1 : u;
        for (int uu = u_first; uu < u_end; ++uu) {
            // (decayed: slot uu ends (u_end - uu - 1) L tokens before this unit starts)
            load_ws<D, B, W, DK>(kv, p.ws + ws_offset<D, W>(p, uu, h, s, wave), lane,
                                 DK ? decay_pow(l2, (u_end - uu - 1) * p.L) : 1.f);
        }
    }
    // a caller-supplied state before the document's first token joins the prefix
    // (decayed: faded by the tokens between the document start and this unit's)
    if (p.kv_in && c0.nb > 0)
        add_state<D, B, W>(kv, p.kv_in + (((int64_t)phys_doc(p, c0.doc) * p.H + h) * D) * D, s * W + col0, p.kv_in_t,
                           g, li, DK ? decay_pow(l2, t0 - cuv[c0.doc]) : 1.f);
    int pb0 = t0, pnb = 0;
    int j = 0;
    // One block (j); its tiles sit in slot SLOT.  This iteration loads block
    // j + NS - 1 into slot FILL, the one block j - 1 used.
    auto step = [&](auto slot) {
        constexpr int SLOT = decltype(slot)::value;
        constexpr int FILL = (SLOT + NS - 1) % NS;
        Cursor cf;
        if constexpr (NS == 2) {
            cf = c0;
            cursor_next(cf, cuv, p.num_seqs, t1, B);
        } else {
            cf = c1;
            if (c1.nb > 0) cursor_next(cf, cuv, p.num_seqs, t1, B);
            else cf.nb = 0;
        }
        // Loads of block j are done.  Vector-memory operations retire in
        // issue order, so the wait lets exactly what was issued after them
        // stay in flight: with two slots, the previous iteration's output
        // stores (issued after its loads); with three, the previous
        // iteration's loads and stores.  The first iteration follows the
        // prologue instead, which issues no stores: there only block 1's
        // loads (three slots) may still be in flight.
        static_assert(NS == 3 || LATE, "two slots always store late");
        if constexpr (NS == 2) {
            if (j == 0) vm_wait<0>();
            else vm_wait<NST>();
        } else {
            if (j == 0) vm_wait<G::LOADS>();
            else vm_wait<G::LOADS + NST>();
        }
        lds_barrier();  // (A) block j visible; block j-1's tiles no longer read
        // Where the next tiles' Q and K go out: around the intra product with
        // three slots (tiles two blocks ahead), after it with two, where that
        // measured faster on short segments (plain loop; the decayed one keeps
        // the first placement).  Either way after (A), past which no wave reads
        // their slot.
        constexpr bool QK_AFTER = NS == 2 && !DK;
        if constexpr (!QK_AFTER) issue_tile(cf, Slot<FILL>{}, Slot<0>{});
        // block j-1's intra product (and its rows, unless they are stored
        // late); in the first iteration pnb = 0 and the stores (of whatever
        // the accumulators hold) fall outside the buffer range
        finish(pb0, pnb);
        if constexpr (!QK_AFTER) issue_tile(cf, Slot<FILL>{}, Slot<1>{});
        lds_barrier();  // (B) scores of block j-1 consumed
        if constexpr (QK_AFTER) {
            issue_tile(cf, Slot<FILL>{}, Slot<0>{});
            issue_tile(cf, Slot<FILL>{}, Slot<1>{});
        }

        const bf16_t* Qs = qbuf(slot);
        const bf16_t* Ks = kbuf(slot);
        const bf16_t* Vs = vbuf(slot);
        // inter: O^T += KV^T Q^T with the state before this block, and the
        // scores S^T = K_w Q^T of key band w (= this wave) against every
        // query band, from the same Q fragments
        f32x4_t sacc[NQT];
#pragma unroll
        for (int b = 0; b < NQT; ++b) sacc[b] = zero4();
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
            Frag<bf16_t> kvf[NCW];
#pragma unroll
            for (int c = 0; c < NCW; ++c) {
                kvf[c].lo = make_uint2(pack2(kv[2 * m][c][0], kv[2 * m][c][1]), pack2(kv[2 * m][c][2], kv[2 * m][c][3]));
                kvf[c].hi = make_uint2(pack2(kv[2 * m + 1][c][0], kv[2 * m + 1][c][1]),
                                       pack2(kv[2 * m + 1][c][2], kv[2 * m + 1][c][3]));
            }
            Frag<bf16_t> kf;
            load_row<D>(kf, Ks, 16 * wave + li, 32 * m, g);
            if constexpr (NCW == 1) {  // (as in finish: all Q fragments of the chunk first)
                Frag<bf16_t> qfs[NQT];
#pragma unroll
                for (int b = 0; b < NQT; ++b) load_row<D>(qfs[b], Qs, 16 * b + li, 32 * m, g);
#pragma unroll
                for (int b = 0; b < NQT; ++b) {
                    mma(oacc[b][0], kvf[0], qfs[b]);
                    mma(sacc[b], kf, qfs[b]);
                }
            } else {
#pragma unroll
                for (int b = 0; b < NQT; ++b) {
                    Frag<bf16_t> qf;
                    load_row<D>(qf, Qs, 16 * b + li, 32 * m, g);
#pragma unroll
                    for (int c = 0; c < NCW; ++c) mma(oacc[b][c], kvf[c], qf);
                    mma(sacc[b], kf, qf);
                }
            }
        }
        // decayed: the state reaches query row r faded r + 1 times, and kv
        // holds it divided by 2^lc
        if constexpr (DK) {
            const float sc = exp2f(lc);
#pragma unroll
            for (int b = 0; b < NQT; ++b)
#pragma unroll
                for (int c = 0; c < NCW; ++c) oacc[b][c] *= ifac[b] * sc;
        }
        issue_tile(cf, Slot<FILL>{}, Slot<2>{});
        // block j-1's rows leave after this iteration's loads: the next
        // iteration's wait for those loads lets these stores stay in flight
        if constexpr (LATE) finish_store(pb0, pnb);
        // state: KV += K^T V (after the inter product read it)
        if constexpr (DK) fade_scale(kv, lc, l2, c0.nb);
        state_update<D, B, W, DK>(kv, vfr, Ks, Vs, col0, lane, l2, c0.nb, lc, DK ? wfull : nullptr);

        // P[query][key] for keys of band w: causal mask (key <= query), the
        // tiles above the diagonal come out as zeros
#pragma unroll
        for (int b = 0; b < NQT; ++b) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (DK) sacc[b][r] *= sfac[b][r];  // lambda^(query - key), 0 above the diagonal
                else if (16 * wave + 4 * g + r > 16 * b + li) sacc[b][r] = 0.f;
            }
            store4(Ps + soff<PP>(16 * b + li, 16 * wave + 4 * g), sacc[b][0], sacc[b][1], sacc[b][2], sacc[b][3]);
        }

        if (c0.b0 + c0.nb == c0.doc_end) {  // the document ends with this block
            vm_wait<0>();  // rare path: keeps the loop's wait bookkeeping exact
            if (p.kv_out)
                store_state<D, B, W, DK>(kv,
                                         p.kv_out + (((int64_t)phys_doc(p, c0.doc) * p.H + h) * D) * D + s * W + col0,
                                         g, li, DK ? exp2f(lc) : 1.f);
#pragma unroll
            for (int a = 0; a < NDT; ++a)
#pragma unroll
                for (int c = 0; c < NCW; ++c) kv[a][c] = zero4();
            lc = 0.f;
            const Cursor& cn = NS == 2 ? cf : c1;  // block j + 1
            if (p.kv_in && cn.nb > 0 && cn.first_of_doc) {  // the next document starts here
                add_state<D, B, W>(kv, p.kv_in + (((int64_t)phys_doc(p, cn.doc) * p.H + h) * D) * D, s * W + col0,
                                   p.kv_in_t, g, li);
                vm_wait<0>();
            }
        }
        pb0 = c0.b0;
        pnb = c0.nb;
        if constexpr (NS == 2) {
            c0 = cf;
        } else {
            c0 = c1;
            c1 = cf;
        }
        ++j;
    };
    while (c0.nb > 0) {
        step(Slot<0>{});
        if (c0.nb <= 0) break;
        step(Slot<1>{});
        if constexpr (NS == 3) {
            if (c0.nb <= 0) break;
            step(Slot<2>{});
        }
    }
    if (j > 0) {
        lds_barrier();  // scores of the last block visible
        finish(pb0, pnb);
        if constexpr (LATE) finish_store(pb0, pnb);
    }

    if (p.kv_out && !p.packed) empty_doc_states<D, W>(p, u, h, s, t0, t1, tid);
    vm_wait<0>();  // no tile load may still be writing into this workgroup's LDS when it ends
}

// ---------------------------------------------------------------------------
// The block loop for 128-token blocks (bf16, 64-column slices, plain variant).
// A block of 128 tokens runs as two halves of 64 rows, a and c, on the tiles,
// fragments and LDS layout of the 64-token loop.  Both halves take the inter
// product against the state at the block's start, so the state update
// (KV += K_a^T V_a + K_c^T V_c) waits for the end of c; c's intra product adds,
// to its own masked scores P_cc = mask(Q_c K_c^T), the unmasked scores of its
// queries against a's keys, P_ca = Q_c K_a^T, times V_a: together the block's
// left product (Q K^T (.) M) V over all 128 tokens.  Blocks restart at each
// document start (a document whose length is an odd number of halves ends with
// an empty c half, which keeps the halves' order fixed).
//
// Slots: a halves alternate between slots 0 and 2, c halves use slot 1, so
// a's tiles stay in place while c runs.  Iteration a loads the same block's c
// half (one iteration ahead) and the next block's a half (two ahead); iteration
// c loads nothing.  A tile load into a slot is issued only after the barrier
// past which no wave reads that slot's previous contents.  The loop is
// unrolled over two blocks, so every slot and every wait count is fixed at
// compile time.
template <int D, int W>
__device__ __forceinline__ void main_v2_b128(const PrefillParams& p, const int64_t wg) {
    constexpr int B = 64;  // rows of a half
    using G = Geo<D, B, W>;
    constexpr int NQT = G::NQT, NCW = G::NCW, NDT = G::NDT;
    static_assert(NQT == kWaves && (NCW == 1 || NCW == 2), "key band w per wave; one or two column tiles");
    constexpr int PP = B;
    constexpr int QN = B * D, VN = B * W;
    __shared__ __align__(16) bf16_t Q0[QN], Q1[QN], Q2[QN];
    __shared__ __align__(16) bf16_t K0[QN], K1[QN], K2[QN];
    __shared__ __align__(16) bf16_t V0[VN], V1[VN], V2[VN];
    __shared__ __align__(16) bf16_t Ps[B * PP];  // masked scores of the half (P_aa or P_cc)
    __shared__ __align__(16) bf16_t Px[B * PP];  // c's queries against a's keys (P_ca)
    constexpr int NST = G::STORES, LOADS = G::LOADS;
    // Full width (two column tiles per wave) has no registers to keep V^T
    // fragments or packed rows from one iteration to the next: there the
    // intra product reads its V^T fragments from LDS (a half's tiles stay in
    // place until after it) and stores its rows at once.
    constexpr bool LIGHT = NCW == 2;
    auto qbuf = [&](auto slot) -> bf16_t* {
        constexpr int X = decltype(slot)::value;
        if constexpr (X == 0) return Q0;
        else if constexpr (X == 1) return Q1;
        else return Q2;
    };
    auto kbuf = [&](auto slot) -> bf16_t* {
        constexpr int X = decltype(slot)::value;
        if constexpr (X == 0) return K0;
        else if constexpr (X == 1) return K1;
        else return K2;
    };
    auto vbuf = [&](auto slot) -> bf16_t* {
        constexpr int X = decltype(slot)::value;
        if constexpr (X == 0) return V0;
        else if constexpr (X == 1) return V1;
        else return V2;
    };

    stamp_key(p, wg);
    int u = 0, h, s, t0, t1;
    int lb0 = 0, lb1 = 0;
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (p.packed) {
        Piece pc;
        if (!piece_of(p, wg, pc, h, s)) return;
        if (pc.len == 0) {
            if (p.kv_out) one_empty_doc_state<D, W>(p, pc.doc, h, s, tid);
            return;
        }
        t0 = pc.t0;
        t1 = pc.t0 + pc.len;
        lb0 = pc.base;
        lb1 = pc.base + (t0 - cu_view(p)[pc.doc]) / p.L;
    } else {
        if (!unit_of(p, wg, u, h, s)) return;
        t0 = u * p.L;
        t1 = min(p.T, t0 + p.L);
    }
    const int col0 = wave * G::CW;
    const bf16_t* qg = static_cast<const bf16_t*>(p.q);
    const bf16_t* kg = static_cast<const bf16_t*>(p.k);
    const bf16_t* vg = static_cast<const bf16_t*>(p.v);
    bf16_t* og = static_cast<bf16_t*>(p.o);
    const uint32_t row_bytes = (uint32_t)(p.H * D * 2);

    DmaTile<D> dq;
    DmaTile<W> dv;
    dq.init(wave, lane, row_bytes);
    dv.init(wave, lane, row_bytes);

    const CuView cuv = cu_view(p);
    Cursor c0;  // the current 128-token block
    cursor_first(c0, cuv, p.num_seqs, t0, t1, 2 * B);

    f32x4_t kv[NDT][NCW];
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int c = 0; c < NCW; ++c) kv[a][c] = zero4();
    f32x4_t oacc[NQT][NCW];
#pragma unroll
    for (int b = 0; b < NQT; ++b)
#pragma unroll
        for (int c = 0; c < NCW; ++c) oacc[b][c] = zero4();
    Frag<bf16_t> vfa[NCW][B / 32];  // V_a^T fragments: a's intra product and c's cross term
    Frag<bf16_t> vfc[NCW][B / 32];  // V_c^T fragments
    u32x4_t opk[NQT];

    int pb0 = t0, pnb = 0;  // the half whose rows the next finish stores
    // Half HF (0 = a, 1 = c) of block c: its first token and length (0 past the end).
    auto half = [&](const Cursor& c, int hf, int& b0h, int& nbh) {
        const int nb = max(c.nb, 0);
        b0h = c.b0 + B * hf;
        nbh = hf == 0 ? min(B, nb) : max(0, nb - B);
    };
    auto issue_tile = [&](const Cursor& c, auto hf, auto slot, auto tile) {
        constexpr int TILE = decltype(tile)::value;
        int b0h, nbh;
        half(c, decltype(hf)::value, b0h, nbh);
        const int64_t e0 = ((int64_t)(nbh > 0 ? phys_block(p, b0h, nbh) : 0) * p.H + h) * D;
        const uint32_t bytes = (uint32_t)nbh * row_bytes;
        const uint32_t last = (uint32_t)(nbh - 1) * row_bytes;
        if constexpr (TILE == 0) dq.issue(make_rsrc(qg + e0, bytes), qbuf(slot), p.rev, last);
        else if constexpr (TILE == 1) dq.issue(make_rsrc(kg + e0, bytes), kbuf(slot), p.rev, last);
        else dv.issue(make_rsrc(vg + e0 + s * W, bytes), vbuf(slot), p.rev, last);
    };
    // O^T += V^T P^T for the previous half (and, after a c half, + V_a^T P_ca^T),
    // then its rows are packed for the late stores.
    auto finish_store = [&](int pb0, int pnb) {
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(og + ((int64_t)phys_block(p, pb0, pnb) * p.H + h) * D + s * W + col0, (uint32_t)pnb * row_bytes);
#pragma unroll
        for (int b = 0; b < NQT; ++b) {
            const int r = 16 * b + li;
            const uint32_t off = (uint32_t)(p.rev ? pnb - 1 - r : r) * row_bytes;
            if constexpr (NCW == 2) {
                __builtin_amdgcn_raw_buffer_store_b128(opk[b], ro, off + (8 * g) * 2, 0, 0);
            } else {
                u32x2_t v;
                v.x = opk[b].x;
                v.y = opk[b].y;
                __builtin_amdgcn_raw_buffer_store_b64(v, ro, off + (4 * g) * 2, 0, 0);
            }
        }
    };
    auto load_vf = [&](Frag<bf16_t> (&vf)[NCW][B / 32], const bf16_t* Vs) {
#pragma unroll
        for (int kc = 0; kc < B / 32; ++kc)
#pragma unroll
            for (int c = 0; c < NCW; ++c) {
                if constexpr (NCW == 2) load_tr<W, 8>(vf[c][kc], Vs, 32 * kc, col0, 4 * c, lane);
                else load_tr<W, 4>(vf[c][kc], Vs, 32 * kc, col0 + 16 * c, 0, lane);
            }
    };
    // (LIGHT: the previous half's rows are stored here; Va = its block's a half's V tile)
    auto finish = [&](auto cross, const bf16_t* Va) {
        constexpr bool X = decltype(cross)::value;
        if constexpr (LIGHT) {
            load_vf(vfa, Va);
            if constexpr (X) load_vf(vfc, vbuf(Slot<1>{}));
        }
        auto& vf = X ? vfc : vfa;  // the half's own V^T fragments
        if constexpr (NCW == 1) {  // registers to fetch every P fragment first
            Frag<bf16_t> pfs[6];  // (band, chunk) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
#pragma unroll
            for (int b = 0, n = 0; b < NQT; ++b)
#pragma unroll
                for (int kc = 0; kc <= b / 2; ++kc, ++n) load_row<PP>(pfs[n], Ps, 16 * b + li, 32 * kc, g);
#pragma unroll
            for (int b = 0, n = 0; b < NQT; ++b)
#pragma unroll
                for (int kc = 0; kc <= b / 2; ++kc, ++n) mma(oacc[b][0], vf[0][kc], pfs[n]);
        } else {
#pragma unroll
            for (int b = 0; b < NQT; ++b)
#pragma unroll
                for (int kc = 0; kc <= b / 2; ++kc) {
                    Frag<bf16_t> pf;
                    load_row<PP>(pf, Ps, 16 * b + li, 32 * kc, g);
#pragma unroll
                    for (int c = 0; c < NCW; ++c) mma(oacc[b][c], vf[c][kc], pf);
                }
        }
        if constexpr (X) {  // c's queries against a's keys
#pragma unroll
            for (int b = 0; b < NQT; ++b)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    Frag<bf16_t> xf;
                    load_row<PP>(xf, Px, 16 * b + li, 32 * kc, g);
#pragma unroll
                    for (int c = 0; c < NCW; ++c) mma(oacc[b][c], vfa[c][kc], xf);
                }
        }
#pragma unroll
        for (int b = 0; b < NQT; ++b) {
            opk[b].x = pack2(oacc[b][0][0], oacc[b][0][1]);
            opk[b].y = pack2(oacc[b][0][2], oacc[b][0][3]);
            if constexpr (NCW == 2) {
                opk[b].z = pack2(oacc[b][1][0], oacc[b][1][1]);
                opk[b].w = pack2(oacc[b][1][2], oacc[b][1][3]);
            }
#pragma unroll
            for (int c = 0; c < NCW; ++c) oacc[b][c] = zero4();
        }
        if constexpr (LIGHT) finish_store(pb0, pnb);
    };
    // inter product O^T += KV^T Q^T of the half in Qs, with its masked scores
    // S^T = K_w Q^T (key band w of Ks), and, with Ka, the unmasked scores of
    // the same queries against key band w of Ka
    auto inter = [&](const bf16_t* Qs, const bf16_t* Ks, const bf16_t* Ka, f32x4_t (&sacc)[NQT],
                     f32x4_t (&xacc)[NQT], auto with_cross) {
#pragma unroll
        for (int b = 0; b < NQT; ++b) {
            sacc[b] = zero4();
            if constexpr (decltype(with_cross)::value) xacc[b] = zero4();
        }
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
            Frag<bf16_t> kvf[NCW];
#pragma unroll
            for (int c = 0; c < NCW; ++c) {
                kvf[c].lo = make_uint2(pack2(kv[2 * m][c][0], kv[2 * m][c][1]), pack2(kv[2 * m][c][2], kv[2 * m][c][3]));
                kvf[c].hi = make_uint2(pack2(kv[2 * m + 1][c][0], kv[2 * m + 1][c][1]),
                                       pack2(kv[2 * m + 1][c][2], kv[2 * m + 1][c][3]));
            }
            Frag<bf16_t> kf, kx;
            load_row<D>(kf, Ks, 16 * wave + li, 32 * m, g);
            if constexpr (decltype(with_cross)::value) load_row<D>(kx, Ka, 16 * wave + li, 32 * m, g);
            if constexpr (NCW == 1) {  // all Q fragments of the chunk first
                Frag<bf16_t> qfs[NQT];
#pragma unroll
                for (int b = 0; b < NQT; ++b) load_row<D>(qfs[b], Qs, 16 * b + li, 32 * m, g);
#pragma unroll
                for (int b = 0; b < NQT; ++b) {
                    mma(oacc[b][0], kvf[0], qfs[b]);
                    mma(sacc[b], kf, qfs[b]);
                    if constexpr (decltype(with_cross)::value) mma(xacc[b], kx, qfs[b]);
                }
            } else {
#pragma unroll
                for (int b = 0; b < NQT; ++b) {
                    Frag<bf16_t> qf;
                    load_row<D>(qf, Qs, 16 * b + li, 32 * m, g);
#pragma unroll
                    for (int c = 0; c < NCW; ++c) mma(oacc[b][c], kvf[c], qf);
                    mma(sacc[b], kf, qf);
                    if constexpr (decltype(with_cross)::value) mma(xacc[b], kx, qf);
                }
            }
        }
    };
    // P[query][key] for keys of band w (masked: key <= query) into buffer P
    auto store_scores = [&](bf16_t* P, f32x4_t (&acc)[NQT], bool masked) {
#pragma unroll
        for (int b = 0; b < NQT; ++b) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (masked && 16 * wave + 4 * g + r > 16 * b + li) acc[b][r] = 0.f;
            store4(P + soff<PP>(16 * b + li, 16 * wave + 4 * g), acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
        }
    };
    // KV += K^T V with the V^T fragments already loaded
    auto kv_add = [&](const bf16_t* Ks, const Frag<bf16_t> (&vf)[NCW][B / 32]) {
#pragma unroll
        for (int kc = 0; kc < B / 32; ++kc)
#pragma unroll
            for (int a = 0; a < NDT; ++a) {
                Frag<bf16_t> kf;
                load_tr<D, 8>(kf, Ks, 32 * kc, 32 * (a >> 1), 4 * (a & 1), lane);
#pragma unroll
                for (int c = 0; c < NCW; ++c) mma(kv[a][c], kf, vf[c][kc]);
            }
    };

    if (c0.nb > 0) {  // the first block's a half, before the prefix loads, so the two overlap
        issue_tile(c0, Slot<0>{}, Slot<0>{}, Slot<0>{});
        issue_tile(c0, Slot<0>{}, Slot<0>{}, Slot<1>{});
        issue_tile(c0, Slot<0>{}, Slot<0>{}, Slot<2>{});
    }
    if (c0.nb > 0 && !c0.first_of_doc) {
        const int u_first = p.packed ? lb0 : p.scan ? u - 1 : cuv[c0.doc] / p.L;
        const int u_end = p.packed ? lb1 : u;
        for (int uu = u_first; uu < u_end; ++uu) load_ws<D, B, W>(kv, p.ws + ws_offset<D, W>(p, uu, h, s, wave), lane);
    }
    if (p.kv_in && c0.nb > 0)
        add_state<D, B, W>(kv, p.kv_in + (((int64_t)phys_doc(p, c0.doc) * p.H + h) * D) * D, s * W + col0, p.kv_in_t,
                           g, li);
    bool first = true;
    Cursor cn = c0;  // the next block
    // Half a of block c0, in slot AS; the next block's a half goes to slot NAS
    // (where the previous block's a half was).
    auto step_a = [&](auto as, auto nas) {
        cn = c0;
        cursor_next(cn, cuv, p.num_seqs, t1, 2 * B);
        // a's loads were issued before the previous block's halves stored their
        // rows (one store group each, or only c's at once with LIGHT); the
        // first block's, by the prologue alone
        if (first) vm_wait<0>();
        else vm_wait<LIGHT ? NST : 2 * NST>();
        first = false;
        lds_barrier();  // (A) a visible; the previous block's tiles no longer read
        issue_tile(c0, Slot<1>{}, Slot<1>{}, Slot<0>{});
        issue_tile(c0, Slot<1>{}, Slot<1>{}, Slot<1>{});
        finish(Slot<1>{}, vbuf(nas));  // the previous c half (nothing stored before the first)
        // c's V tile goes where the previous c half's was, which finish may
        // read (full width): only once every wave is past it.  The next a
        // half's Q follows it, so that a's three tiles stay the last loads
        // issued before the c half's wait.
        lds_barrier();  // (B) scores and V tiles of the previous half consumed
        issue_tile(c0, Slot<1>{}, Slot<1>{}, Slot<2>{});
        issue_tile(cn, Slot<0>{}, nas, Slot<0>{});
        f32x4_t sacc[NQT], xacc[NQT];
        inter(qbuf(as), kbuf(as), nullptr, sacc, xacc, Slot<0>{});
        issue_tile(cn, Slot<0>{}, nas, Slot<1>{});
        issue_tile(cn, Slot<0>{}, nas, Slot<2>{});
        if constexpr (!LIGHT) {
            finish_store(pb0, pnb);
            load_vf(vfa, vbuf(as));
        }
        store_scores(Ps, sacc, true);
        half(c0, 0, pb0, pnb);
    };
    // Half c of block c0 (in slot 1; its a half in slot AS), then the state
    // update of the whole block.
    auto step_c = [&](auto as) {
        // c's loads were followed by the next a half's (and one late store group)
        vm_wait<LIGHT ? LOADS : LOADS + NST>();
        lds_barrier();  // (A)
        finish(Slot<0>{}, vbuf(as));  // a's intra product
        lds_barrier();  // (B)
        if constexpr (LIGHT) {
            // (full width: the cross scores in a second pass over Q_c, so that
            // the two score sets are never live together)
            {
                f32x4_t sacc[NQT], xacc[NQT];
                inter(qbuf(Slot<1>{}), kbuf(Slot<1>{}), nullptr, sacc, xacc, Slot<0>{});
                store_scores(Ps, sacc, true);
            }
            {
                f32x4_t xacc[NQT];
#pragma unroll
                for (int b = 0; b < NQT; ++b) xacc[b] = zero4();
#pragma unroll
                for (int m = 0; m < D / 32; ++m) {
                    Frag<bf16_t> kx;
                    load_row<D>(kx, kbuf(as), 16 * wave + li, 32 * m, g);
#pragma unroll
                    for (int b = 0; b < NQT; ++b) {
                        Frag<bf16_t> qf;
                        load_row<D>(qf, qbuf(Slot<1>{}), 16 * b + li, 32 * m, g);
                        mma(xacc[b], kx, qf);
                    }
                }
                store_scores(Px, xacc, false);
            }
            load_vf(vfa, vbuf(as));
            kv_add(kbuf(as), vfa);                                                         // K_a^T V_a
            state_update<D, B, W>(kv, vfc, kbuf(Slot<1>{}), vbuf(Slot<1>{}), col0, lane);  // K_c^T V_c
        } else {
            f32x4_t sacc[NQT], xacc[NQT];
            inter(qbuf(Slot<1>{}), kbuf(Slot<1>{}), kbuf(as), sacc, xacc, Slot<1>{});
            finish_store(pb0, pnb);
            kv_add(kbuf(as), vfa);                                                         // K_a^T V_a
            state_update<D, B, W>(kv, vfc, kbuf(Slot<1>{}), vbuf(Slot<1>{}), col0, lane);  // K_c^T V_c
            store_scores(Ps, sacc, true);
            store_scores(Px, xacc, false);
        }
        half(c0, 1, pb0, pnb);
        if (c0.b0 + c0.nb == c0.doc_end) {  // the document ends with this block
            vm_wait<0>();  // rare path: keeps the loop's wait bookkeeping exact
            if (p.kv_out)
                store_state<D, B, W>(kv, p.kv_out + (((int64_t)phys_doc(p, c0.doc) * p.H + h) * D) * D + s * W + col0,
                                     g, li);
#pragma unroll
            for (int a = 0; a < NDT; ++a)
#pragma unroll
                for (int c = 0; c < NCW; ++c) kv[a][c] = zero4();
            if (p.kv_in && cn.nb > 0 && cn.first_of_doc) {
                add_state<D, B, W>(kv, p.kv_in + (((int64_t)phys_doc(p, cn.doc) * p.H + h) * D) * D, s * W + col0,
                                   p.kv_in_t, g, li);
                vm_wait<0>();
            }
        }
        c0 = cn;
    };
    // the last block's c half (its a half in slot AS)
    auto last = [&](auto as) {
        lds_barrier();  // scores of the last half visible
        finish(Slot<1>{}, vbuf(as));
        if constexpr (!LIGHT) finish_store(pb0, pnb);
    };
    if (c0.nb > 0) {
        while (true) {
            step_a(Slot<0>{}, Slot<2>{});
            step_c(Slot<0>{});
            if (c0.nb <= 0) {
                last(Slot<0>{});
                break;
            }
            step_a(Slot<2>{}, Slot<0>{});
            step_c(Slot<2>{});
            if (c0.nb <= 0) {
                last(Slot<2>{});
                break;
            }
        }
    }
    if (p.kv_out && !p.packed) empty_doc_states<D, W>(p, u, h, s, t0, t1, tid);
    vm_wait<0>();  // no tile load may still be writing into this workgroup's LDS when it ends
}

template <int D, int W>
__global__ __launch_bounds__(kThreads, 1) void la_prefill_main_v2_b128(PrefillParams p) {
    main_v2_b128<D, W>(p, blockIdx.x);
}

template <int D, int B, int W, int NS, bool DK = false>
__global__ __launch_bounds__(kThreads, 1) void la_prefill_main_v2(PrefillParams p) {
    main_v2<D, B, W, NS, DK>(p, blockIdx.x);
}

// Two passes with the same plan in one launch: the backward's dv and dk
// passes, which read the same Q and dO tiles (one as keys and values, the
// other as values and keys) in the same order.  Workgroup g runs on XCD
// g mod 8 (dispatch is round-robin); of the workgroups of one XCD, in dispatch
// order, the even ones run the units of pass p0 and the odd ones the same
// units of pass p1, so the two workgroups of a unit run side by side on one
// XCD and the second to ask for a shared tile finds it in that XCD's L2.  The
// grid is twice the single pass's (a multiple of 16): pass-local index
// 8 (l / 2) + g mod 8 for local index l = g / 8.
template <int D, int B, int W, int NS>
__global__ __launch_bounds__(kThreads, 1) void la_prefill_pair_v2(PrefillParams p0, PrefillParams p1) {
    const int64_t g = blockIdx.x, l = g >> 3;
    const int64_t wg = ((l >> 1) << 3) | (g & 7);
    main_v2<D, B, W, NS, false>((l & 1) ? p1 : p0, wg);
}

}  // namespace v2
}  // namespace la
