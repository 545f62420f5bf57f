// Prefill kernels (templates; instantiated per dtype in la_prefill_*.hip).
//
// The method ("MiniMax-01技术报告解读（一）模型架构" and "MiniMax-01技术报告解读",
// §2.2 线性注意力): Q, K, V are cut along the sequence into blocks; inside a
// block the masked left product (Q K^T ⊙ M) V, across blocks the right
// product Q . KV against the running state, then KV += K^T V.
//
// Work decomposition.  The packed token range [0, T) is cut into segments of
// L tokens (a multiple of the block).  One workgroup ("unit") handles one
// (segment u, head h, value-column slice s of width W).  A segment can hold
// pieces of several documents; blocks never straddle a document boundary and
// the state restarts at zero at each document start.  When a document starts
// before the segment, the unit starts from the document's state at the
// segment start, obtained the LASP+ way ("MiniMax-01技术报告解读", §3.2 item 3:
// each part computes its local prefix state, then a global prefix is formed
// from them):
//   la_segment_state_kernel  K^T V of each segment's last document piece
//   la_segment_scan_kernel   (long documents) per-document inclusive scan of
//                            those states, in place
//   la_prefill_main_kernel   the block loop from the prefix; writes o and
//                            the final state of every document ending here.
#pragma once
#include "la_device.h"
#include "la_tiles.h"

namespace la {

struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    const int32_t* cu;
    const float* kv_in;  // [num_seqs][H][D][D] state before each document, or null (zero)
    float* kv_out;   // [num_seqs][H][D][D] or null
    float* ws;       // segment states [nseg][H][D][D] (null when nseg == 1)
    int32_t* flags;  // [nseg]: bit 0 = the segment's last document continues past it,
                     //         bit 1 = that piece also continues from the previous segment
    int32_t T;
    int32_t num_seqs;
    int32_t H;
    int32_t L;       // segment length (tokens)
    int32_t nseg;
    int32_t S;       // value slices per head
    int32_t scan;    // 1: ws holds inclusive per-document states (after the scan kernel)
    int32_t rev;     // 1: every document is processed from its last token to its first
    int32_t kv_in_t; // 1: kv_in holds transposed states ([value][key])
    int32_t slots;   // tile slots of the transpose-read block loop (2 or 3)
    int32_t skip_prefix;  // 1: ws already holds this pass's states; run only the block loop
    int32_t prefix_only;  // host side, 1: enqueue the planning, state and scan kernels but not
                          // the block loop (which then runs in a launch of its own)
    int32_t packed;       // 1: the work list is document pieces (pieces / slot_tab, written on the device)
    int32_t max_pieces;   // packed: entries of pieces
    int32_t state_slots;  // packed: entries of slot_tab
    int32_t* pieces;      // packed: [max_pieces][4] first token, length (-1: unused), document,
                          //         the document's first state slot (-1: none); longest first
    int32_t* slot_tab;    // packed: [state_slots][2] first token, length (0: unused)
    const float* decay;   // decayed variant: per-head lambda in [0, 1] (device, [H]), or null
    uint64_t* marker;     // forward calls with segment states: the block loop stores `key` here
                          // (the states are complete once it runs), for a backward to reuse
    const int32_t* reuse; // backward dq pass: 1 here means the workspace already holds this
                          // pass's segment states (so the state and scan kernels do nothing)
    uint64_t key;
    int64_t units;   // block-loop workgroups
    int64_t per_xcd; // ceil(units / 8)
};

// The workspace's segment states are complete before the block loop runs
// (stream order), so any of its workgroups may stamp the call's key: the one
// with (pass-local) workgroup index g = 0.
__device__ __forceinline__ void stamp_key(const PrefillParams& p, int64_t g) {
    if (p.marker && g == 0 && threadIdx.x == 0) *p.marker = p.key;
}
__device__ __forceinline__ void stamp_key(const PrefillParams& p) { stamp_key(p, blockIdx.x); }
// In a backward pass that reuses the forward's states, the state and scan
// kernels have nothing to do.
__device__ __forceinline__ bool states_reused(const PrefillParams& p) { return p.reuse && *p.reuse != 0; }

// One lane: whether the workspace holds the states of the forward call whose
// key is `key` (decision = 1) or anything else (0); either way the key is
// consumed, so a second backward on the same workspace computes its states.
template <int NT>
__global__ __launch_bounds__(NT) void la_ws_claim_kernel(uint64_t* marker, uint64_t key, int32_t* decision) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const uint64_t m = *marker;
        *decision = m == key ? 1 : 0;
        *marker = 0;
    }
}

// Document boundaries as the kernels see them.  In reverse mode the packed
// sequence is read back to front: logical token t is physical token T-1-t,
// logical document k is physical document n-1-k, and the logical boundaries
// are T - cu[n - k].  Everything (segments, blocks, the causal mask) then
// works on logical positions unchanged; only addresses are mirrored.
struct CuView {
    const int32_t* cu;
    int n;
    int T;
    int rev;
    // The first and last boundaries are 0 and T by the interface contract,
    // so they are never read from memory (a one-document call reads none):
    // at kernel start that saves a memory round trip before the first load.
    __device__ __forceinline__ int operator[](int k) const {
        if (k <= 0) return 0;
        if (k >= n) return T;
        return rev ? T - cu[n - k] : cu[k];
    }
};
__device__ __forceinline__ CuView cu_view(const PrefillParams& p) { return CuView{p.cu, p.num_seqs, p.T, p.rev}; }
// Physical document and token of a logical one.
__device__ __forceinline__ int phys_doc(const PrefillParams& p, int doc) { return p.rev ? p.num_seqs - 1 - doc : doc; }
__device__ __forceinline__ int phys_tok(const PrefillParams& p, int t) { return p.rev ? p.T - 1 - t : t; }
// Physical token of the lowest-addressed row of logical block [b0, b0 + nb).
__device__ __forceinline__ int phys_block(const PrefillParams& p, int b0, int nb) { return p.rev ? p.T - b0 - nb : b0; }

// Largest doc in [0, n-1] with cu[doc] <= t.
__device__ __forceinline__ int doc_at(const CuView& cu, int n, int t) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}
// First doc in [0, n] with cu[doc] >= t.
__device__ __forceinline__ int doc_lower(const CuView& cu, int n, int t) {
    int lo = 0, hi = n;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (cu[mid] < t) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// Workgroup -> unit.  Consecutive unit indices x = (h*nseg + u)*S + s go to
// the same XCD (workgroup ids are dealt round-robin over the 8 XCDs), so the S
// slices of one (segment, head) -- which read the same Q and K rows -- share
// that XCD's L2, and so do the segments of one head, whose block loops read
// the same earlier segment states when they sum their prefix.
// g is the workgroup index within the pass (blockIdx.x, except where two
// passes share a launch).
__device__ __forceinline__ bool unit_of(const PrefillParams& p, int64_t g, int& u, int& h, int& s) {
    const int64_t x = (g & 7) * p.per_xcd + (g >> 3);
    if (x >= p.units) return false;
    s = (int)(x % p.S);
    u = (int)((x / p.S) % p.nseg);
    h = (int)(x / ((int64_t)p.S * p.nseg));
    return true;
}
__device__ __forceinline__ bool unit_of(const PrefillParams& p, int& u, int& h, int& s) {
    return unit_of(p, blockIdx.x, u, h, s);
}

// Packed work list: workgroup g takes entry g / (H S) of the piece table,
// which the planning kernel wrote longest first, so that workgroups are
// dispatched longest first; head (g / S) mod H, slice g mod S.  The entry is
// the same for the whole workgroup (readfirstlane keeps it in scalar
// registers).
struct Piece {
    int t0, len, doc, base;
};
__device__ __forceinline__ bool piece_of(const PrefillParams& p, int64_t g, Piece& pc, int& h, int& s) {
    const int64_t r = g / ((int64_t)p.H * p.S);
    if (r >= p.max_pieces) return false;
    const int4 e = reinterpret_cast<const int4*>(p.pieces)[r];
    pc.t0 = __builtin_amdgcn_readfirstlane(e.x);
    pc.len = __builtin_amdgcn_readfirstlane(e.y);
    pc.doc = __builtin_amdgcn_readfirstlane(e.z);
    pc.base = __builtin_amdgcn_readfirstlane(e.w);
    if (pc.len < 0) return false;
    h = (int)((g / p.S) % p.H);
    s = (int)(g % p.S);
    return true;
}
__device__ __forceinline__ bool piece_of(const PrefillParams& p, Piece& pc, int& h, int& s) {
    return piece_of(p, blockIdx.x, pc, h, s);
}
// Packed work list, segment-state kernels: workgroup g takes state slot
// g / (H S) (a piece that is not its document's last), head and slice as above.
__device__ __forceinline__ bool slot_of(const PrefillParams& p, int& j, int& t0, int& len, int& h, int& s) {
    const int64_t g = blockIdx.x;
    const int64_t r = g / ((int64_t)p.H * p.S);
    if (r >= p.state_slots) return false;
    const int2 e = reinterpret_cast<const int2*>(p.slot_tab)[r];
    t0 = __builtin_amdgcn_readfirstlane(e.x);
    len = __builtin_amdgcn_readfirstlane(e.y);
    if (len <= 0) return false;
    j = (int)r;
    h = (int)((g / p.S) % p.H);
    s = (int)(g % p.S);
    return true;
}

// ---------------------------------------------------------------------------
// The packed work list, built on the device (the document boundaries live in
// device memory).  Document n_d tokens long is cut into max(1, ceil(n_d / L))
// pieces: the first ones exactly L tokens from the document start, the last
// one the rest (length 0 for an empty document, whose unit only writes its
// final state).  Every piece but the last of its document owns a state slot
// (K^T V over the piece); a document's slots are consecutive, in document
// order.  Pieces go to the table longest first -- a counting sort over
// kPlanThreads length buckets, ties in any order -- so that the workgroups
// the hardware dispatches first are the longest (longest-processing-time
// list scheduling over the CUs).  Which workgroup runs a piece does not change
// any result.  One workgroup; at most kPlanThreads * 4 documents.
constexpr int kPlanThreads = 1024;
constexpr int kPlanDocsPerThread = 4;  // so at most 4096 documents

// Inclusive scan of one int per lane over the workgroup: a shuffle scan in
// each wave, then the wave totals scanned by the first wave (two barriers).
__device__ __forceinline__ int block_scan_incl(int x, int* wave_tot, int tid) {
    constexpr int NW = kPlanThreads / 64;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int t = lane < NW ? wave_tot[lane] : 0;
#pragma unroll
        for (int off = 1; off < NW; off <<= 1) {
            const int y = __shfl_up(t, off, 64);
            if (lane >= off) t += y;
        }
        if (lane < NW) wave_tot[lane] = t;
    }
    __syncthreads();
    const int before = wave > 0 ? wave_tot[wave - 1] : 0;
    const int total = wave_tot[NW - 1];
    __syncthreads();  // wave_tot may be reused by the next scan
    wave_tot[NW] = total;
    return x + before;
}

template <int NT>
__global__ __launch_bounds__(NT) void la_plan_pieces_kernel(PrefillParams p) {
    static_assert(NT == kPlanThreads, "one lane per length bucket");
    __shared__ int wave_tot[kPlanThreads / 64 + 1];
    __shared__ int cnt[kPlanThreads];  // pieces per length bucket, then each bucket's next table position
    const int tid = threadIdx.x;
    const CuView cu = cu_view(p);
    const int n = p.num_seqs, L = p.L;
    // this lane's documents: a contiguous run, boundaries read once
    const int per = (n + kPlanThreads - 1) / kPlanThreads;
    const int d0 = min(n, tid * per), nd = min(n, d0 + per) - d0;
    int start[kPlanDocsPerThread], len[kPlanDocsPerThread], np[kPlanDocsPerThread];
    int nslots = 0, npieces = 0;
#pragma unroll
    for (int i = 0; i < kPlanDocsPerThread; ++i) {
        start[i] = i < nd ? cu[d0 + i] : 0;
        len[i] = i < nd ? cu[d0 + i + 1] - start[i] : 0;
        np[i] = i < nd ? (len[i] == 0 ? 1 : (len[i] + L - 1) / L) : 0;
        nslots += i < nd ? np[i] - 1 : 0;
        npieces += np[i];
    }
    // bucket of a piece length in [0, L]: longer pieces, higher buckets
    auto bucket = [&](int plen) { return (int)((int64_t)plen * (kPlanThreads - 1) / L); };
    cnt[tid] = 0;
    int slot = block_scan_incl(nslots, wave_tot, tid) - nslots;  // first state slot of this lane's documents
    const int total_slots = wave_tot[kPlanThreads / 64];
    const int total_pieces = (block_scan_incl(npieces, wave_tot, tid), wave_tot[kPlanThreads / 64]);
#pragma unroll
    for (int i = 0; i < kPlanDocsPerThread; ++i) {
        if (i < nd) {
            if (np[i] > 1) atomicAdd(&cnt[bucket(L)], np[i] - 1);
            atomicAdd(&cnt[bucket(len[i] - (np[i] - 1) * L)], 1);
        }
    }
    __syncthreads();
    // descending order of buckets: lane t holds bucket kPlanThreads - 1 - t
    const int mine = cnt[kPlanThreads - 1 - tid];
    const int first = block_scan_incl(mine, wave_tot, tid) - mine;
    cnt[kPlanThreads - 1 - tid] = first;  // first table position of that bucket
    __syncthreads();
    int4* tab = reinterpret_cast<int4*>(p.pieces);
    int2* stab = reinterpret_cast<int2*>(p.slot_tab);
#pragma unroll
    for (int i = 0; i < kPlanDocsPerThread; ++i) {
        if (i < nd) {
            const int base = np[i] > 1 ? slot : -1;
            for (int k = 0; k < np[i]; ++k) {
                const int plen = k < np[i] - 1 ? L : len[i] - (np[i] - 1) * L;
                const int pos = atomicAdd(&cnt[bucket(plen)], 1);
                tab[pos] = make_int4(start[i] + k * L, plen, d0 + i, base);
                if (k < np[i] - 1) stab[slot + k] = make_int2(start[i] + k * L, L);
            }
            slot += np[i] - 1;
        }
    }
    for (int r = total_pieces + tid; r < p.max_pieces; r += kPlanThreads) tab[r] = make_int4(0, -1, 0, -1);
    for (int r = total_slots + tid; r < p.state_slots; r += kPlanThreads) stab[r] = make_int2(0, 0);
}

// Final state of one empty document (the packed work list gives each its own
// unit): the incoming state, or zero.
template <int D, int W>
__device__ __forceinline__ void one_empty_doc_state(const PrefillParams& p, int doc, int h, int s, int tid) {
    const int64_t base = (((int64_t)phys_doc(p, doc) * p.H + h) * D) * D;
    float* dst = p.kv_out + base;
    const float* src = p.kv_in ? p.kv_in + base : nullptr;
    for (int i = tid; i < D * W; i += kThreads) {
        const int r = i / W, c = s * W + i % W;  // key row, value column
        dst[(int64_t)r * D + c] = src ? (p.kv_in_t ? src[(int64_t)c * D + r] : src[(int64_t)r * D + c]) : 0.f;
    }
}

// Walks the blocks of one segment [t0, t1): blocks start at the segment start
// or at a document start, hold at most B tokens and never cross a document end.
struct Cursor {
    int b0;       // first token of the block
    int nb;       // tokens in it (0: no more blocks)
    int doc;
    int doc_end;       // cu[doc + 1]
    int first_of_doc;  // 1 if the block starts its document (an int: the struct stays all-register)
};

__device__ __forceinline__ void cursor_first(Cursor& c, const CuView& cu, int n, int t0, int t1, int B) {
    c.b0 = t0;
    c.nb = 0;
    c.doc = 0;
    c.doc_end = 0;
    c.first_of_doc = 0;
    if (t0 >= t1) return;
    c.doc = doc_at(cu, n, t0);
    c.doc_end = cu[c.doc + 1];
    c.b0 = t0;
    c.nb = min(B, min(t1, c.doc_end) - t0);
    c.first_of_doc = (cu[c.doc] == t0) ? 1 : 0;
}

__device__ __forceinline__ void cursor_next(Cursor& c, const CuView& cu, int n, int t1, int B) {
    int nb0 = c.b0 + c.nb;
    int piece_end = min(t1, c.doc_end);
    if (nb0 < piece_end) {
        c.b0 = nb0;
        c.nb = min(B, piece_end - nb0);
        c.first_of_doc = 0;
        return;
    }
    int d = c.doc + 1;
    while (d < n && cu[d + 1] == cu[d]) ++d;  // skip empty documents
    if (d >= n || cu[d] >= t1) { c.nb = 0; return; }
    c.doc = d;
    c.b0 = cu[d];
    c.doc_end = cu[d + 1];
    c.nb = min(B, min(t1, c.doc_end) - c.b0);
    c.first_of_doc = 1;
}

// Register staging of a ROWS x COLS tile of one head (row stride ld elements):
// each item is 4 consecutive rows x one 16-byte column chunk, so the tile can
// be written to LDS both row-major and transposed (4-token runs).
template <typename T, int ROWS, int COLS>
struct TileRegs {
    static constexpr int CE = 16 / (int)sizeof(T);
    static constexpr int CPR = COLS / CE;
    static constexpr int ITEMS = (ROWS / 4) * CPR;
    static constexpr int PER = (ITEMS + kThreads - 1) / kThreads;
    uint4 r[PER][4];

    __device__ __forceinline__ void load(const T* base, int64_t ld, int nb, int tid) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int item = tid + p * kThreads;
            const int rq = item / CPR, c = item % CPR;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * rq + i;
                if (item < ITEMS && row < nb)
                    r[p][i] = *reinterpret_cast<const uint4*>(base + (int64_t)row * ld + c * CE);
                else
                    r[p][i] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    }
    // row-major: lds[row][col], pitch in elements
    __device__ __forceinline__ void store_rows(T* lds, int pitch, int tid) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int item = tid + p * kThreads;
            if (item < ITEMS) {
                const int rq = item / CPR, c = item % CPR;
#pragma unroll
                for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(lds + (4 * rq + i) * pitch + c * CE) = r[p][i];
            }
        }
    }
    // transposed, each row (token) r scaled by lambda^(nb - 1 - r) and rows
    // from nb on by 0 (the decayed state update's weights; l2 = log2 lambda)
    __device__ __forceinline__ void store_cols_weighted(T* lds, int pitch, int tid, float l2, int nb) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int item = tid + p * kThreads;
            if (item < ITEMS) {
                const int rq = item / CPR, c = item % CPR;
                float w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = 4 * rq + i < nb ? decay_pow(l2, nb - 1 - (4 * rq + i)) : 0.f;
#pragma unroll
                for (int e = 0; e < CE; ++e) {
                    float x[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if constexpr (sizeof(T) == 2) x[i] = __uint_as_float(lane16(r[p][i], e) << 16) * w[i];
                        else x[i] = __uint_as_float(lane32(r[p][i], e)) * w[i];
                    }
                    store4(lds + (c * CE + e) * pitch + 4 * rq, x[0], x[1], x[2], x[3]);
                }
            }
        }
    }
    // transposed: lds[col][row], 4 rows per write
    __device__ __forceinline__ void store_cols(T* lds, int pitch, int tid) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int item = tid + p * kThreads;
            if (item < ITEMS) {
                const int rq = item / CPR, c = item % CPR;
#pragma unroll
                for (int e = 0; e < CE; ++e) store_col4(lds + (c * CE + e) * pitch + 4 * rq, r[p], e);
            }
        }
    }
};

// Round LDS sub-array sizes to 8 elements so every tile starts 16-byte aligned.
constexpr size_t al8(size_t n) { return (n + 7) & ~(size_t)7; }

// KV += K^T V for one block: the state tiles owned by this wave.  kv[j] is the
// 16x16 tile t = wave + 4j of the D x W state, rows = key dim, cols = value dim;
// lane (col li, group g) holds rows 4g..4g+3.
template <typename TIn, int D, int B, int W, int KVPW>
__device__ __forceinline__ void state_update(f32x4_t (&kv)[KVPW], const TIn* Kt, const TIn* Vt, int wave, int li,
                                             int g) {
    constexpr int NCT = W / 16, NKV = (D / 16) * NCT, TP = t_pitch(B);
#pragma unroll
    for (int j = 0; j < KVPW; ++j) {
        const int t = wave + kWaves * j;
        if (t < NKV) {
            const int a = t / NCT, c = t % NCT;
#pragma unroll
            for (int kc = 0; kc < B / 32; ++kc) {
                Frag<TIn> fa, fb;
                load_frag(fa, Kt + (16 * a + li) * TP + 32 * kc, g);  // K^T[d][keys]
                load_frag(fb, Vt + (16 * c + li) * TP + 32 * kc, g);  // V[keys][col]
                mma(kv[j], fa, fb);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Segment states: for every segment whose last document continues into the
// next segment, K^T V over that document's piece of the segment.
template <typename TIn, int D, int B, int W, bool DECAY = false>
__global__ __launch_bounds__(kThreads, 2) void la_segment_state_kernel(PrefillParams p) {
    constexpr int TP = t_pitch(B);
    constexpr int NKV = (D / 16) * (W / 16);
    constexpr int KVPW = (NKV + kWaves - 1) / kWaves;
    __shared__ __align__(16) TIn smem[al8(kt_elems(D, B)) + al8(vt_elems(W, B))];
    TIn* Kt = smem;
    TIn* Vt = smem + al8(kt_elems(D, B));

    if (states_reused(p)) return;
    int u, h, s, b0, t_end;
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (p.packed) {  // state slot u: a whole piece [b0, t_end) of one document
        int len;
        if (!slot_of(p, u, b0, len, h, s)) return;
        t_end = b0 + len;
    } else {
        if (!unit_of(p, u, h, s)) return;
        if (u >= p.nseg - 1) return;  // nothing after the last segment
        const int t_beg = u * p.L;
        t_end = (u + 1) * p.L;  // t_end < T here
        const CuView cu = cu_view(p);
        const int de = doc_at(cu, p.num_seqs, t_end - 1);
        const int dstart = cu[de];
        const bool needs = cu[de + 1] > t_end;
        const bool chain = dstart < t_beg;
        if (h == 0 && s == 0 && tid == 0) p.flags[u] = (needs ? 1 : 0) | (chain ? 2 : 0);
        if (!needs) return;
        b0 = max(t_beg, dstart);
    }

    const TIn* kg = static_cast<const TIn*>(p.k);
    const TIn* vg = static_cast<const TIn*>(p.v);
    const int64_t ld = p.rev ? -(int64_t)p.H * D : (int64_t)p.H * D;  // row step of logical tokens
    f32x4_t kv[KVPW];
#pragma unroll
    for (int j = 0; j < KVPW; ++j) kv[j] = zero4();

    TileRegs<TIn, B, D> lk;
    TileRegs<TIn, B, W> lv;
    // decayed variant: the state is faded to the end of the piece, block by block
    const float l2 = DECAY ? log2f(p.decay[h]) : 0.f;
    int nb = min(B, t_end - b0);
    lk.load(kg + ((int64_t)phys_tok(p, b0) * p.H + h) * D, ld, nb, tid);
    lv.load(vg + ((int64_t)phys_tok(p, b0) * p.H + h) * D + s * W, ld, nb, tid);
    while (nb > 0) {
        __syncthreads();
        if constexpr (DECAY) {
            lk.store_cols_weighted(Kt, TP, tid, l2, nb);
            const float f = decay_pow(l2, nb);
#pragma unroll
            for (int j = 0; j < KVPW; ++j) kv[j] *= f;
        } else {
            lk.store_cols(Kt, TP, tid);
        }
        lv.store_cols(Vt, TP, tid);
        const int nb0 = b0 + nb;
        const int nnb = min(B, t_end - nb0);
        if (nnb > 0) {
            lk.load(kg + ((int64_t)phys_tok(p, nb0) * p.H + h) * D, ld, nnb, tid);
            lv.load(vg + ((int64_t)phys_tok(p, nb0) * p.H + h) * D + s * W, ld, nnb, tid);
        }
        __syncthreads();
        state_update<TIn, D, B, W, KVPW>(kv, Kt, Vt, wave, li, g);
        b0 = nb0;
        nb = nnb;
    }
    float* dst = p.ws + (((int64_t)u * p.H + h) * D) * D + s * W;
#pragma unroll
    for (int j = 0; j < KVPW; ++j) {
        const int t = wave + kWaves * j;
        if (t < NKV) {
            const int a = t / (W / 16), c = t % (W / 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(int64_t)(16 * a + 4 * g + r) * D + 16 * c + li] = kv[j][r];
        }
    }
}

// ---------------------------------------------------------------------------
// Per-document inclusive scan of the segment states, in place: afterwards
// ws[u] is the state of segment u's last document at the end of segment u.
// One thread per 4 consecutive state entries (h, i, j..j+3); the segments are
// taken CH at a time: CH independent 16-byte loads in flight, then the
// running sums and CH stores.  NT threads per workgroup: small workgroups
// spread the scan over every CU (each CU's stream of requests is the limit).
template <int CH, int NT>
__global__ __launch_bounds__(NT) void la_segment_scan_kernel(float* __restrict__ ws, const int32_t* __restrict__ flags,
                                                             int nseg, int64_t entries, const int32_t* reuse,
                                                             const float* decay, int64_t per_head, int L) {
    if (reuse && *reuse) return;  // the workspace already holds the (transposed) prefixes
    const int64_t idx = ((int64_t)blockIdx.x * NT + threadIdx.x) * 4;
    if (idx >= entries) return;
    // decayed variant: a carried prefix fades by lambda^L across one more segment
    const float fL = decay ? decay_pow(log2f(decay[idx / per_head]), L) : 1.f;
    f32x4_t carry = zero4();
    for (int u0 = 0; u0 < nseg - 1; u0 += CH) {
        f32x4_t a[CH];
        int f[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int u = u0 + c;
            f[c] = u < nseg - 1 ? flags[u] : 0;
            a[c] = (f[c] & 1) ? *reinterpret_cast<const f32x4_t*>(ws + (int64_t)u * entries + idx) : zero4();
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (f[c] & 1) {
                carry = (f[c] & 2) ? fL * carry + a[c] : a[c];
                *reinterpret_cast<f32x4_t*>(ws + (int64_t)(u0 + c) * entries + idx) = carry;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Final state of the empty documents whose start lies in segment u (the last
// segment also takes those at the very end): the incoming state, or zero.
template <int D, int W>
__device__ __forceinline__ void empty_doc_states(const PrefillParams& p, int u, int h, int s, int t0, int t1,
                                                 int tid) {
    const CuView cu = cu_view(p);
    const int lo = doc_lower(cu, p.num_seqs, t0);
    const int hi = (u == p.nseg - 1) ? p.num_seqs : doc_lower(cu, p.num_seqs, t1);
    for (int d = lo; d < hi; ++d) {
        if (cu[d + 1] != cu[d]) continue;
        const int64_t base = (((int64_t)phys_doc(p, d) * p.H + h) * D) * D;
        float* dst = p.kv_out + base;
        const float* src = p.kv_in ? p.kv_in + base : nullptr;
        for (int i = tid; i < D * W; i += kThreads) {
            const int r = i / W, c = s * W + i % W;  // key row, value column
            dst[(int64_t)r * D + c] = src ? (p.kv_in_t ? src[(int64_t)c * D + r] : src[(int64_t)r * D + c]) : 0.f;
        }
    }
}

// ---------------------------------------------------------------------------
// The block loop.
template <typename TIn, int D, int B, int W, bool DECAY = false>
__global__ __launch_bounds__(kThreads, 1) void la_prefill_main_kernel(PrefillParams p) {
    constexpr int ES = (int)sizeof(TIn);
    constexpr int CE = 16 / ES;
    constexpr int DK = dk_of(D);
    constexpr int QP = row_pitch(ES, D), TP = t_pitch(B), OP = o_pitch(ES, W), KP = kvt_pitch(D);
    constexpr int NQT = B / 16, NCT = W / 16, NKV = (D / 16) * NCT;
    constexpr int KVPW = (NKV + kWaves - 1) / kWaves;
    constexpr int NTRI = NQT * (NQT + 1) / 2, NZT = NQT / 2;
    constexpr size_t OQ = 0;
    constexpr size_t OK = OQ + al8(qs_elems(ES, D, B));
    constexpr size_t OKT = OK + al8(ks_elems(ES, D, B, W));
    constexpr size_t OVT = OKT + al8(kt_elems(D, B));
    constexpr size_t OPS = OVT + al8(vt_elems(W, B));
    constexpr size_t OKV = OPS + al8(ps_elems(B));
    constexpr size_t NTOT = OKV + al8(kvt_elems(D, W));
    static_assert(NTOT * ES <= kMaxLdsBytes, "LDS budget exceeded");
    __shared__ __align__(16) TIn smem[NTOT];
    TIn* Qs = smem + OQ;
    TIn* Ks = smem + OK;
    TIn* Os = smem + OK;  // O staging reuses the key rows (dead after the score phase)
    TIn* Kt = smem + OKT;
    TIn* Vt = smem + OVT;
    TIn* Ps = smem + OPS;
    TIn* KVt = smem + OKV;

    stamp_key(p);
    int u = 0, h, s, t0, t1;
    int lb0 = 0, lb1 = 0;  // packed: state slots of the document's earlier pieces
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (p.packed) {
        Piece pc;
        if (!piece_of(p, pc, h, s)) return;
        if (pc.len == 0) {  // an empty document: only its final state
            if (p.kv_out) one_empty_doc_state<D, W>(p, pc.doc, h, s, tid);
            return;
        }
        t0 = pc.t0;
        t1 = pc.t0 + pc.len;
        lb0 = pc.base;
        lb1 = pc.base + (t0 - cu_view(p)[pc.doc]) / p.L;
    } else {
        if (!unit_of(p, u, h, s)) return;
        t0 = u * p.L;
        t1 = min(p.T, t0 + p.L);
    }
    const TIn* qg = static_cast<const TIn*>(p.q);
    const TIn* kg = static_cast<const TIn*>(p.k);
    const TIn* vg = static_cast<const TIn*>(p.v);
    TIn* og = static_cast<TIn*>(p.o);
    const int64_t ld = p.rev ? -(int64_t)p.H * D : (int64_t)p.H * D;  // row step of logical tokens
    const CuView cuv = cu_view(p);

    // Zero LDS once: pad columns (d >= D) of Qs and KVt must stay finite zeros.
    {
        uint4* z = reinterpret_cast<uint4*>(smem);
        constexpr int NV = (int)(NTOT * ES / 16);
        for (int i = tid; i < NV; i += kThreads) z[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    Cursor cur;
    cursor_first(cur, cuv, p.num_seqs, t0, t1, B);
    // decayed variant: this head's log2 lambda
    const float l2 = DECAY ? log2f(p.decay[h]) : 0.f;

    // Initial state: zero, or the document's state at the segment start
    // (decayed: each earlier piece's state faded by the tokens between its end
    // and this unit's start).
    f32x4_t kv[KVPW];
#pragma unroll
    for (int j = 0; j < KVPW; ++j) kv[j] = zero4();
    if (cur.nb > 0 && !cur.first_of_doc) {
        const int u_first = p.packed ? lb0 : p.scan ? u - 1 : cuv[cur.doc] / p.L;
        const int u_end = p.packed ? lb1 : u;
        for (int uu = u_first; uu < u_end; ++uu) {
            const float* src = p.ws + (((int64_t)uu * p.H + h) * D) * D + s * W;
            const float f = DECAY ? decay_pow(l2, (u_end - uu - 1) * p.L) : 1.f;
#pragma unroll
            for (int j = 0; j < KVPW; ++j) {
                const int t = wave + kWaves * j;
                if (t < NKV) {
                    const int a = t / NCT, c = t % NCT;
#pragma unroll
                    for (int r = 0; r < 4; ++r) kv[j][r] += f * src[(int64_t)(16 * a + 4 * g + r) * D + 16 * c + li];
                }
            }
        }
    }
    // A caller-supplied state before the document's first token joins the
    // prefix (decayed: faded by factor f).
    auto add_kv_in = [&](int doc, float f) {
        const float* src = p.kv_in + (((int64_t)phys_doc(p, doc) * p.H + h) * D) * D;
#pragma unroll
        for (int j = 0; j < KVPW; ++j) {
            const int t = wave + kWaves * j;
            if (t < NKV) {
                const int a = t / NCT, c = t % NCT;
                const int col = s * W + 16 * c + li;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * a + 4 * g + r;
                    kv[j][r] += f * (p.kv_in_t ? src[(int64_t)col * D + row] : src[(int64_t)row * D + col]);
                }
            }
        }
    };
    if (p.kv_in && cur.nb > 0) add_kv_in(cur.doc, DECAY ? decay_pow(l2, t0 - cuv[cur.doc]) : 1.f);
    __syncthreads();  // LDS zeroed before the state copy below
#pragma unroll
    for (int j = 0; j < KVPW; ++j) {
        const int t = wave + kWaves * j;
        if (t < NKV) {
            const int a = t / NCT, c = t % NCT;
            store4(KVt + (16 * c + li) * KP + 16 * a + 4 * g, kv[j][0], kv[j][1], kv[j][2], kv[j][3]);
        }
    }

    TileRegs<TIn, B, D> lq, lk;
    TileRegs<TIn, B, W> lv;
    if (cur.nb > 0) {
        const int64_t row0 = (int64_t)phys_tok(p, cur.b0) * p.H + h;
        lq.load(qg + row0 * D, ld, cur.nb, tid);
        lk.load(kg + row0 * D, ld, cur.nb, tid);
        lv.load(vg + row0 * D + s * W, ld, cur.nb, tid);
    }

    while (cur.nb > 0) {
        __syncthreads();  // (A) previous block fully consumed
        lq.store_rows(Qs, QP, tid);
        lk.store_rows(Ks, QP, tid);
        if constexpr (DK != D) {  // Ks pad columns were overwritten by the O staging
            for (int i = tid; i < B * (DK - D) / CE; i += kThreads) {
                const int row = i / ((DK - D) / CE), c = i % ((DK - D) / CE);
                *reinterpret_cast<uint4*>(Ks + row * QP + D + c * CE) = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        if constexpr (DECAY) lk.store_cols_weighted(Kt, TP, tid, l2, cur.nb);  // (Kt feeds only the state update)
        else lk.store_cols(Kt, TP, tid);
        lv.store_cols(Vt, TP, tid);
        Cursor nxt = cur;
        cursor_next(nxt, cuv, p.num_seqs, t1, B);
        if (nxt.nb > 0) {
            const int64_t row0 = (int64_t)phys_tok(p, nxt.b0) * p.H + h;
            lq.load(qg + row0 * D, ld, nxt.nb, tid);
            lk.load(kg + row0 * D, ld, nxt.nb, tid);
            lv.load(vg + row0 * D + s * W, ld, nxt.nb, tid);
        }
        __syncthreads();  // (B) tiles in LDS

        // Scores, transposed: S^T = K Q^T on the lower-triangular tiles, causal
        // mask on the diagonal tiles (key <= query kept), stored as P[query][key].
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
            TIn* prow = Ps + (16 * b + li) * TP + 16 * a + 4 * g;
            if (t >= NTRI) {  // above-diagonal tile read by the P.V chunk loop: zeros
                store4_zero(prow);
                continue;
            }
            f32x4_t acc = zero4();
#pragma unroll
            for (int m = 0; m < DK / 32; ++m) {
                Frag<TIn> fa, fb;
                load_frag(fa, Ks + (16 * a + li) * QP + 32 * m, g);
                load_frag(fb, Qs + (16 * b + li) * QP + 32 * m, g);
                mma(acc, fa, fb);
            }
            if constexpr (DECAY) {  // lambda^(query - key), 0 above the diagonal
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = (16 * b + li) - (16 * a + 4 * g + r);
                    acc[r] = m >= 0 ? acc[r] * decay_pow(l2, m) : 0.f;
                }
            } else if (a == b) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g + r > li) acc[r] = 0.f;
            }
            store4(prow, acc[0], acc[1], acc[2], acc[3]);
        }
        __syncthreads();  // (C) P complete

        // Output, transposed: O^T = V^T P^T (intra) + KV^T Q^T (inter, state
        // before this block).
        for (int t = wave; t < NQT * NCT; t += kWaves) {
            const int b = t % NQT, c = t / NQT;
            f32x4_t acc = zero4();
            for (int kc = 0; kc <= b / 2; ++kc) {
                Frag<TIn> fa, fb;
                load_frag(fa, Vt + (16 * c + li) * TP + 32 * kc, g);
                load_frag(fb, Ps + (16 * b + li) * TP + 32 * kc, g);
                mma(acc, fa, fb);
            }
            // inter product; decayed: in its own accumulator, then faded by
            // lambda^(query + 1) for query row 16 b + li
            f32x4_t acce = zero4();
            f32x4_t& ae = DECAY ? acce : acc;
#pragma unroll
            for (int m = 0; m < DK / 32; ++m) {
                Frag<TIn> fa, fb;
                load_frag(fa, KVt + (16 * c + li) * KP + 32 * m, g);
                load_frag(fb, Qs + (16 * b + li) * QP + 32 * m, g);
                mma(ae, fa, fb);
            }
            if constexpr (DECAY) acc += decay_pow(l2, 16 * b + li + 1) * acce;
            store4(Os + (16 * b + li) * OP + 16 * c + 4 * g, acc[0], acc[1], acc[2], acc[3]);
        }
        // State update after the inter product used the old state (decayed:
        // KV <- lambda^nb KV + weighted K^T V, the weights already on Kt).
        if constexpr (DECAY) {
            const float f = decay_pow(l2, cur.nb);
#pragma unroll
            for (int j = 0; j < KVPW; ++j) kv[j] *= f;
        }
        state_update<TIn, D, B, W, KVPW>(kv, Kt, Vt, wave, li, g);
        __syncthreads();  // (D) O staged, old KVt no longer read

        // Coalesced store of the block's output rows.
        {
            constexpr int OCPR = W / CE;
            TIn* obase = og + ((int64_t)phys_tok(p, cur.b0) * p.H + h) * D + s * W;
            for (int i = tid; i < cur.nb * OCPR; i += kThreads) {
                const int row = i / OCPR, c = i % OCPR;
                *reinterpret_cast<uint4*>(obase + (int64_t)row * ld + c * CE) =
                    *reinterpret_cast<const uint4*>(Os + row * OP + c * CE);
            }
        }
        if (cur.b0 + cur.nb == cur.doc_end && p.kv_out) {
            float* dst = p.kv_out + (((int64_t)phys_doc(p, cur.doc) * p.H + h) * D) * D + s * W;
#pragma unroll
            for (int j = 0; j < KVPW; ++j) {
                const int t = wave + kWaves * j;
                if (t < NKV) {
                    const int a = t / NCT, c = t % NCT;
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[(int64_t)(16 * a + 4 * g + r) * D + 16 * c + li] = kv[j][r];
                }
            }
        }
        if (nxt.nb > 0 && nxt.first_of_doc) {
#pragma unroll
            for (int j = 0; j < KVPW; ++j) kv[j] = zero4();
            if (p.kv_in) add_kv_in(nxt.doc, 1.f);  // a document starting here starts from its state
        }
#pragma unroll
        for (int j = 0; j < KVPW; ++j) {
            const int t = wave + kWaves * j;
            if (t < NKV) {
                const int a = t / NCT, c = t % NCT;
                store4(KVt + (16 * c + li) * KP + 16 * a + 4 * g, kv[j][0], kv[j][1], kv[j][2], kv[j][3]);
            }
        }
        cur = nxt;
    }

    // Empty documents placed in this segment keep their incoming state (zero
    // when none is given); the packed work list gives them units of their own.
    if (p.kv_out && !p.packed) empty_doc_states<D, W>(p, u, h, s, t0, t1, tid);
}

}  // namespace la
