// Tile geometry of the prefill kernels, shared by the host planner and the
// device code (pure constexpr C++, no HIP dependency).
#pragma once
#include <cstddef>
#include <cstdint>

namespace la {

constexpr int kThreads = 256;            // 4 wavefronts of 64 lanes per workgroup
constexpr int kWaves = kThreads / 64;
constexpr size_t kMaxLdsBytes = 160 * 1024;  // LDS per CU on gfx950

// LDS layout of the block-loop kernel for element size ES, head dim D, block B
// and value-slice width W (all tiles hold raw input elements):
//   Qs [B][DK + 16/ES]   query rows, d padded to a multiple of 32
//   Ks [B][DK + 16/ES]   key rows (also reused as the O staging tile [B][W + 16/ES])
//   Kt [D][B + 4]        keys transposed (d-major)
//   Vt [W][B + 4]        value slice transposed
//   Ps [B][B + 4]        masked scores P[query][key]
//   KVt[W][DK + 4]       running state transposed, rounded to the input type
constexpr int dk_of(int D) { return D < 32 ? 32 : D; }
constexpr int row_pitch(int ES, int D) { return dk_of(D) + 16 / ES; }
constexpr int t_pitch(int B) { return B + 4; }
constexpr int o_pitch(int ES, int W) { return W + 16 / ES; }
constexpr int kvt_pitch(int D) { return dk_of(D) + 4; }

constexpr size_t qs_elems(int ES, int D, int B) { return (size_t)B * row_pitch(ES, D); }
constexpr size_t ks_elems(int ES, int D, int B, int W) {
    return qs_elems(ES, D, B) > (size_t)B * o_pitch(ES, W) ? qs_elems(ES, D, B) : (size_t)B * o_pitch(ES, W);
}
constexpr size_t kt_elems(int D, int B) { return (size_t)D * t_pitch(B); }
constexpr size_t vt_elems(int W, int B) { return (size_t)W * t_pitch(B); }
constexpr size_t ps_elems(int B) { return (size_t)B * t_pitch(B); }
constexpr size_t kvt_elems(int D, int W) { return (size_t)W * kvt_pitch(D); }

constexpr size_t main_lds_bytes(int ES, int D, int B, int W) {
    return (size_t)ES * (qs_elems(ES, D, B) + ks_elems(ES, D, B, W) + kt_elems(D, B) + vt_elems(W, B) + ps_elems(B) +
                         kvt_elems(D, W));
}
// segment-state kernel: only Kt and Vt
constexpr size_t state_lds_bytes(int ES, int D, int B, int W) {
    return (size_t)ES * (kt_elems(D, B) + vt_elems(W, B));
}

constexpr bool main_fits(int ES, int D, int B, int W) {
    return main_lds_bytes(ES, D, B, W) <= kMaxLdsBytes && W >= 16 && W <= D && D % W == 0;
}

}  // namespace la
