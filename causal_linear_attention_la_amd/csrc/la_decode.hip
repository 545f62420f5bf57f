// Decode kernel instantiations.
#include "la_launch.h"

namespace la {
namespace {
template <typename T, bool DK>
hipError_t run_decode(const DecodeParams& p, int D, hipStream_t st) {
    const dim3 grid((unsigned)p.pairs), block(kThreads);
    switch (D) {
        case 16: return launch_kernel(la_decode_kernel<T, 16, DK>, grid, block, st, p);
        case 32: return launch_kernel(la_decode_kernel<T, 32, DK>, grid, block, st, p);
        case 64: return launch_kernel(la_decode_kernel<T, 64, DK>, grid, block, st, p);
        case 128: return launch_kernel(la_decode_kernel<T, 128, DK>, grid, block, st, p);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_decode(const DecodeParams& p, int D, int dtype, hipStream_t st) {
    if (p.pairs == 0) return hipSuccess;
    if (p.decay) return dtype == 0 ? run_decode<bf16_t, true>(p, D, st) : run_decode<float, true>(p, D, st);
    return dtype == 0 ? run_decode<bf16_t, false>(p, D, st) : run_decode<float, false>(p, D, st);
}
}  // namespace la
