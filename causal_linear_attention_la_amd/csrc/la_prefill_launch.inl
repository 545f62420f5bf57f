// Shared body of la_prefill_bf16.hip / la_prefill_fp32.hip: dispatch from the
// runtime (D, B, W) to the kernel instantiation, skipping combinations whose
// LDS tiles do not fit.
namespace la {
namespace {

// The transpose-read block loops (la_prefill_v2.h) cover bf16, d >= 64, and
// 64-token or 128-token blocks with slices of at least 64 value columns.
template <typename T, int D, int B, int W>
constexpr bool has_v2() {
    return sizeof(T) == 2 && D >= 64 && ((B == 64 && W >= 64) || (B == 128 && (W == 64 || W == 128)));
}

// Launches the block-loop kernel; with events, through hipExtLaunchKernel, so
// that they timestamp the kernel's own start and end.
inline hipError_t launch_main(void (*kernel)(PrefillParams), dim3 grid, dim3 block, const PrefillParams& p,
                              hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    if (!e0 && !e1) return launch_kernel(kernel, grid, block, st, p);
    PrefillParams arg = p;
    void* args[] = {&arg};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, st, e0, e1, 0);
}

// The kernels of one plan, without (DK = false) or with the decay.
template <typename T, int D, int B, int W, bool DK>
hipError_t run_prefill_k(const PrefillParams& p, int variant, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    // (the generic loop's tiles do not fit every shape the transpose-read loops take)
    constexpr bool GEN = main_fits((int)sizeof(T), D, B, W);
    constexpr bool V2 = has_v2<T, D, B, W>();
    if constexpr (!GEN && !V2) {
        return hipErrorInvalidValue;
    } else {
        const dim3 block(kThreads);
        // segments: 8 * ceil(units / 8) workgroups (units numbered per XCD);
        // pieces: one per table entry (head, slice), in table order
        const dim3 grid((unsigned)(p.packed ? p.units : 8 * p.per_xcd));
        bool use_v2 = false;
        if constexpr (V2) use_v2 = (variant != 1);
        if (variant == 2 && !use_v2) return hipErrorInvalidValue;
        if (!GEN && !use_v2) return hipErrorInvalidValue;
        void (*seg_kernel)(PrefillParams) = nullptr;
        if constexpr (GEN) seg_kernel = la_segment_state_kernel<T, D, B, W, DK>;
        if constexpr (V2) {
            // (a segment state is a sum over its piece: the 64-token state kernel serves both block sizes)
            if (use_v2) seg_kernel = v2::la_segment_state_v2<D, 64, W, DK>;
        }
        if (p.packed) {
            hipError_t e = launch_kernel(la_plan_pieces_kernel<kPlanThreads>, dim3(1), dim3(kPlanThreads), st, p);
            if (e != hipSuccess) return e;
            if (p.state_slots > 0 && !p.skip_prefix) {
                e = launch_kernel(seg_kernel, dim3((unsigned)((int64_t)p.state_slots * p.H * p.S)), block, st, p);
                if (e != hipSuccess) return e;
            }
        } else if (p.nseg > 1 && !p.skip_prefix) {
            hipError_t e = launch_kernel(seg_kernel, grid, block, st, p);
            if (e != hipSuccess) return e;
            if (p.scan) {
                const int64_t entries = (int64_t)p.H * D * D;  // a multiple of 4
                const int64_t threads = entries / 4;
                constexpr int NT = 128;
                e = launch_kernel(la_segment_scan_kernel<32, NT>, dim3((unsigned)((threads + NT - 1) / NT)), dim3(NT),
                                  st, p.ws, (const int32_t*)p.flags, (int)p.nseg, entries, p.reuse, p.decay,
                                  (int64_t)D * D, (int)p.L);
                if (e != hipSuccess) return e;
            }
        }
        if (p.prefix_only) return hipSuccess;
        void (*main_kernel)(PrefillParams) = nullptr;
        if constexpr (GEN) main_kernel = la_prefill_main_kernel<T, D, B, W, DK>;
        if constexpr (V2) {
            if (use_v2) {
                if constexpr (B == 128) {
                    // (no decayed form: the planner gives decayed 128-token blocks the generic loop)
                    if constexpr (DK) return hipErrorInvalidValue;
                    else main_kernel = v2::la_prefill_main_v2_b128<D, W>;
                } else if constexpr (D == 128 && DK && W == 128) {
                    // (the decayed full-width loop has no registers for a third slot: the planner gives it two)
                    if (p.slots == 3) return hipErrorInvalidValue;
                    main_kernel = v2::la_prefill_main_v2<D, B, W, 2, DK>;
                } else if constexpr (D == 128) {
                    main_kernel = p.slots == 3 ? v2::la_prefill_main_v2<D, B, W, 3, DK>
                                               : v2::la_prefill_main_v2<D, B, W, 2, DK>;
                } else {
                    if (p.slots == 3) return hipErrorInvalidValue;
                    main_kernel = v2::la_prefill_main_v2<D, B, W, 2, DK>;
                }
            }
        }
        return launch_main(main_kernel, grid, block, p, st, e0, e1);
    }
}

template <typename T, int D, int B, int W>
hipError_t run_prefill(const PrefillParams& p, int variant, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    return p.decay ? run_prefill_k<T, D, B, W, true>(p, variant, st, e0, e1)
                   : run_prefill_k<T, D, B, W, false>(p, variant, st, e0, e1);
}

template <typename T, int D, int B>
hipError_t by_width(const PrefillParams& p, int W, int variant, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    if (W == D) return run_prefill<T, D, B, D>(p, variant, st, e0, e1);
    if constexpr (D / 2 >= 16) {
        if (W == D / 2) return run_prefill<T, D, B, D / 2>(p, variant, st, e0, e1);
    }
    if constexpr (D / 4 >= 16) {
        if (W == D / 4) return run_prefill<T, D, B, D / 4>(p, variant, st, e0, e1);
    }
    return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t by_block(const PrefillParams& p, int B, int W, int variant, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    switch (B) {
        case 32: return by_width<T, D, 32>(p, W, variant, st, e0, e1);
        case 64: return by_width<T, D, 64>(p, W, variant, st, e0, e1);
        case 128: return by_width<T, D, 128>(p, W, variant, st, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t dispatch_prefill(const PrefillParams& p, int D, int B, int W, int variant, hipStream_t st, hipEvent_t e0,
                            hipEvent_t e1) {
    switch (D) {
        case 16: return by_block<T, 16>(p, B, W, variant, st, e0, e1);
        case 32: return by_block<T, 32>(p, B, W, variant, st, e0, e1);
        case 64: return by_block<T, 64>(p, B, W, variant, st, e0, e1);
        case 128: return by_block<T, 128>(p, B, W, variant, st, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace la
