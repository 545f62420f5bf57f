/*
 * la_bench.h -- measurement helper exported by the same library as la.h.
 *
 * Not part of the attention method: a plain contiguous HBM stream that the
 * benchmark times beside the attention kernels, so that their bandwidth can be
 * read against what the part sustains for the same read/write mix, written
 * here rather than taken from a copy engine or a framework's copy.
 */
#ifndef LA_BENCH_H
#define LA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "la.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One pass over `bytes` bytes of each source (device memory, 16-byte aligned,
 * bytes a multiple of 16):
 *   mode 0: dst = a                (1 read + 1 write stream: the decode step's mix)
 *   mode 1: dst = a ^ b ^ c        (3 reads + 1 write: the prefill's q, k, v -> o mix)
 *   mode 2: a is read, nothing is written (dst must still be a valid 16-byte
 *           device buffer; it is never written for any data a caller can supply
 *           short of a fixed 16-byte pattern, and then only its first 16 bytes).
 * workgroups: 256-thread workgroups in the grid (1 .. 2^20); each lane keeps
 * four 16-byte loads in flight.  nontemporal != 0 uses non-temporal loads and
 * stores.  dst must not overlap the sources.  Enqueued on `stream` (a
 * hipStream_t, NULL = null stream); returns LA_ERR_INVALID_ARG for a bad
 * argument (nothing enqueued) or LA_ERR_HIP if the launch fails. */
la_status la_bench_stream(int32_t mode, const void* a, const void* b, const void* c, void* dst, size_t bytes,
                          int32_t workgroups, int32_t nontemporal, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LA_BENCH_H */
