/*
 * moe_streams.h -- C ABI of libmoe_streams, a measurement aid that ships
 * beside libmoe_ep and is not part of dispatch / combine: plain streaming
 * kernels with the 16-byte non-temporal accesses of the row kernels, free of
 * their row lookups and arithmetic, each in the fastest grid form found for
 * its access pattern.  The benchmark times them on the
 * phases' own buffers to give each phase the achievable HBM rate of its
 * access pattern on the same GPU, and counter runs use the copy to calibrate
 * the hardware byte counters.
 *
 * Conventions: device pointers owned by the caller, 16-B aligned; every call
 * only enqueues work on `stream` (a hipStream_t, NULL = the default stream).
 * Return codes are those of moe_ep.h (MOE_OK, MOE_EINVAL, MOE_ENULL,
 * MOE_EALIGN, MOE_ERANGE, MOE_EHIP); a rejected call enqueues nothing.
 */
#ifndef MOE_STREAMS_H
#define MOE_STREAMS_H

#include <stdint.h>

#include "moe_ep.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copy nbytes (a multiple of 16) from src to dst; the buffers must not
 * overlap.  MOE_EINVAL for a negative or ragged size. */
int moe_copy(void *dst, const void *src, int64_t nbytes, void *stream);

/*
 * Streams with the access patterns of two phases; n16 counts 16-byte units,
 * k is in [1, 8], and what is stored is the XOR of the bytes read.
 *   MOE_STREAM_FANOUT: unit i reads 32 bytes (src units 2i and 2i+1) and
 *     stores 16 bytes at dst unit j*n16 + i for every j < k: the dispatch
 *     pack's bf16 row in, k fp8 rows out.  src holds 2*n16 units, dst k*n16.
 *   MOE_STREAM_REDUCE: unit i reads src units j*n16 + i for every j < k and
 *     stores 16 bytes at dst unit i: the receive-side sum's k rows in, one
 *     out.  src holds k*n16 units, dst n16.
 *   MOE_STREAM_FANOUT_ONESHOT: MOE_STREAM_FANOUT's result from another
 *     grid (one unit per thread, workgroups in address order), the faster
 *     form when k is small.
 * Errors: MOE_EINVAL for another pattern, k outside [1, 8] or n16 < 0;
 * MOE_ERANGE for n16 above 2^40 (16 TiB); MOE_ENULL / MOE_EALIGN.
 */
#define MOE_STREAM_FANOUT 1
#define MOE_STREAM_REDUCE 2
#define MOE_STREAM_FANOUT_ONESHOT 3
int moe_stream(int pattern, int k, void *dst, const void *src, int64_t n16, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_STREAMS_H */
