/*
 * fsdpshard_calib.h -- measurement aid exported by libfsdpshard.so.  Not part of the sharded step.
 *
 * A plain streaming copy of 16-byte vectors.  It serves two purposes when the step kernels are
 * measured: its bandwidth is the achievable-HBM reference on the same GPU, and its known byte
 * count calibrates the hardware fetch / write byte counters against which the step kernels' own
 * counter readings are scaled.
 */
#ifndef FSDPSHARD_CALIB_H
#define FSDPSHARD_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fsdpshard_stream_copy -- dst[0 .. bytes) = src[0 .. bytes).
 *   src, dst  device, 16-byte aligned, non-overlapping
 *   bytes     >= 0, a multiple of 16
 *   stream    hipStream_t as void* (NULL = null stream); asynchronous
 * Returns 0 or an fsdpshard_status (INVALID_ARG, ALIGNMENT, HIP).
 */
int fsdpshard_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FSDPSHARD_CALIB_H */
