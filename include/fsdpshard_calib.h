/*
 * fsdpshard_calib.h -- measurement aids exported by libfsdpshard.so.  Not part of the sharded step.
 *
 * fsdpshard_stream_copy is a plain streaming copy of 16-byte vectors: its bandwidth is the
 * achievable-HBM reference on the same GPU, and its known byte count calibrates the hardware
 * fetch / write byte counters against which the step kernel's counter readings are scaled.
 * fsdpshard_stream_mix replays the step's exact access pattern with trivial arithmetic, which
 * separates what the memory system allows for that pattern from what the kernel's code costs.
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

/*
 * fsdpshard_stream_mix -- the fused step's memory traffic without its arithmetic: for every
 * element i < n it reads the F bf16 contributions and s0[i], s1[i], s2[i] and writes s0, s1, s2
 * back, the first element of every 8-element vector XOR-ed with the XOR of that vector's
 * contribution words; out receives 16 bytes per vector (the second element of each state vector
 * and the XOR).  Same vector width, cache hints and one-group-per-wave grid as adamw_shard_step.
 * Its bandwidth is the ceiling of that access pattern on the GPU at hand.
 *   contribs  host array of fan_in device pointers (1 .. 64), n bf16 each, 16-byte aligned
 *   s0,s1,s2  device, n floats each, 16-byte aligned;  out: device, n bf16, 16-byte aligned
 *   n         >= 0, a multiple of 8;  no written buffer may overlap another buffer of the call
 * Returns 0 or an fsdpshard_status (INVALID_ARG, ALIGNMENT, UNSUPPORTED, OVERFLOW, HIP).
 */
int fsdpshard_stream_mix(const uint16_t* const* contribs, int32_t fan_in, float* s0, float* s1,
                         float* s2, uint16_t* out, int64_t n, void* stream);

/*
 * fsdpshard_stream_mix_blocked -- the same replay for the blocked state layout (see
 * adamw_shard_step_blocked): `state` holds state_blocked_elems(n) floats, 16-byte aligned.
 */
int fsdpshard_stream_mix_blocked(const uint16_t* const* contribs, int32_t fan_in, float* state,
                                 uint16_t* out, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FSDPSHARD_CALIB_H */
