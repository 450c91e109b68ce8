/*
 * fsdpshard_calib.h -- measurement aids exported by libfsdpshard.so.  Not part of the sharded step.
 *
 * fsdpshard_stream_copy is a plain streaming copy of 16-byte vectors: its bandwidth is the
 * achievable-HBM reference on the same GPU, and its known byte count calibrates the hardware
 * fetch / write byte counters against which the step kernel's counter readings are scaled.
 * fsdpshard_stream_rw measures pure reads, pure writes and fixed read : write byte ratios.
 * fsdpshard_stream_mix replays the step's exact access pattern with trivial arithmetic, which
 * separates what the memory system allows for that pattern from what the kernel's code costs;
 * fsdpshard_stream_mix_shaped moves the same bytes in other launch shapes, optionally with each
 * work-group's reads and writes in separate phases.
 *
 * The step's bytes per parameter follow the 2 + 2 + 4 + 8 accounting of "FSDP: Fully Sharded
 * Data Parallel Training at Scale" (memory-breakdown passage): at fan-in F it reads 2F + 12 and
 * writes 12 + 2 bytes, so at F = 8 two thirds of its bytes are reads.
 */
#ifndef FSDPSHARD_CALIB_H
#define FSDPSHARD_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSDPSHARD_CALIB_MAX_STREAMS 8

/*
 * fsdpshard_stream_copy -- dst[0 .. bytes) = src[0 .. bytes).
 *   src, dst  device, 16-byte aligned, non-overlapping
 *   bytes     >= 0, a multiple of 16
 *   stream    hipStream_t as void* (NULL = null stream); asynchronous
 * Returns 0 or an fsdpshard_status (INVALID_ARG, ALIGNMENT, HIP).
 */
int fsdpshard_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * fsdpshard_stream_rw -- n_src read streams and n_dst write streams, each `bytes` long, in a
 * chosen launch shape.
 *   Every 16-byte vector of every source is read once (non-temporal); destination vector i of
 *   stream w receives the XOR of the sources' vectors i, as they were before the call, mixed with
 *   i and w (non-temporal).  With n_dst == 0 nothing is written except, for a vector whose XOR
 *   equals a fixed constant (almost never), that value to *sink, so the loads cannot be
 *   optimised away.
 *   src                host array of n_src device pointers (0 .. FSDPSHARD_CALIB_MAX_STREAMS),
 *                      16-byte aligned
 *   dst                host array of n_dst device pointers (0 .. FSDPSHARD_CALIB_MAX_STREAMS),
 *                      16-byte aligned; n_src + n_dst >= 1.  A destination may not overlap
 *                      another destination, nor a source unless it is that source's pointer
 *                      exactly: that stream is then read and written in place, as the step
 *                      does its fp32 state (every vector is loaded before it is stored)
 *   bytes              >= 0, a multiple of 16
 *   vectors_per_thread 1, 2 or 4 (others: UNSUPPORTED); a thread's vectors are a work-group
 *                      width apart
 *   threads_per_group  256, 512 or 1024 (others: UNSUPPORTED)
 *   per_cu             resident work-groups per CU (0: as many as the registers allow)
 *   xcd_run            0 or 1: work-group b takes tile b; r > 1: each XCD streams runs of r
 *                      consecutive tiles (the tile map of the step kernels)
 *   sink               device, one uint32 (4-byte aligned); required when n_dst == 0
 * Pure reads (n_dst 0), pure writes (n_src 0), a copy (1, 1), the fused step's 2 : 1 read :
 * write byte ratio at fan-in 8 (2, 1); in place: one stream (src = dst = {A}) or one read
 * stream and one in-place stream (src = {A, B}, dst = {B}).
 * Returns 0 or an fsdpshard_status (INVALID_ARG, ALIGNMENT, UNSUPPORTED, OVERFLOW, HIP).
 */
int fsdpshard_stream_rw(const void* const* src, int32_t n_src, void* const* dst, int32_t n_dst,
                        int64_t bytes, int32_t vectors_per_thread, int32_t threads_per_group,
                        int32_t per_cu, int32_t xcd_run, uint32_t* sink, void* stream);

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

/*
 * fsdpshard_stream_mix_interleaved -- the same replay for adamw_shard_step_interleaved: the
 * fan_in contributions are read from `grads`, grads_interleaved_elems(fan_in, n) bf16 elements
 * in the interleaved layout (16-byte aligned); `state`, `out`, n as fsdpshard_stream_mix_blocked.
 * Returns 0 or an fsdpshard_status (INVALID_ARG, ALIGNMENT, UNSUPPORTED, OVERFLOW, HIP).
 */
int fsdpshard_stream_mix_interleaved(const uint16_t* grads, int32_t fan_in, float* state,
                                     uint16_t* out, int64_t n, void* stream);

/*
 * fsdpshard_stream_mix_shaped -- the bytes of fsdpshard_stream_mix_blocked in another launch
 * shape: each wavefront owns `groups_per_wave` consecutive 512-element groups and issues every
 * load of them (state, then contributions) before any store.  With phased == 1 the work-group
 * of 4 wavefronts also meets at a barrier once every wavefront holds its data, so no store of
 * the work-group precedes its last load; with per_cu == 1 each CU then alternates between a
 * read phase of 4 * groups_per_wave groups and a write phase of the same groups.
 *   contribs, fan_in   fan_in 1, 4 or 8 (others: UNSUPPORTED); state, out, n as
 *                      fsdpshard_stream_mix_blocked
 *   groups_per_wave    1, 2 or 4 (others: UNSUPPORTED)
 *   per_cu             resident work-groups per CU (0: as many as the registers allow)
 *   xcd_run            as in fsdpshard_stream_rw
 *   phased             0 or 1
 * Returns 0 or an fsdpshard_status (INVALID_ARG, ALIGNMENT, UNSUPPORTED, OVERFLOW, HIP).
 */
int fsdpshard_stream_mix_shaped(const uint16_t* const* contribs, int32_t fan_in, float* state,
                                uint16_t* out, int64_t n, int32_t groups_per_wave, int32_t per_cu,
                                int32_t xcd_run, int32_t phased, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FSDPSHARD_CALIB_H */
