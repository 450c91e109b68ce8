/*
 * fsdpshard.h -- C ABI of libfsdpshard.so: one rank's share of a fully sharded (ZeRO-3 / FSDP
 * FULL_SHARD) training step on one AMD Instinct MI355X (gfx950).
 *
 * The pages this follows (titles as published):
 *   [FSDP]  "FSDP: Fully Sharded Data Parallel Training at Scale"
 *   [DDL]   "Distributed Deep Learning & Model Sharding"
 *
 * Conventions for every call below
 *   - Counts and indices are int64_t.  bf16 values travel as uint16_t bit patterns.
 *   - "device" pointers are HIP device allocations on the current HIP device; "host" pointers are
 *     ordinary process memory.  The caller owns every buffer; the library never allocates device
 *     memory and keeps no state besides, per device, the cached LDS size of one compute unit
 *     (queried once, used to size launches).
 *   - `stream` is a hipStream_t passed as void* (NULL = the device's null stream).  GPU calls are
 *     asynchronous and stream-ordered: they validate their arguments on the host, enqueue their
 *     kernels (one for most calls; two for the sums of squares; reshard_copy one per 96 pieces)
 *     and return.  A fault inside a kernel surfaces at the caller's next synchronisation.
 *   - Every call returns 0 (FSDPSHARD_OK) or a positive fsdpshard_status.  Argument errors are
 *     found before anything is enqueued; a launch the HIP runtime refuses (FSDPSHARD_ERR_HIP)
 *     may leave a multi-kernel call's earlier kernels enqueued.  Nothing is thrown and nothing
 *     aborts.
 *   - n == 0 is a successful no-op, except that the calls with a sum of squares still write +0
 *     into their result (one small kernel).
 */
#ifndef FSDPSHARD_H
#define FSDPSHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSDPSHARD_ABI_VERSION 1
#define FSDPSHARD_MAX_FAN_IN 64
#define FSDPSHARD_STATE_BLOCK 512   /* elements per block of the blocked state layout */

typedef enum fsdpshard_status {
    FSDPSHARD_OK = 0,
    FSDPSHARD_ERR_INVALID_ARG = 1,  /* null pointer, negative size, rank >= world, overlap, ... */
    FSDPSHARD_ERR_OVERFLOW = 2,     /* a flat offset, P, or k*P does not fit the int64 range */
    FSDPSHARD_ERR_CAPACITY = 3,     /* a caller array (segments, pieces) or workspace too small */
    FSDPSHARD_ERR_ALIGNMENT = 4,    /* an fp32 or gradient pointer is not 16-byte aligned, ... */
    FSDPSHARD_ERR_UNSUPPORTED = 5,  /* fan_in above FSDPSHARD_MAX_FAN_IN */
    FSDPSHARD_ERR_HIP = 6           /* the HIP runtime refused a query or the kernel launch */
} fsdpshard_status;

/* Segment flags. */
#define FSDPSHARD_SEG_WEIGHT_DECAY 1u  /* decoupled weight decay applies to these elements */
#define FSDPSHARD_SEG_PADDING 2u       /* padding: never updated, served as +0 */

/*
 * One run of a rank's slice that belongs to a single tensor and is either all real elements or
 * all padding.  32 bytes, 8-byte aligned; the same struct is used on the host and, uploaded by
 * the caller, on the device.
 */
typedef struct fsdpshard_segment {
    int64_t shard_begin;    /* first element of the run, counted from the slice start lo   */
    int64_t length;         /* elements in the run, >= 1                                    */
    int64_t tensor_offset;  /* position of shard_begin inside its tensor's padded extent    */
    int32_t tensor_id;      /* index of the tensor in the flatten order                     */
    uint32_t flags;         /* FSDPSHARD_SEG_* bits                                         */
} fsdpshard_segment;

typedef struct fsdpshard_layout {
    int64_t P;           /* flat length, padding included                                  */
    int64_t lo, hi;      /* the rank's slice [lo, hi) of the flat vector                   */
    int64_t n;           /* hi - lo                                                        */
    int64_t n_real;      /* elements of the slice that are not padding                     */
    int32_t n_segments;  /* segments needed to describe the slice (always reported)        */
    int32_t n_tensors;   /* tensors that intersect the slice                               */
} fsdpshard_layout;

/* AdamW hyperparameters of one step (float64 on the host; see adamw_shard_step). */
typedef struct fsdpshard_adamw {
    double lr;
    double beta1, beta2;        /* each in [0, 1)                                          */
    double eps;
    double weight_decay;        /* decoupled, scaled by lr                                 */
    double grad_scale;          /* multiplies the reduced gradient; 1.0 = plain sum        */
    int64_t step;               /* 1-based step counter t, incremented by the caller       */
    double max_grad_norm;       /* > 0: clip by the global gradient norm; 0: no clipping   */
    const double* grad_sumsq;   /* device: global sum of g^2 (see grad_sumsq_shard); read
                                   by the kernel when max_grad_norm > 0, else ignored      */
} fsdpshard_adamw;

/*
 * shard_layout -- flatten tensors and cut rank `rank`'s slice.            (host only, no GPU)
 *
 * [FSDP], passage on sharding a linear layer: a unit's parameters are viewed as one 1-D tensor
 * of length P; with N ranks, rank k owns the contiguous elements floor(kP/N) .. floor((k+1)P/N)-1,
 * and its gradient, m and v shards cover the same positions.  Several tensors are laid out one
 * after another in the order given, each padded up to a multiple of `pad_multiple` elements
 * (1 = no padding).
 *
 *   numels        host, n_tensors sizes (each >= 0); may be NULL when n_tensors == 0
 *   pad_multiple  >= 1
 *   wd_mask       host, n_tensors bytes (nonzero = weight decay on), or NULL = on everywhere
 *   world_size    N >= 1;  rank: 0 <= rank < N
 *   out           host, receives P, lo, hi, n, n_real, n_segments, n_tensors (required)
 *   segs          host, room for seg_capacity segments, or NULL to only count
 *   seg_capacity  >= 0
 * Segments tile [0, n) in flat order.  k*P is formed in 128-bit arithmetic.  If segs is non-NULL
 * and n_segments > seg_capacity, `out` is still filled, the first seg_capacity segments are
 * written and FSDPSHARD_ERR_CAPACITY is returned (call again with a larger array).
 * Errors: INVALID_ARG (nulls, negative sizes, bad rank or world size, pad_multiple < 1),
 *         OVERFLOW (P or a padded size beyond INT64_MAX).
 */
int shard_layout(const int64_t* numels, int32_t n_tensors, int64_t pad_multiple,
                 const uint8_t* wd_mask, int32_t world_size, int32_t rank,
                 fsdpshard_layout* out, fsdpshard_segment* segs, int32_t seg_capacity);

/*
 * Blocked state layout (an alternative to three separate master / m / v arrays).
 *
 * The optimizer state of an n-element slice kept in one array of state_blocked_elems(n) floats:
 * for block b = i / FSDPSHARD_STATE_BLOCK and o = i % FSDPSHARD_STATE_BLOCK, element i's master
 * is at state[(3b + 0) * FSDPSHARD_STATE_BLOCK + o], its m at (3b + 1) * ... + o and its v at
 * (3b + 2) * ... + o.  Positions past n in the last block are never read or written.  The values
 * and their positions in the slice are those of the separate layout ([FSDP], sharding a linear
 * layer: grad, m and v shards cover the same positions); only the placement in memory differs:
 * on MI355X the step streams one state array instead of three and runs 3-8 % faster.
 */
int64_t state_blocked_elems(int64_t n);   /* 3 * ceil(n / 512) * 512, or -1 if n is out of range */

/*
 * adamw_shard_step_blocked, adamw_shard_step_f32grad_blocked -- adamw_shard_step and
 * adamw_shard_step_f32grad with the state in the blocked layout.
 *   state  device, state_blocked_elems(n) floats, 16-byte aligned, updated in place; it must not
 *          overlap the gradient inputs, the bf16 window or grad_sumsq
 * Every other argument, the results and the errors are those of the separate-layout calls.
 */
int adamw_shard_step_blocked(float* state, const uint16_t* const* contribs, int32_t fan_in,
                             int64_t n, const fsdpshard_segment* segs, int32_t n_segments,
                             const fsdpshard_adamw* hp, uint16_t* flat_bf16, int64_t flat_index0,
                             int64_t lo, void* stream);
int adamw_shard_step_f32grad_blocked(float* state, const float* grad, int64_t n,
                                     const fsdpshard_segment* segs, int32_t n_segments,
                                     const fsdpshard_adamw* hp, uint16_t* flat_bf16,
                                     int64_t flat_index0, int64_t lo, void* stream);

/*
 * Interleaved gradient layout (an alternative to F separate contribution arrays).
 *
 * The F bf16 contributions of an n-element slice kept in one array of
 * grads_interleaved_elems(F, n) elements: for block b = i / FSDPSHARD_STATE_BLOCK and
 * o = i % FSDPSHARD_STATE_BLOCK, contribution r's element i is at
 * grads[(b * F + r) * FSDPSHARD_STATE_BLOCK + o].  Positions past n in the last block are never
 * read.  The values are the slice's F contributions of [FSDP], communication pattern of one unit
 * (what the reduce-scatter sums); only their placement differs: a receive buffer the peers write
 * into block by block.  With it the step streams one gradient array instead of F.
 */
int64_t grads_interleaved_elems(int32_t fan_in, int64_t n);  /* F * ceil(n / 512) * 512, or -1 if
                                                               fan_in or n is out of range     */

/*
 * adamw_shard_step_interleaved -- adamw_shard_step_blocked with the contributions interleaved.
 *   grads   device, grads_interleaved_elems(fan_in, n) bf16 bit patterns, 16-byte aligned, read
 *           only; it must not overlap the state, the bf16 window or grad_sumsq
 *   fan_in  1 .. FSDPSHARD_MAX_FAN_IN; contributions are added in rank order r = 0 .. F-1
 * The results are bit-identical to adamw_shard_step_blocked on the same contributions; every
 * other argument and error is that call's (OVERFLOW also when the gradient array's size in bytes
 * does not fit int64).
 */
int adamw_shard_step_interleaved(float* state, const uint16_t* grads, int32_t fan_in, int64_t n,
                                 const fsdpshard_segment* segs, int32_t n_segments,
                                 const fsdpshard_adamw* hp, uint16_t* flat_bf16,
                                 int64_t flat_index0, int64_t lo, void* stream);

/*
 * grads_to_interleaved -- copy F separate contributions (n elements each) into the interleaved
 * array `grads` (grads_interleaved_elems(fan_in, n) elements; positions past n in the last block
 * are left untouched).  All pointers device and 16-byte aligned; `grads` must not overlap a
 * contribution.  Errors: INVALID_ARG, UNSUPPORTED (fan_in > FSDPSHARD_MAX_FAN_IN), ALIGNMENT,
 * OVERFLOW, HIP.
 */
int grads_to_interleaved(const uint16_t* const* contribs, int32_t fan_in, int64_t n,
                         uint16_t* grads, void* stream);

/*
 * state_to_blocked, state_from_blocked -- copy an n-element slice's state between the separate
 * arrays (n floats each) and the blocked array (state_blocked_elems(n) floats), e.g. to
 * checkpoint or reshard blocked state with reshard_plan / reshard_copy, which move the separate
 * arrays.  All pointers device, 16-byte aligned, pairwise non-overlapping.
 * Errors: INVALID_ARG, ALIGNMENT, OVERFLOW, HIP.
 */
int state_to_blocked(const float* master, const float* m, const float* v, int64_t n, float* state,
                     void* stream);
int state_from_blocked(const float* state, int64_t n, float* master, float* m, float* v,
                       void* stream);

/*
 * reduce_shard -- out[i] = scale * (((+0 + G_0[i]) + G_1[i]) + ... + G_{F-1}[i]),  0 <= i < n.
 *
 * [FSDP], communication pattern of one unit: the reduce-scatter after backward sums the ranks'
 * gradients and leaves rank k only the part matching its slice; mixed-precision passage: the
 * reduction runs in float32.  Here the F contributions of the slice are already on this GPU
 * (no collective); each is widened exactly from bf16 and added in rank order 0..F-1 in float32.
 *
 *   contribs  host array of `fan_in` device pointers, each to n bf16 values, 16-byte aligned
 *   fan_in    1 .. FSDPSHARD_MAX_FAN_IN
 *   scale     multiplies the sum once (float32)
 *   out       device, n floats, 16-byte aligned, must not overlap any contribution
 * Errors: INVALID_ARG, ALIGNMENT, UNSUPPORTED, HIP.
 */
int reduce_shard(const uint16_t* const* contribs, int32_t fan_in, int64_t n, float scale,
                 float* out, void* stream);

/*
 * adamw_shard_step -- the fused local step of one slice: reduce the F bf16 contributions,
 * AdamW-update the fp32 master, m and v shards in place, and write the bf16 copy of the updated
 * master into the flat parameter layout.
 *
 * [FSDP], communication pattern: the optimizer step runs on each rank with only its own
 * parameter, gradient and optimizer-state slices; the next all-gather serves the bf16 params.
 * [FSDP], memory breakdown, and [DDL], "The constraint is rarely FLOPs": bf16 params and grads,
 * fp32 master weights, fp32 first moment (moving average of g) and second moment (moving average
 * of g^2).  The pages do not print the update; it is bias-corrected Adam with decoupled weight
 * decay scaled by lr.  Per real element, each step an IEEE float32 operation on its own:
 *   g = scale * sum_r G_r             (as reduce_shard)
 *   m = b1*m + c1*g;  v = b2*v + c2*(g*g)
 *   den = sqrt(v / bc2) + eps;  th = th*dec (decay flag);  th = th - lr*((m / bc1) / den)
 *   flat[lo + i] = bf16 round-to-nearest-even of th  (NaN stays a quiet NaN)
 * with c1 = 1-beta1, c2 = 1-beta2, bc1 = 1-beta1^t, bc2 = 1-beta2^t, dec = 1-lr*weight_decay
 * formed in float64 and rounded to float32 once.  Padding elements keep master, m and v bit for
 * bit and are served as +0; their gradient values are ignored.
 * Clipping ([FSDP], gradient-clipping passage: the norm must be the global one, not the rank's):
 * when hp->max_grad_norm > 0 the scale above is float32(grad_scale * min(1, max_grad_norm /
 * (sqrt(*hp->grad_sumsq) + 1e-6))), formed in float64 on the device from the global sum of
 * squares, so no host synchronisation is needed between the norm and the step.
 *
 *   master, m, v  device, n floats each, 16-byte aligned, updated in place
 *   contribs      host array of fan_in device pointers, each to n bf16 values, 16-byte aligned
 *   segs          device copy of the slice's segments (as shard_layout emits them), 8-byte
 *                 aligned, or NULL with n_segments == 0 (all elements real, decay everywhere).
 *                 Segments must tile [0, n) in order; elements they do not cover take the flags
 *                 of the nearest preceding segment (never an out-of-bounds read).
 *   hp            host
 *   flat_bf16     device window of the flat bf16 parameter vector whose element 0 is flat index
 *                 flat_index0 (2-byte aligned; any phase); the call writes exactly the elements
 *                 of flat indices [lo, lo + n) and nothing else.  NULL skips the bf16 output.
 *   lo            flat index of the slice start, flat_index0 <= lo
 * No written buffer (master, m, v, the bf16 window) may overlap another buffer of the call,
 * the segment table and grad_sumsq included.
 * Errors: INVALID_ARG (nulls, n < 0, step < 1, betas outside [0,1), non-finite values,
 *         negative max_grad_norm, clipping without grad_sumsq, overlaps, n_segments < 0),
 *         ALIGNMENT, UNSUPPORTED, HIP.
 */
int adamw_shard_step(float* master, float* m, float* v,
                     const uint16_t* const* contribs, int32_t fan_in, int64_t n,
                     const fsdpshard_segment* segs, int32_t n_segments,
                     const fsdpshard_adamw* hp,
                     uint16_t* flat_bf16, int64_t flat_index0, int64_t lo, void* stream);

/*
 * adamw_shard_step_f32grad -- adamw_shard_step fed by one fp32 gradient shard instead of F bf16
 * contributions: g = grad[i] * scale (scale as in adamw_shard_step, clipping included).
 *
 * [FSDP], mixed-precision passage: gradients accumulated in float32 (reduce_dtype) keep small
 * values; gradient accumulation over micro-batches suppresses the synchronisation until the last
 * one.  reduce_shard / reduce_shard_accumulate build `grad` over the micro-batches.
 *   grad   device, n floats, 16-byte aligned, read only, must not overlap a written buffer
 *   other arguments as in adamw_shard_step.
 * Errors: as adamw_shard_step.
 */
int adamw_shard_step_f32grad(float* master, float* m, float* v, const float* grad, int64_t n,
                             const fsdpshard_segment* segs, int32_t n_segments,
                             const fsdpshard_adamw* hp, uint16_t* flat_bf16, int64_t flat_index0,
                             int64_t lo, void* stream);

/*
 * reduce_shard_accumulate -- acc[i] = acc[i] + scale * (((+0 + G_0[i]) + ...) + G_{F-1}[i]).
 *
 * [FSDP], mixed-precision passage (float32 gradient accumulation) and its note on accumulating
 * over micro-batches before synchronising: one micro-batch's reduced contributions added to an
 * fp32 gradient shard, each of the three steps one float32 rounding.
 *   acc    device, n floats, 16-byte aligned, updated in place; other arguments as reduce_shard.
 * Errors: as reduce_shard.
 */
int reduce_shard_accumulate(const uint16_t* const* contribs, int32_t fan_in, int64_t n,
                            float scale, float* acc, void* stream);

/*
 * reduce_shard_interleaved -- reduce_shard (accumulate = 0) or reduce_shard_accumulate
 * (accumulate = 1, `out` is the accumulator) of fan_in contributions held in the interleaved
 * layout (see grads_interleaved_elems); the results are bit-identical to those calls on the same
 * contributions.
 *   grads  device, grads_interleaved_elems(fan_in, n) bf16 bit patterns, 16-byte aligned; it
 *          must not overlap `out`
 * Errors: those of reduce_shard; INVALID_ARG also for accumulate other than 0 or 1; OVERFLOW
 * also when the gradient array's size in bytes does not fit int64.
 */
int reduce_shard_interleaved(const uint16_t* grads, int32_t fan_in, int64_t n, float scale,
                             float* out, int32_t accumulate, void* stream);

/*
 * grad_sumsq_workspace_bytes -- device workspace grad_sumsq_shard needs for an n-element slice
 * (8 bytes per 32,768 elements, rounded up); -1 for n < 0.
 */
int64_t grad_sumsq_workspace_bytes(int64_t n);

/*
 * grad_sumsq_shard -- this rank's share of the squared global gradient norm: the sum over the
 * slice's real elements of g_i^2, g_i the float32 reduced gradient times `scale` (as in
 * reduce_shard), each square exact in float64, the sum in float64 in a fixed order (so the
 * result depends only on n and the data).
 *
 * [FSDP], gradient-clipping passage: a norm computed from one rank's slice underestimates the
 * global norm; the ranks' sums of squares are added (a scalar all-reduce across ranks) and the
 * total feeds adamw_shard_step's clipping through hp->grad_sumsq.
 *   contribs, fan_in  the bf16 contributions as in reduce_shard (fan_in 1 .. 64), or
 *   grad              with fan_in == 0: one fp32 gradient shard (16-byte aligned)
 *   segs, n_segments  as in adamw_shard_step (padding does not count)
 *   workspace         device, >= grad_sumsq_workspace_bytes(n) bytes, 8-byte aligned, scratch
 *   sumsq             device, one double, receives the sum (+0 for n == 0)
 * The written buffers (workspace, sumsq) may not overlap each other, a gradient input or the
 * segment table.  Two kernels are enqueued on `stream`; the workspace may be reused once they
 * have run.
 * Errors: INVALID_ARG (nulls, negative sizes, overlaps), ALIGNMENT, UNSUPPORTED,
 *         CAPACITY (workspace too small), OVERFLOW, HIP.
 */
int grad_sumsq_shard(const uint16_t* const* contribs, int32_t fan_in, const float* grad,
                     int64_t n, const fsdpshard_segment* segs, int32_t n_segments, float scale,
                     void* workspace, int64_t workspace_bytes, double* sumsq, void* stream);

/*
 * grad_sumsq_shard_interleaved -- grad_sumsq_shard of fan_in contributions held in the
 * interleaved layout (see grads_interleaved_elems): the same sum, bit for bit, in the same
 * order.
 *   grads   device, grads_interleaved_elems(fan_in, n) bf16 bit patterns, 16-byte aligned
 *   fan_in  1 .. FSDPSHARD_MAX_FAN_IN
 * Every other argument and error is grad_sumsq_shard's (the interleaved array is the input that
 * the workspace, sumsq and the segment table must not overlap; OVERFLOW also when its size in
 * bytes does not fit int64).
 */
int grad_sumsq_shard_interleaved(const uint16_t* grads, int32_t fan_in, int64_t n,
                                 const fsdpshard_segment* segs, int32_t n_segments, float scale,
                                 void* workspace, int64_t workspace_bytes, double* sumsq,
                                 void* stream);

/*
 * grad_sumsq_shard_noalloc -- grad_sumsq_shard with no workspace argument.
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine).  Its float64 partials live in a library-owned array of
 * FSDPSHARD_NOALLOC_MAX_PARTIALS doubles (512 KiB) in each device's global segment, held by every
 * GPU the library runs on until the process ends; its device address is looked up once per
 * device, on the first call whose stream belongs to that device (make that first call outside a
 * graph capture).  Slices of up to FSDPSHARD_NOALLOC_MAX_ELEMS elements are accepted; a longer
 * slice returns CAPACITY.  Every partial the second kernel reads is written by the first kernel
 * of the same call, so nothing has to be cleared between calls; but all calls on one GPU share
 * the one array, so calls that overlap in time on one GPU (work on different streams, or host
 * threads without an ordering between their calls) race and give wrong sums.
 * Arguments, results and the other errors are those of grad_sumsq_shard.
 */
#define FSDPSHARD_NOALLOC_MAX_PARTIALS 65536
#define FSDPSHARD_NOALLOC_MAX_ELEMS ((int64_t)FSDPSHARD_NOALLOC_MAX_PARTIALS * 32768)
int grad_sumsq_shard_noalloc(const uint16_t* const* contribs, int32_t fan_in, const float* grad,
                             int64_t n, const fsdpshard_segment* segs, int32_t n_segments,
                             float scale, double* sumsq, void* stream);

/*
 * unflatten_bf16 -- flat[lo + i] = bf16_rne(master[i]) for real elements, +0 for padding.
 *
 * [FSDP], communication pattern: after the all-gather every rank holds the full bf16 parameter
 * tensor, each rank's slice sitting at [lo, hi) of the flat layout; this writes one slice's part.
 * Arguments as in adamw_shard_step (master 16-byte aligned; flat_bf16 any 2-byte phase; segs
 * may be NULL with n_segments == 0).  The written window may not overlap master or the segment
 * table.
 * Errors: INVALID_ARG, ALIGNMENT, HIP.
 */
int unflatten_bf16(const float* master, int64_t n, const fsdpshard_segment* segs,
                   int32_t n_segments, uint16_t* flat_bf16, int64_t flat_index0, int64_t lo,
                   void* stream);

/*
 * reduce_shard_sumsq -- reduce_shard (accumulate == 0) or reduce_shard_accumulate
 * (accumulate == 1) into the fp32 shard `out`, fused with the sum of squares of the result:
 *   *sumsq = sum over real elements i of (double)out[i]^2   (float64, fixed order)
 *
 * [FSDP], gradient clipping passage (each rank contributes its part of the squared global norm;
 * see grad_sumsq_shard) and mixed-precision passage (float32 gradient shards).  With a large
 * fan-in this reads the contributions once: the reduction plus the fp32-gradient step move
 * 2F + 4 + 30 bytes per parameter against 2F + 26 + 2F for grad_sumsq_shard plus the fused step.
 * After the last micro-batch (accumulate == 1) it yields the norm of the accumulated gradient.
 *   contribs, fan_in, n, scale, out   as reduce_shard; out also receives padding positions
 *                                      (their values are whatever the reduction gives)
 *   segs, n_segments   device segment table of the slice (padding does not count), or NULL/0
 *   workspace          device, >= grad_sumsq_workspace_bytes(n) bytes, 8-byte aligned
 *   sumsq              device, one double, receives this rank's part (+0 when n == 0)
 * The written buffers (out, workspace, sumsq) may not overlap each other, a contribution or the
 * segment table.
 * Errors: INVALID_ARG (nulls, overlaps, accumulate not 0 or 1), ALIGNMENT, UNSUPPORTED,
 *         CAPACITY (workspace too small), OVERFLOW, HIP.
 */
int reduce_shard_sumsq(const uint16_t* const* contribs, int32_t fan_in, int64_t n, float scale,
                       float* out, int32_t accumulate, const fsdpshard_segment* segs,
                       int32_t n_segments, void* workspace, int64_t workspace_bytes, double* sumsq,
                       void* stream);

/*
 * reduce_shard_sumsq_interleaved -- reduce_shard_sumsq of fan_in contributions held in the
 * interleaved layout: bit-identical results.  `grads` as for reduce_shard_interleaved; every
 * other argument and error as for reduce_shard_sumsq.
 */
int reduce_shard_sumsq_interleaved(const uint16_t* grads, int32_t fan_in, int64_t n, float scale,
                                   float* out, int32_t accumulate, const fsdpshard_segment* segs,
                                   int32_t n_segments, void* workspace, int64_t workspace_bytes,
                                   double* sumsq, void* stream);

/*
 * One piece of a reshard plan: `length` elements that land at `dst_offset` of the destination
 * shard, read from `src_offset` of source rank `src_rank`'s shard, or zeros when src_rank is -1
 * (destination padding).  32 bytes.
 */
typedef struct fsdpshard_piece {
    int64_t src_offset;
    int64_t dst_offset;
    int64_t length;
    int32_t src_rank;
    int32_t reserved;   /* 0 */
} fsdpshard_piece;

/*
 * reshard_plan -- how destination rank `dst_rank` of a new layout gathers its shard from the
 * shards of an old one.                                                       (host only, no GPU)
 *
 * [FSDP], checkpointing passage: a local state dict holds each rank's own shard and loads only
 * with the same number of GPUs and wrapping; resharding turns one world size's shards into
 * another's.  Both layouts flatten the same tensors (numels, in order) under the floor rule of
 * shard_layout, each with its own padding multiple and world size.  Every tensor keeps its
 * values; destination padding is zero.  Pieces come in destination order, tile the destination
 * shard exactly, and contiguous neighbours are merged.
 *   pieces    host, room for `capacity` pieces, or NULL to count only
 *   n_pieces  host, receives the number of pieces (always)
 * Errors: INVALID_ARG, OVERFLOW, CAPACITY (pieces written up to capacity; call again).
 */
int reshard_plan(const int64_t* numels, int32_t n_tensors, int64_t src_pad, int32_t src_world,
                 int64_t dst_pad, int32_t dst_world, int32_t dst_rank, fsdpshard_piece* pieces,
                 int32_t capacity, int32_t* n_pieces);

/*
 * reshard_copy -- execute a reshard plan on the GPU: for every piece, copy `length` elements of
 * `elem_bytes` bytes from src_shards[src_rank] + src_offset to dst + dst_offset, or write zeros.
 *   src_shards  host array of src_world device pointers (a NULL entry is allowed for a rank no
 *               piece reads); src_elems: host array, the element count of each source shard
 *   dst         device pointer to the destination shard of dst_elems elements (may be NULL
 *               when dst_elems == 0: an empty shard, as P < N produces)
 *   pieces      host array of n_pieces pieces (as reshard_plan emits them)
 *   elem_bytes  2, 4 or 8; every pointer aligned to elem_bytes
 * Every piece is checked against the shard sizes before anything is enqueued.  Pieces may not
 * overlap in the destination, and no source shard may overlap the destination.
 * Errors: INVALID_ARG (out-of-range piece, bad rank, overlap), ALIGNMENT, HIP.
 */
int reshard_copy(const void* const* src_shards, const int64_t* src_elems, int32_t src_world,
                 void* dst, int64_t dst_elems, const fsdpshard_piece* pieces, int32_t n_pieces,
                 int32_t elem_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* fsdpshard_strerror(int code);

/* FSDPSHARD_ABI_VERSION of the loaded library. */
int fsdpshard_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FSDPSHARD_H */
