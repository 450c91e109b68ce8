// Device side of libfsdpshard.so: the fused local step of one rank's slice on gfx950 (MI355X).
//
// What is computed (page titles as published):
//   "FSDP: Fully Sharded Data Parallel Training at Scale" -- communication pattern of one unit:
//   the reduce-scatter sums the ranks' gradients and leaves rank k the part of its slice; the
//   optimizer step then runs locally on the rank's parameter, gradient and Adam-state slices; the
//   next all-gather serves the bf16 parameters.  Memory breakdown and mixed-precision passages:
//   fp32 master weights, fp32 first / second moments, bf16 params and grads, fp32 reduction.
//   "Distributed Deep Learning & Model Sharding", "The constraint is rarely FLOPs": the same
//   2 + 2 + 12 bytes of state per parameter.
//
// How it maps to the hardware.  The step is a pure stream: per parameter it reads 2F bytes of
// bf16 gradient contributions and 12 bytes of fp32 state and writes 12 + 2 bytes, with ~30 ALU
// operations -- about 0.5 flop per byte, so HBM bandwidth bounds it and MFMA has no role.
//   * Every lane owns a vector of 8 consecutive elements: one 16-byte load per gradient stream,
//     two 16-byte loads / stores per fp32 stream, one 16-byte bf16 store.  A wave covers 512
//     elements (1 KiB per bf16 stream, 2 KiB per fp32 stream, all fully coalesced).
//   * Each work-group owns one contiguous chunk of the slice; its 4 waves take interleaved 512-
//     element groups of it.  The grid is a few work-groups per compute unit (256 CUs), sized so
//     every wave has the same number of groups.
//   * Contributions are reduced in registers in rank order 0..F-1 from +0 (fixed order, so the
//     result is deterministic and matches a sequential float32 sum bit for bit).
//   * Segment flags (padding, weight decay) come from a per-wave cursor over the segment table:
//     one binary search when a wave starts, a compare per group after that, and a per-element
//     scan only in the rare groups that contain a tensor edge.
//   * The bf16 destination may start at any 2-byte phase inside a 16-byte vector (a slice starts
//     wherever floor(kP/N) falls).  The state streams stay aligned; the bf16 result is re-phased
//     across lanes (each lane borrows its right neighbour's first elements through a lane
//     permute) so interior stores stay 16-byte aligned, and only the two edge lanes of a group
//     write their leftover elements with 2-byte stores.
// Arithmetic is IEEE float32 with no contraction (the library is built with -ffp-contract=off),
// correctly rounded division and square root, denormals kept.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "fsdpshard.h"
#include "fsdpshard_calib.h"

namespace {

constexpr int kVec = 8;            // elements per lane
constexpr int kWave = 64;          // lanes per wavefront
constexpr int kBlock = 256;        // threads per work-group
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kDefaultBlocksPerCu = 4;
constexpr int kMaxDevices = 64;

// ------------------------------------------------------------------------------------------------
// Kernel parameter blocks (passed by value in the kernel-argument segment).

struct StepParams {
    float* master;
    float* m;
    float* v;
    const uint16_t* contrib[FSDPSHARD_MAX_FAN_IN];
    const fsdpshard_segment* segs;
    uint16_t* out;           // destination of slice element 0 (flat index lo), or null
    int64_t n;               // elements in the slice
    int64_t block_vecs;      // 8-element vectors per work-group (multiple of 64 * waves)
    int32_t n_segs;
    int32_t fan_in;
    int32_t out_shift;       // first slice element whose destination is 16-byte aligned (0..7)
    float b1, b2, c1, c2, bc1, bc2, eps, lr, dec, scale;
};

struct ReduceParams {
    const uint16_t* contrib[FSDPSHARD_MAX_FAN_IN];
    float* out;
    int64_t n;
    int64_t block_vecs;
    int32_t fan_in;
    float scale;
};

struct UnflattenParams {
    const float* master;
    const fsdpshard_segment* segs;
    uint16_t* out;
    int64_t n;
    int64_t block_vecs;
    int32_t n_segs;
    int32_t out_shift;
};

// ------------------------------------------------------------------------------------------------
// Small helpers.

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16 bits, round to nearest even; NaN stays NaN, made quiet, sign kept.
__device__ __forceinline__ uint32_t to_bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x40u;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? quiet : rounded;
}

// Accumulate one 8-element bf16 vector into g (each element added after the previous ranks').
__device__ __forceinline__ void accumulate(float (&g)[kVec], const uint4 raw) {
    g[0] = g[0] + bf16_lo(raw.x);
    g[1] = g[1] + bf16_hi(raw.x);
    g[2] = g[2] + bf16_lo(raw.y);
    g[3] = g[3] + bf16_hi(raw.y);
    g[4] = g[4] + bf16_lo(raw.z);
    g[5] = g[5] + bf16_hi(raw.z);
    g[6] = g[6] + bf16_lo(raw.w);
    g[7] = g[7] + bf16_hi(raw.w);
}

__device__ __forceinline__ uint4 ld_u4(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ float4 ld_f4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ void st_f4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }

// Partial vector (slice tail): element-wise loads of the first `cnt` elements, zeros after.
__device__ __forceinline__ uint4 ld_u4_partial(const uint16_t* p, int cnt) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int e = 0; e < cnt; ++e) w[e >> 1] |= static_cast<uint32_t>(p[e]) << (16 * (e & 1));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ void load8(const float* p, bool full, int cnt, float (&x)[kVec]) {
    if (full) {
        const float4 a = ld_f4(p), b = ld_f4(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) x[e] = (e < cnt) ? p[e] : 0.0f;
    }
}

__device__ __forceinline__ void store8(float* p, bool full, int cnt, const float (&x)[kVec]) {
    if (full) {
        st_f4(p, make_float4(x[0], x[1], x[2], x[3]));
        st_f4(p + 4, make_float4(x[4], x[5], x[6], x[7]));
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (e < cnt) p[e] = x[e];
    }
}

// ------------------------------------------------------------------------------------------------
// Segment cursor: wave-uniform view of the segment that holds a position.

struct SegCursor {
    const fsdpshard_segment* segs;
    int32_t n_segs;
    int32_t idx;
    int64_t end;      // one past the last element of segment idx
    uint32_t flags;

    __device__ void load(int32_t i) {
        idx = i;
        const int64_t b = segs[i].shard_begin;
        end = b + segs[i].length;
        flags = segs[i].flags;
    }

    // Position the cursor on the last segment that begins at or before `pos` (binary search).
    __device__ void init(const fsdpshard_segment* s, int32_t ns, int64_t pos) {
        segs = s;
        n_segs = ns;
        if (ns <= 0) {
            idx = 0;
            end = INT64_MAX;
            flags = FSDPSHARD_SEG_WEIGHT_DECAY;
            return;
        }
        int32_t a = 0, b = ns;
        while (b - a > 1) {
            const int32_t mid = a + ((b - a) >> 1);
            if (segs[mid].shard_begin <= pos) a = mid; else b = mid;
        }
        load(a);
    }

    // Move forward until segment idx ends after `pos` (or idx is the last segment).
    __device__ void seek(int64_t pos) {
        while (end <= pos && idx + 1 < n_segs) load(idx + 1);
    }
};

// Flags of the 8 elements starting at e0.  Uniform when the group, which ends at g1, sits in the
// cursor's segment; otherwise each lane scans forward from the cursor.
__device__ __forceinline__ void element_flags(const SegCursor& cur, int64_t g1, int64_t e0,
                                              uint32_t (&fl)[kVec]) {
    if (g1 <= cur.end) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) fl[e] = cur.flags;
        return;
    }
    int32_t t = cur.idx;
    int64_t end = cur.end;
    uint32_t f = cur.flags;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        const int64_t pos = e0 + e;
        while (end <= pos && t + 1 < cur.n_segs) {
            ++t;
            end = cur.segs[t].shard_begin + cur.segs[t].length;
            f = cur.segs[t].flags;
        }
        fl[e] = f;
    }
}

// ------------------------------------------------------------------------------------------------
// bf16 output path shared by the fused step and the standalone unflatten.
//
// `w` holds this lane's 8 results (element 2k in the low half of w[k]).  Element i of the slice
// goes to out[i].  With shift s = 0 every lane's vector is 16-byte aligned.  With s in 1..7 the
// aligned 16-byte vector starting at element 8j+s holds this lane's elements s..7 and the next
// lane's elements 0..s-1; lane j stores it when the next lane holds a complete vector in the same
// group, and every element no aligned store covers is written with a 2-byte store.
//   group_valid: this lane holds a vector of the slice;  cnt: how many of its elements are real.
//   next_ok:     the next lane holds elements 0..s-1 of its vector (and is in this group).
//   prev_ok:     the previous lane stored the aligned vector that covers our elements 0..s-1.
template <int S>
__device__ __forceinline__ uint4 rephase(const uint32_t (&w)[4], const uint32_t (&x)[4]) {
    constexpr int Q = S >> 1;
    uint32_t all[8] = {w[0], w[1], w[2], w[3], x[0], x[1], x[2], x[3]};
    uint32_t r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if constexpr ((S & 1) == 0) r[k] = all[Q + k];
        else r[k] = __builtin_amdgcn_alignbit(all[Q + k + 1], all[Q + k], 16);
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ void store_bf16_vec(uint16_t* out, int64_t e0, int shift,
                                               const uint32_t (&w)[4], bool valid, int cnt,
                                               bool next_ok, bool prev_ok) {
    // Every lane takes part in the permutes (inactive lanes would read back zeros).
    uint32_t x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = __shfl_down(w[k], 1, kWave);
    if (!valid) return;

    uint32_t narrow = 0;  // bit e: write element e with a 2-byte store
    if (shift == 0) {
        if (cnt == kVec) *reinterpret_cast<uint4*>(out + e0) = make_uint4(w[0], w[1], w[2], w[3]);
        else narrow = (1u << cnt) - 1u;
    } else {
        const uint32_t lo_mask = (1u << shift) - 1u;
        const uint32_t real_mask = (cnt >= kVec) ? 0xFFu : ((1u << cnt) - 1u);
        if (next_ok) {
            uint4 r;
            switch (shift) {
                case 1: r = rephase<1>(w, x); break;
                case 2: r = rephase<2>(w, x); break;
                case 3: r = rephase<3>(w, x); break;
                case 4: r = rephase<4>(w, x); break;
                case 5: r = rephase<5>(w, x); break;
                case 6: r = rephase<6>(w, x); break;
                default: r = rephase<7>(w, x); break;
            }
            *reinterpret_cast<uint4*>(out + e0 + shift) = r;
        } else {
            narrow |= ~lo_mask & real_mask;
        }
        if (!prev_ok) narrow |= lo_mask & real_mask;
    }
    if (narrow) {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (narrow & (1u << e))
                out[e0 + e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
    }
}

// ------------------------------------------------------------------------------------------------
// The fused step.

// Contributions of one vector, summed in rank order from +0.  Every HBM load of the vector is
// issued before the first add: the compile-time fan-ins load all F vectors at once, the generic
// path loads four at a time.
template <int F>
__device__ __forceinline__ void load_contribs(const StepParams& p, int64_t e0, bool full, int cnt,
                                              uint4 (&raw)[F > 0 ? F : 1]) {
    if constexpr (F > 0) {
#pragma unroll
        for (int r = 0; r < F; ++r)
            raw[r] = full ? ld_u4(p.contrib[r] + e0) : ld_u4_partial(p.contrib[r] + e0, cnt);
    }
}

template <int F>
__device__ __forceinline__ void sum_contribs(const StepParams& p, int64_t e0, bool full, int cnt,
                                             const uint4 (&raw)[F > 0 ? F : 1], float (&g)[kVec]) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) g[e] = 0.0f;
    if constexpr (F > 0) {
#pragma unroll
        for (int r = 0; r < F; ++r) accumulate(g, raw[r]);
    } else {
        const int fan_in = p.fan_in;
        for (int r0 = 0; r0 < fan_in; r0 += 4) {
            uint4 q4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (r0 + q < fan_in) {
                    const uint16_t* src = p.contrib[r0 + q] + e0;
                    q4[q] = full ? ld_u4(src) : ld_u4_partial(src, cnt);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (r0 + q < fan_in) accumulate(g, q4[q]);
        }
    }
}

// One 512-element group of the fused step.  TAIL = false is the interior case (all 64 vectors of
// the group are complete slice elements) and compiles to straight-line loads; TAIL = true handles
// the last, partial group of a work-group's chunk with per-lane bounds.
template <int F, bool OUT, bool TAIL>
__device__ __forceinline__ void step_group(const StepParams& p, const SegCursor& cur, int64_t vec,
                                           int64_t group_end_vec, int lane) {
    const int64_t n = p.n;
    const int64_t e0 = vec * kVec;
    const bool valid = !TAIL || vec < group_end_vec;
    const int cnt =
        !TAIL ? kVec : (valid ? static_cast<int>((n - e0) < kVec ? (n - e0) : kVec) : 0);
    const bool full = !TAIL || cnt == kVec;

    float g[kVec], th[kVec], mm[kVec], vv[kVec];
    uint4 raw[F > 0 ? F : 1];
    if (valid) {
        load_contribs<F>(p, e0, full, cnt, raw);
        load8(p.master + e0, full, cnt, th);
        load8(p.m + e0, full, cnt, mm);
        load8(p.v + e0, full, cnt, vv);
        sum_contribs<F>(p, e0, full, cnt, raw, g);
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = th[e] = mm[e] = vv[e] = 0.0f;
    }

    uint32_t fl[kVec];
    int64_t g1 = group_end_vec * kVec;
    if (g1 > n) g1 = n;
    element_flags(cur, g1, e0, fl);

#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        const float gs = g[e] * p.scale;
        const float m1 = p.b1 * mm[e] + p.c1 * gs;
        const float v1 = p.b2 * vv[e] + p.c2 * (gs * gs);
        const float mh = m1 / p.bc1;
        const float vh = v1 / p.bc2;
        const float den = sqrtf(vh) + p.eps;
        const float decayed = (fl[e] & FSDPSHARD_SEG_WEIGHT_DECAY) ? th[e] * p.dec : th[e];
        const float t1 = decayed - p.lr * (mh / den);
        const bool real = (fl[e] & FSDPSHARD_SEG_PADDING) == 0u;
        th[e] = real ? t1 : th[e];
        mm[e] = real ? m1 : mm[e];
        vv[e] = real ? v1 : vv[e];
    }

    if (valid) {
        store8(p.master + e0, full, cnt, th);
        store8(p.m + e0, full, cnt, mm);
        store8(p.v + e0, full, cnt, vv);
    }

    if constexpr (OUT) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bool r0 = (fl[2 * k] & FSDPSHARD_SEG_PADDING) == 0u;
            const bool r1 = (fl[2 * k + 1] & FSDPSHARD_SEG_PADDING) == 0u;
            const uint32_t lo16 = r0 ? to_bf16_bits(th[2 * k]) : 0u;
            const uint32_t hi16 = r1 ? to_bf16_bits(th[2 * k + 1]) : 0u;
            w[k] = lo16 | (hi16 << 16);
        }
        const int s = p.out_shift;
        const bool next_ok = (lane < kWave - 1) && (vec + 1 < group_end_vec) &&
                             ((vec + 1) * kVec + s <= n);
        const bool prev_ok = (lane > 0) && (e0 + s <= n);
        store_bf16_vec(p.out, e0, s, w, valid, cnt, next_ok, prev_ok);
    }
}

template <int F, bool OUT>
__global__ __launch_bounds__(kBlock) void fused_step_kernel(StepParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t nvec = (p.n + kVec - 1) / kVec;
    const int64_t blk0 = static_cast<int64_t>(blockIdx.x) * p.block_vecs;
    int64_t blk1 = blk0 + p.block_vecs;
    if (blk1 > nvec) blk1 = nvec;

    SegCursor cur;
    cur.init(p.segs, p.n_segs, (blk0 + static_cast<int64_t>(wave) * kWave) * kVec);
    for (int64_t base = blk0 + static_cast<int64_t>(wave) * kWave; base < blk1;
         base += kWavesPerBlock * kWave) {
        int64_t gend = base + kWave;
        if (gend > blk1) gend = blk1;
        cur.seek(base * kVec);
        if (gend == base + kWave && gend * kVec <= p.n)
            step_group<F, OUT, false>(p, cur, base + lane, gend, lane);
        else
            step_group<F, OUT, true>(p, cur, base + lane, gend, lane);
    }
}

// ------------------------------------------------------------------------------------------------
// Standalone reduce and unflatten.

__global__ __launch_bounds__(kBlock) void reduce_kernel(ReduceParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t nvec = (p.n + kVec - 1) / kVec;
    const int64_t blk0 = static_cast<int64_t>(blockIdx.x) * p.block_vecs;
    int64_t blk1 = blk0 + p.block_vecs;
    if (blk1 > nvec) blk1 = nvec;
    for (int64_t base = blk0 + static_cast<int64_t>(wave) * kWave; base < blk1;
         base += kWavesPerBlock * kWave) {
        const int64_t vec = base + lane;
        if (vec >= blk1) continue;
        const int64_t e0 = vec * kVec;
        const int cnt = static_cast<int>((p.n - e0) < kVec ? (p.n - e0) : kVec);
        const bool full = cnt == kVec;
        float g[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = 0.0f;
        for (int r0 = 0; r0 < p.fan_in; r0 += 4) {
            uint4 raw[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (r0 + q < p.fan_in) {
                    const uint16_t* src = p.contrib[r0 + q] + e0;
                    raw[q] = full ? ld_u4(src) : ld_u4_partial(src, cnt);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (r0 + q < p.fan_in) accumulate(g, raw[q]);
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = g[e] * p.scale;
        store8(p.out + e0, full, cnt, g);
    }
}

__global__ __launch_bounds__(kBlock) void unflatten_kernel(UnflattenParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t nvec = (p.n + kVec - 1) / kVec;
    const int64_t blk0 = static_cast<int64_t>(blockIdx.x) * p.block_vecs;
    int64_t blk1 = blk0 + p.block_vecs;
    if (blk1 > nvec) blk1 = nvec;

    SegCursor cur;
    cur.init(p.segs, p.n_segs, (blk0 + static_cast<int64_t>(wave) * kWave) * kVec);
    for (int64_t base = blk0 + static_cast<int64_t>(wave) * kWave; base < blk1;
         base += kWavesPerBlock * kWave) {
        int64_t gend = base + kWave;
        if (gend > blk1) gend = blk1;
        cur.seek(base * kVec);
        const int64_t vec = base + lane;
        const int64_t e0 = vec * kVec;
        const bool valid = vec < gend;
        const int cnt = valid ? static_cast<int>((p.n - e0) < kVec ? (p.n - e0) : kVec) : 0;
        float th[kVec];
        if (valid) load8(p.master + e0, cnt == kVec, cnt, th);
        else {
#pragma unroll
            for (int e = 0; e < kVec; ++e) th[e] = 0.0f;
        }
        uint32_t fl[kVec];
        int64_t g1 = gend * kVec;
        if (g1 > p.n) g1 = p.n;
        element_flags(cur, g1, e0, fl);
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo16 = (fl[2 * k] & FSDPSHARD_SEG_PADDING) ? 0u : to_bf16_bits(th[2 * k]);
            const uint32_t hi16 =
                (fl[2 * k + 1] & FSDPSHARD_SEG_PADDING) ? 0u : to_bf16_bits(th[2 * k + 1]);
            w[k] = lo16 | (hi16 << 16);
        }
        const int s = p.out_shift;
        const bool next_ok = (lane < kWave - 1) && (vec + 1 < gend) && ((vec + 1) * kVec + s <= p.n);
        const bool prev_ok = (lane > 0) && (e0 + s <= p.n);
        store_bf16_vec(p.out, e0, s, w, valid, cnt, next_ok, prev_ok);
    }
}

__global__ __launch_bounds__(kBlock) void stream_copy_kernel(const uint4* __restrict__ src,
                                                             uint4* __restrict__ dst,
                                                             int64_t nvec) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < nvec; i += stride)
        dst[i] = src[i];
}

// ------------------------------------------------------------------------------------------------
// Host-side launch helpers.

std::atomic<int> g_cu_count[kMaxDevices];
std::atomic<int> g_blocks_per_cu{kDefaultBlocksPerCu};

int cu_count(int* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FSDPSHARD_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *out = cached;
            return FSDPSHARD_OK;
        }
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return FSDPSHARD_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
    *out = cus;
    return FSDPSHARD_OK;
}

// Grid for n elements: a few resident work-groups per CU, each owning an equal contiguous
// chunk whose size is a multiple of one group per wave.
int plan_grid(int64_t n, int64_t* block_vecs, unsigned* blocks) {
    int cus = 0;
    const int rc = cu_count(&cus);
    if (rc != FSDPSHARD_OK) return rc;
    const int64_t nvec = (n + kVec - 1) / kVec;
    const int64_t unit = static_cast<int64_t>(kWave) * kWavesPerBlock;  // vectors per block round
    const int64_t max_blocks = static_cast<int64_t>(cus) * g_blocks_per_cu.load();
    int64_t want = (nvec + unit - 1) / unit;
    if (want > max_blocks) want = max_blocks;
    if (want < 1) want = 1;
    int64_t per = (nvec + want - 1) / want;
    per = (per + unit - 1) / unit * unit;
    *block_vecs = per;
    *blocks = static_cast<unsigned>((nvec + per - 1) / per);
    return FSDPSHARD_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + static_cast<uintptr_t>(bbytes) && y < x + static_cast<uintptr_t>(abytes);
}

int launch(const void* kernel, unsigned blocks, void* params, void* stream) {
    void* args[] = {params};
    const hipError_t e = hipLaunchKernel(kernel, dim3(blocks), dim3(kBlock), args, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FSDPSHARD_OK : FSDPSHARD_ERR_HIP;
}

template <int F>
const void* step_kernel(bool out) {
    return out ? reinterpret_cast<const void*>(&fused_step_kernel<F, true>)
               : reinterpret_cast<const void*>(&fused_step_kernel<F, false>);
}

const void* pick_step_kernel(int fan_in, bool out) {
    switch (fan_in) {
        case 1: return step_kernel<1>(out);
        case 2: return step_kernel<2>(out);
        case 4: return step_kernel<4>(out);
        case 8: return step_kernel<8>(out);
        default: return step_kernel<0>(out);
    }
}

// First slice element whose bf16 destination starts a 16-byte vector.
int out_shift_of(const uint16_t* out) {
    const unsigned phase = static_cast<unsigned>(reinterpret_cast<uintptr_t>(out) & 15u) / 2u;
    return static_cast<int>((kVec - phase) % kVec);
}

int check_contribs(const uint16_t* const* contribs, int32_t fan_in, int64_t n) {
    if (contribs == nullptr || fan_in < 1) return FSDPSHARD_ERR_INVALID_ARG;
    if (fan_in > FSDPSHARD_MAX_FAN_IN) return FSDPSHARD_ERR_UNSUPPORTED;
    for (int r = 0; r < fan_in; ++r) {
        if (contribs[r] == nullptr) return FSDPSHARD_ERR_INVALID_ARG;
        if (!aligned16(contribs[r])) return FSDPSHARD_ERR_ALIGNMENT;
    }
    (void)n;
    return FSDPSHARD_OK;
}

bool is_finite(double x) { return std::isfinite(x); }

}  // namespace

// ------------------------------------------------------------------------------------------------
// C ABI.

extern "C" int adamw_shard_step(float* master, float* m, float* v,
                                const uint16_t* const* contribs, int32_t fan_in, int64_t n,
                                const fsdpshard_segment* segs, int32_t n_segments,
                                const fsdpshard_adamw* hp, uint16_t* flat_bf16,
                                int64_t flat_index0, int64_t lo, void* stream) {
    if (master == nullptr || m == nullptr || v == nullptr || hp == nullptr || n < 0 ||
        n_segments < 0 || (n_segments > 0 && segs == nullptr) || lo < 0)
        return FSDPSHARD_ERR_INVALID_ARG;
    int rc = check_contribs(contribs, fan_in, n);
    if (rc != FSDPSHARD_OK) return rc;
    if (hp->step < 1 || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
        !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !is_finite(hp->lr) || !is_finite(hp->eps) ||
        !is_finite(hp->weight_decay) || !is_finite(hp->grad_scale))
        return FSDPSHARD_ERR_INVALID_ARG;
    if (!aligned16(master) || !aligned16(m) || !aligned16(v)) return FSDPSHARD_ERR_ALIGNMENT;
    if (segs != nullptr && (reinterpret_cast<uintptr_t>(segs) & 7u) != 0)
        return FSDPSHARD_ERR_ALIGNMENT;
    uint16_t* out = nullptr;
    if (flat_bf16 != nullptr) {
        if (flat_index0 > lo) return FSDPSHARD_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(flat_bf16) & 1u) != 0) return FSDPSHARD_ERR_ALIGNMENT;
        out = flat_bf16 + (lo - flat_index0);
    }
    if (n > INT64_MAX / 4) return FSDPSHARD_ERR_OVERFLOW;
    // Written buffers must not overlap each other or the inputs.
    const int64_t fb = n * 4, hb = n * 2;
    const void* wr[4] = {master, m, v, out};
    const int64_t wb[4] = {fb, fb, fb, hb};
    for (int i = 0; i < 4; ++i) {
        if (wr[i] == nullptr || n == 0) continue;
        for (int j = i + 1; j < 4; ++j)
            if (wr[j] != nullptr && overlaps(wr[i], wb[i], wr[j], wb[j]))
                return FSDPSHARD_ERR_INVALID_ARG;
        for (int r = 0; r < fan_in; ++r)
            if (overlaps(wr[i], wb[i], contribs[r], hb)) return FSDPSHARD_ERR_INVALID_ARG;
    }
    if (n == 0) return FSDPSHARD_OK;

    StepParams p;
    p.master = master;
    p.m = m;
    p.v = v;
    for (int r = 0; r < FSDPSHARD_MAX_FAN_IN; ++r) p.contrib[r] = r < fan_in ? contribs[r] : nullptr;
    p.segs = segs;
    p.out = out;
    p.n = n;
    p.n_segs = segs == nullptr ? 0 : n_segments;
    p.fan_in = fan_in;
    p.out_shift = out == nullptr ? 0 : out_shift_of(out);
    const double t = static_cast<double>(hp->step);
    p.b1 = static_cast<float>(hp->beta1);
    p.b2 = static_cast<float>(hp->beta2);
    p.c1 = static_cast<float>(1.0 - hp->beta1);
    p.c2 = static_cast<float>(1.0 - hp->beta2);
    p.bc1 = static_cast<float>(1.0 - std::pow(hp->beta1, t));
    p.bc2 = static_cast<float>(1.0 - std::pow(hp->beta2, t));
    p.eps = static_cast<float>(hp->eps);
    p.lr = static_cast<float>(hp->lr);
    p.dec = static_cast<float>(1.0 - hp->lr * hp->weight_decay);
    p.scale = static_cast<float>(hp->grad_scale);

    unsigned blocks = 0;
    rc = plan_grid(n, &p.block_vecs, &blocks);
    if (rc != FSDPSHARD_OK) return rc;
    return launch(pick_step_kernel(fan_in, out != nullptr), blocks, &p, stream);
}

extern "C" int reduce_shard(const uint16_t* const* contribs, int32_t fan_in, int64_t n,
                            float scale, float* out, void* stream) {
    if (out == nullptr || n < 0) return FSDPSHARD_ERR_INVALID_ARG;
    int rc = check_contribs(contribs, fan_in, n);
    if (rc != FSDPSHARD_OK) return rc;
    if (!aligned16(out)) return FSDPSHARD_ERR_ALIGNMENT;
    if (n > INT64_MAX / 4) return FSDPSHARD_ERR_OVERFLOW;
    for (int r = 0; r < fan_in && n > 0; ++r)
        if (overlaps(out, n * 4, contribs[r], n * 2)) return FSDPSHARD_ERR_INVALID_ARG;
    if (n == 0) return FSDPSHARD_OK;
    ReduceParams p;
    for (int r = 0; r < FSDPSHARD_MAX_FAN_IN; ++r) p.contrib[r] = r < fan_in ? contribs[r] : nullptr;
    p.out = out;
    p.n = n;
    p.fan_in = fan_in;
    p.scale = scale;
    unsigned blocks = 0;
    rc = plan_grid(n, &p.block_vecs, &blocks);
    if (rc != FSDPSHARD_OK) return rc;
    return launch(reinterpret_cast<const void*>(&reduce_kernel), blocks, &p, stream);
}

extern "C" int unflatten_bf16(const float* master, int64_t n, const fsdpshard_segment* segs,
                              int32_t n_segments, uint16_t* flat_bf16, int64_t flat_index0,
                              int64_t lo, void* stream) {
    if (master == nullptr || flat_bf16 == nullptr || n < 0 || n_segments < 0 ||
        (n_segments > 0 && segs == nullptr) || lo < 0 || flat_index0 > lo)
        return FSDPSHARD_ERR_INVALID_ARG;
    if (!aligned16(master) || (reinterpret_cast<uintptr_t>(flat_bf16) & 1u) != 0)
        return FSDPSHARD_ERR_ALIGNMENT;
    if (segs != nullptr && (reinterpret_cast<uintptr_t>(segs) & 7u) != 0)
        return FSDPSHARD_ERR_ALIGNMENT;
    if (n > INT64_MAX / 4) return FSDPSHARD_ERR_OVERFLOW;
    uint16_t* out = flat_bf16 + (lo - flat_index0);
    if (n > 0 && overlaps(out, n * 2, master, n * 4)) return FSDPSHARD_ERR_INVALID_ARG;
    if (n == 0) return FSDPSHARD_OK;
    UnflattenParams p;
    p.master = master;
    p.segs = segs;
    p.out = out;
    p.n = n;
    p.n_segs = segs == nullptr ? 0 : n_segments;
    p.out_shift = out_shift_of(out);
    unsigned blocks = 0;
    int rc = plan_grid(n, &p.block_vecs, &blocks);
    if (rc != FSDPSHARD_OK) return rc;
    return launch(reinterpret_cast<const void*>(&unflatten_kernel), blocks, &p, stream);
}

extern "C" int fsdpshard_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (src == nullptr || dst == nullptr || bytes < 0 || (bytes & 15) != 0)
        return FSDPSHARD_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(dst)) return FSDPSHARD_ERR_ALIGNMENT;
    if (bytes > 0 && overlaps(src, bytes, dst, bytes)) return FSDPSHARD_ERR_INVALID_ARG;
    if (bytes == 0) return FSDPSHARD_OK;
    int cus = 0;
    const int rc = cu_count(&cus);
    if (rc != FSDPSHARD_OK) return rc;
    const int64_t nvec = bytes / 16;
    int64_t blocks = static_cast<int64_t>(cus) * 8;
    const int64_t need = (nvec + kBlock - 1) / kBlock;
    if (blocks > need) blocks = need;
    void* args[3];
    const uint4* s = static_cast<const uint4*>(src);
    uint4* d = static_cast<uint4*>(dst);
    int64_t nv = nvec;
    args[0] = &s;
    args[1] = &d;
    args[2] = &nv;
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&stream_copy_kernel),
                                         dim3(static_cast<unsigned>(blocks)), dim3(kBlock), args,
                                         0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FSDPSHARD_OK : FSDPSHARD_ERR_HIP;
}

extern "C" int fsdpshard_set_blocks_per_cu(int blocks_per_cu) {
    if (blocks_per_cu < 0 || blocks_per_cu > 16) return -1;
    const int v = blocks_per_cu == 0 ? kDefaultBlocksPerCu : blocks_per_cu;
    return g_blocks_per_cu.exchange(v);
}
