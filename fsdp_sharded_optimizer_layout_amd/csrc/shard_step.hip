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
//   * One 512-element group per wave: each wave issues every HBM load of its group before the
//     first arithmetic instruction; the grid has one work-group of 4 waves per 4 groups
//     (hundreds of thousands for a 7B-model slice), enough to keep all 256 CUs fed.  Work-groups
//     map to tiles so that each of the 8 XCDs streams runs of consecutive tiles (tile_index).
//     Gradient loads and all full-vector stores carry the non-temporal hint (single-use
//     streams); the state loads do not.
//   * Contributions are reduced in registers in rank order 0..F-1 from +0 (fixed order, so the
//     result is deterministic and matches a sequential float32 sum bit for bit).  They come as F
//     arrays, or interleaved per 512-element block in one array (grad_src), which the step then
//     streams as a single gradient array.
//   * Segment flags (padding, weight decay) come from a per-wave cursor over the segment table:
//     one binary search when a wave starts (issued after the tile's loads, so it overlaps them),
//     a compare per group after that, and a per-element scan only in groups that hold an edge.
//   * The bf16 destination may start at any 2-byte phase inside a 16-byte vector (a slice starts
//     wherever floor(kP/N) falls).  The state streams stay aligned; the bf16 result is re-phased
//     across lanes (lane permutes, and LDS between the waves of a work-group) so that every
//     store inside a work-group is an aligned 16-byte vector and each wave writes whole 64-byte
//     lines; only the elements at a work-group's two ends, whose lines it shares with its
//     neighbours, go out as 2-byte stores.
//   * Resident work-groups per CU are capped (2 or 3, by gradient source and launch size) by
//     reserving LDS the kernel never touches: fewer concurrent streams suit the HBM.
// Arithmetic is IEEE float32 with no contraction (the library is built with -ffp-contract=off),
// correctly rounded division and square root, denormals kept.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "fsdpshard.h"
#include "stream_common.h"

namespace {

using namespace fsdpshard_detail;

// ------------------------------------------------------------------------------------------------
// Kernel parameter blocks (passed by value in the kernel-argument segment).

struct StepParams {
    float* master;
    float* m;
    float* v;
    const uint16_t* contrib[FSDPSHARD_MAX_FAN_IN];
    const fsdpshard_segment* segs;
    const float* grad32;     // fp32 gradient shard (fan-in -1 kernels), else null
    uint16_t* out;           // destination of slice element 0 (flat index lo), or null
    const double* sumsq;     // global sum of squares of the gradient when clipping, else null
    double max_norm;         // clip threshold (> 0 when clipping)
    double grad_scale;       // grad_scale in float64 (the clipped scale is formed from it)
    int64_t n;               // elements in the slice
    int32_t n_segs;
    int32_t fan_in;
    int32_t out_shift;       // first slice element whose destination is 16-byte aligned (0..7)
    int32_t out_line_vecs;   // with out_shift: element 8 * out_line_vecs + out_shift is the first
                             // whose destination starts a 64-byte line (0..3)
    float b1, b2, c1, c2, bc1, bc2, eps, lr, dec, scale;
};

struct ReduceParams {
    const uint16_t* contrib[FSDPSHARD_MAX_FAN_IN];
    float* out;              // receives scale * sum (plus its old value when accumulating)
    int64_t n;
    int32_t fan_in;
    float scale;
};

struct SumsqParams {
    const uint16_t* contrib[FSDPSHARD_MAX_FAN_IN];
    const float* grad32;     // fp32 gradient shard when fan_in == 0
    const fsdpshard_segment* segs;
    double* partials;        // one float64 per work-group
    double* result;
    int64_t n;
    int64_t groups_per_wave;
    int32_t n_segs;
    int32_t fan_in;
    int32_t n_partials;
    float scale;
};

struct UnflattenParams {
    const float* master;
    const fsdpshard_segment* segs;
    uint16_t* out;
    int64_t n;
    int32_t n_segs;
    int32_t out_shift;
};

// ------------------------------------------------------------------------------------------------
// Small helpers.

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

// Partial vector (slice tail): element-wise loads of the first `cnt` elements, zeros after.
__device__ __forceinline__ uint4 ld_u4_partial(const uint16_t* p, int cnt) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int e = 0; e < cnt; ++e) w[e >> 1] |= static_cast<uint32_t>(p[e]) << (16 * (e & 1));
    return make_uint4(w[0], w[1], w[2], w[3]);
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

    // Position the cursor on the last segment that begins at or before `pos`.  An 8-ary search:
    // each level issues its seven probes together (indices clamped into [a, b), so every load is
    // in range), then narrows [a, b) to one eighth; the first segment begins at 0 <= pos.  The
    // probes are wave-uniform scalar loads, so the levels overlap the group's data loads.  Against
    // a binary search (one dependent probe per level) the step on a 237-segment slice ran
    // 1.0-1.5 % faster (measured on MI355X, three boxes, 8 alternating rounds, cache flushed),
    // and the 7B- and 70B-shaped slices were unchanged.
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
            const int32_t step = (b - a - 1) / 8 + 1;             // ceil((b - a) / 8), no overflow
            int32_t probe[7];
            int64_t begin[7];
#pragma unroll
            for (int j = 0; j < 7; ++j) {
                const int64_t m = static_cast<int64_t>(a) + static_cast<int64_t>(j + 1) * step;
                probe[j] = static_cast<int32_t>(m < b - 1 ? m : b - 1);
                begin[j] = segs[probe[j]].shard_begin;
            }
            __builtin_amdgcn_sched_barrier(0);   // all seven loads before the first compare
            int32_t na = a;
#pragma unroll
            for (int j = 0; j < 7; ++j)
                if (begin[j] <= pos) na = max(na, probe[j]);
            b = step < b - na ? na + step : b;
            a = na;
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

// The next lane's 8 packed words (every lane must take part in the permutes: inactive lanes
// would read back zeros).  The last lane of the wave gets its own words back.
__device__ __forceinline__ void next_lane_words(const uint32_t (&w)[4], uint32_t (&x)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = __shfl_down(w[k], 1, kWave);
}

// Stores this lane's part of the bf16 slice given the next lane's words x (see above).
__device__ __forceinline__ void store_bf16_words(uint16_t* out, int64_t e0, int shift,
                                                 const uint32_t (&w)[4], const uint32_t (&x)[4],
                                                 bool valid, int cnt, bool next_ok, bool prev_ok) {
    if (!valid) return;

    uint32_t narrow = 0;  // bit e: write element e with a 2-byte store
    if (shift == 0) {
        if (cnt == kVec) st_u4_nt(out + e0, make_uint4(w[0], w[1], w[2], w[3]));
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
            st_u4_nt(out + e0 + shift, r);
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

__device__ __forceinline__ void store_bf16_vec(uint16_t* out, int64_t e0, int shift,
                                               const uint32_t (&w)[4], bool valid, int cnt,
                                               bool next_ok, bool prev_ok) {
    uint32_t x[4];
    next_lane_words(w, x);
    store_bf16_words(out, e0, shift, w, x, valid, cnt, next_ok, prev_ok);
}

// LDS-only work-group barrier: this wave's LDS writes are complete before it waits, and no LDS
// read after it is issued before every wave has arrived.  (Global stores in flight are not
// waited for, unlike __syncthreads.)
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The aligned 16-byte vector made of x's elements s..7 followed by y's elements 0..s-1.
__device__ __forceinline__ uint4 rephase_rt(const uint32_t (&x)[4], const uint32_t (&y)[4], int s) {
    switch (s) {
        case 0: return make_uint4(x[0], x[1], x[2], x[3]);
        case 1: return rephase<1>(x, y);
        case 2: return rephase<2>(x, y);
        case 3: return rephase<3>(x, y);
        case 4: return rephase<4>(x, y);
        case 5: return rephase<5>(x, y);
        case 6: return rephase<6>(x, y);
        default: return rephase<7>(x, y);
    }
}

// bf16 stores of one whole 512-element group whose destination does not start a 64-byte line.
// S = 8q + s (q = out_line_vecs, s = out_shift) is the first slice element whose destination
// does.  U_i is the aligned 16-byte destination vector of group elements 8i + s .. 8i + s + 7
// (lane i's elements s..7, lane i + 1's elements 0..s-1).  Lane j stores U_{j+q}, so a wave
// writes the 16 whole 64-byte lines that begin at its group element S, and no line inside a
// work-group has two writing waves.  U_63 (when s != 0) and U_64..U_{63+q} hold the next
// wave's first elements; with the exchange (`exch`: the work-group's four groups are whole)
// their words come from the next wave's lanes 0..q through LDS, and the previous wave likewise
// stores this wave's U_0..U_{q-1} and elements 0..s-1.  A wave without an exchanging neighbour
// on a side stores that side itself: U_0..U_{q-1} from lanes 0..q-1, and 2-byte stores for
// what none of its aligned vectors covers.  Group element e goes to out[8 * gb + e].
__device__ __forceinline__ void store_bf16_lines(uint16_t* out, int s, int q, int64_t gb, int lane,
                                                 int wave, bool exch, const uint32_t (&w)[4]) {
    __shared__ uint4 head_words[kWavesPerBlock][4];
    const bool prev_ex = exch && wave > 0;
    const bool next_ex = exch && wave < kWavesPerBlock - 1;
    const int a = lane + q;                    // this lane stores U_a
    uint32_t x[4], y[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {              // every lane takes part in the permutes
        x[k] = __shfl(w[k], a & (kWave - 1), kWave);
        y[k] = __shfl(w[k], (a + 1) & (kWave - 1), kWave);
    }
    if (exch) {
        if (lane <= q) head_words[wave][lane] = make_uint4(w[0], w[1], w[2], w[3]);
        lds_barrier();
        if (next_ex && a >= kWave) {
            const uint4 t = head_words[wave + 1][a - kWave];
            x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
        }
        if (next_ex && a + 1 >= kWave) {
            const uint4 t = head_words[wave + 1][a + 1 - kWave];
            y[0] = t.x; y[1] = t.y; y[2] = t.z; y[3] = t.w;
        }
    }
    const bool own = a + 1 < kWave || (a + 1 == kWave && s == 0);   // U_a from this wave alone
    if (own || next_ex) st_u4_nt(out + (gb + a) * kVec + s, rephase_rt(x, y, s));
    if (!prev_ex) {
        if (q > 0) {                           // wave-uniform: lanes 0..q-1 store U_0..U_{q-1}
            uint32_t z[4];
            next_lane_words(w, z);
            if (lane < q) st_u4_nt(out + (gb + lane) * kVec + s, rephase_rt(w, z, s));
        }
        if (lane == 0) {
#pragma unroll
            for (int e = 0; e < kVec; ++e)
                if (e < s) out[gb * kVec + e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
        }
    }
    if (!next_ex && lane == kWave - 1 && s != 0) {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (e >= s)
                out[(gb + lane) * kVec + e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
    }
}

// ------------------------------------------------------------------------------------------------
// The fused step.

// Gradient sources.  F >= 1: F bf16 contributions, a compile-time count; F == 0: run-time fan-in
// (p.fan_in); F == -1: one fp32 gradient shard (accumulated over micro-batches).
//
// Reduced gradient of one vector, before the scale: the contributions summed in rank order from
// +0.  Every HBM load is issued before the first add (the run-time fan-in loads four at a time).
//
// Where rank r's vector at slice element e0 lives: its own array (p.contrib[r]), or with GIL the
// interleaved buffer at p.contrib[0], whose block b holds every rank's elements
// [512b, 512b + 512) one rank after another: rank r's element i at
// ((i / 512) * fan_in + r) * 512 + i % 512.
template <int F, bool GIL, class Params>
__device__ __forceinline__ const uint16_t* grad_src(const Params& p, int r, int64_t e0) {
    if constexpr (GIL) {
        const uint64_t u = static_cast<uint64_t>(e0);
        const int64_t fan_in = F > 0 ? F : p.fan_in;
        return p.contrib[0] +
               (static_cast<int64_t>(u / kStateBlock) * fan_in + r) * kStateBlock +
               static_cast<int64_t>(u % kStateBlock);
    } else {
        return p.contrib[r] + e0;
    }
}

template <int F, bool GIL = false>
__device__ __forceinline__ void load_grad(const StepParams& p, int64_t e0, bool full, int cnt,
                                          uint4 (&raw)[F > 0 ? F : 1], float (&gf)[kVec]) {
    if constexpr (F > 0) {
#pragma unroll
        for (int r = 0; r < F; ++r) {
            const uint16_t* src = grad_src<F, GIL>(p, r, e0);
            raw[r] = full ? ld_u4_nt(src) : ld_u4_partial(src, cnt);
        }
    } else if constexpr (F == -1) {
        if (full) ld8_f32_nt(p.grad32 + e0, gf);
        else load8(p.grad32 + e0, false, cnt, gf);
    }
}

template <int F, bool GIL = false>
__device__ __forceinline__ void sum_grad(const StepParams& p, int64_t e0, bool full, int cnt,
                                         const uint4 (&raw)[F > 0 ? F : 1],
                                         const float (&gf)[kVec], float (&g)[kVec]) {
    if constexpr (F == -1) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = gf[e];
        return;
    }
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
                    const uint16_t* src = grad_src<F, GIL>(p, r0 + q, e0);
                    q4[q] = full ? ld_u4_nt(src) : ld_u4_partial(src, cnt);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (r0 + q < fan_in) accumulate(g, q4[q]);
        }
    }
}

// AdamW on 8 elements in registers; padding elements keep their state.
__device__ __forceinline__ void adam8(const StepParams& p, float scale, const uint32_t (&fl)[kVec],
                                      const float (&g)[kVec], float (&th)[kVec],
                                      float (&mm)[kVec], float (&vv)[kVec]) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        const float gs = g[e] * scale;
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
}

// Scale applied to the reduced gradient: grad_scale, or with clipping
// float32(grad_scale * min(1, max_norm / (sqrt(global sum of squares) + 1e-6))) in float64.
__device__ __forceinline__ float step_scale(const StepParams& p) {
    if (p.sumsq == nullptr) return p.scale;
    const double s = *p.sumsq;
    double coef = p.max_norm / (sqrt(s) + 1e-6);
    coef = coef < 1.0 ? coef : 1.0;
    return static_cast<float>(p.grad_scale * coef);
}

// bf16 bits of 8 updated weights, +0 for padding, packed two per dword.
__device__ __forceinline__ void pack_out(const uint32_t (&fl)[kVec], const float (&th)[kVec],
                                         uint32_t (&w)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo16 = (fl[2 * k] & FSDPSHARD_SEG_PADDING) ? 0u : to_bf16_bits(th[2 * k]);
        const uint32_t hi16 =
            (fl[2 * k + 1] & FSDPSHARD_SEG_PADDING) ? 0u : to_bf16_bits(th[2 * k + 1]);
        w[k] = lo16 | (hi16 << 16);
    }
}

// Where element e0 (a multiple of 8) of state array k (0 master, 1 m, 2 v) lives: three separate
// arrays, or the blocked array (blocked_index).
template <bool BLK>
__device__ __forceinline__ float* state_ptr(const StepParams& p, int k, int64_t e0) {
    if constexpr (BLK) {
        return p.master + blocked_index(k, e0);
    } else {
        return k == 0 ? p.master + e0 : (k == 1 ? p.m + e0 : p.v + e0);
    }
}

// One 512-element group with per-lane bounds: the slice's last, partial group, and every group
// of the run-time fan-in kernel.  TAIL = false drops the bounds for complete groups.
template <int F, bool OUT, bool TAIL, bool BLK, bool GIL>
__device__ __forceinline__ void step_group(const StepParams& p, float scale, const SegCursor& cur,
                                           int64_t vec, int64_t group_end_vec, int lane) {
    const int64_t n = p.n;
    const int64_t e0 = vec * kVec;
    const bool valid = !TAIL || vec < group_end_vec;
    const int cnt =
        !TAIL ? kVec : (valid ? static_cast<int>((n - e0) < kVec ? (n - e0) : kVec) : 0);
    const bool full = !TAIL || cnt == kVec;

    float g[kVec], gf[kVec], th[kVec], mm[kVec], vv[kVec];
    uint4 raw[F > 0 ? F : 1];
    if (valid) {
        load_grad<F, GIL>(p, e0, full, cnt, raw, gf);
        load8(state_ptr<BLK>(p, 0, e0), full, cnt, th);
        load8(state_ptr<BLK>(p, 1, e0), full, cnt, mm);
        load8(state_ptr<BLK>(p, 2, e0), full, cnt, vv);
        sum_grad<F, GIL>(p, e0, full, cnt, raw, gf, g);
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = th[e] = mm[e] = vv[e] = 0.0f;
    }

    uint32_t fl[kVec];
    int64_t g1 = group_end_vec * kVec;
    if (g1 > n) g1 = n;
    element_flags(cur, g1, e0, fl);
    adam8(p, scale, fl, g, th, mm, vv);

    if (valid) {
        store8(state_ptr<BLK>(p, 0, e0), full, cnt, th);
        store8(state_ptr<BLK>(p, 1, e0), full, cnt, mm);
        store8(state_ptr<BLK>(p, 2, e0), full, cnt, vv);
    }
    if constexpr (OUT) {
        uint32_t w[4];
        pack_out(fl, th, w);
        const int s = p.out_shift;
        const bool next_ok = (lane < kWave - 1) && (vec + 1 < group_end_vec) &&
                             ((vec + 1) * kVec + s <= n);
        const bool prev_ok = (lane > 0) && (e0 + s <= n);
        store_bf16_vec(p.out, e0, s, w, valid, cnt, next_ok, prev_ok);
    }
}

// A wave's complete group (compile-time gradient source F >= 1 or F == -1): every HBM load of
// the group is issued first (gradients non-temporal), then the segment cursor is placed, then
// the group is reduced, updated and stored.
// With `edges` (a destination that does not start a 64-byte line, and a work-group whose four
// groups are all whole) the waves of the work-group exchange their first lanes' bf16 words
// through LDS so that every 64-byte line of bf16 output inside the work-group is written by one
// wave in whole 16-byte vectors (store_bf16_lines).
// Pause before a group's stores, in units of 64 cycles (see step_whole_group).
constexpr int kStorePace = 28;

template <int F, bool OUT, bool BLK, bool GIL>
__device__ __forceinline__ void step_whole_group(const StepParams& p, int64_t gb, int lane,
                                                 int wave, bool edges) {
    uint4 raw[F > 0 ? F : 1];
    float gf[kVec], th[kVec], mm[kVec], vv[kVec];
    const int64_t e0 = (gb + lane) * kVec;
    // Issue order of the group's loads, pinned with scheduling barriers because it moves the
    // kernel's bandwidth on MI355X (measured): with the blocked state, or with one gradient
    // stream, every state load goes first (blocked, fan-in 8: 5 % faster than the order below);
    // with separate state arrays and several gradient streams, master and m go first, then the
    // gradients, then v (about 2 % better than the alternatives).
    if constexpr (BLK || F == 1 || F == -1) {
        load8(state_ptr<BLK>(p, 0, e0), true, kVec, th);
        load8(state_ptr<BLK>(p, 1, e0), true, kVec, mm);
        load8(state_ptr<BLK>(p, 2, e0), true, kVec, vv);
        __builtin_amdgcn_sched_barrier(0);
        load_grad<F, GIL>(p, e0, true, kVec, raw, gf);
    } else {
        load8(state_ptr<BLK>(p, 0, e0), true, kVec, th);
        load8(state_ptr<BLK>(p, 1, e0), true, kVec, mm);
        __builtin_amdgcn_sched_barrier(0);
        load_grad<F>(p, e0, true, kVec, raw, gf);
        __builtin_amdgcn_sched_barrier(0);
        load8(state_ptr<BLK>(p, 2, e0), true, kVec, vv);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float scale = step_scale(p);     // after the loads: its own reads overlap them
    SegCursor cur;
    cur.init(p.segs, p.n_segs, gb * kVec);
    uint32_t fl[kVec];
    element_flags(cur, (gb + kWave) * kVec, e0, fl);
    float g[kVec];
    sum_grad<F, GIL>(p, e0, true, kVec, raw, gf, g);
    adam8(p, scale, fl, g, th, mm, vv);
    if constexpr (BLK && (F == 1 || F == 8)) {
        // Store pacing: the wave waits kStorePace x 64 cycles before its stores.  Measured on
        // one GPU (compile-time variants, 8 alternating rounds), with the blocked state a pause of
        // 24-32 made the step 1.0-1.8 % faster at fan-in 8 (7B-shaped and one-layer slices) and
        // fan-in 1 (70B-shaped slice); 64 and longer were slower.  At fan-in 2 and 4 it cost
        // 0.7-2.4 % on 2^28-element slices (within 1 % on small ones), at the run-time fan-ins
        // 3 and 16 it gained nothing, and it slowed the separate-array step (0.5-1 %) and the
        // fp32-gradient step (1.6-1.8 %): those store at once.
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_sleep(kStorePace);
        __builtin_amdgcn_sched_barrier(0);
    }
    auto store_out = [&]() {
        if constexpr (OUT) {
            uint32_t w[4];
            pack_out(fl, th, w);
            if (p.out_shift == 0 && p.out_line_vecs == 0)
                st_u4_nt(p.out + e0, make_uint4(w[0], w[1], w[2], w[3]));
            else
                store_bf16_lines(p.out, p.out_shift, p.out_line_vecs, gb, lane, wave, edges, w);
        }
    };
    // Store order: at fan-in 1 and for the fp32 gradient the bf16 copy goes first (measured on
    // one GPU, 8-10 alternating rounds: with the blocked state 1.0-2.4 % faster at fan-in 1 on
    // the 70B-shaped slice and on 2^25- and 2^28-element slices; with separate arrays 1.2-1.4 %
    // faster at fan-in 1 on the 70B-shaped slice; 0.5-0.7 % faster for the fp32 gradient on
    // the 7B- and 70B-shaped slices in both layouts); at fan-in 8 the state goes first (bf16
    // first was 1.4-1.6 % slower with the blocked state, 3.5 % with separate arrays, on the
    // 7B-shaped slice).
    constexpr bool kOutFirst = F == 1 || F == -1;
    if constexpr (kOutFirst) store_out();
    store8(state_ptr<BLK>(p, 0, e0), true, kVec, th);
    store8(state_ptr<BLK>(p, 1, e0), true, kVec, mm);
    store8(state_ptr<BLK>(p, 2, e0), true, kVec, vv);
    if constexpr (!kOutFirst) store_out();
}

// Wave w of the grid owns vectors [64w, 64w + 64) of the slice (one group), placed by the
// XCD-aware tile map.  One group per wave was measured fastest on MI355X for every fan-in and
// state layout: waves owning 2 or 4 consecutive groups (all loads first) ran 7-15 % slower on
// the 7B- and 70B-shaped slices.
template <int F, bool OUT, bool BLK, bool GIL>
__device__ __forceinline__ void fused_step_body(StepParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t nvec = (p.n + kVec - 1) / kVec;
    const int64_t gb = tile_base<kStepXcdRun>(wave, 1);
    if (gb >= nvec) return;
    if constexpr (F != 0) {
        if (gb + kWave <= p.n / kVec) {
            // The edge exchange needs all four waves of the work-group here (a barrier): the
            // condition is the same for all of them.
            const int64_t tile_end = (gb / (kWave * kWavesPerBlock) + 1) * (kWave * kWavesPerBlock);
            const bool edges =
                OUT && (p.out_shift != 0 || p.out_line_vecs != 0) && tile_end <= p.n / kVec;
            step_whole_group<F, OUT, BLK, GIL>(p, gb, lane, wave, edges);
            return;
        }
    }
    const float scale = step_scale(p);
    SegCursor cur;
    cur.init(p.segs, p.n_segs, gb * kVec);
    int64_t gend = gb + kWave;
    if (gend > nvec) gend = nvec;
    if (gend == gb + kWave && gend * kVec <= p.n)
        step_group<F, OUT, false, BLK, GIL>(p, scale, cur, gb + lane, gend, lane);
    else
        step_group<F, OUT, true, BLK, GIL>(p, scale, cur, gb + lane, gend, lane);
}

template <int F, bool OUT, bool BLK>
__global__ __launch_bounds__(kBlock) void fused_step_kernel(StepParams p) {
    fused_step_body<F, OUT, BLK, false>(p);
}

// The blocked state with the F bf16 contributions interleaved per 512-element block in one
// buffer (grad_src): the step then streams one gradient array instead of F.
template <int F, bool OUT>
__global__ __launch_bounds__(kBlock) void fused_step_interleaved_kernel(StepParams p) {
    fused_step_body<F, OUT, true, true>(p);
}

// ------------------------------------------------------------------------------------------------
// Sum of squares of the reduced gradient (the rank's share of the global norm).
//
// Each wave walks G consecutive groups; every lane squares its elements in float64 (exact squares
// of float32 values), adds each vector's 8 squares in a fixed pairwise tree and the vectors in
// group order, padding excluded; the wave and the work-group then add their lanes in a fixed
// tree, and one float64 partial per work-group goes to the workspace.
// A second kernel adds the partials in a fixed order.  The result depends only on n and the data.

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_down(x, off, kWave);
    return x;   // valid in lane 0
}

// Sum-of-squares grid: each wave walks kSumsqGroups groups; one float64 partial per work-group.
constexpr int64_t kSumsqGroups = 16;

// Groups whose loads a wave issues back to back in the sum-of-squares kernel, in tiles that lie
// wholly inside the slice.  Measured on one GPU: the fp32 gradient reads 4-5 % faster with 8
// groups per batch than with 1; bf16 contributions are fastest one group at a time (batches of
// 2-16 were 2-25 % slower at fan-in 1, equal at fan-in 8).
template <int F>
constexpr int sumsq_batch() { return F == -1 ? 8 : 1; }

// One group's squares for this lane: the 8 float32 values x, padding and elements past the slice
// (n elements) left out, each squared in float64 (exact) and added as a fixed pairwise tree, then
// into the lane's running sum.
__device__ __forceinline__ void add_squares(SegCursor& cur, int64_t n, int64_t gb, int64_t nvec,
                                            int lane, const float (&x)[kVec], int cnt,
                                            double& acc) {
    int64_t gend = gb + kWave;
    if (gend > nvec) gend = nvec;
    cur.seek(gb * kVec);
    const int64_t e0 = (gb + lane) * kVec;
    uint32_t fl[kVec];
    int64_t g1 = gend * kVec;
    if (g1 > n) g1 = n;
    element_flags(cur, g1, e0, fl);
    double q[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        const double d = static_cast<double>(x[e]);
        const bool use = e < cnt && (fl[e] & FSDPSHARD_SEG_PADDING) == 0u;
        q[e] = use ? d * d : 0.0;
    }
    acc += ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
}

// The sum of squares of scale * g for one group.
__device__ __forceinline__ void square_group(const SumsqParams& p, SegCursor& cur, int64_t gb,
                                             int64_t nvec, int lane, const float (&g)[kVec],
                                             int cnt, double& acc) {
    float gs[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) gs[e] = g[e] * p.scale;
    add_squares(cur, p.n, gb, nvec, lane, gs, cnt, acc);
}

template <int F, bool GIL>
__device__ __forceinline__ void sumsq_body(SumsqParams p) {
    constexpr int B = sumsq_batch<F>();
    static_assert(kSumsqGroups % B == 0, "a batch must divide a wave's groups");
    __shared__ double wave_part[kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t nvec = (p.n + kVec - 1) / kVec;
    // Identity map (runs of one tile): a tile here is 16 groups per wave, and longer runs were
    // slower on one GPU.
    const int64_t tile = tile_index<1>();
    const int64_t base0 = (tile * kWavesPerBlock + wave) * (kWave * p.groups_per_wave);
    double acc = 0.0;
    if (base0 < nvec) {
        SegCursor cur;
        cur.init(p.segs, p.n_segs, base0 * kVec);
        bool done = false;
        if constexpr (F != 0) {
            // Every vector of the tile is whole: straight-line loads, B groups at a time, then
            // the squares in group order (the same order as the general path below).
            if (base0 + static_cast<int64_t>(p.groups_per_wave) * kWave <= p.n / kVec) {
                for (int g0 = 0; g0 < p.groups_per_wave; g0 += B) {
                    float g[B][kVec];
                    if constexpr (F == -1) {
#pragma unroll
                        for (int b = 0; b < B; ++b)
                            ld8_f32_nt(p.grad32 + (base0 + (g0 + b) * kWave + lane) * kVec, g[b]);
                    } else {
                        uint4 raw[B][F];
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            const int64_t e0 = (base0 + (g0 + b) * kWave + lane) * kVec;
#pragma unroll
                            for (int r = 0; r < F; ++r)
                                raw[b][r] = ld_u4_nt(grad_src<F, GIL>(p, r, e0));
                        }
#pragma unroll
                        for (int b = 0; b < B; ++b) {
#pragma unroll
                            for (int e = 0; e < kVec; ++e) g[b][e] = 0.0f;
#pragma unroll
                            for (int r = 0; r < F; ++r) accumulate(g[b], raw[b][r]);
                        }
                    }
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        square_group(p, cur, base0 + (g0 + b) * kWave, nvec, lane, g[b], kVec, acc);
                }
                done = true;
            }
        }
        if (!done) {
            // General path (the slice's last tile, or a run-time fan-in): one group at a time;
            // lanes past the slice end load nothing.
            for (int64_t g0 = 0; g0 < p.groups_per_wave; ++g0) {
                const int64_t gb = base0 + g0 * kWave;
                if (gb >= nvec) break;
                const int64_t e0 = (gb + lane) * kVec;
                const int64_t left = p.n - e0;
                const int cnt = left <= 0 ? 0 : static_cast<int>(left < kVec ? left : kVec);
                const bool full = cnt == kVec;
                float g[kVec];
#pragma unroll
                for (int e = 0; e < kVec; ++e) g[e] = 0.0f;
                if (cnt > 0) {
                    if constexpr (F == -1) {
                        if (full) ld8_f32_nt(p.grad32 + e0, g);
                        else load8(p.grad32 + e0, false, cnt, g);
                    } else if constexpr (F > 0) {
                        uint4 raw[F];
#pragma unroll
                        for (int r = 0; r < F; ++r) {
                            const uint16_t* src = grad_src<F, GIL>(p, r, e0);
                            raw[r] = full ? ld_u4_nt(src) : ld_u4_partial(src, cnt);
                        }
#pragma unroll
                        for (int r = 0; r < F; ++r) accumulate(g, raw[r]);
                    } else {
                        for (int r = 0; r < p.fan_in; ++r) {
                            const uint16_t* src = grad_src<F, GIL>(p, r, e0);
                            const uint4 q = full ? ld_u4_nt(src) : ld_u4_partial(src, cnt);
                            accumulate(g, q);
                        }
                    }
                }
                square_group(p, cur, gb, nvec, lane, g, cnt, acc);
            }
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) wave_part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double b = wave_part[0];
#pragma unroll
        for (int w = 1; w < kWavesPerBlock; ++w) b += wave_part[w];
        p.partials[tile] = b;
    }
}

template <int F>
__global__ __launch_bounds__(kBlock) void sumsq_kernel(SumsqParams p) {
    sumsq_body<F, false>(p);
}

// The F bf16 contributions interleaved per 512-element block in one array (grad_src).
template <int F>
__global__ __launch_bounds__(kBlock) void sumsq_interleaved_kernel(SumsqParams p) {
    sumsq_body<F, true>(p);
}

// Finish: thread t adds partials t, t + 256, t + 512, ... in that order, then the fixed wave and
// work-group trees.  The loads go out 16 at a time ahead of their adds (the addition order is
// unchanged), so a thread waits for memory once per 16 partials instead of once per partial.
constexpr int kFinishBatch = 16;

__global__ __launch_bounds__(kBlock) void sumsq_finish_kernel(SumsqParams p) {
    __shared__ double wave_part[kWavesPerBlock];
    double acc = 0.0;
    int64_t i = threadIdx.x;   // 64-bit: i + 15 * 256 stays exact for any partial count
    for (; i + (kFinishBatch - 1) * kBlock < p.n_partials; i += kFinishBatch * kBlock) {
        double x[kFinishBatch];
#pragma unroll
        for (int k = 0; k < kFinishBatch; ++k) x[k] = p.partials[i + k * kBlock];
#pragma unroll
        for (int k = 0; k < kFinishBatch; ++k) acc += x[k];
    }
    for (; i < p.n_partials; i += kBlock) acc += p.partials[i];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    acc = wave_sum(acc);
    if (lane == 0) wave_part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double b = wave_part[0];
#pragma unroll
        for (int w = 1; w < kWavesPerBlock; ++w) b += wave_part[w];
        *p.result = b;
    }
}

// Reduction into an fp32 shard fused with that shard's sum of squares: out = scale * sum (or
// out + scale * sum when ACC), exactly as reduce_kernel computes it, and one float64 partial per
// work-group of the sum of out^2 over the real elements, added in the same fixed order as
// sumsq_kernel (each work-group covers kSumsqGroups groups per wave, so the partials fill the
// same workspace).  Whole tiles take a straight-line path; the slice's last tile and run-time
// fan-ins take the bounds-checked path.
//
// Where many bytes per element arrive (eight contribution streams, or four plus the accumulator),
// the straight-line path is software-pipelined: the next group's loads are issued before the
// current group is reduced and stored, which the kernel cannot otherwise do because the
// compiler must assume the stores may alias the next loads (the entry point rejects overlaps).
// Those instances run one work-group per CU.  Measured on MI355X at the 7B-shaped slice against
// one group at a time with 2 work-groups per CU: fan-in 8 9 % faster, fan-in 8 accumulating 2.5 %,
// fan-in 4 accumulating 5.5 %; at fan-in 1, 2 and 4 without accumulation the pipeline is 4-10 %
// slower, so they keep the plain loop.
template <int F, bool ACC>
constexpr bool reduce_sq_pipelined() { return F >= 8 || (F >= 4 && ACC); }
static_assert(kSumsqGroups % 2 == 0, "the pipelined path takes groups in pairs");

struct ReduceSqParams {
    const uint16_t* contrib[FSDPSHARD_MAX_FAN_IN];
    float* out;
    const fsdpshard_segment* segs;
    double* partials;
    int64_t n;
    int32_t n_segs;
    int32_t fan_in;
    float scale;
};

template <int F, bool ACC, bool GIL>
__device__ __forceinline__ void reduce_sumsq_body(ReduceSqParams p) {
    __shared__ double wave_part[kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t nvec = (p.n + kVec - 1) / kVec;
    const int64_t tile = tile_index<1>();
    const int64_t base0 = (tile * kWavesPerBlock + wave) * (kWave * kSumsqGroups);
    double sq = 0.0;
    if (base0 < nvec) {
        SegCursor cur;
        cur.init(p.segs, p.n_segs, base0 * kVec);
        bool done = false;
        if constexpr (reduce_sq_pipelined<F, ACC>()) {
            if (base0 + kSumsqGroups * kWave <= p.n / kVec) {
                // Two register slots: slot (g0 & 1) holds group g0's loads.
                uint4 raw[2][F];
                float acc[2][kVec];
                auto issue = [&](int slot, int g0) {
                    const int64_t e0 = (base0 + g0 * kWave + lane) * kVec;
#pragma unroll
                    for (int r = 0; r < F; ++r) raw[slot][r] = ld_u4_nt(grad_src<F, GIL>(p, r, e0));
                    if constexpr (ACC) load8(p.out + e0, true, kVec, acc[slot]);
                };
                auto finish = [&](int slot, int g0) {
                    const int64_t gb = base0 + g0 * kWave;
                    const int64_t e0 = (gb + lane) * kVec;
                    float g[kVec];
#pragma unroll
                    for (int e = 0; e < kVec; ++e) g[e] = 0.0f;
#pragma unroll
                    for (int r = 0; r < F; ++r) accumulate(g, raw[slot][r]);
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        g[e] = g[e] * p.scale;
                        if constexpr (ACC) g[e] = acc[slot][e] + g[e];
                    }
                    store8(p.out + e0, true, kVec, g);
                    add_squares(cur, p.n, gb, nvec, lane, g, kVec, sq);
                };
                issue(0, 0);
#pragma unroll 1
                for (int g0 = 0; g0 < kSumsqGroups; g0 += 2) {
                    issue(1, g0 + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    finish(0, g0);
                    if (g0 + 2 < kSumsqGroups) issue(0, g0 + 2);
                    __builtin_amdgcn_sched_barrier(0);
                    finish(1, g0 + 1);
                }
                done = true;
            }
        } else if constexpr (F > 0) {
            if (base0 + kSumsqGroups * kWave <= p.n / kVec) {
                for (int g0 = 0; g0 < kSumsqGroups; ++g0) {
                    const int64_t gb = base0 + g0 * kWave;
                    const int64_t e0 = (gb + lane) * kVec;
                    uint4 raw[F];
                    float acc[kVec];
                    if constexpr (ACC) load8(p.out + e0, true, kVec, acc);
#pragma unroll
                    for (int r = 0; r < F; ++r) raw[r] = ld_u4_nt(grad_src<F, GIL>(p, r, e0));
                    float g[kVec];
#pragma unroll
                    for (int e = 0; e < kVec; ++e) g[e] = 0.0f;
#pragma unroll
                    for (int r = 0; r < F; ++r) accumulate(g, raw[r]);
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        g[e] = g[e] * p.scale;
                        if constexpr (ACC) g[e] = acc[e] + g[e];
                    }
                    store8(p.out + e0, true, kVec, g);
                    add_squares(cur, p.n, gb, nvec, lane, g, kVec, sq);
                }
                done = true;
            }
        }
        if (!done) {
            for (int g0 = 0; g0 < kSumsqGroups; ++g0) {
                const int64_t gb = base0 + g0 * kWave;
                if (gb >= nvec) break;
                const int64_t e0 = (gb + lane) * kVec;
                const int64_t left = p.n - e0;
                const int cnt = left <= 0 ? 0 : static_cast<int>(left < kVec ? left : kVec);
                const bool full = cnt == kVec;
                float g[kVec];
#pragma unroll
                for (int e = 0; e < kVec; ++e) g[e] = 0.0f;
                if (cnt > 0) {
                    float acc[kVec];
                    if constexpr (ACC) load8(p.out + e0, full, cnt, acc);
                    for (int r = 0; r < p.fan_in; ++r) {
                        const uint16_t* src = grad_src<0, GIL>(p, r, e0);
                        const uint4 q = full ? ld_u4_nt(src) : ld_u4_partial(src, cnt);
                        accumulate(g, q);
                    }
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        g[e] = g[e] * p.scale;
                        if constexpr (ACC) g[e] = acc[e] + g[e];
                    }
                    store8(p.out + e0, full, cnt, g);
                }
                add_squares(cur, p.n, gb, nvec, lane, g, cnt, sq);
            }
        }
    }
    sq = wave_sum(sq);
    if (lane == 0) wave_part[wave] = sq;
    __syncthreads();
    if (threadIdx.x == 0) {
        double b = wave_part[0];
#pragma unroll
        for (int w = 1; w < kWavesPerBlock; ++w) b += wave_part[w];
        p.partials[tile] = b;
    }
}

template <int F, bool ACC>
__global__ __launch_bounds__(kBlock) void reduce_sumsq_kernel(ReduceSqParams p) {
    reduce_sumsq_body<F, ACC, false>(p);
}

// The F contributions interleaved per 512-element block in one array (grad_src).
template <int F, bool ACC>
__global__ __launch_bounds__(kBlock) void reduce_sumsq_interleaved_kernel(ReduceSqParams p) {
    reduce_sumsq_body<F, ACC, true>(p);
}

// ------------------------------------------------------------------------------------------------
// Standalone reduce and unflatten: one 512-element group per wave.

// Groups per wave of the reduce kernels (measured on MI355X: two groups per wave pay off only for
// the plain reduction of eight or more separate contribution arrays; below that, for the fp32
// accumulation under the work-group cap, and for interleaved contributions, one group per wave
// is fastest: the plain interleaved reduction of eight runs 7.5-8 % faster with one than with
// two on 2^27- and 905M-element slices).
// Pause before the stores of the fan-in-8 fp32 accumulation, in units of 64 cycles.
constexpr int kAccumulatePace = 16;

template <int F, bool ACC, bool GIL = false>
constexpr int reduce_groups() { return F >= 8 && !ACC && !GIL ? 2 : 1; }

// ACC = false: out = scale * sum.  ACC = true: out = out + scale * sum (fp32 accumulation of
// micro-batches; one rounding for the sum, one for the scale, one for the addition).
// F >= 1 is a compile-time fan-in, F == 0 the run-time one; each wave owns reduce_groups<F, ACC, GIL>()
// consecutive groups, and a complete tile issues all its loads before the first add.
template <int F, bool ACC, bool GIL>
__device__ __forceinline__ void reduce_body(ReduceParams p) {
    constexpr int U = reduce_groups<F, ACC, GIL>();
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t nvec = (p.n + kVec - 1) / kVec;
    const int64_t base0 = tile_base(wave, U);
    if (base0 >= nvec) return;
    if constexpr (F > 0) {
        if (base0 + kWave * U <= p.n / kVec) {
            uint4 raw[U][F];
            float acc[U][kVec];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t e0 = (base0 + u * kWave + lane) * kVec;
                if constexpr (ACC) load8(p.out + e0, true, kVec, acc[u]);
#pragma unroll
                for (int r = 0; r < F; ++r) raw[u][r] = ld_u4_nt(grad_src<F, GIL>(p, r, e0));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t e0 = (base0 + u * kWave + lane) * kVec;
                float g[kVec];
#pragma unroll
                for (int e = 0; e < kVec; ++e) g[e] = 0.0f;
#pragma unroll
                for (int r = 0; r < F; ++r) accumulate(g, raw[u][r]);
#pragma unroll
                for (int e = 0; e < kVec; ++e) {
                    g[e] = g[e] * p.scale;
                    if constexpr (ACC) g[e] = acc[u][e] + g[e];
                }
                if constexpr (ACC && F == 8) {
                    // Store pacing, as in the fused step (measured on one GPU, 10 alternating
                    // rounds): a pause of 16 x 64 cycles made the fp32 accumulation of eight
                    // contributions 2.3-3.1 % faster on a 905M-element shard and 0.8-1.3 % on a
                    // 134M-element one.  The plain reduction and the other fan-ins were the
                    // same or slower with a pause (fan-in 1 by 30 %).
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_sleep(kAccumulatePace);
                    __builtin_amdgcn_sched_barrier(0);
                }
                store8(p.out + e0, true, kVec, g);
            }
            return;
        }
    }
    for (int u = 0; u < U; ++u) {
        const int64_t vec = base0 + u * kWave + lane;
        if (vec >= nvec) continue;
        const int64_t e0 = vec * kVec;
        const int cnt = static_cast<int>((p.n - e0) < kVec ? (p.n - e0) : kVec);
        const bool full = cnt == kVec;
        float acc[kVec];
        if constexpr (ACC) load8(p.out + e0, full, cnt, acc);
        float g[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = 0.0f;
        for (int r0 = 0; r0 < p.fan_in; r0 += 4) {
            uint4 q4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (r0 + q < p.fan_in) {
                    const uint16_t* src = grad_src<0, GIL>(p, r0 + q, e0);
                    q4[q] = full ? ld_u4_nt(src) : ld_u4_partial(src, cnt);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (r0 + q < p.fan_in) accumulate(g, q4[q]);
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            g[e] = g[e] * p.scale;
            if constexpr (ACC) g[e] = acc[e] + g[e];
        }
        store8(p.out + e0, full, cnt, g);
    }
}

template <int F, bool ACC>
__global__ __launch_bounds__(kBlock) void reduce_kernel(ReduceParams p) {
    reduce_body<F, ACC, false>(p);
}

// The F contributions interleaved per 512-element block in one array (grad_src).
template <int F, bool ACC>
__global__ __launch_bounds__(kBlock) void reduce_interleaved_kernel(ReduceParams p) {
    reduce_body<F, ACC, true>(p);
}

__global__ __launch_bounds__(kBlock) void unflatten_kernel(UnflattenParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t nvec = (p.n + kVec - 1) / kVec;
    const int64_t gb = tile_base(wave, 1);
    if (gb >= nvec) return;
    int64_t gend = gb + kWave;
    if (gend > nvec) gend = nvec;
    const int64_t vec = gb + lane;
    const int64_t e0 = vec * kVec;
    const bool valid = vec < gend;
    const int cnt = valid ? static_cast<int>((p.n - e0) < kVec ? (p.n - e0) : kVec) : 0;
    float th[kVec];
    if (valid) {
        load8(p.master + e0, cnt == kVec, cnt, th);
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) th[e] = 0.0f;
    }
    SegCursor cur;
    cur.init(p.segs, p.n_segs, gb * kVec);
    uint32_t fl[kVec];
    int64_t g1 = gend * kVec;
    if (g1 > p.n) g1 = p.n;
    element_flags(cur, g1, e0, fl);
    uint32_t w[4];
    pack_out(fl, th, w);
    const int s = p.out_shift;
    const bool next_ok = (lane < kWave - 1) && (vec + 1 < gend) && ((vec + 1) * kVec + s <= p.n);
    const bool prev_ok = (lane > 0) && (e0 + s <= p.n);
    store_bf16_vec(p.out, e0, s, w, valid, cnt, next_ok, prev_ok);
}

// Conversion between the separate state arrays and the blocked state array (plain copies).
struct StatePackParams {
    float* sep[3];           // master, m, v
    float* blocked;
    int64_t n;
};

template <bool TO_BLOCKED>
__global__ __launch_bounds__(kBlock) void state_pack_kernel(StatePackParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t vec = tile_base(wave, 1) + lane;
    const int64_t e0 = vec * kVec;
    if (e0 >= p.n) return;
    const int cnt = static_cast<int>((p.n - e0) < kVec ? (p.n - e0) : kVec);
    const bool full = cnt == kVec;
    const int64_t b0 = ((e0 / kStateBlock) * 3) * kStateBlock + e0 % kStateBlock;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        float x[kVec];
        float* bp = p.blocked + b0 + k * kStateBlock;
        if constexpr (TO_BLOCKED) {
            load8(p.sep[k] + e0, full, cnt, x);
            store8(bp, full, cnt, x);
        } else {
            load8(bp, full, cnt, x);
            store8(p.sep[k] + e0, full, cnt, x);
        }
    }
}

// Copy of F separate contributions into the interleaved buffer (grad_src): lane by lane, one
// 16-byte vector per contribution, elements past the slice in the last block left untouched.
struct InterleaveParams {
    const uint16_t* contrib[FSDPSHARD_MAX_FAN_IN];
    uint16_t* dst;
    int64_t n;
    int32_t fan_in;
};

__global__ __launch_bounds__(kBlock) void interleave_kernel(InterleaveParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t vec = tile_base(wave, 1) + lane;
    const int64_t e0 = vec * kVec;
    if (e0 >= p.n) return;
    const int cnt = static_cast<int>((p.n - e0) < kVec ? (p.n - e0) : kVec);
    const uint64_t u = static_cast<uint64_t>(e0);
    uint16_t* dst = p.dst + static_cast<int64_t>(u / kStateBlock) * p.fan_in * kStateBlock +
                    static_cast<int64_t>(u % kStateBlock);
    for (int r = 0; r < p.fan_in; ++r) {
        const uint16_t* src = p.contrib[r] + e0;
        uint16_t* d = dst + static_cast<int64_t>(r) * kStateBlock;
        if (cnt == kVec) {
            st_u4_nt(d, ld_u4_nt(src));
        } else {
            for (int e = 0; e < cnt; ++e) d[e] = src[e];
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Host-side launch helpers.

// Work-groups per CU of the reduction kernels (see occupancy_lds).  Measured on one GPU at
// 2^24..2^29.75 elements against the other caps (0-4), 4 alternating rounds per point:
//   plain reduction:  fan-in 1 takes 4 (2-6 % ahead of uncapped, 2 costs a third), fan-in 2
//                     takes 3 (10-12 % ahead of 2); other fan-ins 2 (within 1 % of the best
//                     at 4, 8 and 16 from 2^26 up; at 3, 3 per CU is 3 % slower at 2^26 and
//                     3-5 % faster from 2^28);
//   fp32 accumulation: fan-in 1 takes 2 (4-5 % ahead of 4), fan-in 2 and run-time fan-ins
//                     above 8 take 3 (2 % and 5 % ahead of 2), others 2;
// the reduction fused with the sum of squares wants 2 per CU, 3 for a single contribution and 1
// where its loads are software-pipelined (reduce_sq_pipelined); unflatten is fastest uncapped
// (the sum of squares has its own rule, sumsq_groups_per_cu); the blocked-state packing takes 2
// (14-20 % ahead of uncapped).
inline int reduce_groups_per_cu(int fan_in, bool accumulate) {
    if (fan_in == 1) return accumulate ? 2 : 4;
    if (fan_in == 2 || (accumulate && fan_in > 8)) return 3;
    return 2;
}

constexpr int kReduceSqGroupsPerCU = 2;
constexpr int kReduceOneStreamSqGroupsPerCU = 3;
constexpr int kReduceSqPipelinedGroupsPerCU = 1;
constexpr int kStatePackGroupsPerCU = 2;

template <int F, bool BLK>
const void* step_kernel(bool out) {
    return out ? reinterpret_cast<const void*>(&fused_step_kernel<F, true, BLK>)
               : reinterpret_cast<const void*>(&fused_step_kernel<F, false, BLK>);
}

// fan_in -1 selects the fp32-gradient kernels.
template <bool BLK>
const void* pick_step_kernel(int fan_in, bool out) {
    switch (fan_in) {
        case -1: return step_kernel<-1, BLK>(out);
        case 1: return step_kernel<1, BLK>(out);
        case 2: return step_kernel<2, BLK>(out);
        case 4: return step_kernel<4, BLK>(out);
        case 8: return step_kernel<8, BLK>(out);
        default: return step_kernel<0, BLK>(out);
    }
}

template <int F>
const void* interleaved_step_kernel(bool out) {
    return out ? reinterpret_cast<const void*>(&fused_step_interleaved_kernel<F, true>)
               : reinterpret_cast<const void*>(&fused_step_interleaved_kernel<F, false>);
}

const void* pick_interleaved_step_kernel(int fan_in, bool out) {
    switch (fan_in) {
        case 1: return interleaved_step_kernel<1>(out);
        case 2: return interleaved_step_kernel<2>(out);
        case 4: return interleaved_step_kernel<4>(out);
        case 8: return interleaved_step_kernel<8>(out);
        default: return interleaved_step_kernel<0>(out);
    }
}

// First slice element whose bf16 destination starts a 16-byte vector.
int out_shift_of(const uint16_t* out) {
    const unsigned phase = static_cast<unsigned>(reinterpret_cast<uintptr_t>(out) & 15u) / 2u;
    return static_cast<int>((kVec - phase) % kVec);
}

// First slice element whose bf16 destination starts a 64-byte line (0..31; out_shift_of(out)
// is this value mod 8).
int out_line_shift_of(const uint16_t* out) {
    const unsigned off = static_cast<unsigned>(reinterpret_cast<uintptr_t>(out) & 63u);
    return static_cast<int>(((64u - off) & 63u) / 2u);
}

bool is_finite(double x) { return std::isfinite(x); }

// Bytes of a device segment table.
int64_t seg_bytes(const fsdpshard_segment* segs, int32_t n_segments) {
    return segs == nullptr ? 0 : static_cast<int64_t>(n_segments) * sizeof(fsdpshard_segment);
}

// Shared by the step entry points: exactly one of (contribs, fan_in >= 1), (grad32,
// fan_in == -1) and (interleaved, fan_in >= 1) is the gradient source.  With `blocked`, `master`
// is the blocked state array and m, v are null; the interleaved source needs the blocked state.
int launch_step(float* master, float* m, float* v, const uint16_t* const* contribs, int32_t fan_in,
                const float* grad32, int64_t n, const fsdpshard_segment* segs, int32_t n_segments,
                const fsdpshard_adamw* hp, uint16_t* flat_bf16, int64_t flat_index0, int64_t lo,
                void* stream, bool blocked = false, const uint16_t* interleaved = nullptr) {
    if (master == nullptr || (!blocked && (m == nullptr || v == nullptr)) || hp == nullptr ||
        n < 0 || n_segments < 0 || (n_segments > 0 && segs == nullptr) || lo < 0)
        return FSDPSHARD_ERR_INVALID_ARG;
    int rc = FSDPSHARD_OK;
    int64_t il_elems = 0;
    if (interleaved != nullptr) {
        if (!blocked || fan_in < 1) return FSDPSHARD_ERR_INVALID_ARG;
        if (fan_in > FSDPSHARD_MAX_FAN_IN) return FSDPSHARD_ERR_UNSUPPORTED;
        if (!aligned16(interleaved)) return FSDPSHARD_ERR_ALIGNMENT;
        il_elems = interleaved_elems(fan_in, n);
        if (il_elems < 0) return FSDPSHARD_ERR_OVERFLOW;
    } else if (fan_in == -1) {
        if (grad32 == nullptr) return FSDPSHARD_ERR_INVALID_ARG;
        if (!aligned16(grad32)) return FSDPSHARD_ERR_ALIGNMENT;
    } else {
        rc = check_contribs(contribs, fan_in);
        if (rc != FSDPSHARD_OK) return rc;
    }
    if (hp->step < 1 || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
        !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !is_finite(hp->lr) || !is_finite(hp->eps) ||
        !is_finite(hp->weight_decay) || !is_finite(hp->grad_scale) ||
        !is_finite(hp->max_grad_norm) || hp->max_grad_norm < 0.0 ||
        (hp->max_grad_norm > 0.0 && hp->grad_sumsq == nullptr))
        return FSDPSHARD_ERR_INVALID_ARG;
    if (!aligned16(master) || (!blocked && (!aligned16(m) || !aligned16(v))))
        return FSDPSHARD_ERR_ALIGNMENT;
    if (segs != nullptr && !aligned8(segs)) return FSDPSHARD_ERR_ALIGNMENT;
    if (hp->max_grad_norm > 0.0 && !aligned8(hp->grad_sumsq)) return FSDPSHARD_ERR_ALIGNMENT;
    uint16_t* out = nullptr;
    if (flat_bf16 != nullptr) {
        if (flat_index0 > lo) return FSDPSHARD_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(flat_bf16) & 1u) != 0) return FSDPSHARD_ERR_ALIGNMENT;
        out = flat_bf16 + (lo - flat_index0);
    }
    if (n > INT64_MAX / 16) return FSDPSHARD_ERR_OVERFLOW;
    // Written buffers must not overlap each other or any input (gradients, segment table, the
    // global sum of squares).
    if (n == 0) return FSDPSHARD_OK;
    const int64_t fb = n * 4, hb = n * 2;
    const void* wr[4] = {master, blocked ? nullptr : m, blocked ? nullptr : v, out};
    const int64_t wb[4] = {blocked ? blocked_elems(n) * 4 : fb, fb, fb, hb};
    const int64_t sb = seg_bytes(segs, n_segments);
    for (int i = 0; i < 4; ++i) {
        if (wr[i] == nullptr) continue;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(wr[i], wb[i], wr[j], wb[j])) return FSDPSHARD_ERR_INVALID_ARG;
        if (interleaved != nullptr) {
            if (overlaps(wr[i], wb[i], interleaved, il_elems * 2)) return FSDPSHARD_ERR_INVALID_ARG;
        } else if (fan_in == -1) {
            if (overlaps(wr[i], wb[i], grad32, fb)) return FSDPSHARD_ERR_INVALID_ARG;
        } else {
            for (int r = 0; r < fan_in; ++r)
                if (overlaps(wr[i], wb[i], contribs[r], hb)) return FSDPSHARD_ERR_INVALID_ARG;
        }
        if (overlaps(wr[i], wb[i], segs, sb)) return FSDPSHARD_ERR_INVALID_ARG;
        if (hp->max_grad_norm > 0.0 && overlaps(wr[i], wb[i], hp->grad_sumsq, 8))
            return FSDPSHARD_ERR_INVALID_ARG;
    }

    StepParams p;
    p.master = master;
    p.m = blocked ? nullptr : m;
    p.v = blocked ? nullptr : v;
    for (int r = 0; r < FSDPSHARD_MAX_FAN_IN; ++r)
        p.contrib[r] = (interleaved == nullptr && fan_in > 0 && r < fan_in) ? contribs[r] : nullptr;
    if (interleaved != nullptr) p.contrib[0] = interleaved;
    p.segs = segs;
    p.grad32 = fan_in == -1 ? grad32 : nullptr;
    p.out = out;
    p.sumsq = hp->max_grad_norm > 0.0 ? hp->grad_sumsq : nullptr;
    p.max_norm = hp->max_grad_norm;
    p.grad_scale = hp->grad_scale;
    p.n = n;
    p.n_segs = segs == nullptr ? 0 : n_segments;
    p.fan_in = fan_in;
    p.out_shift = out == nullptr ? 0 : out_shift_of(out);
    p.out_line_vecs = out == nullptr ? 0 : out_line_shift_of(out) / kVec;
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
    rc = tile_grid(n, 1, &blocks);
    if (rc != FSDPSHARD_OK) return rc;
    const void* k = interleaved != nullptr ? pick_interleaved_step_kernel(fan_in, out != nullptr)
                    : blocked              ? pick_step_kernel<true>(fan_in, out != nullptr)
                                           : pick_step_kernel<false>(fan_in, out != nullptr);
    return launch(k, blocks, &p, stream, step_groups_per_cu(fan_in, blocks));
}

// The gradient source of the reductions: F separate arrays, or (`interleaved` non-null) the F
// contributions in that one interleaved array.  Checks it as the step does; `elems` receives the
// interleaved array's length.
int check_grad_source(const uint16_t* const* contribs, const uint16_t* interleaved,
                      int32_t fan_in, int64_t n, int64_t* elems) {
    *elems = 0;
    if (interleaved == nullptr) return check_contribs(contribs, fan_in);
    if (fan_in < 1) return FSDPSHARD_ERR_INVALID_ARG;
    if (fan_in > FSDPSHARD_MAX_FAN_IN) return FSDPSHARD_ERR_UNSUPPORTED;
    if (!aligned16(interleaved)) return FSDPSHARD_ERR_ALIGNMENT;
    *elems = interleaved_elems(fan_in, n);
    return *elems < 0 ? FSDPSHARD_ERR_OVERFLOW : FSDPSHARD_OK;
}

// Whether a written buffer overlaps the gradient source (n elements per separate array).
bool overlaps_grad_source(const void* w, int64_t wbytes, const uint16_t* const* contribs,
                          const uint16_t* interleaved, int32_t fan_in, int64_t n,
                          int64_t il_elems) {
    if (interleaved != nullptr) return overlaps(w, wbytes, interleaved, il_elems * 2);
    for (int r = 0; r < fan_in; ++r)
        if (overlaps(w, wbytes, contribs[r], n * 2)) return true;
    return false;
}

template <int F>
const void* reduce_kernel_for(bool accumulate, bool interleaved) {
    if (interleaved)
        return accumulate ? reinterpret_cast<const void*>(&reduce_interleaved_kernel<F, true>)
                          : reinterpret_cast<const void*>(&reduce_interleaved_kernel<F, false>);
    return accumulate ? reinterpret_cast<const void*>(&reduce_kernel<F, true>)
                      : reinterpret_cast<const void*>(&reduce_kernel<F, false>);
}

template <int F>
int reduce_groups_for(bool accumulate, bool interleaved) {
    if (interleaved)
        return accumulate ? reduce_groups<F, true, true>() : reduce_groups<F, false, true>();
    return accumulate ? reduce_groups<F, true>() : reduce_groups<F, false>();
}

int launch_reduce(const uint16_t* const* contribs, int32_t fan_in, int64_t n, float scale,
                  float* out, bool accumulate, void* stream,
                  const uint16_t* interleaved = nullptr) {
    if (out == nullptr || n < 0) return FSDPSHARD_ERR_INVALID_ARG;
    int64_t il_elems = 0;
    int rc = check_grad_source(contribs, interleaved, fan_in, n, &il_elems);
    if (rc != FSDPSHARD_OK) return rc;
    if (!aligned16(out)) return FSDPSHARD_ERR_ALIGNMENT;
    if (n > INT64_MAX / 4) return FSDPSHARD_ERR_OVERFLOW;
    if (n > 0 && overlaps_grad_source(out, n * 4, contribs, interleaved, fan_in, n, il_elems))
        return FSDPSHARD_ERR_INVALID_ARG;
    if (n == 0) return FSDPSHARD_OK;
    ReduceParams p;
    for (int r = 0; r < FSDPSHARD_MAX_FAN_IN; ++r)
        p.contrib[r] = (interleaved == nullptr && r < fan_in) ? contribs[r] : nullptr;
    if (interleaved != nullptr) p.contrib[0] = interleaved;
    p.out = out;
    p.n = n;
    p.fan_in = fan_in;
    p.scale = scale;
    const bool il = interleaved != nullptr;
    const void* k = nullptr;
    int groups = 1;
    switch (fan_in) {
#define FSDPSHARD_REDUCE_CASE(FI)                                                               \
    case FI:                                                                                    \
        k = reduce_kernel_for<FI>(accumulate, il);                                              \
        groups = reduce_groups_for<FI>(accumulate, il);                                         \
        break;
        FSDPSHARD_REDUCE_CASE(1)
        FSDPSHARD_REDUCE_CASE(2)
        FSDPSHARD_REDUCE_CASE(4)
        FSDPSHARD_REDUCE_CASE(8)
#undef FSDPSHARD_REDUCE_CASE
        default:
            k = reduce_kernel_for<0>(accumulate, il);
            groups = reduce_groups_for<0>(accumulate, il);
    }
    unsigned blocks = 0;
    rc = tile_grid(n, groups, &blocks);
    if (rc != FSDPSHARD_OK) return rc;
    return launch(k, blocks, &p, stream, reduce_groups_per_cu(fan_in, accumulate));
}

int64_t sumsq_partials(int64_t n) {
    const int64_t nvec = (n + kVec - 1) / kVec;
    const int64_t per_block = static_cast<int64_t>(kWavesPerBlock) * kWave * kSumsqGroups;
    return (nvec + per_block - 1) / per_block;
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// C ABI.

extern "C" int adamw_shard_step(float* master, float* m, float* v,
                                const uint16_t* const* contribs, int32_t fan_in, int64_t n,
                                const fsdpshard_segment* segs, int32_t n_segments,
                                const fsdpshard_adamw* hp, uint16_t* flat_bf16,
                                int64_t flat_index0, int64_t lo, void* stream) {
    if (fan_in < 1) return FSDPSHARD_ERR_INVALID_ARG;
    return launch_step(master, m, v, contribs, fan_in, nullptr, n, segs, n_segments, hp, flat_bf16,
                       flat_index0, lo, stream);
}

extern "C" int adamw_shard_step_f32grad(float* master, float* m, float* v, const float* grad,
                                        int64_t n, const fsdpshard_segment* segs,
                                        int32_t n_segments, const fsdpshard_adamw* hp,
                                        uint16_t* flat_bf16, int64_t flat_index0, int64_t lo,
                                        void* stream) {
    return launch_step(master, m, v, nullptr, -1, grad, n, segs, n_segments, hp, flat_bf16,
                       flat_index0, lo, stream);
}

extern "C" int64_t state_blocked_elems(int64_t n) { return blocked_elems(n); }

extern "C" int adamw_shard_step_blocked(float* state, const uint16_t* const* contribs,
                                        int32_t fan_in, int64_t n, const fsdpshard_segment* segs,
                                        int32_t n_segments, const fsdpshard_adamw* hp,
                                        uint16_t* flat_bf16, int64_t flat_index0, int64_t lo,
                                        void* stream) {
    if (fan_in < 1) return FSDPSHARD_ERR_INVALID_ARG;
    return launch_step(state, nullptr, nullptr, contribs, fan_in, nullptr, n, segs, n_segments, hp,
                       flat_bf16, flat_index0, lo, stream, true);
}

extern "C" int adamw_shard_step_f32grad_blocked(float* state, const float* grad, int64_t n,
                                                const fsdpshard_segment* segs, int32_t n_segments,
                                                const fsdpshard_adamw* hp, uint16_t* flat_bf16,
                                                int64_t flat_index0, int64_t lo, void* stream) {
    return launch_step(state, nullptr, nullptr, nullptr, -1, grad, n, segs, n_segments, hp,
                       flat_bf16, flat_index0, lo, stream, true);
}

extern "C" int64_t grads_interleaved_elems(int32_t fan_in, int64_t n) {
    return interleaved_elems(fan_in, n);
}

extern "C" int adamw_shard_step_interleaved(float* state, const uint16_t* grads, int32_t fan_in,
                                            int64_t n, const fsdpshard_segment* segs,
                                            int32_t n_segments, const fsdpshard_adamw* hp,
                                            uint16_t* flat_bf16, int64_t flat_index0, int64_t lo,
                                            void* stream) {
    if (grads == nullptr || fan_in < 1) return FSDPSHARD_ERR_INVALID_ARG;
    return launch_step(state, nullptr, nullptr, nullptr, fan_in, nullptr, n, segs, n_segments, hp,
                       flat_bf16, flat_index0, lo, stream, true, grads);
}

extern "C" int grads_to_interleaved(const uint16_t* const* contribs, int32_t fan_in, int64_t n,
                                    uint16_t* grads, void* stream) {
    if (grads == nullptr || n < 0) return FSDPSHARD_ERR_INVALID_ARG;
    const int rc = check_contribs(contribs, fan_in);
    if (rc != FSDPSHARD_OK) return rc;
    if (!aligned16(grads)) return FSDPSHARD_ERR_ALIGNMENT;
    const int64_t elems = interleaved_elems(fan_in, n);
    if (elems < 0) return FSDPSHARD_ERR_OVERFLOW;
    for (int r = 0; r < fan_in && n > 0; ++r)
        if (overlaps(grads, elems * 2, contribs[r], n * 2)) return FSDPSHARD_ERR_INVALID_ARG;
    if (n == 0) return FSDPSHARD_OK;
    InterleaveParams p;
    for (int r = 0; r < FSDPSHARD_MAX_FAN_IN; ++r) p.contrib[r] = r < fan_in ? contribs[r] : nullptr;
    p.dst = grads;
    p.n = n;
    p.fan_in = fan_in;
    unsigned blocks = 0;
    const int grc = tile_grid(n, 1, &blocks);
    if (grc != FSDPSHARD_OK) return grc;
    return launch(reinterpret_cast<const void*>(&interleave_kernel), blocks, &p, stream);
}

namespace {
int launch_state_pack(float* master, float* m, float* v, int64_t n, float* state, bool to_blocked,
                      void* stream) {
    if (master == nullptr || m == nullptr || v == nullptr || state == nullptr || n < 0)
        return FSDPSHARD_ERR_INVALID_ARG;
    if (!aligned16(master) || !aligned16(m) || !aligned16(v) || !aligned16(state))
        return FSDPSHARD_ERR_ALIGNMENT;
    const int64_t sb = blocked_elems(n);
    if (sb < 0) return FSDPSHARD_ERR_OVERFLOW;
    const void* sep[3] = {master, m, v};
    for (int i = 0; i < 3 && n > 0; ++i) {
        if (overlaps(sep[i], n * 4, state, sb * 4)) return FSDPSHARD_ERR_INVALID_ARG;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(sep[i], n * 4, sep[j], n * 4)) return FSDPSHARD_ERR_INVALID_ARG;
    }
    if (n == 0) return FSDPSHARD_OK;
    StatePackParams p;
    p.sep[0] = master;
    p.sep[1] = m;
    p.sep[2] = v;
    p.blocked = state;
    p.n = n;
    unsigned blocks = 0;
    const int rc = tile_grid(n, 1, &blocks);
    if (rc != FSDPSHARD_OK) return rc;
    return launch(to_blocked ? reinterpret_cast<const void*>(&state_pack_kernel<true>)
                             : reinterpret_cast<const void*>(&state_pack_kernel<false>),
                  blocks, &p, stream, kStatePackGroupsPerCU);
}
}  // namespace

extern "C" int state_to_blocked(const float* master, const float* m, const float* v, int64_t n,
                                float* state, void* stream) {
    return launch_state_pack(const_cast<float*>(master), const_cast<float*>(m),
                             const_cast<float*>(v), n, state, true, stream);
}

extern "C" int state_from_blocked(const float* state, int64_t n, float* master, float* m, float* v,
                                  void* stream) {
    return launch_state_pack(master, m, v, n, const_cast<float*>(state), false, stream);
}

extern "C" int reduce_shard(const uint16_t* const* contribs, int32_t fan_in, int64_t n,
                            float scale, float* out, void* stream) {
    return launch_reduce(contribs, fan_in, n, scale, out, false, stream);
}

extern "C" int reduce_shard_accumulate(const uint16_t* const* contribs, int32_t fan_in,
                                       int64_t n, float scale, float* acc, void* stream) {
    return launch_reduce(contribs, fan_in, n, scale, acc, true, stream);
}

extern "C" int reduce_shard_interleaved(const uint16_t* grads, int32_t fan_in, int64_t n,
                                       float scale, float* out, int32_t accumulate,
                                       void* stream) {
    if (grads == nullptr || (accumulate != 0 && accumulate != 1)) return FSDPSHARD_ERR_INVALID_ARG;
    return launch_reduce(nullptr, fan_in, n, scale, out, accumulate != 0, stream, grads);
}

extern "C" int64_t grad_sumsq_workspace_bytes(int64_t n) {
    if (n < 0) return -1;
    return sumsq_partials(n) * static_cast<int64_t>(sizeof(double));
}

namespace {

// Checks of grad_sumsq_shard's inputs and result pointer shared by its two entry points.
int check_sumsq_args(const uint16_t* const* contribs, int32_t fan_in, const float* grad, int64_t n,
                     const fsdpshard_segment* segs, int32_t n_segments, double* sumsq,
                     int64_t* parts) {
    if (n < 0 || sumsq == nullptr || n_segments < 0 || (n_segments > 0 && segs == nullptr))
        return FSDPSHARD_ERR_INVALID_ARG;
    if (fan_in == 0) {
        if (grad == nullptr) return FSDPSHARD_ERR_INVALID_ARG;
        if (!aligned16(grad)) return FSDPSHARD_ERR_ALIGNMENT;
    } else {
        const int rc = check_contribs(contribs, fan_in);
        if (rc != FSDPSHARD_OK) return rc;
    }
    if (!aligned8(sumsq)) return FSDPSHARD_ERR_ALIGNMENT;
    if (segs != nullptr && !aligned8(segs)) return FSDPSHARD_ERR_ALIGNMENT;
    if (n > INT64_MAX / 4) return FSDPSHARD_ERR_OVERFLOW;
    *parts = sumsq_partials(n);
    if (*parts > 0x7FFFFFFF) return FSDPSHARD_ERR_OVERFLOW;
    return FSDPSHARD_OK;
}

// The written buffers (the partials when they are the caller's, and sumsq) must not overlap
// each other or an input.
int check_sumsq_overlaps(const uint16_t* const* contribs, int32_t fan_in, const float* grad,
                         int64_t n, const fsdpshard_segment* segs, int32_t n_segments,
                         const void* workspace, int64_t need, const double* sumsq) {
    const void* wr[2] = {workspace, sumsq};
    const int64_t wb[2] = {need, 8};
    const int64_t sb = seg_bytes(segs, n_segments);
    if (overlaps(wr[0], wb[0], wr[1], wb[1])) return FSDPSHARD_ERR_INVALID_ARG;
    for (int i = 0; i < 2 && n > 0; ++i) {
        if (fan_in == 0) {
            if (overlaps(wr[i], wb[i], grad, n * 4)) return FSDPSHARD_ERR_INVALID_ARG;
        } else {
            for (int r = 0; r < fan_in; ++r)
                if (overlaps(wr[i], wb[i], contribs[r], n * 2)) return FSDPSHARD_ERR_INVALID_ARG;
        }
        if (overlaps(wr[i], wb[i], segs, sb)) return FSDPSHARD_ERR_INVALID_ARG;
    }
    return FSDPSHARD_OK;
}

// The two kernels of the sum of squares: one float64 partial per work-group into `partials`,
// then their fixed-order sum into *sumsq.
// Work-groups per CU of sumsq_kernel (see occupancy_lds; 0 = uncapped).  Measured on one GPU at
// 2^25..2^29.75 elements, caps 1-4 against uncapped, 4 alternating rounds: uncapped is best for
// one, two, three and sixteen contributions and for an fp32 gradient (every cap 1-4 is 0-330 %
// slower at 2^28 and above); four contributions do 0.4-3.6 % better with 2; eight do 2.4 %
// better with 1 from 8,192 work-groups (2^28 elements) up.  Against uncapped in a second run:
// 1-3 % faster for four and eight contributions at 2^28 and above, within 1 % at 2^25.
inline int sumsq_groups_per_cu(int32_t fan_in, int64_t work_groups) {
    if (fan_in == 4) return 2;
    if (fan_in == 8) return work_groups >= 8192 ? 1 : 0;
    return 0;
}

// fan_in 0 selects the fp32 gradient `grad`; with `interleaved`, the fan_in contributions are
// read from that one interleaved array (contribs unused).
int launch_sumsq(const uint16_t* const* contribs, int32_t fan_in, const float* grad, int64_t n,
                 const fsdpshard_segment* segs, int32_t n_segments, float scale, double* partials,
                 int64_t parts, double* sumsq, void* stream,
                 const uint16_t* interleaved = nullptr) {
    SumsqParams p;
    for (int r = 0; r < FSDPSHARD_MAX_FAN_IN; ++r)
        p.contrib[r] = (interleaved == nullptr && fan_in > 0 && r < fan_in) ? contribs[r] : nullptr;
    if (interleaved != nullptr) p.contrib[0] = interleaved;
    p.grad32 = fan_in == 0 ? grad : nullptr;
    p.segs = segs;
    p.partials = partials;
    p.result = sumsq;
    p.n = n;
    p.groups_per_wave = kSumsqGroups;
    p.n_segs = segs == nullptr ? 0 : n_segments;
    p.fan_in = fan_in;
    p.n_partials = static_cast<int32_t>(parts);
    p.scale = scale;
    if (parts > 0) {
        const void* k =
            interleaved != nullptr
                ? (fan_in == 1   ? reinterpret_cast<const void*>(&sumsq_interleaved_kernel<1>)
                   : fan_in == 4 ? reinterpret_cast<const void*>(&sumsq_interleaved_kernel<4>)
                   : fan_in == 8 ? reinterpret_cast<const void*>(&sumsq_interleaved_kernel<8>)
                                 : reinterpret_cast<const void*>(&sumsq_interleaved_kernel<0>))
            : fan_in == 0 ? reinterpret_cast<const void*>(&sumsq_kernel<-1>)
            : fan_in == 1 ? reinterpret_cast<const void*>(&sumsq_kernel<1>)
            : fan_in == 4 ? reinterpret_cast<const void*>(&sumsq_kernel<4>)
            : fan_in == 8 ? reinterpret_cast<const void*>(&sumsq_kernel<8>)
                          : reinterpret_cast<const void*>(&sumsq_kernel<0>);
        const int rc = launch(k, static_cast<unsigned>(parts), &p, stream,
                              sumsq_groups_per_cu(fan_in, parts));
        if (rc != FSDPSHARD_OK) return rc;
    }
    // One work-group adds the partials (or writes +0 for an empty slice).
    return launch(reinterpret_cast<const void*>(&sumsq_finish_kernel), 1, &p, stream);
}

}  // namespace

extern "C" int grad_sumsq_shard(const uint16_t* const* contribs, int32_t fan_in,
                                const float* grad, int64_t n, const fsdpshard_segment* segs,
                                int32_t n_segments, float scale, void* workspace,
                                int64_t workspace_bytes, double* sumsq, void* stream) {
    int64_t parts = 0;
    int rc = check_sumsq_args(contribs, fan_in, grad, n, segs, n_segments, sumsq, &parts);
    if (rc != FSDPSHARD_OK) return rc;
    const int64_t need = parts * static_cast<int64_t>(sizeof(double));
    if (parts > 0 && (workspace == nullptr || workspace_bytes < need))
        return FSDPSHARD_ERR_CAPACITY;
    if (parts > 0 && !aligned8(workspace)) return FSDPSHARD_ERR_ALIGNMENT;
    rc = check_sumsq_overlaps(contribs, fan_in, grad, n, segs, n_segments,
                              parts > 0 ? workspace : nullptr, need, sumsq);
    if (rc != FSDPSHARD_OK) return rc;
    return launch_sumsq(contribs, fan_in, grad, n, segs, n_segments, scale,
                        static_cast<double*>(workspace), parts, sumsq, stream);
}

extern "C" int grad_sumsq_shard_interleaved(const uint16_t* grads, int32_t fan_in, int64_t n,
                                            const fsdpshard_segment* segs, int32_t n_segments,
                                            float scale, void* workspace, int64_t workspace_bytes,
                                            double* sumsq, void* stream) {
    if (grads == nullptr || fan_in < 1) return FSDPSHARD_ERR_INVALID_ARG;
    if (fan_in > FSDPSHARD_MAX_FAN_IN) return FSDPSHARD_ERR_UNSUPPORTED;
    // The interleaved array is checked as one input of grads_interleaved_elems elements.
    const uint16_t* one[1] = {grads};
    int64_t parts = 0;
    int rc = check_sumsq_args(one, 1, nullptr, n, segs, n_segments, sumsq, &parts);
    if (rc != FSDPSHARD_OK) return rc;
    const int64_t elems = interleaved_elems(fan_in, n);
    if (elems < 0) return FSDPSHARD_ERR_OVERFLOW;
    const int64_t need = parts * static_cast<int64_t>(sizeof(double));
    if (parts > 0 && (workspace == nullptr || workspace_bytes < need))
        return FSDPSHARD_ERR_CAPACITY;
    if (parts > 0 && !aligned8(workspace)) return FSDPSHARD_ERR_ALIGNMENT;
    rc = check_sumsq_overlaps(one, 1, nullptr, elems, segs, n_segments,
                              parts > 0 ? workspace : nullptr, need, sumsq);
    if (rc != FSDPSHARD_OK) return rc;
    return launch_sumsq(nullptr, fan_in, nullptr, n, segs, n_segments, scale,
                        static_cast<double*>(workspace), parts, sumsq, stream, grads);
}

// ------------------------------------------------------------------------------------------------
// grad_sumsq_shard without a caller workspace, for callers that cannot allocate device memory.
// The float64 partials go to `scratch`, a library-owned array in each device's global segment
// (one copy per GPU, held until the process ends).  In host code `scratch` names a host-side
// stand-in, never the device array: kernels receive the device address that hipGetSymbolAddress
// returned for the device the call runs on, looked up once per device and kept.

static __device__ __align__(256) double scratch[FSDPSHARD_NOALLOC_MAX_PARTIALS];

namespace {

std::mutex g_scratch_mutex;
double* g_scratch_addr[kMaxDevices];   // device address of `scratch` per device; null until set

// Device of `stream` (the null stream: the current device).
int stream_device(void* stream, int* dev) {
    if (stream != nullptr) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &d) != hipSuccess)
            return FSDPSHARD_ERR_HIP;
        *dev = d;
        return FSDPSHARD_OK;
    }
    return hipGetDevice(dev) == hipSuccess ? FSDPSHARD_OK : FSDPSHARD_ERR_HIP;
}

// The device address of `scratch` on device `dev`: on the first call for that device, looked up
// with that device current (then the caller's current device is restored).
int scratch_address(int dev, double** out) {
    if (dev < 0 || dev >= kMaxDevices) return FSDPSHARD_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_addr[dev] == nullptr) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return FSDPSHARD_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return FSDPSHARD_ERR_HIP;
        void* addr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return FSDPSHARD_ERR_HIP;
        if (e != hipSuccess || addr == nullptr) return FSDPSHARD_ERR_HIP;
        g_scratch_addr[dev] = static_cast<double*>(addr);
    }
    *out = g_scratch_addr[dev];
    return FSDPSHARD_OK;
}

}  // namespace

extern "C" int grad_sumsq_shard_noalloc(const uint16_t* const* contribs, int32_t fan_in,
                                        const float* grad, int64_t n,
                                        const fsdpshard_segment* segs, int32_t n_segments,
                                        float scale, double* sumsq, void* stream) {
    int64_t parts = 0;
    int rc = check_sumsq_args(contribs, fan_in, grad, n, segs, n_segments, sumsq, &parts);
    if (rc != FSDPSHARD_OK) return rc;
    if (parts > FSDPSHARD_NOALLOC_MAX_PARTIALS) return FSDPSHARD_ERR_CAPACITY;
    rc = check_sumsq_overlaps(contribs, fan_in, grad, n, segs, n_segments, nullptr, 0, sumsq);
    if (rc != FSDPSHARD_OK) return rc;
    int dev = 0;
    rc = stream_device(stream, &dev);
    if (rc != FSDPSHARD_OK) return rc;
    double* partials = nullptr;
    rc = scratch_address(dev, &partials);
    if (rc != FSDPSHARD_OK) return rc;
    return launch_sumsq(contribs, fan_in, grad, n, segs, n_segments, scale, partials, parts, sumsq,
                        stream);
}

namespace {

template <int F>
const void* reduce_sq_kernel_for(bool acc, bool interleaved) {
    if (interleaved)
        return acc ? reinterpret_cast<const void*>(&reduce_sumsq_interleaved_kernel<F, true>)
                   : reinterpret_cast<const void*>(&reduce_sumsq_interleaved_kernel<F, false>);
    return acc ? reinterpret_cast<const void*>(&reduce_sumsq_kernel<F, true>)
               : reinterpret_cast<const void*>(&reduce_sumsq_kernel<F, false>);
}

// reduce_shard_sumsq from F separate arrays, or from the interleaved array when `interleaved`
// is non-null (contribs unused).
int launch_reduce_sumsq(const uint16_t* const* contribs, const uint16_t* interleaved,
                        int32_t fan_in, int64_t n, float scale, float* out, int32_t accumulate,
                        const fsdpshard_segment* segs, int32_t n_segments, void* workspace,
                        int64_t workspace_bytes, double* sumsq, void* stream) {
    if (out == nullptr || n < 0 || sumsq == nullptr || n_segments < 0 ||
        (n_segments > 0 && segs == nullptr) || (accumulate != 0 && accumulate != 1))
        return FSDPSHARD_ERR_INVALID_ARG;
    int64_t il_elems = 0;
    int rc = check_grad_source(contribs, interleaved, fan_in, n, &il_elems);
    if (rc != FSDPSHARD_OK) return rc;
    if (!aligned16(out)) return FSDPSHARD_ERR_ALIGNMENT;
    if (!aligned8(sumsq)) return FSDPSHARD_ERR_ALIGNMENT;
    if (segs != nullptr && !aligned8(segs)) return FSDPSHARD_ERR_ALIGNMENT;
    if (n > INT64_MAX / 4) return FSDPSHARD_ERR_OVERFLOW;
    const int64_t parts = sumsq_partials(n);
    if (parts > 0x7FFFFFFF) return FSDPSHARD_ERR_OVERFLOW;
    const int64_t need = parts * static_cast<int64_t>(sizeof(double));
    if (parts > 0 && (workspace == nullptr || workspace_bytes < need)) return FSDPSHARD_ERR_CAPACITY;
    if (parts > 0 && !aligned8(workspace)) return FSDPSHARD_ERR_ALIGNMENT;
    // The three written buffers (out, workspace, sumsq) must not overlap each other or an input.
    const void* wr[3] = {n > 0 ? out : nullptr, parts > 0 ? workspace : nullptr, sumsq};
    const int64_t wb[3] = {n * 4, need, 8};
    const int64_t sb = seg_bytes(segs, n_segments);
    for (int i = 0; i < 3; ++i) {
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(wr[i], wb[i], wr[j], wb[j])) return FSDPSHARD_ERR_INVALID_ARG;
        if (n > 0 && overlaps_grad_source(wr[i], wb[i], contribs, interleaved, fan_in, n, il_elems))
            return FSDPSHARD_ERR_INVALID_ARG;
        if (overlaps(wr[i], wb[i], segs, sb)) return FSDPSHARD_ERR_INVALID_ARG;
    }
    ReduceSqParams p;
    for (int r = 0; r < FSDPSHARD_MAX_FAN_IN; ++r)
        p.contrib[r] = (interleaved == nullptr && r < fan_in) ? contribs[r] : nullptr;
    if (interleaved != nullptr) p.contrib[0] = interleaved;
    p.out = out;
    p.segs = segs;
    p.partials = static_cast<double*>(workspace);
    p.n = n;
    p.n_segs = segs == nullptr ? 0 : n_segments;
    p.fan_in = fan_in;
    p.scale = scale;
    if (parts > 0) {
        const bool acc = accumulate != 0;
        const bool il = interleaved != nullptr;
        const void* k = nullptr;
        bool pipelined = false;
        switch (fan_in) {
#define FSDPSHARD_REDUCE_SQ_CASE(FI)                                                            \
    case FI:                                                                                    \
        k = reduce_sq_kernel_for<FI>(acc, il);                                                  \
        pipelined = acc ? reduce_sq_pipelined<FI, true>() : reduce_sq_pipelined<FI, false>();   \
        break;
            FSDPSHARD_REDUCE_SQ_CASE(1)
            FSDPSHARD_REDUCE_SQ_CASE(2)
            FSDPSHARD_REDUCE_SQ_CASE(4)
            FSDPSHARD_REDUCE_SQ_CASE(8)
#undef FSDPSHARD_REDUCE_SQ_CASE
            default:
                k = reduce_sq_kernel_for<0>(acc, il);
        }
        rc = launch(k, static_cast<unsigned>(parts), &p, stream,
                    pipelined                ? kReduceSqPipelinedGroupsPerCU
                    : fan_in == 1 && !acc    ? kReduceOneStreamSqGroupsPerCU
                                             : kReduceSqGroupsPerCU);
        if (rc != FSDPSHARD_OK) return rc;
    }
    SumsqParams f;
    for (int r = 0; r < FSDPSHARD_MAX_FAN_IN; ++r) f.contrib[r] = nullptr;
    f.grad32 = nullptr;
    f.segs = nullptr;
    f.partials = static_cast<double*>(workspace);
    f.result = sumsq;
    f.n = n;
    f.groups_per_wave = kSumsqGroups;
    f.n_segs = 0;
    f.fan_in = 0;
    f.n_partials = static_cast<int32_t>(parts);
    f.scale = 1.0f;
    // One work-group adds the partials (or writes +0 for an empty slice).
    return launch(reinterpret_cast<const void*>(&sumsq_finish_kernel), 1, &f, stream);
}

}  // namespace

extern "C" int reduce_shard_sumsq(const uint16_t* const* contribs, int32_t fan_in, int64_t n,
                                 float scale, float* out, int32_t accumulate,
                                 const fsdpshard_segment* segs, int32_t n_segments,
                                 void* workspace, int64_t workspace_bytes, double* sumsq,
                                 void* stream) {
    return launch_reduce_sumsq(contribs, nullptr, fan_in, n, scale, out, accumulate, segs,
                               n_segments, workspace, workspace_bytes, sumsq, stream);
}

extern "C" int reduce_shard_sumsq_interleaved(const uint16_t* grads, int32_t fan_in, int64_t n,
                                             float scale, float* out, int32_t accumulate,
                                             const fsdpshard_segment* segs, int32_t n_segments,
                                             void* workspace, int64_t workspace_bytes,
                                             double* sumsq, void* stream) {
    if (grads == nullptr) return FSDPSHARD_ERR_INVALID_ARG;
    return launch_reduce_sumsq(nullptr, grads, fan_in, n, scale, out, accumulate, segs,
                               n_segments, workspace, workspace_bytes, sumsq, stream);
}

extern "C" int unflatten_bf16(const float* master, int64_t n, const fsdpshard_segment* segs,
                              int32_t n_segments, uint16_t* flat_bf16, int64_t flat_index0,
                              int64_t lo, void* stream) {
    if (master == nullptr || flat_bf16 == nullptr || n < 0 || n_segments < 0 ||
        (n_segments > 0 && segs == nullptr) || lo < 0 || flat_index0 > lo)
        return FSDPSHARD_ERR_INVALID_ARG;
    if (!aligned16(master) || (reinterpret_cast<uintptr_t>(flat_bf16) & 1u) != 0)
        return FSDPSHARD_ERR_ALIGNMENT;
    if (segs != nullptr && !aligned8(segs)) return FSDPSHARD_ERR_ALIGNMENT;
    if (n > INT64_MAX / 4) return FSDPSHARD_ERR_OVERFLOW;
    uint16_t* out = flat_bf16 + (lo - flat_index0);
    if (n == 0) return FSDPSHARD_OK;
    if (overlaps(out, n * 2, master, n * 4) || overlaps(out, n * 2, segs, seg_bytes(segs, n_segments)))
        return FSDPSHARD_ERR_INVALID_ARG;
    UnflattenParams p;
    p.master = master;
    p.segs = segs;
    p.out = out;
    p.n = n;
    p.n_segs = segs == nullptr ? 0 : n_segments;
    p.out_shift = out_shift_of(out);
    unsigned blocks = 0;
    int rc = tile_grid(n, 1, &blocks);
    if (rc != FSDPSHARD_OK) return rc;
    return launch(reinterpret_cast<const void*>(&unflatten_kernel), blocks, &p, stream);
}
