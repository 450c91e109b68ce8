// Private header of libfsdpshard.so: pieces shared by the step kernels (shard_step.hip) and the
// measurement aids (calib.hip).  Not installed; the C ABI is include/fsdpshard.h.
//
// Every kernel here is a stream over 16-byte vectors.  One lane owns 8 consecutive elements (one
// 16-byte vector of a bf16 stream, two of an fp32 stream); one 64-lane wavefront covers a
// 512-element group; a 256-thread work-group covers 4 consecutive groups (a tile).
#ifndef FSDPSHARD_STREAM_COMMON_H
#define FSDPSHARD_STREAM_COMMON_H

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "fsdpshard.h"

namespace fsdpshard_detail {

constexpr int kVec = 8;            // elements per lane
constexpr int kWave = 64;          // lanes per wavefront
// Threads per work-group: 4 waves.  Measured on MI355X for the fused step (7B- and 70B-shaped
// slices, per-CU cap and XCD run rescaled): 2-, 3- and 8-wave work-groups at 6-12 waves per CU
// were 1-18 % slower than 4-wave ones at 2 per CU.
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int64_t kStateBlock = FSDPSHARD_STATE_BLOCK;

// ------------------------------------------------------------------------------------------------
// Device helpers.

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_u4(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ float4 ld_f4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}

// Non-temporal forms for single-use streams (global_load / global_store with the nt bit).
__device__ __forceinline__ uint4 ld_u4_nt(const uint16_t* p) {
    const u32x4_t r = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(r.x, r.y, r.z, r.w);
}
__device__ __forceinline__ void ld8_f32_nt(const float* p, float (&x)[8]) {
    const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 4));
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void st_f4_nt(float* p, float a, float b, float c, float d) {
    const f32x4_t v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void st_u4_nt(uint16_t* p, uint4 x) {
    const u32x4_t v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// 8 floats: two 16-byte loads when the vector is whole, else the first `cnt` elements (zeros after).
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

// 8 floats: two non-temporal 16-byte stores when whole, else the first `cnt` elements.
__device__ __forceinline__ void store8(float* p, bool full, int cnt, const float (&x)[kVec]) {
    if (full) {
        st_f4_nt(p, x[0], x[1], x[2], x[3]);
        st_f4_nt(p + 4, x[4], x[5], x[6], x[7]);
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (e < cnt) p[e] = x[e];
    }
}

// Blocked state layout: element e0 (a multiple of 8) of state array k (0 master, 1 m, 2 v) in
// one array whose blocks of kStateBlock slice elements hold the block's masters, then its m,
// then its v (an 8-element vector never straddles a block).
__device__ __forceinline__ int64_t blocked_index(int k, int64_t e0) {
    return ((e0 / kStateBlock) * 3 + k) * kStateBlock + e0 % kStateBlock;
}

// Work-group -> tile.  MI355X deals a launch's work-groups to its 8 XCDs in turn, so with the
// identity map neighbouring tiles run on different XCDs at the same moment.  Here work-group b on
// XCD x = b mod 8 takes the (b / 8 mod Run)-th tile of the x-th run of Run consecutive tiles in
// each block of 8 * Run tiles: every XCD streams its own run of tiles.  Work-groups past the last
// whole block keep the identity map, so the map is a permutation of [0, gridDim.x) for any grid.
// Measured on one GPU against the identity map, with runs of 64 tiles (512 KiB of each fp32
// stream): the fused step 3-4 % faster on the 7B-shaped slice and 0.4-1.4 % on the 70B-shaped
// one, the fp32 accumulation 2-5 % faster; runs of 8 or 96 tiles were slower than 64 or 128.  With
// the cap on work-groups per CU (launch), the fused step does 0.5-1 % better with runs of 32 tiles
// on the large slices, while the reduction keeps 64 (2 % better than 32).  Results never depend
// on the map: a tile's work is the same wherever it runs.
constexpr int64_t kXcds = 8;
constexpr int64_t kXcdRun = 64;       // reduction, unflatten
constexpr int64_t kStepXcdRun = 32;   // fused step and its traffic replicas

template <int64_t Run = kXcdRun>
__device__ __forceinline__ int64_t tile_index() {
    const int64_t b = blockIdx.x;
    const int64_t whole = static_cast<int64_t>(gridDim.x) / (kXcds * Run) * (kXcds * Run);
    if (b >= whole) return b;
    const int64_t x = b % kXcds, q = b / kXcds;
    return (q / Run) * (kXcds * Run) + x * Run + q % Run;
}

// First vector of wave `wave`'s tile when each wave owns `groups` consecutive groups.
template <int64_t Run = kXcdRun>
__device__ __forceinline__ int64_t tile_base(int wave, int groups) {
    return (tile_index<Run>() * kWavesPerBlock + wave) * (kWave * groups);
}

// ------------------------------------------------------------------------------------------------
// Host helpers.

// One work-group of 4 waves per 4 * groups * 64 vectors of 8 elements.
inline int tile_grid(int64_t n, int groups, unsigned* blocks) {
    const int64_t nvec = (n + kVec - 1) / kVec;
    const int64_t per_block = static_cast<int64_t>(kWavesPerBlock) * kWave * groups;
    const int64_t b = (nvec + per_block - 1) / per_block;
    if (b > 0x7FFFFFFF) return FSDPSHARD_ERR_OVERFLOW;
    *blocks = static_cast<unsigned>(b);
    return FSDPSHARD_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

inline bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (a == nullptr || b == nullptr || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + static_cast<uintptr_t>(bbytes) && y < x + static_cast<uintptr_t>(abytes);
}

// Elements of a blocked state array for an n-element slice (-1 when it does not fit int64).
inline int64_t blocked_elems(int64_t n) {
    if (n < 0 || n > INT64_MAX / 16) return -1;
    return 3 * ((n + kStateBlock - 1) / kStateBlock) * kStateBlock;
}

// Elements of a buffer holding fan_in contributions of an n-element slice interleaved per block
// of kStateBlock elements (-1 when its size in bytes does not fit int64 or fan_in is out of range).
inline int64_t interleaved_elems(int32_t fan_in, int64_t n) {
    if (n < 0 || fan_in < 1 || fan_in > FSDPSHARD_MAX_FAN_IN) return -1;
    const int64_t blocks = n / kStateBlock + (n % kStateBlock != 0 ? 1 : 0);
    if (blocks > INT64_MAX / (2 * kStateBlock * fan_in)) return -1;
    return blocks * kStateBlock * fan_in;
}

inline int check_contribs(const uint16_t* const* contribs, int32_t fan_in) {
    if (contribs == nullptr || fan_in < 1) return FSDPSHARD_ERR_INVALID_ARG;
    if (fan_in > FSDPSHARD_MAX_FAN_IN) return FSDPSHARD_ERR_UNSUPPORTED;
    for (int r = 0; r < fan_in; ++r) {
        if (contribs[r] == nullptr) return FSDPSHARD_ERR_INVALID_ARG;
        if (!aligned16(contribs[r])) return FSDPSHARD_ERR_ALIGNMENT;
    }
    return FSDPSHARD_OK;
}

// Resident work-groups per CU.  The streaming kernels lose bandwidth when every CU holds as
// many work-groups as its registers allow: with fewer waves in flight the HBM sees fewer
// concurrent access streams.  The cap is set by reserving LDS that the kernels never touch (a
// dynamic LDS size at launch), sized from the device's LDS per CU so that exactly `per_cu`
// work-groups fit: halfway between lds/(per_cu+1) and lds/per_cu, which leaves room for the few
// bytes of static LDS a kernel declares itself.
//
// The fused step takes 2 or 3 per CU by its gradient source and the size of the launch.  With
// few gradient streams a third work-group per CU keeps more requests in flight through the ramp
// and tail of a short launch; in a long one the steady state dominates, and there the extra
// streams cost more than they bring.  Measured on one GPU (blocked and separate state, slices of
// 2^23..2^28 elements, 4 alternating rounds of 10 launches per point, a cache flush before each
// launch that moves under 2 GB), 3 against 2 per CU:
//   fan-in 2 and 4:      1-5 % faster up to 32,768 work-groups, 2-8 % slower from 65,536;
//   fp32 gradient:       2-5 % faster up to 32,768 (65,536 separate), 2 % slower at 131,072;
//   fan-in 3 (run-time): 1-10 % faster up to 65,536, 1.5 % slower at 131,072;
//   fan-in 16:           2 % faster up to 8,192, 3-8 % slower from 32,768;
//   fan-in 8:            4 % faster at 4,096, 3-11 % slower from 16,384;
//   fan-in 1:            2-10 % slower at every size (blocked state).
// three_up_to is the largest launch, in work-groups, that still takes 3.
inline int step_groups_per_cu(int fan_in, int64_t work_groups) {
    int64_t three_up_to;
    switch (fan_in) {
        case 1: three_up_to = 0; break;
        case 8: three_up_to = 4096; break;
        case 2:
        case 4: three_up_to = 32768; break;
        case -1: three_up_to = 65536; break;                              // fp32 gradient
        default: three_up_to = fan_in < 8 ? 65536 : 8192; break;          // run-time fan-in loop
    }
    return work_groups <= three_up_to ? 3 : 2;
}

constexpr int kMaxDevices = 64;
inline std::atomic<int64_t> g_lds_per_cu[kMaxDevices];   // 0: not queried yet; -1: unknown

inline int64_t lds_per_cu() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    int64_t v = g_lds_per_cu[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int bytes = 0;
        const hipError_t e = hipDeviceGetAttribute(
            &bytes, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
        v = (e == hipSuccess && bytes > 0) ? bytes : -1;
        g_lds_per_cu[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Dynamic LDS bytes that leave room for exactly `per_cu` work-groups (0: no cap).
inline size_t occupancy_lds(int per_cu) {
    if (per_cu <= 0) return 0;
    const int64_t lds = lds_per_cu();
    if (lds <= 0) return 0;
    const int64_t bytes = (lds / (per_cu + 1) + lds / per_cu) / 2;
    return static_cast<size_t>(bytes & ~static_cast<int64_t>(1023));
}

inline int launch(const void* kernel, unsigned blocks, void* params, void* stream, int per_cu = 0) {
    void* args[] = {params};
    const hipError_t e = hipLaunchKernel(kernel, dim3(blocks), dim3(kBlock), args,
                                         occupancy_lds(per_cu), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FSDPSHARD_OK : FSDPSHARD_ERR_HIP;
}

}  // namespace fsdpshard_detail

#endif  // FSDPSHARD_STREAM_COMMON_H
