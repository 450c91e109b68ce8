// Measurement aids of libfsdpshard.so (declared in include/fsdpshard_calib.h).  None of these is
// part of the sharded step; they bound what the memory system allows for the step's traffic.
//
//   * stream_copy_kernel   one read and one write stream (the classic copy).
//   * stream_rw_kernel     R read streams and W write streams of equal length: pure reads
//                          (W = 0), pure writes (R = 0), a copy (1, 1), or the 2 : 1 read : write
//                          byte ratio of the fused step at fan-in 8 (2, 1), any of them with a
//                          write stream that is one of the read streams (read and written in
//                          place, as the step's state), in any launch shape (vectors per thread,
//                          threads per work-group, work-groups per CU, XCD run length).
//   * stream_mix_kernel    the fused step's exact loads and stores (same vector width, cache
//                          hints, tile map, load issue order and work-groups per CU) with
//                          trivial integer arithmetic in place of the reduction and the update;
//                          stream_mix_interleaved_kernel the same for the step fed by
//                          contributions interleaved in one array.
//   * stream_mix_shaped_kernel
//                          the same bytes as the blocked-state step in other shapes: G groups
//                          per wave, any work-groups per CU and XCD run, and optionally in phases
//                          (the work-group meets at a barrier after its loads, before any store;
//                          with one work-group per CU a CU alternates between a pure-read and a
//                          pure-write phase).
//
// Every kernel checks each vector index against the stream length, so any grid is safe.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fsdpshard.h"
#include "fsdpshard_calib.h"
#include "stream_common.h"

namespace {

using namespace fsdpshard_detail;

__global__ __launch_bounds__(kBlock) void stream_copy_kernel(const uint4* __restrict__ src,
                                                             uint4* __restrict__ dst,
                                                             int64_t nvec) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= nvec) return;
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + i));
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst + i));
}

// ------------------------------------------------------------------------------------------------
// Work-group -> tile with a run length chosen at launch (the library kernels fix theirs at
// compile time): run <= 1 is the identity, otherwise each XCD streams runs of `run` tiles.
__device__ __forceinline__ int64_t tile_index_rt(int64_t run) {
    const int64_t b = blockIdx.x;
    if (run <= 1) return b;
    const int64_t whole = static_cast<int64_t>(gridDim.x) / (kXcds * run) * (kXcds * run);
    if (b >= whole) return b;
    const int64_t x = b % kXcds, q = b / kXcds;
    return (q / run) * (kXcds * run) + x * run + q % run;
}

inline int launch_shaped(const void* kernel, unsigned blocks, int threads, void* params,
                         void* stream, int per_cu) {
    void* args[] = {params};
    const hipError_t e = hipLaunchKernel(kernel, dim3(blocks), dim3(threads), args,
                                         occupancy_lds(per_cu), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FSDPSHARD_OK : FSDPSHARD_ERR_HIP;
}

// ------------------------------------------------------------------------------------------------
// R read streams, W write streams.

constexpr int kRwMaxStreams = FSDPSHARD_CALIB_MAX_STREAMS;
constexpr uint32_t kSinkMagic = 0x9E3779B9u;

struct RwParams {
    const u32x4_t* src[kRwMaxStreams];
    u32x4_t* dst[kRwMaxStreams];
    uint32_t* sink;
    int64_t nvec;
    int64_t run;
    int32_t n_src, n_dst;
};

// Thread t of the work-group on tile b handles vectors b * T * V + u * T + t, u < V (T threads
// per work-group, V vectors per thread), of every stream: all loads first, then the XOR of the
// loaded words (mixed with the index) to every write stream.  A vector is read and written by the
// same thread only, loads before stores, so a write stream may be one of the read streams.  With no write stream, a lane whose
// XOR equals a fixed constant stores it to `sink`, so the loads cannot be dropped and almost no
// bytes are written.
template <int V>
__global__ __launch_bounds__(1024) void stream_rw_kernel(RwParams p) {
    const int64_t T = blockDim.x;
    const int64_t base = tile_index_rt(p.run) * T * V + threadIdx.x;
    u32x4_t x[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const uint32_t i32 = static_cast<uint32_t>(base + u * T);
        x[u] = u32x4_t{i32, i32 ^ 0x55555555u, i32 ^ 0x33333333u, i32 ^ 0x0F0F0F0Fu};
    }
#pragma unroll
    for (int r = 0; r < kRwMaxStreams; ++r) {
        if (r >= p.n_src) break;
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int64_t i = base + u * T;
            if (i < p.nvec) x[u] ^= __builtin_nontemporal_load(p.src[r] + i);
        }
    }
    if (p.n_dst == 0) {
#pragma unroll
        for (int u = 0; u < V; ++u)
            if ((x[u].x ^ x[u].y ^ x[u].z ^ x[u].w) == kSinkMagic) *p.sink = x[u].x;
        return;
    }
#pragma unroll
    for (int w = 0; w < kRwMaxStreams; ++w) {
        if (w >= p.n_dst) break;
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int64_t i = base + u * T;
            if (i < p.nvec) {
                u32x4_t y = x[u];
                y.x += static_cast<uint32_t>(w);
                __builtin_nontemporal_store(y, p.dst[w] + i);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Replicas of the fused step's traffic.

struct MixParams {
    const uint16_t* contrib[FSDPSHARD_MAX_FAN_IN];
    float* s[3];
    uint16_t* out;
    int64_t nvec;
    int64_t run;             // XCD run length of the shaped replica
    int32_t fan_in;
};

// One 512-element group per wave, exactly as the step: F non-temporal bf16 loads (from F arrays,
// or with GIL from one array interleaved per 512-element block: contribution r's element i at
// ((i / 512) * F + r) * 512 + i % 512), three fp32 read-modify-write streams (separate, or the
// blocked array in s[0]), one bf16 store per 8-element vector.
template <int F, bool BLK, bool GIL>
__device__ __forceinline__ const uint16_t* mix_src(const MixParams& p, int r, int64_t e0) {
    if constexpr (GIL) {
        const uint64_t u = static_cast<uint64_t>(e0);
        const int64_t fan_in = F > 0 ? F : p.fan_in;
        return p.contrib[0] + (static_cast<int64_t>(u / kStateBlock) * fan_in + r) * kStateBlock +
               static_cast<int64_t>(u % kStateBlock);
    } else {
        return p.contrib[r] + e0;
    }
}

template <int F, bool BLK, bool GIL>
__device__ __forceinline__ void stream_mix_body(MixParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t vec = tile_base<kStepXcdRun>(wave, 1) + lane;
    if (vec >= p.nvec) return;
    const int64_t e0 = vec * kVec;
    const int fan_in = F > 0 ? F : p.fan_in;
    uint4 raw[F > 0 ? F : 1];
    float st[3][kVec];
    uint32_t x = 0;
    float* sp[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) sp[k] = BLK ? p.s[0] + blocked_index(k, e0) : p.s[k] + e0;
    // The step's issue order: all state first (blocked state, or one gradient stream), else
    // master and m, then the gradients, then v.
    constexpr bool kStateFirst = BLK || F == 1;
    load8(sp[0], true, kVec, st[0]);
    load8(sp[1], true, kVec, st[1]);
    if constexpr (kStateFirst) load8(sp[2], true, kVec, st[2]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (F > 0) {
#pragma unroll
        for (int r = 0; r < F; ++r) raw[r] = ld_u4_nt(mix_src<F, BLK, GIL>(p, r, e0));
    }
    if constexpr (!kStateFirst) {
        __builtin_amdgcn_sched_barrier(0);
        load8(sp[2], true, kVec, st[2]);
    }
    if constexpr (F > 0) {
#pragma unroll
        for (int r = 0; r < F; ++r) x ^= raw[r].x ^ raw[r].y ^ raw[r].z ^ raw[r].w;
    } else {
        for (int r = 0; r < fan_in; ++r) {
            const uint4 q = ld_u4_nt(mix_src<F, BLK, GIL>(p, r, e0));
            x ^= q.x ^ q.y ^ q.z ^ q.w;
        }
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        st[k][0] = __uint_as_float(__float_as_uint(st[k][0]) ^ x);
        store8(sp[k], true, kVec, st[k]);
    }
    st_u4_nt(p.out + e0, make_uint4(__float_as_uint(st[0][1]), __float_as_uint(st[1][1]),
                                    __float_as_uint(st[2][1]), x));
}

template <int F, bool BLK>
__global__ __launch_bounds__(kBlock) void stream_mix_kernel(MixParams p) {
    stream_mix_body<F, BLK, false>(p);
}

// The replica of the step fed by interleaved contributions (blocked state).
template <int F>
__global__ __launch_bounds__(kBlock) void stream_mix_interleaved_kernel(MixParams p) {
    stream_mix_body<F, true, true>(p);
}

// Blocked-state replica of any shape: wave w owns G consecutive groups and issues every load of
// them (state first, then the contributions), folding all loaded words into one XOR so that it
// holds all its data; with PHASED no wave of the work-group stores before every wave has loaded
// (a work-group barrier), otherwise each wave stores as soon as it can.  Same bytes per element
// as stream_mix_kernel; work-groups take tiles through the XCD map with run length p.run.
template <int F, int G, bool PHASED>
__global__ __launch_bounds__(kBlock) void stream_mix_shaped_kernel(MixParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int64_t base = (tile_index_rt(p.run) * kWavesPerBlock + wave) * (kWave * G);
    float st[G][3][kVec];
    uint4 raw[G][F];
    uint32_t x[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t vec = base + g * kWave + lane;
        x[g] = 0u;
        if (vec < p.nvec) {
            const int64_t e0 = vec * kVec;
#pragma unroll
            for (int k = 0; k < 3; ++k) load8(p.s[0] + blocked_index(k, e0), true, kVec, st[g][k]);
#pragma unroll
            for (int r = 0; r < F; ++r) raw[g][r] = ld_u4_nt(p.contrib[r] + e0);
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (base + g * kWave + lane < p.nvec) {
#pragma unroll
            for (int r = 0; r < F; ++r) x[g] ^= raw[g][r].x ^ raw[g][r].y ^ raw[g][r].z ^ raw[g][r].w;
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int e = 1; e < kVec; ++e) x[g] ^= __float_as_uint(st[g][k][e]);
        }
    }
    if constexpr (PHASED) {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t vec = base + g * kWave + lane;
        if (vec < p.nvec) {
            const int64_t e0 = vec * kVec;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                st[g][k][0] = __uint_as_float(__float_as_uint(st[g][k][0]) ^ x[g]);
                store8(p.s[0] + blocked_index(k, e0), true, kVec, st[g][k]);
            }
            st_u4_nt(p.out + e0, make_uint4(__float_as_uint(st[g][0][1]),
                                            __float_as_uint(st[g][1][1]),
                                            __float_as_uint(st[g][2][1]), x[g]));
        }
    }
}

template <int G, bool PHASED>
const void* shaped_kernel(int fan_in) {
    switch (fan_in) {
        case 1: return reinterpret_cast<const void*>(&stream_mix_shaped_kernel<1, G, PHASED>);
        case 4: return reinterpret_cast<const void*>(&stream_mix_shaped_kernel<4, G, PHASED>);
        case 8: return reinterpret_cast<const void*>(&stream_mix_shaped_kernel<8, G, PHASED>);
        default: return nullptr;
    }
}

// Checks shared by the mix replicas.  With `blocked`, s0 is the blocked state array and s1, s2
// are null.
int check_mix(const uint16_t* const* contribs, int32_t fan_in, float* s0, float* s1, float* s2,
              uint16_t* out, int64_t n, bool blocked) {
    if (s0 == nullptr || (!blocked && (s1 == nullptr || s2 == nullptr)) || out == nullptr ||
        n < 0 || n % kVec)
        return FSDPSHARD_ERR_INVALID_ARG;
    const int rc = check_contribs(contribs, fan_in);
    if (rc != FSDPSHARD_OK) return rc;
    if (!aligned16(s0) || (!blocked && (!aligned16(s1) || !aligned16(s2))) || !aligned16(out))
        return FSDPSHARD_ERR_ALIGNMENT;
    if (n > INT64_MAX / 16) return FSDPSHARD_ERR_OVERFLOW;
    const void* wr[4] = {s0, blocked ? nullptr : s1, blocked ? nullptr : s2, out};
    const int64_t wb[4] = {blocked ? blocked_elems(n) * 4 : n * 4, n * 4, n * 4, n * 2};
    for (int i = 0; i < 4 && n > 0; ++i) {
        if (wr[i] == nullptr) continue;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(wr[i], wb[i], wr[j], wb[j])) return FSDPSHARD_ERR_INVALID_ARG;
        for (int r = 0; r < fan_in; ++r)
            if (overlaps(wr[i], wb[i], contribs[r], n * 2)) return FSDPSHARD_ERR_INVALID_ARG;
    }
    return FSDPSHARD_OK;
}

void fill_mix(MixParams& p, const uint16_t* const* contribs, int32_t fan_in, float* s0, float* s1,
              float* s2, uint16_t* out, int64_t n) {
    for (int r = 0; r < FSDPSHARD_MAX_FAN_IN; ++r) p.contrib[r] = r < fan_in ? contribs[r] : nullptr;
    p.s[0] = s0;
    p.s[1] = s1;
    p.s[2] = s2;
    p.out = out;
    p.nvec = n / kVec;
    p.fan_in = fan_in;
    p.run = 1;
}

int stream_mix_impl(const uint16_t* const* contribs, int32_t fan_in, float* s0, float* s1,
                    float* s2, uint16_t* out, int64_t n, bool blocked, void* stream) {
    int rc = check_mix(contribs, fan_in, s0, s1, s2, out, n, blocked);
    if (rc != FSDPSHARD_OK || n == 0) return rc;
    MixParams p;
    fill_mix(p, contribs, fan_in, s0, s1, s2, out, n);
    unsigned blocks = 0;
    rc = tile_grid(n, 1, &blocks);
    if (rc != FSDPSHARD_OK) return rc;
    const void* k =
        blocked ? (fan_in == 1   ? reinterpret_cast<const void*>(&stream_mix_kernel<1, true>)
                   : fan_in == 8 ? reinterpret_cast<const void*>(&stream_mix_kernel<8, true>)
                                 : reinterpret_cast<const void*>(&stream_mix_kernel<0, true>))
                : (fan_in == 1   ? reinterpret_cast<const void*>(&stream_mix_kernel<1, false>)
                   : fan_in == 8 ? reinterpret_cast<const void*>(&stream_mix_kernel<8, false>)
                                 : reinterpret_cast<const void*>(&stream_mix_kernel<0, false>));
    return launch(k, blocks, &p, stream, step_groups_per_cu(fan_in, blocks));   // as the step
}

}  // namespace

extern "C" int fsdpshard_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (src == nullptr || dst == nullptr || bytes < 0 || (bytes & 15) != 0)
        return FSDPSHARD_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(dst)) return FSDPSHARD_ERR_ALIGNMENT;
    if (overlaps(src, bytes, dst, bytes)) return FSDPSHARD_ERR_INVALID_ARG;
    if (bytes == 0) return FSDPSHARD_OK;
    const int64_t nvec = bytes / 16;
    const int64_t blocks = (nvec + kBlock - 1) / kBlock;
    if (blocks > 0x7FFFFFFF) return FSDPSHARD_ERR_OVERFLOW;
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

extern "C" int fsdpshard_stream_rw(const void* const* src, int32_t n_src, void* const* dst,
                                   int32_t n_dst, int64_t bytes, int32_t vectors_per_thread,
                                   int32_t threads_per_group, int32_t per_cu, int32_t xcd_run,
                                   uint32_t* sink, void* stream) {
    if (n_src < 0 || n_dst < 0 || n_src > kRwMaxStreams || n_dst > kRwMaxStreams ||
        n_src + n_dst == 0 || bytes < 0 || (bytes & 15) != 0 || per_cu < 0 || xcd_run < 0 ||
        (n_src > 0 && src == nullptr) || (n_dst > 0 && dst == nullptr) ||
        (n_dst == 0 && sink == nullptr))
        return FSDPSHARD_ERR_INVALID_ARG;
    const void* k = vectors_per_thread == 1   ? reinterpret_cast<const void*>(&stream_rw_kernel<1>)
                    : vectors_per_thread == 2 ? reinterpret_cast<const void*>(&stream_rw_kernel<2>)
                    : vectors_per_thread == 4 ? reinterpret_cast<const void*>(&stream_rw_kernel<4>)
                                              : nullptr;
    if (k == nullptr || (threads_per_group != 256 && threads_per_group != 512 &&
                         threads_per_group != 1024))
        return FSDPSHARD_ERR_UNSUPPORTED;
    for (int r = 0; r < n_src; ++r) {
        if (src[r] == nullptr) return FSDPSHARD_ERR_INVALID_ARG;
        if (!aligned16(src[r])) return FSDPSHARD_ERR_ALIGNMENT;
    }
    for (int w = 0; w < n_dst; ++w) {
        if (dst[w] == nullptr) return FSDPSHARD_ERR_INVALID_ARG;
        if (!aligned16(dst[w])) return FSDPSHARD_ERR_ALIGNMENT;
        for (int j = w + 1; j < n_dst; ++j)
            if (overlaps(dst[w], bytes, dst[j], bytes)) return FSDPSHARD_ERR_INVALID_ARG;
        for (int r = 0; r < n_src; ++r)   // a destination may be a source itself (in place)
            if (dst[w] != src[r] && overlaps(dst[w], bytes, src[r], bytes))
                return FSDPSHARD_ERR_INVALID_ARG;
    }
    if (sink != nullptr && (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return FSDPSHARD_ERR_ALIGNMENT;
    if (bytes == 0) return FSDPSHARD_OK;
    RwParams p;
    for (int r = 0; r < kRwMaxStreams; ++r) {
        p.src[r] = r < n_src ? static_cast<const u32x4_t*>(src[r]) : nullptr;
        p.dst[r] = r < n_dst ? static_cast<u32x4_t*>(dst[r]) : nullptr;
    }
    p.sink = sink;
    p.nvec = bytes / 16;
    p.run = xcd_run;
    p.n_src = n_src;
    p.n_dst = n_dst;
    const int64_t per_block = static_cast<int64_t>(threads_per_group) * vectors_per_thread;
    const int64_t blocks = (p.nvec + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFF) return FSDPSHARD_ERR_OVERFLOW;
    return launch_shaped(k, static_cast<unsigned>(blocks), threads_per_group, &p, stream, per_cu);
}

extern "C" int fsdpshard_stream_mix(const uint16_t* const* contribs, int32_t fan_in, float* s0,
                                    float* s1, float* s2, uint16_t* out, int64_t n, void* stream) {
    return stream_mix_impl(contribs, fan_in, s0, s1, s2, out, n, false, stream);
}

extern "C" int fsdpshard_stream_mix_blocked(const uint16_t* const* contribs, int32_t fan_in,
                                            float* state, uint16_t* out, int64_t n, void* stream) {
    return stream_mix_impl(contribs, fan_in, state, nullptr, nullptr, out, n, true, stream);
}

extern "C" int fsdpshard_stream_mix_interleaved(const uint16_t* grads, int32_t fan_in,
                                                float* state, uint16_t* out, int64_t n,
                                                void* stream) {
    if (grads == nullptr || state == nullptr || out == nullptr || n < 0 || n % kVec != 0 ||
        fan_in < 1)
        return FSDPSHARD_ERR_INVALID_ARG;
    if (fan_in > FSDPSHARD_MAX_FAN_IN) return FSDPSHARD_ERR_UNSUPPORTED;
    if (!aligned16(grads) || !aligned16(state) || !aligned16(out)) return FSDPSHARD_ERR_ALIGNMENT;
    if (n > INT64_MAX / 16) return FSDPSHARD_ERR_OVERFLOW;
    const int64_t ge = interleaved_elems(fan_in, n);
    if (ge < 0) return FSDPSHARD_ERR_OVERFLOW;
    const int64_t sb = blocked_elems(n) * 4;
    if (n > 0 && (overlaps(state, sb, out, n * 2) || overlaps(state, sb, grads, ge * 2) ||
                  overlaps(out, n * 2, grads, ge * 2)))
        return FSDPSHARD_ERR_INVALID_ARG;
    if (n == 0) return FSDPSHARD_OK;
    MixParams p;
    const uint16_t* one[1] = {grads};
    fill_mix(p, one, 1, state, nullptr, nullptr, out, n);
    p.fan_in = fan_in;
    unsigned blocks = 0;
    const int rc = tile_grid(n, 1, &blocks);
    if (rc != FSDPSHARD_OK) return rc;
    const void* k = fan_in == 1   ? reinterpret_cast<const void*>(&stream_mix_interleaved_kernel<1>)
                    : fan_in == 8 ? reinterpret_cast<const void*>(&stream_mix_interleaved_kernel<8>)
                                  : reinterpret_cast<const void*>(&stream_mix_interleaved_kernel<0>);
    return launch(k, blocks, &p, stream, step_groups_per_cu(fan_in, blocks));   // as the step
}

extern "C" int fsdpshard_stream_mix_shaped(const uint16_t* const* contribs, int32_t fan_in,
                                           float* state, uint16_t* out, int64_t n,
                                           int32_t groups_per_wave, int32_t per_cu,
                                           int32_t xcd_run, int32_t phased, void* stream) {
    int rc = check_mix(contribs, fan_in, state, nullptr, nullptr, out, n, true);
    if (rc != FSDPSHARD_OK) return rc;
    if (per_cu < 0 || xcd_run < 0 || (phased != 0 && phased != 1)) return FSDPSHARD_ERR_INVALID_ARG;
    const bool ph = phased != 0;
    const void* k = groups_per_wave == 1   ? (ph ? shaped_kernel<1, true>(fan_in)
                                                 : shaped_kernel<1, false>(fan_in))
                    : groups_per_wave == 2 ? (ph ? shaped_kernel<2, true>(fan_in)
                                                 : shaped_kernel<2, false>(fan_in))
                    : groups_per_wave == 4 ? (ph ? shaped_kernel<4, true>(fan_in)
                                                 : shaped_kernel<4, false>(fan_in))
                                           : nullptr;
    if (k == nullptr) return FSDPSHARD_ERR_UNSUPPORTED;
    if (n == 0) return FSDPSHARD_OK;
    MixParams p;
    fill_mix(p, contribs, fan_in, state, nullptr, nullptr, out, n);
    p.run = xcd_run;
    unsigned blocks = 0;
    rc = tile_grid(n, groups_per_wave, &blocks);
    if (rc != FSDPSHARD_OK) return rc;
    return launch(k, blocks, &p, stream, per_cu);
}
