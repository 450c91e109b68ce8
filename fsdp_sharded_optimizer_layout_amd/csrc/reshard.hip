// Reshard execution of libfsdpshard.so on gfx950: copy the pieces of a reshard plan.
//
// "FSDP: Fully Sharded Data Parallel Training at Scale", checkpointing passage: local state
// dicts (each rank's own shard) load only under the same rank count; a reshard plan (host code,
// reshard_plan) maps another rank count's shards onto one destination shard as a list of pieces,
// each a contiguous run of elements from one source shard, or zeros for destination padding.
//
// The copy is a bandwidth-bound stream.  One launch carries up to kMaxPieces pieces in its
// kernel arguments; every piece is cut into 4 KiB chunks of its destination, one work-group per
// chunk (XCD-aware order, chunk_index), and a work-group finds its piece by binary search over
// the pieces' first chunks.  Each
// lane stores one 16-byte destination-aligned vector.  Source and destination of a piece may sit
// at different offsets within 16 bytes (a new world size or padding multiple moves every shard
// boundary); then every lane still issues one aligned 16-byte load, takes the next aligned
// vector from its neighbour lane, and funnel-shifts the pair into place, so the source stream is
// read with full-width loads whatever its phase.  Loads and stores are non-temporal: every byte
// is touched once.  The at most 14 bytes before the first aligned destination vector and after
// the last one are copied 2 bytes at a time (every element is at least 2 bytes wide).
//
// An aligned 16-byte load that holds at least one byte of a piece may also cover a few bytes on
// either side of it; those lie in the same 16-byte block, hence in the same page, and are
// discarded.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

#include "fsdpshard.h"

namespace {

constexpr int kBlock = 256;
constexpr int64_t kChunk = 16 * kBlock;   // destination bytes per work-group
constexpr int kMaxPieces = 96;            // keeps the kernel arguments under 4 KiB
constexpr int kWaveShl1 = 0x130;          // DPP control: lane l reads lane l + 1 of the wave

struct CopyPiece {
    const unsigned char* src;   // null: write zeros
    unsigned char* dst;
    int64_t bytes;
};

struct ReshardParams {
    CopyPiece piece[kMaxPieces];
    int64_t first_block[kMaxPieces + 1];   // work-group index where each piece starts
    int32_t n;
};

using u32x4_t = uint32_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t load_nt(const unsigned char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ void store_nt(unsigned char* p, u32x4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// Bytes [4W + sh/8, 4W + sh/8 + 16) of the 32 bytes lo:hi (little-endian words).
template <int W>
__device__ __forceinline__ u32x4_t funnel(u32x4_t lo, u32x4_t hi, uint32_t sh) {
    const uint32_t c[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    u32x4_t r;
    r.x = __builtin_amdgcn_alignbit(c[W + 1], c[W], sh);
    r.y = __builtin_amdgcn_alignbit(c[W + 2], c[W + 1], sh);
    r.z = __builtin_amdgcn_alignbit(c[W + 3], c[W + 2], sh);
    r.w = __builtin_amdgcn_alignbit(c[W + 4], c[W + 3], sh);
    return r;
}

// Work-group -> chunk.  The hardware deals work-groups to the 8 XCDs in turn; this permutation
// gives each XCD runs of kXcdRun consecutive chunks (1 MiB of destination) instead of every
// eighth chunk, and keeps the identity past the last whole block of 8 * kXcdRun chunks.
// Measured on one GPU against the identity map: 3-5 % faster on misaligned pieces, 1 % on
// aligned ones; runs of 16 chunks were slower, 128-512 about the same as 256.
constexpr int64_t kXcds = 8;
constexpr int64_t kXcdRun = 256;

__device__ __forceinline__ int64_t chunk_index() {
    const int64_t b = blockIdx.x;
    const int64_t whole = static_cast<int64_t>(gridDim.x) / (kXcds * kXcdRun) * (kXcds * kXcdRun);
    if (b >= whole) return b;
    const int64_t x = b % kXcds, q = b / kXcds;
    return (q / kXcdRun) * (kXcds * kXcdRun) + x * kXcdRun + q % kXcdRun;
}

__global__ __launch_bounds__(kBlock) void reshard_kernel(ReshardParams p) {
    const int64_t b = chunk_index();
    int a = 0, z = p.n;   // largest piece index with first_block <= b
    while (z - a > 1) {
        const int mid = (a + z) >> 1;
        if (p.first_block[mid] <= b) a = mid; else z = mid;
    }
    const CopyPiece pc = p.piece[a];
    const int64_t chunk = b - p.first_block[a];
    const int64_t head_raw = static_cast<int64_t>((16u - (reinterpret_cast<uintptr_t>(pc.dst) & 15u)) & 15u);
    const int64_t head = head_raw < pc.bytes ? head_raw : pc.bytes;
    const int64_t body_end = head + ((pc.bytes - head) & ~static_cast<int64_t>(15));
    const int64_t tail = pc.bytes - body_end;

    const int lane = threadIdx.x & 63;
    const int64_t off = head + chunk * kChunk + static_cast<int64_t>(threadIdx.x) * 16;
    const bool active = off + 16 <= body_end;
    if (pc.src == nullptr) {
        if (active) store_nt(pc.dst + off, u32x4_t{0u, 0u, 0u, 0u});
    } else {
        // The source phase is the same for every lane of the piece (off is head + 16k).
        const uint32_t ph = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(pc.src + off) & 15u);
        const unsigned char* base = pc.src + (off - ph);
        if (ph == 0) {
            if (active) store_nt(pc.dst + off, load_nt(base));
        } else {
            // Each active lane loads its own aligned vector; the next one comes from lane + 1
            // through a one-lane wave shift (DPP wave_shl), except where lane + 1 is past the
            // piece or in the next wave: there the lane loads it itself, issued together with its
            // first load so that no wave waits for a second round trip.
            const bool next_active = lane < 63 && off + 32 <= body_end;
            u32x4_t lo = {0u, 0u, 0u, 0u}, extra = {0u, 0u, 0u, 0u};
            if (active) lo = load_nt(base);
            if (active && !next_active) extra = load_nt(base + 16);
            u32x4_t hi;
            hi.x = __builtin_amdgcn_mov_dpp(static_cast<int>(lo.x), kWaveShl1, 0xF, 0xF, false);
            hi.y = __builtin_amdgcn_mov_dpp(static_cast<int>(lo.y), kWaveShl1, 0xF, 0xF, false);
            hi.z = __builtin_amdgcn_mov_dpp(static_cast<int>(lo.z), kWaveShl1, 0xF, 0xF, false);
            hi.w = __builtin_amdgcn_mov_dpp(static_cast<int>(lo.w), kWaveShl1, 0xF, 0xF, false);
            if (!next_active) hi = extra;
            if (active) {
                const uint32_t sh = (ph & 3u) * 8u;
                u32x4_t v;
                switch (ph >> 2) {
                    case 0: v = funnel<0>(lo, hi, sh); break;
                    case 1: v = funnel<1>(lo, hi, sh); break;
                    case 2: v = funnel<2>(lo, hi, sh); break;
                    default: v = funnel<3>(lo, hi, sh); break;
                }
                // Store pacing (measured on one GPU, 8 alternating rounds): a pause of 8 x 64
                // cycles before the store made re-phased copies (8 -> 6 ranks of a 2^31-element
                // fp32 vector) 1.6-2.0 % faster; aligned copies were the same or slower with it.
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_sleep(8);
                __builtin_amdgcn_sched_barrier(0);
                store_nt(pc.dst + off, v);
            }
        }
    }
    if (chunk == 0) {
        const int64_t t2 = static_cast<int64_t>(threadIdx.x) * 2;
        if (t2 < head) {
            const uint16_t x = pc.src ? *reinterpret_cast<const uint16_t*>(pc.src + t2) : 0;
            *reinterpret_cast<uint16_t*>(pc.dst + t2) = x;
        }
        if (t2 < tail) {
            const int64_t o = body_end + t2;
            const uint16_t x = pc.src ? *reinterpret_cast<const uint16_t*>(pc.src + o) : 0;
            *reinterpret_cast<uint16_t*>(pc.dst + o) = x;
        }
    }
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + static_cast<uintptr_t>(bbytes) && y < x + static_cast<uintptr_t>(abytes);
}

}  // namespace

extern "C" int reshard_copy(const void* const* src_shards, const int64_t* src_elems,
                            int32_t src_world, void* dst, int64_t dst_elems,
                            const fsdpshard_piece* pieces, int32_t n_pieces, int32_t elem_bytes,
                            void* stream) {
    if (src_shards == nullptr || src_elems == nullptr || src_world < 1 ||
        (dst == nullptr && dst_elems != 0) || dst_elems < 0 || n_pieces < 0 ||
        (n_pieces > 0 && pieces == nullptr))
        return FSDPSHARD_ERR_INVALID_ARG;
    if (elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return FSDPSHARD_ERR_INVALID_ARG;
    if (dst_elems > INT64_MAX / 8) return FSDPSHARD_ERR_OVERFLOW;
    const uintptr_t amask = static_cast<uintptr_t>(elem_bytes - 1);
    if ((reinterpret_cast<uintptr_t>(dst) & amask) != 0) return FSDPSHARD_ERR_ALIGNMENT;
    for (int32_t r = 0; r < src_world; ++r) {
        if (src_elems[r] < 0 || src_elems[r] > INT64_MAX / 8) return FSDPSHARD_ERR_INVALID_ARG;
        if (src_shards[r] == nullptr) continue;
        if ((reinterpret_cast<uintptr_t>(src_shards[r]) & amask) != 0) return FSDPSHARD_ERR_ALIGNMENT;
        if (src_elems[r] > 0 && dst_elems > 0 &&
            overlaps(src_shards[r], src_elems[r] * elem_bytes, dst, dst_elems * elem_bytes))
            return FSDPSHARD_ERR_INVALID_ARG;
    }
    // Every piece inside its shards; destination pieces pairwise disjoint.
    int64_t prev_end = -1;
    bool sorted = true;
    for (int32_t i = 0; i < n_pieces; ++i) {
        const fsdpshard_piece& q = pieces[i];
        if (q.length < 0 || q.dst_offset < 0 || q.dst_offset > dst_elems - q.length)
            return FSDPSHARD_ERR_INVALID_ARG;
        if (q.src_rank >= 0) {
            if (q.src_rank >= src_world || src_shards[q.src_rank] == nullptr || q.src_offset < 0 ||
                q.src_offset > src_elems[q.src_rank] - q.length)
                return FSDPSHARD_ERR_INVALID_ARG;
        } else if (q.src_rank != -1) {
            return FSDPSHARD_ERR_INVALID_ARG;
        }
        if (q.dst_offset < prev_end) sorted = false;
        prev_end = q.dst_offset + q.length;
    }
    if (!sorted) {
        std::vector<std::pair<int64_t, int64_t>> spans;
        spans.reserve(static_cast<size_t>(n_pieces));
        for (int32_t i = 0; i < n_pieces; ++i)
            if (pieces[i].length > 0) spans.emplace_back(pieces[i].dst_offset, pieces[i].length);
        std::sort(spans.begin(), spans.end());
        for (size_t i = 1; i < spans.size(); ++i)
            if (spans[i - 1].first + spans[i - 1].second > spans[i].first)
                return FSDPSHARD_ERR_INVALID_ARG;
    }
    unsigned char* d = static_cast<unsigned char*>(dst);
    int32_t i = 0;   // next piece to place; empty pieces are skipped
    while (i < n_pieces) {
        ReshardParams p;
        int32_t cnt = 0;
        int64_t blocks = 0;
        for (; i < n_pieces && cnt < kMaxPieces; ++i) {
            const fsdpshard_piece& q = pieces[i];
            if (q.length == 0) continue;
            CopyPiece& c = p.piece[cnt];
            c.src = q.src_rank < 0 ? nullptr
                                   : static_cast<const unsigned char*>(src_shards[q.src_rank]) +
                                         q.src_offset * elem_bytes;
            c.dst = d + q.dst_offset * elem_bytes;
            c.bytes = q.length * elem_bytes;
            const int64_t head = static_cast<int64_t>((16u - (reinterpret_cast<uintptr_t>(c.dst) & 15u)) & 15u);
            const int64_t body = c.bytes > head ? c.bytes - head : 0;
            const int64_t nb = (body + kChunk - 1) / kChunk;
            p.first_block[cnt] = blocks;
            blocks += nb > 0 ? nb : 1;
            ++cnt;
        }
        if (cnt == 0) continue;
        p.first_block[cnt] = blocks;
        p.n = cnt;
        if (blocks > 0x7FFFFFFF) return FSDPSHARD_ERR_OVERFLOW;
        void* args[] = {&p};
        const hipError_t e =
            hipLaunchKernel(reinterpret_cast<const void*>(&reshard_kernel),
                            dim3(static_cast<unsigned>(blocks)), dim3(kBlock), args, 0,
                            static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return FSDPSHARD_ERR_HIP;
    }
    return FSDPSHARD_OK;
}
