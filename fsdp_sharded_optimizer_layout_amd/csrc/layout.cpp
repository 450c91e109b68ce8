// Host side of libfsdpshard.so: the flat layout and floor-rule slice of one rank, status strings.
//
// "FSDP: Fully Sharded Data Parallel Training at Scale", passage on sharding a linear layer:
// parameters are flattened to one 1-D vector of length P and rank k owns the contiguous range
// [floor(kP/N), floor((k+1)P/N)); gradients and both Adam moments use the same positions.
// Tensors are laid out back to back, each padded to a multiple of pad_multiple elements; the
// slice is described as runs (segments) of one tensor's real elements or of its padding.

#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include "fsdpshard.h"

namespace {

constexpr int64_t kI64Max = std::numeric_limits<int64_t>::max();

// ceil(s / m) * m, or -1 when it does not fit int64.
int64_t padded_size(int64_t s, int64_t m) {
    const int64_t q = s / m + (s % m != 0);
    if (q > kI64Max / m) return -1;
    return q * m;
}

// floor(k * P / N) with a 128-bit product (k <= N, so the quotient fits int64).
int64_t floor_kp_over_n(int64_t k, int64_t P, int64_t N) {
    const __int128 prod = static_cast<__int128>(k) * static_cast<__int128>(P);
    return static_cast<int64_t>(prod / N);
}

}  // namespace

extern "C" int shard_layout(const int64_t* numels, int32_t n_tensors, int64_t pad_multiple,
                            const uint8_t* wd_mask, int32_t world_size, int32_t rank,
                            fsdpshard_layout* out, fsdpshard_segment* segs,
                            int32_t seg_capacity) {
    if (out == nullptr || n_tensors < 0 || (n_tensors > 0 && numels == nullptr) ||
        pad_multiple < 1 || world_size < 1 || rank < 0 || rank >= world_size ||
        seg_capacity < 0) {
        return FSDPSHARD_ERR_INVALID_ARG;
    }
    // Flat offsets: offs[i] is where tensor i starts; offs[T] = P.
    std::vector<int64_t> offs(static_cast<size_t>(n_tensors) + 1);
    int64_t pos = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (numels[i] < 0) return FSDPSHARD_ERR_INVALID_ARG;
        const int64_t ps = padded_size(numels[i], pad_multiple);
        if (ps < 0 || ps > kI64Max - pos) return FSDPSHARD_ERR_OVERFLOW;
        offs[i] = pos;
        pos += ps;
    }
    offs[n_tensors] = pos;
    const int64_t P = pos;
    const int64_t lo = floor_kp_over_n(rank, P, world_size);
    const int64_t hi = floor_kp_over_n(static_cast<int64_t>(rank) + 1, P, world_size);

    // First tensor whose padded extent reaches past lo: largest i with offs[i] <= lo, then skip
    // forward over tensors that end at or before lo (empty tensors share an offset).
    int32_t first = 0;
    {
        int32_t a = 0, b = n_tensors;  // search in [a, b)
        while (b - a > 1) {
            const int32_t mid = a + (b - a) / 2;
            if (offs[mid] <= lo) a = mid; else b = mid;
        }
        first = a;
        while (first < n_tensors && offs[first + 1] <= lo) ++first;
    }

    int64_t n_real = 0;
    int32_t count = 0, tensors = 0;
    bool over = false;
    for (int32_t i = first; i < n_tensors && offs[i] < hi; ++i) {
        const int64_t base = offs[i];
        const int64_t real_end = base + numels[i];
        const uint32_t wd = (wd_mask == nullptr || wd_mask[i] != 0) ? FSDPSHARD_SEG_WEIGHT_DECAY : 0u;
        bool touched = false;
        const int64_t run_a[2] = {base, real_end};
        const int64_t run_b[2] = {real_end, offs[i + 1]};
        for (int part = 0; part < 2; ++part) {
            const int64_t x = run_a[part] > lo ? run_a[part] : lo;
            const int64_t y = run_b[part] < hi ? run_b[part] : hi;
            if (x >= y) continue;
            touched = true;
            if (part == 0) n_real += y - x;
            if (count == std::numeric_limits<int32_t>::max()) return FSDPSHARD_ERR_OVERFLOW;
            if (segs != nullptr) {
                if (count < seg_capacity) {
                    fsdpshard_segment& s = segs[count];
                    s.shard_begin = x - lo;
                    s.length = y - x;
                    s.tensor_offset = x - base;
                    s.tensor_id = i;
                    s.flags = wd | (part == 1 ? FSDPSHARD_SEG_PADDING : 0u);
                } else {
                    over = true;
                }
            }
            ++count;
        }
        tensors += touched ? 1 : 0;
    }

    out->P = P;
    out->lo = lo;
    out->hi = hi;
    out->n = hi - lo;
    out->n_real = n_real;
    out->n_segments = count;
    out->n_tensors = tensors;
    return over ? FSDPSHARD_ERR_CAPACITY : FSDPSHARD_OK;
}

namespace {

// Flat offsets of the tensors under one padding multiple; offs[T] = P.  Returns a status.
int flat_offsets(const int64_t* numels, int32_t n_tensors, int64_t pad, std::vector<int64_t>* offs) {
    offs->assign(static_cast<size_t>(n_tensors) + 1, 0);
    int64_t pos = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (numels[i] < 0) return FSDPSHARD_ERR_INVALID_ARG;
        const int64_t ps = padded_size(numels[i], pad);
        if (ps < 0 || ps > kI64Max - pos) return FSDPSHARD_ERR_OVERFLOW;
        (*offs)[i] = pos;
        pos += ps;
    }
    (*offs)[n_tensors] = pos;
    return FSDPSHARD_OK;
}

// Rank that owns flat position u (0 <= u < P) under the floor rule: the k with
// floor(kP/N) <= u < floor((k+1)P/N), i.e. k = ceil((u+1)N/P) - 1 = floor(((u+1)N - 1)/P).
int32_t owner_of(int64_t u, int64_t P, int32_t N) {
    const __int128 a = (static_cast<__int128>(u) + 1) * N - 1;
    return static_cast<int32_t>(a / P);
}

struct PieceSink {
    fsdpshard_piece* out;
    int32_t capacity;
    int32_t count;
    bool over;
    bool have;
    fsdpshard_piece cur;

    void flush() {
        if (!have) return;
        if (out != nullptr) {
            if (count < capacity) out[count] = cur;
            else over = true;
        }
        ++count;
        have = false;
    }
    // Append a piece, merging it into the previous one when both are contiguous.
    void add(int32_t src_rank, int64_t src_off, int64_t dst_off, int64_t len) {
        if (len <= 0) return;
        if (have && cur.src_rank == src_rank && cur.dst_offset + cur.length == dst_off &&
            (src_rank < 0 || cur.src_offset + cur.length == src_off)) {
            cur.length += len;
            return;
        }
        flush();
        cur.src_offset = src_rank < 0 ? 0 : src_off;
        cur.dst_offset = dst_off;
        cur.length = len;
        cur.src_rank = src_rank;
        cur.reserved = 0;
        have = true;
    }
};

}  // namespace

extern "C" int reshard_plan(const int64_t* numels, int32_t n_tensors, int64_t src_pad,
                            int32_t src_world, int64_t dst_pad, int32_t dst_world, int32_t dst_rank,
                            fsdpshard_piece* pieces, int32_t capacity, int32_t* n_pieces) {
    if (n_pieces == nullptr || n_tensors < 0 || (n_tensors > 0 && numels == nullptr) ||
        src_pad < 1 || dst_pad < 1 || src_world < 1 || dst_world < 1 || dst_rank < 0 ||
        dst_rank >= dst_world || capacity < 0)
        return FSDPSHARD_ERR_INVALID_ARG;
    std::vector<int64_t> oa, ob;
    int rc = flat_offsets(numels, n_tensors, src_pad, &oa);
    if (rc != FSDPSHARD_OK) return rc;
    rc = flat_offsets(numels, n_tensors, dst_pad, &ob);
    if (rc != FSDPSHARD_OK) return rc;
    const int64_t Pa = oa[n_tensors], Pb = ob[n_tensors];
    const int64_t lo = floor_kp_over_n(dst_rank, Pb, dst_world);
    const int64_t hi = floor_kp_over_n(static_cast<int64_t>(dst_rank) + 1, Pb, dst_world);

    PieceSink sink{pieces, capacity, 0, false, false, {}};
    // First tensor whose destination extent reaches past lo.
    int32_t first = 0;
    {
        int32_t a = 0, b = n_tensors;
        while (b - a > 1) {
            const int32_t mid = a + (b - a) / 2;
            if (ob[mid] <= lo) a = mid; else b = mid;
        }
        first = a;
        while (first < n_tensors && ob[first + 1] <= lo) ++first;
    }
    for (int32_t i = first; i < n_tensors && ob[i] < hi; ++i) {
        // Real elements of tensor i inside the destination shard: flat [x, y) of the new layout.
        const int64_t x = ob[i] > lo ? ob[i] : lo;
        const int64_t real_end = ob[i] + numels[i];
        const int64_t y = real_end < hi ? real_end : hi;
        if (x < y) {
            // The same tensor positions in the source layout, cut by the source ranks' slices.
            int64_t u = oa[i] + (x - ob[i]);
            const int64_t w = oa[i] + (y - ob[i]);
            int32_t r = owner_of(u, Pa, src_world);
            while (u < w) {
                const int64_t rlo = floor_kp_over_n(r, Pa, src_world);
                const int64_t rhi = floor_kp_over_n(static_cast<int64_t>(r) + 1, Pa, src_world);
                const int64_t e = w < rhi ? w : rhi;
                if (u < e) sink.add(r, u - rlo, (u - oa[i]) + ob[i] - lo, e - u);
                u = e > u ? e : u;
                ++r;
            }
        }
        // Destination padding of tensor i: zero.
        const int64_t px = real_end > lo ? real_end : lo;
        const int64_t py = ob[i + 1] < hi ? ob[i + 1] : hi;
        if (px < py) sink.add(-1, 0, px - lo, py - px);
    }
    sink.flush();
    *n_pieces = sink.count;
    return sink.over ? FSDPSHARD_ERR_CAPACITY : FSDPSHARD_OK;
}

extern "C" const char* fsdpshard_strerror(int code) {
    switch (code) {
        case FSDPSHARD_OK: return "ok";
        case FSDPSHARD_ERR_INVALID_ARG: return "invalid argument";
        case FSDPSHARD_ERR_OVERFLOW: return "integer overflow in the flat layout";
        case FSDPSHARD_ERR_CAPACITY: return "output array or workspace too small";
        case FSDPSHARD_ERR_ALIGNMENT: return "misaligned pointer";
        case FSDPSHARD_ERR_UNSUPPORTED: return "unsupported fan-in";
        case FSDPSHARD_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" int fsdpshard_abi_version(void) { return FSDPSHARD_ABI_VERSION; }
