/*
 * host_edges.c -- edge cases of the host-only entry points (shard_layout, reshard_plan,
 * fsdpshard_strerror, fsdpshard_abi_version), called from plain C.  Test program; not part of the
 * library.  Built both against libfsdpshard.so and, with AddressSanitizer and UBSan, against the
 * host layout source alone: every caller array is allocated at exactly the size passed as its
 * capacity, so a write past it, a signed overflow in the offset arithmetic or an out-of-range
 * index inside the library stops the sanitized run.
 *
 * stdout: one "ok <case>" line per case; exit status 0 when all pass, 1 at the first failure
 * (with a message on stderr).
 */
#include <inttypes.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fsdpshard.h"

#define I64MAX INT64_MAX
#define I32MAX INT32_MAX

static int failures = 0;

#define CHECK(cond, ...)                                                        \
    do {                                                                        \
        if (!(cond)) {                                                          \
            fprintf(stderr, "%s:%d: ", __FILE__, __LINE__);                     \
            fprintf(stderr, __VA_ARGS__);                                       \
            fprintf(stderr, "\n");                                              \
            ++failures;                                                         \
            return;                                                             \
        }                                                                       \
    } while (0)

/* floor(k * P / N) in 128-bit arithmetic, as the floor rule defines the slice bounds. */
static int64_t floor_kp(int64_t k, int64_t P, int64_t N) {
    return (int64_t)(((__int128)k * (__int128)P) / N);
}

static int seg_equal(const fsdpshard_segment* a, const fsdpshard_segment* b) {
    return a->shard_begin == b->shard_begin && a->length == b->length &&
           a->tensor_offset == b->tensor_offset && a->tensor_id == b->tensor_id &&
           a->flags == b->flags;
}

static int piece_equal(const fsdpshard_piece* a, const fsdpshard_piece* b) {
    return a->src_offset == b->src_offset && a->dst_offset == b->dst_offset &&
           a->length == b->length && a->src_rank == b->src_rank && a->reserved == b->reserved;
}

/* Segments must tile [0, n) in order, each of positive length. */
static int segs_tile(const fsdpshard_segment* s, int32_t count, int64_t n) {
    int64_t pos = 0;
    for (int32_t i = 0; i < count; ++i) {
        if (s[i].shard_begin != pos || s[i].length < 1) return 0;
        pos += s[i].length;
    }
    return pos == n;
}

/* A short segment array: CAPACITY, `out` still complete, the first `cap` segments written. */
static void case_layout_capacity(void) {
    int64_t sizes[9] = {3, 0, 17, 1, 100, 0, 5, 64, 2};
    uint8_t wd[9] = {1, 0, 1, 1, 0, 1, 0, 1, 1};
    for (int32_t N = 1; N <= 4; ++N) {
        for (int32_t k = 0; k < N; ++k) {
            fsdpshard_layout full;
            int rc = shard_layout(sizes, 9, 8, wd, N, k, &full, NULL, 0);
            CHECK(rc == FSDPSHARD_OK, "count call: %d", rc);
            fsdpshard_segment* all = malloc((size_t)full.n_segments * sizeof *all + 1);
            CHECK(all != NULL, "malloc");
            rc = shard_layout(sizes, 9, 8, wd, N, k, &full, all, full.n_segments);
            CHECK(rc == FSDPSHARD_OK, "fill call: %d", rc);
            CHECK(segs_tile(all, full.n_segments, full.n), "segments do not tile the slice");
            for (int32_t cap = 0; cap < full.n_segments; ++cap) {
                /* Exactly cap elements; malloc(0) gives a pointer that may not be written. */
                fsdpshard_segment* part = malloc((size_t)cap * sizeof *part);
                if (part == NULL) continue;
                fsdpshard_layout L;
                memset(&L, 0xff, sizeof L);
                rc = shard_layout(sizes, 9, 8, wd, N, k, &L, part, cap);
                CHECK(rc == FSDPSHARD_ERR_CAPACITY, "N=%d k=%d cap=%d: rc %d", N, k, cap, rc);
                CHECK(L.P == full.P && L.lo == full.lo && L.hi == full.hi && L.n == full.n &&
                          L.n_real == full.n_real && L.n_segments == full.n_segments &&
                          L.n_tensors == full.n_tensors,
                      "layout differs under a short array");
                for (int32_t i = 0; i < cap; ++i)
                    CHECK(seg_equal(&part[i], &all[i]), "segment %d differs", i);
                free(part);
            }
            free(all);
        }
    }
    printf("ok layout_capacity\n");
}

/* A short piece array: CAPACITY, the count still reported, the first `cap` pieces written. */
static void case_plan_capacity(void) {
    int64_t sizes[7] = {5, 100, 0, 17, 1, 33, 8};
    for (int32_t N = 1; N <= 5; ++N) {
        for (int32_t N2 = 1; N2 <= 4; ++N2) {
            for (int32_t k2 = 0; k2 < N2; ++k2) {
                int32_t count = -1;
                int rc = reshard_plan(sizes, 7, 4, N, 16, N2, k2, NULL, 0, &count);
                CHECK(rc == FSDPSHARD_OK && count >= 0, "count call: %d", rc);
                fsdpshard_piece* all = malloc((size_t)count * sizeof *all + 1);
                CHECK(all != NULL, "malloc");
                int32_t c2 = -1;
                rc = reshard_plan(sizes, 7, 4, N, 16, N2, k2, all, count, &c2);
                CHECK(rc == FSDPSHARD_OK && c2 == count, "fill call: %d %d", rc, c2);
                for (int32_t cap = 0; cap < count; ++cap) {
                    fsdpshard_piece* part = malloc((size_t)cap * sizeof *part);
                    if (part == NULL) continue;
                    int32_t c3 = -1;
                    rc = reshard_plan(sizes, 7, 4, N, 16, N2, k2, part, cap, &c3);
                    CHECK(rc == FSDPSHARD_ERR_CAPACITY && c3 == count,
                          "N=%d N2=%d k2=%d cap=%d: rc %d count %d", N, N2, k2, cap, rc, c3);
                    for (int32_t i = 0; i < cap; ++i)
                        CHECK(piece_equal(&part[i], &all[i]), "piece %d differs", i);
                    free(part);
                }
                free(all);
            }
        }
    }
    printf("ok plan_capacity\n");
}

/* Flat lengths at the top of the int64 range: the slice bounds need k*P in 128 bits. */
static void case_int64_extremes(void) {
    fsdpshard_layout L;
    fsdpshard_segment segs[4];
    int64_t one[1] = {I64MAX};
    /* P = INT64_MAX exactly (pad 1), a rank near the top of a huge world. */
    int32_t ranks[3] = {0, I32MAX / 2, I32MAX - 1};
    for (int i = 0; i < 3; ++i) {
        int rc = shard_layout(one, 1, 1, NULL, I32MAX, ranks[i], &L, segs, 4);
        CHECK(rc == FSDPSHARD_OK, "rank %d: rc %d", ranks[i], rc);
        CHECK(L.P == I64MAX, "P");
        CHECK(L.lo == floor_kp(ranks[i], I64MAX, I32MAX) &&
                  L.hi == floor_kp((int64_t)ranks[i] + 1, I64MAX, I32MAX),
              "bounds of rank %d", ranks[i]);
        CHECK(L.n_segments == 1 && segs[0].tensor_offset == L.lo && segs[0].length == L.n &&
                  L.n_real == L.n,
              "one real segment");
    }
    /* Padding past INT64_MAX, and two tensors whose sum passes it. */
    int rc = shard_layout(one, 1, 2, NULL, 1, 0, &L, NULL, 0);
    CHECK(rc == FSDPSHARD_ERR_OVERFLOW, "padded size: rc %d", rc);
    int64_t two[2] = {I64MAX / 2 + 1, I64MAX / 2 + 1};
    rc = shard_layout(two, 2, 1, NULL, 1, 0, &L, NULL, 0);
    CHECK(rc == FSDPSHARD_ERR_OVERFLOW, "sum: rc %d", rc);
    /* pad_multiple = INT64_MAX: one element pads to P = INT64_MAX; a second tensor overflows. */
    int64_t ones[2] = {1, 1};
    rc = shard_layout(ones, 1, I64MAX, NULL, 3, 2, &L, segs, 4);
    CHECK(rc == FSDPSHARD_OK && L.P == I64MAX && L.n_real == 0, "huge pad: rc %d", rc);
    CHECK(L.n_segments == 1 && (segs[0].flags & FSDPSHARD_SEG_PADDING), "padding segment");
    rc = shard_layout(ones, 2, I64MAX, NULL, 3, 2, &L, NULL, 0);
    CHECK(rc == FSDPSHARD_ERR_OVERFLOW, "huge pad, two tensors: rc %d", rc);
    /* The plan under the same extremes (a few source ranks, so the plan stays short). */
    int32_t count = -1;
    fsdpshard_piece pieces[8];
    rc = reshard_plan(one, 1, 1, 5, 1, 2, 1, pieces, 8, &count);
    CHECK(rc == FSDPSHARD_OK && count >= 1, "plan at INT64_MAX: rc %d count %d", rc, count);
    int64_t pos = 0;
    for (int32_t i = 0; i < count; ++i) {
        CHECK(pieces[i].dst_offset == pos && pieces[i].length > 0 && pieces[i].src_rank >= 0,
              "piece %d", i);
        pos += pieces[i].length;
    }
    CHECK(pos == I64MAX - floor_kp(1, I64MAX, 2), "pieces cover the shard");
    rc = reshard_plan(one, 1, 2, 1, 1, 1, 0, NULL, 0, &count);
    CHECK(rc == FSDPSHARD_ERR_OVERFLOW, "plan, source padding overflows: rc %d", rc);
    rc = reshard_plan(one, 1, 1, 1, 2, 1, 0, NULL, 0, &count);
    CHECK(rc == FSDPSHARD_ERR_OVERFLOW, "plan, destination padding overflows: rc %d", rc);
    printf("ok int64_extremes\n");
}

/* No tensors, only empty tensors, and more ranks than elements (empty slices). */
static void case_empty(void) {
    fsdpshard_layout L;
    int rc = shard_layout(NULL, 0, 1, NULL, 4, 3, &L, NULL, 0);
    CHECK(rc == FSDPSHARD_OK && L.P == 0 && L.n == 0 && L.n_segments == 0 && L.n_tensors == 0,
          "no tensors: rc %d", rc);
    int32_t count = -1;
    rc = reshard_plan(NULL, 0, 1, 2, 8, 3, 2, NULL, 0, &count);
    CHECK(rc == FSDPSHARD_OK && count == 0, "plan, no tensors: rc %d count %d", rc, count);

    int64_t zeros[5] = {0, 0, 0, 0, 0};
    rc = shard_layout(zeros, 5, 16, NULL, 2, 1, &L, NULL, 0);
    CHECK(rc == FSDPSHARD_OK && L.P == 0 && L.n_segments == 0, "empty tensors: rc %d", rc);
    rc = reshard_plan(zeros, 5, 16, 3, 4, 2, 0, NULL, 0, &count);
    CHECK(rc == FSDPSHARD_OK && count == 0, "plan, empty tensors: rc %d", rc);

    /* P = 5 over 8 ranks: three ranks own nothing; all slices together tile [0, P). */
    int64_t sizes[5] = {0, 0, 5, 0, 0};
    int64_t covered = 0;
    for (int32_t k = 0; k < 8; ++k) {
        fsdpshard_segment segs[4];
        rc = shard_layout(sizes, 5, 1, NULL, 8, k, &L, segs, 4);
        CHECK(rc == FSDPSHARD_OK, "k=%d: rc %d", k, rc);
        CHECK(L.lo == covered && L.n == L.hi - L.lo && L.n >= 0, "k=%d bounds", k);
        CHECK(L.n_segments == (L.n > 0 ? 1 : 0), "k=%d segments", k);
        CHECK(L.n == 0 || (segs[0].tensor_id == 2 && segs[0].tensor_offset == L.lo), "k=%d id", k);
        covered = L.hi;
        int32_t c = -1;
        fsdpshard_piece pieces[4];
        rc = reshard_plan(sizes, 5, 1, 3, 1, 8, k, pieces, 4, &c);
        CHECK(rc == FSDPSHARD_OK && c >= 0 && c <= 4, "plan k=%d: rc %d", k, rc);
        int64_t pos = 0;
        for (int32_t i = 0; i < c; ++i) pos += pieces[i].length;
        CHECK(pos == L.n, "plan k=%d covers %" PRId64 " of %" PRId64, k, pos, L.n);
    }
    CHECK(covered == 5, "slices cover P");
    printf("ok empty\n");
}

/* Many tensors, most empty: the search for the first tensor of each slice. */
static void case_many_tensors(void) {
    const int32_t T = 200000;
    int64_t* sizes = malloc((size_t)T * sizeof *sizes);
    CHECK(sizes != NULL, "malloc");
    uint64_t x = 88172645463325252ull;  /* xorshift64 */
    for (int32_t i = 0; i < T; ++i) {
        x ^= x << 13;
        x ^= x >> 7;
        x ^= x << 17;
        sizes[i] = (x % 4 == 0) ? (int64_t)(x % 37) : 0;
    }
    for (int32_t N = 1; N <= 64; N = N * 3 + 1) {
        int64_t covered = 0;
        for (int32_t k = 0; k < N; ++k) {
            fsdpshard_layout L;
            int rc = shard_layout(sizes, T, 4, NULL, N, k, &L, NULL, 0);
            CHECK(rc == FSDPSHARD_OK, "count: rc %d", rc);
            fsdpshard_segment* segs = malloc((size_t)L.n_segments * sizeof *segs + 1);
            CHECK(segs != NULL, "malloc");
            rc = shard_layout(sizes, T, 4, NULL, N, k, &L, segs, L.n_segments);
            CHECK(rc == FSDPSHARD_OK, "fill: rc %d", rc);
            CHECK(L.lo == covered && segs_tile(segs, L.n_segments, L.n), "N=%d k=%d tiles", N, k);
            for (int32_t i = 0; i < L.n_segments; ++i)
                CHECK(sizes[segs[i].tensor_id] > 0, "segment of an empty tensor");
            covered = L.hi;
            free(segs);
        }
        CHECK(covered > 0, "P > 0");
    }
    free(sizes);
    printf("ok many_tensors\n");
}

/* Argument errors are reported, never fatal, and write nothing through NULL. */
static void case_invalid(void) {
    int64_t sizes[3] = {4, 5, 6};
    int64_t neg[2] = {4, -1};
    fsdpshard_layout L;
    fsdpshard_segment segs[4];
    CHECK(shard_layout(sizes, 3, 1, NULL, 2, 0, NULL, segs, 4) == FSDPSHARD_ERR_INVALID_ARG, "out");
    CHECK(shard_layout(NULL, 3, 1, NULL, 2, 0, &L, segs, 4) == FSDPSHARD_ERR_INVALID_ARG, "numels");
    CHECK(shard_layout(sizes, -1, 1, NULL, 2, 0, &L, segs, 4) == FSDPSHARD_ERR_INVALID_ARG, "T");
    CHECK(shard_layout(neg, 2, 1, NULL, 2, 0, &L, segs, 4) == FSDPSHARD_ERR_INVALID_ARG, "size");
    CHECK(shard_layout(sizes, 3, 0, NULL, 2, 0, &L, segs, 4) == FSDPSHARD_ERR_INVALID_ARG, "pad");
    CHECK(shard_layout(sizes, 3, 1, NULL, 0, 0, &L, segs, 4) == FSDPSHARD_ERR_INVALID_ARG, "N");
    CHECK(shard_layout(sizes, 3, 1, NULL, 2, -1, &L, segs, 4) == FSDPSHARD_ERR_INVALID_ARG, "k<0");
    CHECK(shard_layout(sizes, 3, 1, NULL, 2, 2, &L, segs, 4) == FSDPSHARD_ERR_INVALID_ARG, "k=N");
    CHECK(shard_layout(sizes, 3, 1, NULL, 2, 0, &L, segs, -1) == FSDPSHARD_ERR_INVALID_ARG, "cap");

    fsdpshard_piece pieces[4];
    int32_t c = 0;
    CHECK(reshard_plan(sizes, 3, 1, 2, 1, 2, 0, pieces, 4, NULL) == FSDPSHARD_ERR_INVALID_ARG,
          "n_pieces");
    CHECK(reshard_plan(NULL, 3, 1, 2, 1, 2, 0, pieces, 4, &c) == FSDPSHARD_ERR_INVALID_ARG, "nums");
    CHECK(reshard_plan(neg, 2, 1, 2, 1, 2, 0, pieces, 4, &c) == FSDPSHARD_ERR_INVALID_ARG, "size");
    CHECK(reshard_plan(sizes, 3, 0, 2, 1, 2, 0, pieces, 4, &c) == FSDPSHARD_ERR_INVALID_ARG, "pad");
    CHECK(reshard_plan(sizes, 3, 1, 2, 0, 2, 0, pieces, 4, &c) == FSDPSHARD_ERR_INVALID_ARG, "pad2");
    CHECK(reshard_plan(sizes, 3, 1, 0, 1, 2, 0, pieces, 4, &c) == FSDPSHARD_ERR_INVALID_ARG, "N");
    CHECK(reshard_plan(sizes, 3, 1, 2, 1, 0, 0, pieces, 4, &c) == FSDPSHARD_ERR_INVALID_ARG, "N2");
    CHECK(reshard_plan(sizes, 3, 1, 2, 1, 2, 2, pieces, 4, &c) == FSDPSHARD_ERR_INVALID_ARG, "k2");
    CHECK(reshard_plan(sizes, 3, 1, 2, 1, 2, -1, pieces, 4, &c) == FSDPSHARD_ERR_INVALID_ARG, "k2<0");
    CHECK(reshard_plan(sizes, 3, 1, 2, 1, 2, 0, pieces, -1, &c) == FSDPSHARD_ERR_INVALID_ARG, "cap");
    printf("ok invalid\n");
}

static void case_status_strings(void) {
    for (int code = -2; code <= 8; ++code) {
        const char* s = fsdpshard_strerror(code);
        CHECK(s != NULL && s[0] != '\0', "strerror(%d)", code);
        int known = code >= FSDPSHARD_OK && code <= FSDPSHARD_ERR_HIP;
        CHECK(known == (strcmp(s, "unknown status") != 0), "strerror(%d) = %s", code, s);
    }
    CHECK(fsdpshard_abi_version() == FSDPSHARD_ABI_VERSION, "abi version");
    printf("ok status_strings\n");
}


/* ---- randomized cases: exact bounds and invariants checked with 128-bit arithmetic ---- */

static uint64_t rng_s = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) {  /* xorshift64* */
    rng_s ^= rng_s >> 12;
    rng_s ^= rng_s << 25;
    rng_s ^= rng_s >> 27;
    return rng_s * 0x2545F4914F6CDD1Dull;
}

static int64_t pick_size(void) {
    switch (rnd() % 8) {
        case 0: return 0;
        case 1: case 2: case 3: return (int64_t)(rnd() % 100);
        case 4: return (int64_t)(rnd() % 100000);
        case 5: return (int64_t)(rnd() % (1ull << 40));
        case 6: return I64MAX - (int64_t)(rnd() % 1000);
        default: return I64MAX / (int64_t)(2 + rnd() % 20);
    }
}

static int64_t pick_pad(void) {
    static const int64_t small[6] = {1, 2, 8, 16, 512, 1 << 20};
    if (rnd() % 8 == 0) return I64MAX / (int64_t)(1 + rnd() % 4);
    return small[rnd() % 6];
}

static int32_t pick_world(int big) {
    switch (rnd() % (big ? 4 : 2)) {
        case 0: return (int32_t)(1 + rnd() % 9);
        case 1: return (int32_t)(1 + rnd() % 64);
        case 2: return I32MAX - (int32_t)(rnd() % 10);
        default: return (int32_t)(1 + rnd() % (uint64_t)I32MAX);
    }
}

/* Flat offsets under one padding multiple in 128 bits; returns 0 when P exceeds INT64_MAX. */
static int offsets128(const int64_t* sizes, int T, int64_t pad, __int128* off) {
    __int128 pos = 0;
    for (int i = 0; i < T; ++i) {
        off[i] = pos;
        pos += ((__int128)sizes[i] + pad - 1) / pad * pad;
    }
    off[T] = pos;
    return pos <= (__int128)I64MAX;
}

/* The tensor whose padded extent holds flat position u (empty extents hold nothing). */
static int tensor_at(const __int128* off, int T, __int128 u) {
    for (int i = 0; i < T; ++i)
        if (off[i] <= u && u < off[i + 1]) return i;
    return -1;
}

static void case_fuzz_layout(void) {
    enum { MAXT = 20 };
    int64_t sizes[MAXT];
    uint8_t wd[MAXT];
    __int128 off[MAXT + 1];
    fsdpshard_segment segs[2 * MAXT + 2];
    for (int trial = 0; trial < 40000; ++trial) {
        const int T = (int)(rnd() % (MAXT + 1));
        for (int i = 0; i < T; ++i) {
            sizes[i] = pick_size();
            wd[i] = (uint8_t)(rnd() & 1);
        }
        const int64_t pad = pick_pad();
        const int32_t N = pick_world(1);
        const int32_t k = (int32_t)(rnd() % (uint64_t)N);
        const int fits = offsets128(sizes, T, pad, off);
        fsdpshard_layout L;
        int rc = shard_layout(sizes, T, pad, wd, N, k, &L, segs, 2 * MAXT + 2);
        if (!fits) {
            CHECK(rc == FSDPSHARD_ERR_OVERFLOW, "trial %d: rc %d, expected overflow", trial, rc);
            continue;
        }
        CHECK(rc == FSDPSHARD_OK, "trial %d: rc %d", trial, rc);
        const int64_t P = (int64_t)off[T];
        CHECK(L.P == P && L.lo == floor_kp(k, P, N) && L.hi == floor_kp((int64_t)k + 1, P, N) &&
                  L.n == L.hi - L.lo,
              "trial %d: bounds", trial);
        CHECK(L.n_segments <= 2 * T, "trial %d: %d segments for %d tensors", trial,
              L.n_segments, T);
        CHECK(segs_tile(segs, L.n_segments, L.n), "trial %d: segments do not tile", trial);
        int64_t real = 0;
        int32_t tensors = 0, last = -1;
        for (int32_t j = 0; j < L.n_segments; ++j) {
            const fsdpshard_segment* g = &segs[j];
            const int id = g->tensor_id;
            CHECK(id >= 0 && id < T && id >= last, "trial %d: tensor id %d", trial, id);
            if (id != last) ++tensors;
            last = id;
            CHECK((__int128)L.lo + g->shard_begin == off[id] + g->tensor_offset,
                  "trial %d: segment %d position", trial, j);
            CHECK(off[id] + g->tensor_offset + g->length <= off[id + 1],
                  "trial %d: segment %d leaves its tensor", trial, j);
            const int pad_run = (g->flags & FSDPSHARD_SEG_PADDING) != 0;
            if (pad_run) {
                CHECK(g->tensor_offset >= sizes[id], "trial %d: padding over real data", trial);
            } else {
                CHECK(g->tensor_offset + g->length <= sizes[id], "trial %d: real run past the end",
                      trial);
                real += g->length;
            }
            CHECK(((g->flags & FSDPSHARD_SEG_WEIGHT_DECAY) != 0) == (wd[id] != 0),
                  "trial %d: weight-decay flag", trial);
        }
        CHECK(real == L.n_real && tensors == L.n_tensors, "trial %d: counts", trial);
    }
    printf("ok fuzz_layout\n");
}

static void case_fuzz_plan(void) {
    enum { MAXT = 12, CAP = 4096 };
    int64_t sizes[MAXT];
    __int128 oa[MAXT + 1], ob[MAXT + 1];
    static fsdpshard_piece pieces[CAP];
    for (int trial = 0; trial < 10000; ++trial) {
        const int T = (int)(rnd() % (MAXT + 1));
        for (int i = 0; i < T; ++i) sizes[i] = pick_size();
        const int64_t pa = pick_pad(), pb = pick_pad();
        const int32_t N = pick_world(0), N2 = pick_world(0);
        const int32_t k2 = (int32_t)(rnd() % (uint64_t)N2);
        const int fits = offsets128(sizes, T, pa, oa) & offsets128(sizes, T, pb, ob);
        int32_t count = -1;
        int rc = reshard_plan(sizes, T, pa, N, pb, N2, k2, pieces, CAP, &count);
        if (!fits) {
            CHECK(rc == FSDPSHARD_ERR_OVERFLOW, "trial %d: rc %d, expected overflow", trial, rc);
            continue;
        }
        CHECK(rc == FSDPSHARD_OK && count >= 0 && count <= CAP, "trial %d: rc %d count %d",
              trial, rc, count);
        const int64_t Pa = (int64_t)oa[T], Pb = (int64_t)ob[T];
        const int64_t lo2 = floor_kp(k2, Pb, N2), hi2 = floor_kp((int64_t)k2 + 1, Pb, N2);
        int64_t pos = 0;
        for (int32_t j = 0; j < count; ++j) {
            const fsdpshard_piece* q = &pieces[j];
            CHECK(q->dst_offset == pos && q->length > 0 && q->reserved == 0,
                  "trial %d: piece %d placement", trial, j);
            pos += q->length;
            /* Walk the piece tensor by tensor (merged neighbours may span several). */
            __int128 d = (__int128)lo2 + q->dst_offset;
            __int128 left = q->length;
            if (q->src_rank < 0) {
                CHECK(q->src_offset == 0, "trial %d: zero piece %d source offset", trial, j);
                while (left > 0) {      /* every element is destination padding */
                    const int i = tensor_at(ob, T, d);
                    CHECK(i >= 0 && d >= ob[i] + sizes[i], "trial %d: zero piece %d over data",
                          trial, j);
                    const __int128 c = left < ob[i + 1] - d ? left : ob[i + 1] - d;
                    d += c;
                    left -= c;
                }
                continue;
            }
            const int32_t r = q->src_rank;
            CHECK(r < N, "trial %d: source rank %d of %d", trial, r, N);
            const int64_t rlo = floor_kp(r, Pa, N), rhi = floor_kp((int64_t)r + 1, Pa, N);
            CHECK(q->src_offset >= 0 && q->src_offset + q->length <= rhi - rlo,
                  "trial %d: piece %d outside source shard", trial, j);
            __int128 u = (__int128)rlo + q->src_offset;
            while (left > 0) {          /* same tensor, same offset, real data on both sides */
                const int i = tensor_at(oa, T, u);
                CHECK(i >= 0 && tensor_at(ob, T, d) == i && u - oa[i] == d - ob[i] &&
                          u - oa[i] < sizes[i],
                      "trial %d: piece %d maps an element wrongly", trial, j);
                const __int128 avail = oa[i] + sizes[i] - u;
                const __int128 c = left < avail ? left : avail;
                u += c;
                d += c;
                left -= c;
            }
        }
        CHECK(pos == hi2 - lo2, "trial %d: pieces cover %lld of %lld", trial, (long long)pos,
              (long long)(hi2 - lo2));
    }
    printf("ok fuzz_plan\n");
}

int main(void) {
    case_layout_capacity();
    case_plan_capacity();
    case_int64_extremes();
    case_empty();
    case_many_tensors();
    case_invalid();
    case_status_strings();
    case_fuzz_layout();
    case_fuzz_plan();
    if (failures) {
        fprintf(stderr, "%d case(s) failed\n", failures);
        return 1;
    }
    return 0;
}
