/*
 * host_check.c -- calls the host-only entry points of libfsdpshard.so from plain C (no HIP, no
 * Python) and prints what they return, one item per line, for the test suite to compare with the
 * oracle.  Test program; not part of the library.
 *
 * stdin:  T pad N k pad2 N2 k2
 *         T tensor sizes
 *         T weight-decay flags (0 or 1)
 * stdout: abi <version>
 *         layout <P> <lo> <hi> <n> <n_real> <n_segments> <n_tensors>
 *         seg <shard_begin> <length> <tensor_offset> <tensor_id> <flags>      (n_segments lines)
 *         plan <count>
 *         piece <src_rank> <src_offset> <dst_offset> <length>               (count lines)
 *         badrank <status> <status string>
 * Exit status 0 on success, 1 on malformed input or an unexpected status.
 */
#include <inttypes.h>
#include <stdio.h>
#include <stdlib.h>

#include "fsdpshard.h"

int main(void) {
    long long T, pad, N, k, pad2, N2, k2;
    if (scanf("%lld %lld %lld %lld %lld %lld %lld", &T, &pad, &N, &k, &pad2, &N2, &k2) != 7 ||
        T < 0 || T > 1000000) {
        fprintf(stderr, "bad header\n");
        return 1;
    }
    int64_t* sizes = malloc((size_t)(T > 0 ? T : 1) * sizeof(int64_t));
    uint8_t* wd = malloc((size_t)(T > 0 ? T : 1));
    if (sizes == NULL || wd == NULL) return 1;
    for (long long i = 0; i < T; ++i) {
        long long s;
        if (scanf("%lld", &s) != 1) return 1;
        sizes[i] = (int64_t)s;
    }
    for (long long i = 0; i < T; ++i) {
        int f;
        if (scanf("%d", &f) != 1) return 1;
        wd[i] = (uint8_t)(f != 0);
    }
    printf("abi %d\n", fsdpshard_abi_version());

    /* Two-call pattern: count, then fill. */
    fsdpshard_layout L;
    int rc = shard_layout(sizes, (int32_t)T, pad, wd, (int32_t)N, (int32_t)k, &L, NULL, 0);
    if (rc != FSDPSHARD_OK) {
        fprintf(stderr, "shard_layout: %s\n", fsdpshard_strerror(rc));
        return 1;
    }
    fsdpshard_segment* segs = malloc((size_t)(L.n_segments > 0 ? L.n_segments : 1) * sizeof *segs);
    if (segs == NULL) return 1;
    rc = shard_layout(sizes, (int32_t)T, pad, wd, (int32_t)N, (int32_t)k, &L, segs, L.n_segments);
    if (rc != FSDPSHARD_OK) {
        fprintf(stderr, "shard_layout: %s\n", fsdpshard_strerror(rc));
        return 1;
    }
    printf("layout %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %d %d\n", L.P, L.lo,
           L.hi, L.n, L.n_real, L.n_segments, L.n_tensors);
    for (int32_t i = 0; i < L.n_segments; ++i)
        printf("seg %" PRId64 " %" PRId64 " %" PRId64 " %d %u\n", segs[i].shard_begin,
               segs[i].length, segs[i].tensor_offset, segs[i].tensor_id, segs[i].flags);

    int32_t count = 0;
    rc = reshard_plan(sizes, (int32_t)T, pad, (int32_t)N, pad2, (int32_t)N2, (int32_t)k2, NULL, 0,
                      &count);
    if (rc != FSDPSHARD_OK) {
        fprintf(stderr, "reshard_plan: %s\n", fsdpshard_strerror(rc));
        return 1;
    }
    fsdpshard_piece* pieces = malloc((size_t)(count > 0 ? count : 1) * sizeof *pieces);
    if (pieces == NULL) return 1;
    rc = reshard_plan(sizes, (int32_t)T, pad, (int32_t)N, pad2, (int32_t)N2, (int32_t)k2, pieces,
                      count, &count);
    if (rc != FSDPSHARD_OK) {
        fprintf(stderr, "reshard_plan: %s\n", fsdpshard_strerror(rc));
        return 1;
    }
    printf("plan %d\n", count);
    for (int32_t i = 0; i < count; ++i)
        printf("piece %d %" PRId64 " %" PRId64 " %" PRId64 "\n", pieces[i].src_rank,
               pieces[i].src_offset, pieces[i].dst_offset, pieces[i].length);

    /* A rank outside the world is an argument error, reported and not fatal. */
    rc = shard_layout(sizes, (int32_t)T, pad, wd, (int32_t)N, (int32_t)N, &L, NULL, 0);
    printf("badrank %d %s\n", rc, fsdpshard_strerror(rc));

    free(pieces);
    free(segs);
    free(wd);
    free(sizes);
    return 0;
}
