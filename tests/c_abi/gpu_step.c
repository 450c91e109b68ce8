/*
 * gpu_step.c -- drives the fused sharded AdamW step of libfsdpshard.so from plain C through the
 * HIP runtime (no Python, no torch): shard_layout on the host, device buffers from hipMalloc,
 * S calls of adamw_shard_step on the null stream, results copied back.  Test program; not part of
 * the library.
 *
 *   gpu_step <input file> <output file>
 *
 * Input (little-endian): 8-byte magic "FSDPIN1", then int64 T, pad, N, k, F, S; float64 lr,
 * beta1, beta2, eps, weight_decay, grad_scale; int64 sizes[T]; uint8 wd[T]; then for the slice
 * of n = hi - lo elements: float32 master[n], m[n], v[n]; uint16 contributions[F][n] (bf16 bit
 * patterns, used by every step).
 * Output: int64 n, lo, phase; float32 master[n], m[n], v[n]; uint16 window[n + phase + 16]: the
 * flat bf16 positions lo - phase - 8 .. hi + 7, prefilled with 0xABCD (phase = lo mod 8).
 * Exit status 0 on success; 1 on a bad file, 2 on a library status, 3 on a HIP error.
 */
#include <inttypes.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fsdpshard.h"

#define HIP_CHECK(call)                                                                \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                \
            return 3;                                                                  \
        }                                                                              \
    } while (0)

static int read_all(FILE* f, void* dst, size_t bytes) { return fread(dst, 1, bytes, f) == bytes; }

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: gpu_step <input> <output>\n");
        return 1;
    }
    FILE* in = fopen(argv[1], "rb");
    if (in == NULL) return 1;
    char magic[8];
    int64_t hdr[6];
    double hpd[6];
    if (!read_all(in, magic, 8) || memcmp(magic, "FSDPIN1", 8) != 0 || !read_all(in, hdr, sizeof hdr) ||
        !read_all(in, hpd, sizeof hpd))
        return 1;
    const int64_t T = hdr[0], pad = hdr[1], N = hdr[2], k = hdr[3], F = hdr[4], S = hdr[5];
    if (T < 0 || T > 1000000 || F < 1 || F > FSDPSHARD_MAX_FAN_IN || S < 1 || S > 1000 || N < 1 ||
        N > 1000000 || k < 0 || k >= N)
        return 1;
    int64_t* sizes = malloc((size_t)(T ? T : 1) * sizeof(int64_t));
    uint8_t* wd = malloc((size_t)(T ? T : 1));
    if (sizes == NULL || wd == NULL || !read_all(in, sizes, (size_t)T * sizeof(int64_t)) ||
        !read_all(in, wd, (size_t)T))
        return 1;

    fsdpshard_layout L;
    int rc = shard_layout(sizes, (int32_t)T, pad, wd, (int32_t)N, (int32_t)k, &L, NULL, 0);
    if (rc != FSDPSHARD_OK) {
        fprintf(stderr, "shard_layout: %s\n", fsdpshard_strerror(rc));
        return 2;
    }
    fsdpshard_segment* segs = malloc((size_t)(L.n_segments ? L.n_segments : 1) * sizeof *segs);
    if (segs == NULL) return 1;
    rc = shard_layout(sizes, (int32_t)T, pad, wd, (int32_t)N, (int32_t)k, &L, segs, L.n_segments);
    if (rc != FSDPSHARD_OK) {
        fprintf(stderr, "shard_layout: %s\n", fsdpshard_strerror(rc));
        return 2;
    }
    const int64_t n = L.n, lo = L.lo, phase = lo % 8;
    if (n < 1 || n > ((int64_t)1 << 31)) return 1;   /* a test-sized slice */
    const size_t nf = (size_t)n * sizeof(float), nh = (size_t)n * sizeof(uint16_t);
    const int64_t win = n + phase + 16;

    float* h_state = malloc(3 * nf);
    uint16_t* h_g = malloc((size_t)F * nh);
    uint16_t* h_win = malloc((size_t)win * sizeof(uint16_t));
    if (h_state == NULL || h_g == NULL || h_win == NULL) return 1;
    if (!read_all(in, h_state, 3 * nf) || !read_all(in, h_g, (size_t)F * nh)) return 1;
    fclose(in);
    for (int64_t i = 0; i < win; ++i) h_win[i] = 0xABCD;

    float *d_master, *d_m, *d_v;
    uint16_t* d_win;
    fsdpshard_segment* d_segs;
    const uint16_t* d_g[FSDPSHARD_MAX_FAN_IN];
    HIP_CHECK(hipMalloc((void**)&d_master, nf));
    HIP_CHECK(hipMalloc((void**)&d_m, nf));
    HIP_CHECK(hipMalloc((void**)&d_v, nf));
    HIP_CHECK(hipMalloc((void**)&d_win, (size_t)win * sizeof(uint16_t)));
    HIP_CHECK(hipMalloc((void**)&d_segs, (size_t)(L.n_segments ? L.n_segments : 1) * sizeof *segs));
    for (int64_t r = 0; r < F; ++r) {
        uint16_t* p;
        HIP_CHECK(hipMalloc((void**)&p, nh));
        HIP_CHECK(hipMemcpy(p, h_g + (size_t)r * (size_t)n, nh, hipMemcpyHostToDevice));
        d_g[r] = p;
    }
    HIP_CHECK(hipMemcpy(d_master, h_state, nf, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_m, h_state + n, nf, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_v, h_state + 2 * n, nf, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_win, h_win, (size_t)win * sizeof(uint16_t), hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_segs, segs, (size_t)L.n_segments * sizeof *segs, hipMemcpyHostToDevice));

    fsdpshard_adamw hp;
    memset(&hp, 0, sizeof hp);
    hp.lr = hpd[0];
    hp.beta1 = hpd[1];
    hp.beta2 = hpd[2];
    hp.eps = hpd[3];
    hp.weight_decay = hpd[4];
    hp.grad_scale = hpd[5];
    hp.max_grad_norm = 0.0;
    hp.grad_sumsq = NULL;
    for (int64_t t = 1; t <= S; ++t) {
        hp.step = t;
        /* The window starts 8 elements before the 16-byte aligned vector that holds lo. */
        rc = adamw_shard_step(d_master, d_m, d_v, d_g, (int32_t)F, n, d_segs, L.n_segments, &hp,
                              d_win, lo - phase - 8, lo, NULL);
        if (rc != FSDPSHARD_OK) {
            fprintf(stderr, "adamw_shard_step: %s\n", fsdpshard_strerror(rc));
            return 2;
        }
    }
    HIP_CHECK(hipDeviceSynchronize());
    HIP_CHECK(hipMemcpy(h_state, d_master, nf, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(h_state + n, d_m, nf, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(h_state + 2 * n, d_v, nf, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(h_win, d_win, (size_t)win * sizeof(uint16_t), hipMemcpyDeviceToHost));

    FILE* out = fopen(argv[2], "wb");
    if (out == NULL) return 1;
    const int64_t oh[3] = {n, lo, phase};
    if (fwrite(oh, sizeof oh, 1, out) != 1 || fwrite(h_state, 1, 3 * nf, out) != 3 * nf ||
        fwrite(h_win, sizeof(uint16_t), (size_t)win, out) != (size_t)win)
        return 1;
    fclose(out);

    for (int64_t r = 0; r < F; ++r) HIP_CHECK(hipFree((void*)d_g[r]));
    HIP_CHECK(hipFree(d_segs));
    HIP_CHECK(hipFree(d_win));
    HIP_CHECK(hipFree(d_v));
    HIP_CHECK(hipFree(d_m));
    HIP_CHECK(hipFree(d_master));
    free(h_win);
    free(h_g);
    free(h_state);
    free(segs);
    free(wd);
    free(sizes);
    printf("gpu_step ok: n=%" PRId64 " lo=%" PRId64 " segments=%d fan-in %" PRId64 ", %" PRId64
           " steps\n", n, lo, L.n_segments, F, S);
    return 0;
}
