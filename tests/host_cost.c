/*
 * Host cost of the dispatch layer: descriptor validation, extent and overlap
 * checks, route decision and launch-family resolution of mm_gemm and mm_id,
 * stopped just before the enqueue by the resolve-failure test hook (so no GPU
 * is needed). rlx-metal 0.2.14 mps_blas.rs, module doc: the per-call cost of
 * crossing into the GPU library is what decides whether small products are
 * worth sending there; this measures the part of that cost this library adds
 * before the HIP runtime's own launch.
 *
 * The buffers are fake device addresses: validation reads no memory. Each
 * case runs `iters` calls, `reps` times; the printed figure is the fastest
 * repetition's mean, in nanoseconds per call. "hook" times the hook and an
 * error-string read alone, the floor under every case.
 *
 * Build: gcc -O2 -I include tests/host_cost.c -L<libdir> -lmm -Wl,-rpath,<libdir>
 * Output: one JSON object on stdout.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "mm.h"

static double now_ns(void) {
    struct timespec t;
    clock_gettime(CLOCK_MONOTONIC, &t);
    return (double)t.tv_sec * 1e9 + (double)t.tv_nsec;
}

/* Distinct, far-apart, 256-byte aligned fake addresses. */
static mm_buf fake(int slot, uint64_t bytes) {
    mm_buf b;
    b.ptr = (void *)(uintptr_t)((uint64_t)(slot + 1) << 40);
    b.bytes = bytes;
    return b;
}

static mm_gemm_desc nt(mm_dtype dt, int64_t m, int64_t n, int64_t k) {
    mm_gemm_desc d;
    memset(&d, 0, sizeof d);
    d.dtype = dt;
    d.trans_a = 0;
    d.trans_b = 1;
    d.batch = 1;
    d.m = m;
    d.n = n;
    d.k = k;
    return d;
}

typedef struct {
    const char *name;
    const char *family; /* launch family whose resolution fails */
    int kind;           /* 0 gemm, 1 id, 2 hook floor */
    mm_gemm_desc g;
    mm_id_params p;
} Case;

static int run_one(const Case *c, mm_buf a, mm_buf b, mm_buf out, const mm_id_capability *cap) {
    if (c->kind == 2) {
        mm_test_inject_resolve_failure(c->family);
        (void)mm_last_error();
        mm_test_inject_resolve_failure(NULL);
        return MM_ERR_UNSUPPORTED;
    }
    mm_test_inject_resolve_failure(c->family);
    if (c->kind == 0) return mm_gemm(&c->g, a, b, out, NULL, NULL);
    return mm_id(&c->p, MM_BF16, fake(0, cap->weight_bytes), fake(1, cap->input_bytes),
                 fake(2, cap->ids_bytes), fake(3, cap->output_bytes), fake(4, cap->counts_bytes),
                 fake(5, cap->routed_rows_bytes), NULL, NULL);
}

int main(int argc, char **argv) {
    long iters = argc > 1 ? atol(argv[1]) : 100000;
    int reps = argc > 2 ? atoi(argv[2]) : 5;
    Case cases[6];
    memset(cases, 0, sizeof cases);
    cases[0].name = "gemm_f16_8192_nt"; cases[0].family = "gemm"; cases[0].kind = 0;
    cases[0].g = nt(MM_F16, 8192, 8192, 8192);
    cases[1].name = "gemv_f16_1x4096_11008"; cases[1].family = "gemv"; cases[1].kind = 0;
    cases[1].g = nt(MM_F16, 1, 11008, 4096);
    cases[2].name = "skinny_f16_8x4096_11008"; cases[2].family = "gemv_wide"; cases[2].kind = 0;
    cases[2].g = nt(MM_F16, 8, 11008, 4096);
    mm_id_params prefill = {512, 1408, 2048, 8, 64, 1408ull * 2048 * 2, 0, 0, 1};
    mm_id_params decode = {1, 1408, 2048, 8, 64, 1408ull * 2048 * 2, 0, 1, 0};
    cases[3].name = "id_prefill_bf16_512x8_of_64"; cases[3].family = "id_grouped"; cases[3].kind = 1;
    cases[3].p = prefill;
    cases[4].name = "id_decode_bf16_1x8_of_64"; cases[4].family = "id_direct"; cases[4].kind = 1;
    cases[4].p = decode;
    cases[5].name = "hook"; cases[5].family = "gemm"; cases[5].kind = 2;

    printf("{\"iters\": %ld, \"reps\": %d", iters, reps);
    for (int ci = 0; ci < 6; ++ci) {
        const Case *c = &cases[ci];
        mm_id_capability cap;
        memset(&cap, 0, sizeof cap);
        mm_buf a = fake(0, 0), b = fake(1, 0), out = fake(2, 0);
        if (c->kind == 0) {
            const uint64_t es = c->g.dtype == MM_F32 ? 4 : 2;
            a.bytes = (uint64_t)(c->g.m * c->g.k) * es;
            b.bytes = (uint64_t)(c->g.n * c->g.k) * es;
            out.bytes = (uint64_t)(c->g.m * c->g.n) * es;
        } else if (c->kind == 1) {
            if (mm_id_query(MM_BF16, &c->p, &cap) != MM_OK) {
                fprintf(stderr, "%s: query failed: %s\n", c->name, mm_last_error());
                return 1;
            }
        }
        /* One checked call: the hook must be what stops it. */
        int st = run_one(c, a, b, out, &cap);
        if (st != MM_ERR_UNSUPPORTED || (c->kind != 2 && !strstr(mm_last_error(), "injected"))) {
            fprintf(stderr, "%s: expected the injected refusal, got %d: %s\n", c->name, st,
                    mm_last_error());
            return 1;
        }
        double best = 1e30;
        for (int r = 0; r < reps; ++r) {
            const double t0 = now_ns();
            for (long i = 0; i < iters; ++i) run_one(c, a, b, out, &cap);
            const double per = (now_ns() - t0) / (double)iters;
            if (per < best) best = per;
        }
        printf(", \"%s\": %.1f", c->name, best);
    }
    printf("}\n");
    return 0;
}
