/* Host-side exercise of libmuon's C ABI for the sanitizer build: table
 * validation (every error class, the size limits, int64 extremes), planning
 * of the five workloads' tables, argument checks of every entry point with
 * NULL or invalid handles, and the host schedules. No device is used: the one
 * muon_init that passes validation names a device index that cannot exist,
 * so it stops at the device check. Exit status 0 when every expectation
 * holds; the sanitizers abort on any report. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "libmuon.h"

static int fails = 0;
#define EXPECT(c)                                                      \
    do {                                                               \
        if (!(c)) {                                                    \
            fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #c);       \
            ++fails;                                                   \
        }                                                              \
    } while (0)

static muon_matrix mat(int64_t r, int64_t c, int64_t count, int64_t off) {
    muon_matrix m;
    memset(&m, 0, sizeof(m));
    m.rows = r;
    m.cols = c;
    m.count = count;
    m.offset = off;
    m.lr_mul = 1.0f;
    m.wd_mul = 1.0f;
    return m;
}

/* layers x (qkvo [4, d, d] + c_fc [d, 4d] + c_proj [4d, d]) */
static int body(muon_matrix* t, int layers, int64_t d) {
    int n = 0;
    int64_t off = 0;
    for (int l = 0; l < layers; ++l) {
        t[n++] = mat(d, d, 4, off);
        off += 4 * d * d;
        t[n++] = mat(d, 4 * d, 1, off);
        off += 4 * d * d;
        t[n++] = mat(4 * d, d, 1, off);
        off += 4 * d * d;
    }
    return n;
}

static size_t ws(const muon_matrix* t, int n, const muon_hparams* hp, muon_status* st) {
    size_t b = 0;
    *st = muon_workspace_bytes(t, n, hp, &b);
    return b;
}

int main(void) {
    static muon_matrix t[300];
    muon_hparams hp;
    muon_hparams_default(&hp);
    muon_status st;
    size_t b;

    /* the five workloads' tables plan cleanly */
    int n = body(t, 1, 128);
    b = ws(t, n, &hp, &st);
    EXPECT(st == MUON_OK && b > 0);
    n = body(t, 12, 768);
    b = ws(t, n, &hp, &st);
    EXPECT(st == MUON_OK && b > (size_t)3 * 84934656 * 2);
    n = body(t, 48, 1600);
    b = ws(t, n, &hp, &st);
    EXPECT(st == MUON_OK && b > (size_t)3 * 1474560000 * 2);
    hp.normuon = 1;
    n = body(t, 12, 768);
    b = ws(t, n, &hp, &st);
    EXPECT(st == MUON_OK);
    hp.normuon = 0;
    t[0] = mat(64, 64, 4096, 0);
    t[1] = mat(256, 1024, 256, 4096 * 64 * 64);
    b = ws(t, 2, &hp, &st);
    EXPECT(st == MUON_OK);
    hp.ns_precision = MUON_NS_FP32;
    n = body(t, 1, 128);
    b = ws(t, n, &hp, &st);
    EXPECT(st == MUON_OK);
    muon_hparams_default(&hp);

    /* shapes */
    t[0] = mat(0, 4, 1, 0);
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_SHAPE);
    t[0] = mat(4, 4, 0, 0);
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_SHAPE);
    t[0] = mat((int64_t)1 << 21, 4, 1, 0);
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_SHAPE);
    /* every dimension at its limit: rows x cols x count would overflow int64 */
    t[0] = mat((int64_t)1 << 20, (int64_t)1 << 20, (int64_t)1 << 24, 0);
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_SHAPE);
    t[0] = mat(INT64_MAX, INT64_MAX, INT64_MAX, 0);
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_SHAPE);
    t[0] = mat(INT64_MIN, 4, 1, 0);
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_SHAPE);
    t[0] = mat(1, (int64_t)1 << 20, 1, 0); /* a single row at the dimension limit is fine */
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_OK);

    /* layout */
    t[0] = mat(4, 4, 1, -1);
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_LAYOUT);
    t[0] = mat(4, 4, 1, INT64_MAX);
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_LAYOUT);
    t[0] = mat(4, 4, 1, ((int64_t)1 << 62) - 8);
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_LAYOUT);
    t[0] = mat(4, 4, 2, 0);
    t[1] = mat(4, 4, 1, 16); /* overlaps the second matrix of entry 0 */
    ws(t, 2, &hp, &st);
    EXPECT(st == MUON_E_LAYOUT);
    t[1] = mat(4, 4, 1, 32); /* touching is fine */
    ws(t, 2, &hp, &st);
    EXPECT(st == MUON_OK);

    /* entries and arguments */
    t[0] = mat(4, 4, 1, 0);
    t[0].reserved = 1;
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_INVALID_ARG && strstr(muon_last_error(NULL), "reserved") != NULL);
    t[0] = mat(4, 4, 1, 0);
    t[0].lr_mul = NAN;
    ws(t, 1, &hp, &st);
    EXPECT(st == MUON_E_INVALID_ARG);
    t[0] = mat(4, 4, 1, 0);
    ws(NULL, 1, &hp, &st);
    EXPECT(st == MUON_E_INVALID_ARG);
    ws(t, -1, &hp, &st);
    EXPECT(st == MUON_E_INVALID_ARG);
    EXPECT(muon_workspace_bytes(t, 1, &hp, NULL) == MUON_E_INVALID_ARG);
    ws(NULL, 0, &hp, &st);
    EXPECT(st == MUON_OK);
    ws(t, 1, NULL, &st);
    EXPECT(st == MUON_OK);

    /* hyper-parameters */
    {
        muon_hparams bad;
        muon_hparams_default(&bad);
        bad.ns_steps = 0;
        ws(t, 1, &bad, &st);
        EXPECT(st == MUON_E_INVALID_ARG);
        muon_hparams_default(&bad);
        bad.ns_steps = MUON_MAX_NS_STEPS + 1;
        ws(t, 1, &bad, &st);
        EXPECT(st == MUON_E_INVALID_ARG);
        muon_hparams_default(&bad);
        bad.momentum = NAN;
        ws(t, 1, &bad, &st);
        EXPECT(st == MUON_E_INVALID_ARG);
        muon_hparams_default(&bad);
        bad.ns_coeffs[2][1] = INFINITY;
        ws(t, 1, &bad, &st);
        EXPECT(st == MUON_E_INVALID_ARG);
        muon_hparams_default(&bad);
        bad.stream_groups = -1; /* 0 is the library's choice, 1 .. 4 explicit */
        ws(t, 1, &bad, &st);
        EXPECT(st == MUON_E_INVALID_ARG);
        muon_hparams_default(&bad);
        bad.stream_groups = 5;
        ws(t, 1, &bad, &st);
        EXPECT(st == MUON_E_INVALID_ARG);
        muon_hparams_default(&bad);
        bad.ns_precision = 7;
        ws(t, 1, &bad, &st);
        EXPECT(st == MUON_E_INVALID_ARG);
    }

    /* muon_init: argument and workspace checks come before any device call */
    {
        muon_handle* h = (muon_handle*)1;
        n = body(t, 1, 128);
        b = ws(t, n, &hp, &st);
        EXPECT(muon_init(NULL, t, n, &hp, NULL, 0, 0) == MUON_E_INVALID_ARG);
        EXPECT(muon_init(&h, t, n, &hp, NULL, b, 0) == MUON_E_WORKSPACE && h == NULL);
        h = (muon_handle*)1;
        EXPECT(muon_init(&h, t, n, &hp, (void*)(uintptr_t)0x100010, b, 0) == MUON_E_WORKSPACE && h == NULL);
        EXPECT(muon_init(&h, t, n, &hp, (void*)(uintptr_t)0x100000, b - 1, 0) == MUON_E_WORKSPACE && h == NULL);
        t[0].rows = 0;
        EXPECT(muon_init(&h, t, n, &hp, (void*)(uintptr_t)0x100000, b, 0) == MUON_E_SHAPE && h == NULL);
        t[0].rows = 128;
        /* passes validation; device 1000 does not exist on any host */
        EXPECT(muon_init(&h, t, n, &hp, (void*)(uintptr_t)0x100000, b, 1000) == MUON_E_NO_DEVICE && h == NULL);
        EXPECT(strlen(muon_last_error(NULL)) > 0);
    }

    /* muon_init_static: the same checks, and tables beyond the static workspace */
    {
        muon_handle* h = (muon_handle*)1;
        EXPECT(muon_init_static(NULL, t, 1, &hp, 0) == MUON_E_INVALID_ARG);
        n = body(t, 12, 768); /* the 124M body needs far more than the static workspace */
        EXPECT(muon_init_static(&h, t, n, &hp, 0) == MUON_E_WORKSPACE && h == NULL);
        EXPECT(strstr(muon_last_error(NULL), "static workspace") != NULL);
        n = body(t, 1, 128);
        h = (muon_handle*)1;
        EXPECT(muon_init_static(&h, t, n, NULL, 1000) == MUON_E_NO_DEVICE && h == NULL);
        t[0].count = 0;
        EXPECT(muon_init_static(&h, t, n, &hp, 0) == MUON_E_SHAPE && h == NULL);
        t[0].count = 4;
    }

    /* every entry point taking a handle rejects NULL */
    {
        float x[4] = {0, 0, 0, 0};
        muon_layout lay;
        muon_work wk;
        void* p = NULL;
        size_t bytes = 0;
        int64_t launches = 0;
        double ms = 0;
        EXPECT(muon_step(NULL, x, x, x, 4, 0.1f, -1.0f, NULL) == MUON_E_INVALID_ARG);
        EXPECT(muon_reset(NULL, x, 4, NULL) == MUON_E_INVALID_ARG);
        EXPECT(muon_matrix_layout(NULL, 0, &lay) == MUON_E_INVALID_ARG);
        EXPECT(muon_debug_view(NULL, MUON_VIEW_V, &p, &bytes) == MUON_E_INVALID_ARG);
        EXPECT(muon_work_stats(NULL, &wk) == MUON_E_INVALID_ARG);
        EXPECT(muon_profile_enable(NULL, 1) == MUON_E_INVALID_ARG);
        EXPECT(muon_profile_read(NULL, 0, 0, &launches, &ms) == MUON_E_INVALID_ARG);
        EXPECT(muon_num_matrices(NULL) == 0);
        muon_destroy(NULL);
    }

    /* status strings */
    for (int s = -8; s <= 0; ++s) EXPECT(muon_status_string((muon_status)s) != NULL);
    EXPECT(strcmp(muon_status_string((muon_status)-99), "unknown status") == 0);
    EXPECT(strcmp(muon_status_string(MUON_E_HOST), "host-side failure") == 0);

    /* host schedules, in range and out of range */
    EXPECT(fabsf(muon_lr_wsd(0, 100, 0, 20) - 1.0f) < 1e-6f);
    EXPECT(fabsf(muon_lr_wsd(90, 100, 0, 20) - 0.5f) < 1e-6f);
    EXPECT(isnan(muon_lr_wsd(-1, 100, 0, 20)));
    EXPECT(isnan(muon_lr_wsd(0, 0, 0, 0)));
    EXPECT(fabsf(muon_lr_cooldown_floor(1000, 100, 0.8f, 0.3f) - 0.3f) < 1e-6f);
    EXPECT(isnan(muon_lr_cooldown_floor(0, 100, 0.0f, 0.3f)));
    EXPECT(fabsf(muon_momentum_warmup(250, 500, 0.85f, 0.95f) - 0.90f) < 1e-6f);
    EXPECT(isnan(muon_momentum_warmup(0, 0, 0.85f, 0.95f)));
    EXPECT(muon_lr_wsd(INT64_MAX - 1, INT64_MAX, 0, INT64_MAX) >= 0.0f);
    EXPECT(isnan(muon_lr_wsd(0, INT64_MAX, INT64_MAX, INT64_MAX))); /* warmup + warmdown overflows int64 */
    EXPECT(isnan(muon_lr_wsd(INT64_MAX, INT64_MAX, 0, 0)));

    if (fails) fprintf(stderr, "%d expectation(s) failed\n", fails);
    else printf("abi_check: all expectations hold\n");
    return fails ? 1 : 0;
}
