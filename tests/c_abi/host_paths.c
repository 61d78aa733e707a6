/*
 * Drives every host-side path of libfnorm that needs no GPU: the variant
 * tables and their descriptions (including truncated buffers), the
 * per-thread candidate cache, the RoPE shape rules, and every entry point's
 * validation, overlap checks and error text.  Calls that pass validation
 * ask for variant 1000000, which no table serves, so nothing is launched.
 * Built with AddressSanitizer and UBSan on the host code by a CPU test;
 * exit status 0 when every documented status is met.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fnorm.h"

#define NOLAUNCH 1000000

static int failures = 0;

static void expect(const char *what, long long line, int got, int want)
{
    if (got != want) {
        fprintf(stderr, "%s (line %lld): %s, expected %s: %s\n", what, line,
                fnorm_status_string(got), fnorm_status_string(want), fnorm_last_error());
        ++failures;
    }
}
#define EXPECT(what, got, want) expect(what, __LINE__, got, want)
#define CHECK(cond)                                                            \
    do {                                                                       \
        if (!(cond)) {                                                         \
            fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #cond); \
            ++failures;                                                        \
        }                                                                      \
    } while (0)

static void tables(void)
{
    static const int64_t widths[] = {1,    2,    3,    7,    8,    15,   16,    17,   31,
                                     64,   100,  128,  255,  256,  768,  1000,  1024, 2048,
                                     4096, 4097, 8192, 8193, 20000, 65536, 65537, 1 << 20};
    char big[256], tiny[4];
    for (int op = -1; op <= 5; ++op)
        for (int dt = -1; dt <= 3; ++dt)
            for (size_t i = 0; i < sizeof widths / sizeof widths[0]; ++i)
                for (int al = 0; al <= 1; ++al) {
                    const int n = fnorm_variant_count(op, dt, widths[i], al);
                    CHECK(n >= 0);
                    for (int v = -1; v <= n; ++v) {
                        const int s = fnorm_describe_shape(op, dt, widths[i], al, v, big,
                                                           sizeof big);
                        const int valid = op >= 0 && op <= 4 && dt >= 0 && dt <= 2;
                        CHECK(!(valid && n > 0 && v < n && s != FNORM_OK));
                        CHECK(s != FNORM_OK || strlen(big) < sizeof big);
                        (void)fnorm_describe_shape(op, dt, widths[i], al, v, tiny, sizeof tiny);
                        CHECK(strlen(tiny) < sizeof tiny);
                    }
                }
    for (int dt = 0; dt <= 2; ++dt)
        for (int64_t hd = 2; hd <= 1024; hd *= 2)
            for (int64_t dims = 2; dims <= hd + 2; dims += dims < 16 ? 2 : dims)
                for (int trad = 0; trad <= 1; ++trad)
                    for (int al = 0; al <= 1; ++al) {
                        const int n = fnorm_rope_variant_count(dt, hd, dims, trad, al);
                        for (int v = -1; v <= n; ++v) {
                            (void)fnorm_describe_rope(dt, hd, dims, trad, al, v, big, sizeof big);
                            (void)fnorm_describe_rope(dt, hd, dims, trad, al, v, tiny, 1);
                        }
                    }
    EXPECT("describe null buf", fnorm_describe_shape(0, 1, 128, 1, -1, NULL, 8), FNORM_ERR_NULL);
    EXPECT("describe zero len", fnorm_describe_shape(0, 1, 128, 1, -1, big, 0), FNORM_ERR_NULL);
    EXPECT("describe call null buf", fnorm_describe(0, (void *)0x1000, 8, NULL, 0, (void *)0x2000,
                                                    NULL, (void *)0x3000, 8, 1, 8, 1, -1, NULL,
                                                    8),
           FNORM_ERR_NULL);
    /* a LayerNorm without bias has its own kernel list (fewer shapes at some
       widths): the shape query of FNORM_OP_LAYER_NOBIAS and the call with
       b == NULL agree */
    {
        static const int64_t nb_widths[] = {6144, 18432, 24576, 65536, 4096, 768};
        for (size_t i = 0; i < sizeof nb_widths / sizeof nb_widths[0]; ++i) {
            char a[256], c[256];
            const int n = fnorm_variant_count(FNORM_OP_LAYER_NOBIAS, FNORM_BF16, nb_widths[i], 1);
            CHECK(n >= 2);
            for (int v = -1; v < n; ++v) {
                EXPECT("nobias shape", fnorm_describe_shape(FNORM_OP_LAYER_NOBIAS, FNORM_BF16,
                                                            nb_widths[i], 1, v, a, sizeof a),
                       FNORM_OK);
                EXPECT("nobias call", fnorm_describe(FNORM_OP_LAYER, (void *)0x100000, nb_widths[i],
                                                     NULL, 0, (void *)0x20000000, NULL,
                                                     (void *)0x40000000, nb_widths[i], 16,
                                                     nb_widths[i], FNORM_BF16, v, c, sizeof c),
                       FNORM_OK);
                CHECK(strcmp(a, c) == 0);
            }
            /* one past the last no-bias variant is refused by the call too */
            EXPECT("nobias past end", fnorm_describe(FNORM_OP_LAYER, (void *)0x100000,
                                                     nb_widths[i], NULL, 0, (void *)0x20000000,
                                                     NULL, (void *)0x40000000, nb_widths[i], 16,
                                                     nb_widths[i], FNORM_BF16, n, c, sizeof c),
                   FNORM_ERR_UNSUPPORTED);
        }
    }
    for (int s = -2; s <= 10; ++s)
        CHECK(fnorm_status_string(s) != NULL);
}

static void entry_points(void)
{
    char *const A = (char *)0x100000, *const B = (char *)0x20000000, *const C = (char *)0x40000000;
    char *const D = (char *)0x60000000, *const E = (char *)0x70000000, *const F = (char *)0x7c000000;
    /* validation passes, no variant: nothing launches */
    for (int dt = 0; dt <= 2; ++dt) {
        EXPECT("rms", fnorm_rms_v(A, B, C, 64, 4096, 1e-6f, dt, NULL, NOLAUNCH), FNORM_ERR_UNSUPPORTED);
        EXPECT("layer", fnorm_layer_v(A, B, D, C, 64, 4096, 1e-6f, dt, NULL, NOLAUNCH),
               FNORM_ERR_UNSUPPORTED);
        EXPECT("gate", fnorm_rms_swiglu_v(A, D, B, C, 64, 4096, 1e-6f, dt, NULL, NOLAUNCH),
               FNORM_ERR_UNSUPPORTED);
        EXPECT("dual", fnorm_dual_head_rms_v(A, D, B, E, C, F, 1024, 256, 128, 1e-6f, dt, NULL,
                                             NOLAUNCH),
               FNORM_ERR_UNSUPPORTED);
        EXPECT("rope", fnorm_dual_head_rms_rope_v(A, D, B, E, C, F, 32, 32, 8, 128, 1e-6f, 128, 1,
                                                  10000.0f, 1.0f, 3, NULL, dt, NULL, NOLAUNCH),
               FNORM_ERR_UNSUPPORTED);
    }
    /* strided forms: interleaved views of one buffer, and clashes */
    EXPECT("strided gaps", fnorm_rms_strided(A, 256, B, A + 256, 256, 64, 64, 1e-6f, FNORM_BF16,
                                             NULL, NOLAUNCH),
           FNORM_ERR_UNSUPPORTED);
    EXPECT("strided clash", fnorm_rms_strided(A, 256, B, A + 64, 256, 64, 64, 1e-6f, FNORM_BF16,
                                              NULL, NOLAUNCH),
           FNORM_ERR_ALIAS);
    EXPECT("strided stride", fnorm_layer_strided(A, 8, B, NULL, C, 64, 4, 64, 1e-6f, FNORM_F32,
                                                 NULL, NOLAUNCH),
           FNORM_ERR_SHAPE);
    EXPECT("strided overflow", fnorm_rms_strided(A, INT64_MAX / 2, B, C, 64, 4, 64, 1e-6f,
                                                 FNORM_F32, NULL, NOLAUNCH),
           FNORM_ERR_SHAPE);
    EXPECT("gate strided", fnorm_rms_swiglu_strided(A, 128, A + 128, 128, B, C, 64, 64, 64, 1e-6f,
                                                    FNORM_BF16, NULL, NOLAUNCH),
           FNORM_ERR_UNSUPPORTED);
    {   /* packed q | k | v per token: in place on q and k is legal */
        const int64_t hd = 128, qh = 8, kh = 2, ts = (qh + 2 * kh) * hd, tok = 16;
        char *q = A, *k = A + qh * hd * 2;
        EXPECT("packed", fnorm_dual_head_rms_strided(q, ts, k, ts, B, D, q, ts, k, ts, tok, qh, kh,
                                                     hd, 1e-6f, FNORM_BF16, NULL, NOLAUNCH),
               FNORM_ERR_UNSUPPORTED);
        EXPECT("packed rope", fnorm_dual_head_rms_rope_strided(
                                  q, ts, k, ts, B, D, q, ts, k, ts, tok, qh, kh, hd, 1e-6f, hd, 0,
                                  10000.0f, 1.0f, 0, NULL, FNORM_BF16, NULL, NOLAUNCH),
               FNORM_ERR_UNSUPPORTED);
        EXPECT("packed clash", fnorm_dual_head_rms_strided(q, ts, k, ts, B, D, k, ts, k, ts, tok,
                                                           qh, kh, hd, 1e-6f, FNORM_BF16, NULL,
                                                           NOLAUNCH),
               FNORM_ERR_ALIAS);
    }
    /* invalid arguments of every kind */
    EXPECT("rms rows", fnorm_rms(A, B, C, -1, 8, 1e-6f, FNORM_F32, NULL), FNORM_ERR_SHAPE);
    EXPECT("rms overflow", fnorm_rms(A, B, C, INT64_MAX / 4, 64, 1e-6f, FNORM_F32, NULL),
           FNORM_ERR_SHAPE);
    /* row counts whose product with head_dim overflows int64: rejected, and
       no overflowing product is formed on the way (UBSan watches) */
    EXPECT("dual overflow", fnorm_dual_head_rms(A, D, B, E, C, F, INT64_MAX / 4, 1, 128, 1e-6f,
                                                FNORM_BF16, NULL),
           FNORM_ERR_SHAPE);
    EXPECT("dual overflow k", fnorm_dual_head_rms(A, D, B, E, C, F, 1, INT64_MAX / 4, 128, 1e-6f,
                                                  FNORM_BF16, NULL),
           FNORM_ERR_SHAPE);
    EXPECT("rope overflow", fnorm_dual_head_rms_rope(A, D, B, E, C, F, 4, INT64_MAX / 4, 1, 128,
                                                     1e-6f, 128, 0, 10000.0f, 1.0f, 0, NULL,
                                                     FNORM_BF16, NULL),
           FNORM_ERR_SHAPE);
    /* no tokens: heads * head_dim alone overflows */
    EXPECT("dual overflow no tokens",
           fnorm_dual_head_rms_strided(A, 0, D, 0, B, E, C, 0, F, 0, 0, INT64_MAX / 8, 1, 1024,
                                       1e-6f, FNORM_BF16, NULL, -1),
           FNORM_ERR_SHAPE);
    EXPECT("rope overflow no tokens",
           fnorm_dual_head_rms_rope_strided(A, 0, D, 0, B, E, C, 0, F, 0, 0, 1, INT64_MAX / 8,
                                            1024, 1e-6f, 64, 0, 10000.0f, 1.0f, 0, NULL,
                                            FNORM_BF16, NULL, -1),
           FNORM_ERR_SHAPE);
    {
        char nb[64];
        EXPECT("describe dual overflow", fnorm_describe_dual(A, 0, D, 0, B, E, C, 0, F, 0, 1,
                                                             INT64_MAX / 4, 1, 128, FNORM_BF16,
                                                             -1, nb, sizeof nb),
               FNORM_ERR_SHAPE);
        EXPECT("describe dual call", fnorm_describe_dual(A, 0, D, 0, B, E, C, 0, F, 0, 1, 4096, 1024,
                                                         128, FNORM_BF16, -1, nb, sizeof nb),
               FNORM_OK);
        CHECK(strncmp(nb, "dual.bf16.vec8.", 15) == 0);
        EXPECT("describe rope call", fnorm_describe_dual_rope(
                                         A, 32 * 128, D, 8 * 128, B, E, C, 32 * 128, F, 8 * 128,
                                         16, 32, 8, 128, 128, 0, 10000.0f, 1.0f, 0, NULL,
                                         FNORM_BF16, -1, nb, sizeof nb),
               FNORM_OK);
        CHECK(strncmp(nb, "ropesplit.bf16.", 15) == 0);
        EXPECT("describe no rows", fnorm_describe(FNORM_OP_RMS, NULL, 8, NULL, 0, NULL, NULL, NULL,
                                                  8, 0, 8, FNORM_F32, -1, nb, sizeof nb),
               FNORM_OK);
        CHECK(strcmp(nb, "none") == 0);
    }
    EXPECT("rms eps", fnorm_rms(A, B, C, 4, 8, -0.5f, FNORM_F32, NULL), FNORM_ERR_EPS);
    EXPECT("dual heads", fnorm_dual_head_rms_strided(A, 64, D, 64, B, E, C, 64, F, 64, 4, -1, 1,
                                                     64, 1e-6f, FNORM_BF16, NULL, -1),
           FNORM_ERR_SHAPE);
    EXPECT("rope dims", fnorm_dual_head_rms_rope(A, D, B, E, C, F, 4, 2, 1, 128, 1e-6f, 3, 0,
                                                 10000.0f, 1.0f, 0, NULL, FNORM_BF16, NULL),
           FNORM_ERR_SHAPE);
    EXPECT("rope base", fnorm_dual_head_rms_rope(A, D, B, E, C, F, 4, 2, 1, 128, 1e-6f, 128, 0,
                                                 -1.0f, 1.0f, 0, NULL, FNORM_BF16, NULL),
           FNORM_ERR_SHAPE);
    EXPECT("rope offset", fnorm_dual_head_rms_rope(A, D, B, E, C, F, 4, 2, 1, 128, 1e-6f, 128, 0,
                                                   10000.0f, 1.0f, INT64_MAX, NULL, FNORM_BF16,
                                                   NULL),
           FNORM_ERR_SHAPE);
    EXPECT("composed ws", fnorm_layer_composed(A, B, NULL, C, 4, 8, 1e-6f, FNORM_F32, D, 3, NULL),
           FNORM_ERR_WORKSPACE);
    /* beyond the static scratch: refused before any HIP call */
    EXPECT("noalloc size", fnorm_rms_composed_noalloc(A, B, C, 4096, 4096, 1e-6f, FNORM_F32, NULL),
           FNORM_ERR_WORKSPACE);
    EXPECT("noalloc rows", fnorm_rms_composed_noalloc(A, B, C, -1, 8, 1e-6f, FNORM_F32, NULL),
           FNORM_ERR_SHAPE);
    EXPECT("noalloc none", fnorm_rms_composed_noalloc(NULL, NULL, NULL, 0, 8, 1e-6f, FNORM_F32,
                                                      NULL),
           FNORM_OK);
    EXPECT("copy alias", fnorm_bench_copy(A, A + 16, 64, NULL), FNORM_ERR_ALIAS);
    CHECK(fnorm_composed_workspace_bytes(0, INT64_MAX / 2, 1 << 20) == -1);
    CHECK(strlen(fnorm_last_error()) != 0);
    EXPECT("no rows", fnorm_layer(NULL, NULL, NULL, NULL, 0, 8, 1e-5f, FNORM_BF16, NULL), FNORM_OK);
    CHECK(strlen(fnorm_last_error()) == 0);
}

int main(void)
{
    for (int pass = 0; pass < 2; ++pass) {   /* second pass: the candidate cache is warm */
        tables();
        entry_points();
    }
    if (failures == 0) printf("host paths ok\n");
    return failures == 0 ? 0 : 1;
}
