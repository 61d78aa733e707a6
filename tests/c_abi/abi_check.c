/*
 * Compiles against include/fnorm.h as plain C11 and links libfnorm.so: every
 * call below fails argument validation, which the library does before any
 * HIP call, so this runs without a GPU.  Exit status 0 when every status
 * code is the one the header documents.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fnorm.h"

static int failures = 0;

static void expect(const char *what, int got, int want)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d (%s), expected %d: %s\n", what, got,
                fnorm_status_string(got), want, fnorm_last_error());
        ++failures;
    }
}

int main(void)
{
    void *x = (void *)0x10000, *w = (void *)0x20000000, *y = (void *)0x40000000;
    char buf[128];

    expect("rms rows<0", fnorm_rms(x, w, y, -1, 8, 1e-6f, FNORM_BF16, NULL), FNORM_ERR_SHAPE);
    expect("rms eps<0", fnorm_rms(x, w, y, 4, 8, -1.0f, FNORM_BF16, NULL), FNORM_ERR_EPS);
    expect("rms dtype", fnorm_rms(x, w, y, 4, 8, 1e-6f, 9, NULL), FNORM_ERR_DTYPE);
    expect("rms null", fnorm_rms(NULL, w, y, 4, 8, 1e-6f, FNORM_F32, NULL), FNORM_ERR_NULL);
    expect("rms alias", fnorm_rms(x, w, (char *)x + 16, 4, 8, 1e-6f, FNORM_F32, NULL),
           FNORM_ERR_ALIAS);
    expect("rms no rows", fnorm_rms(NULL, NULL, NULL, 0, 8, 1e-6f, FNORM_F16, NULL), FNORM_OK);
    expect("layer width", fnorm_layer(x, w, NULL, y, 4, 0, 1e-5f, FNORM_BF16, NULL),
           FNORM_ERR_SHAPE);
    expect("dual null k", fnorm_dual_head_rms(x, NULL, w, w, y, (char *)y + 4096, 4, 4, 128,
                                              1e-6f, FNORM_BF16, NULL),
           FNORM_ERR_NULL);
    expect("rope dims", fnorm_dual_head_rms_rope(x, x, w, w, y, y, 4, 2, 1, 128, 1e-6f, 127, 0,
                                                 10000.0f, 1.0f, 0, NULL, FNORM_BF16, NULL),
           FNORM_ERR_SHAPE);
    expect("swiglu gate", fnorm_rms_swiglu(x, NULL, w, y, 4, 8, 1e-6f, FNORM_BF16, NULL),
           FNORM_ERR_NULL);
    expect("strided stride", fnorm_rms_strided(x, 4, w, y, 8, 4, 8, 1e-6f, FNORM_F32, NULL, -1),
           FNORM_ERR_SHAPE);
    expect("composed ws", fnorm_rms_composed(x, w, y, 4, 8, 1e-6f, FNORM_F32, NULL, 0, NULL),
           FNORM_ERR_WORKSPACE);
    expect("copy size", fnorm_bench_copy(x, y, 24, NULL), FNORM_ERR_SHAPE);
    expect("describe shape", fnorm_describe_shape(FNORM_OP_RMS, FNORM_BF16, 8192, 1, -1, buf,
                                                  sizeof buf),
           FNORM_OK);
    if (strncmp(buf, "rms.bf16.", 9) != 0) {
        fprintf(stderr, "describe_shape gave '%s'\n", buf);
        ++failures;
    }
    /* the call form: a misaligned x takes the scalar-access kernel */
    expect("describe call", fnorm_describe(FNORM_OP_LAYER, (char *)x + 2, 8192, NULL, 0, w, NULL,
                                           y, 8192, 4, 8192, FNORM_BF16, -1, buf, sizeof buf),
           FNORM_OK);
    if (strncmp(buf, "layer.bf16.vec1.", 16) != 0) {
        fprintf(stderr, "describe gave '%s'\n", buf);
        ++failures;
    }
    expect("describe call error", fnorm_describe(FNORM_OP_RMS, x, 8, NULL, 0, w, NULL,
                                                 (char *)x + 16, 8, 4, 8, FNORM_F32, -1, buf,
                                                 sizeof buf),
           FNORM_ERR_ALIAS);
    if (fnorm_variant_count(FNORM_OP_DUAL, FNORM_BF16, 128, 1) < 2) ++failures;
    if (fnorm_version() < 100) ++failures;
    if (failures == 0) printf("c abi ok (version %d)\n", fnorm_version());
    return failures == 0 ? 0 : 1;
}
