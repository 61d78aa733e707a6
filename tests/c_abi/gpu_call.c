/*
 * The library called from plain C on the GPU, with no Python in the call
 * path: reads bf16 inputs from files in DIR, runs every fused entry point
 * on the null stream, writes the outputs back to DIR.  The GPU test that
 * drives it compares the files bitwise with the same calls made through the
 * Python binding.
 *
 *   gpu_call DIR ROWS WIDTH TOKENS Q_HEADS K_HEADS HEAD_DIM
 *
 * Inputs (raw little-endian bf16): x, g [ROWS, WIDTH]; w, b [WIDTH];
 * q [TOKENS, Q_HEADS, HEAD_DIM], k [TOKENS, K_HEADS, HEAD_DIM];
 * qw, kw [HEAD_DIM].  Outputs: rms, layer, swiglu, qy, ky, qr, kr.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fnorm.h"

static const char *dir;

static void *read_to_device(const char *name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s.bin", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
    void *host = malloc(bytes);
    if (!host || fread(host, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
    fclose(f);
    void *dev = NULL;
    if (hipMalloc(&dev, bytes) != hipSuccess ||
        hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        fprintf(stderr, "device copy of %s failed\n", name);
        exit(3);
    }
    free(host);
    return dev;
}

static void *device_buffer(size_t bytes)
{
    void *dev = NULL;
    if (hipMalloc(&dev, bytes) != hipSuccess) { fprintf(stderr, "hipMalloc failed\n"); exit(3); }
    return dev;
}

static void write_from_device(const char *name, const void *dev, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s.bin", dir, name);
    void *host = malloc(bytes);
    if (!host || hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
        fprintf(stderr, "copy back of %s failed\n", name);
        exit(3);
    }
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(host, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
    fclose(f);
    free(host);
}

static void check(const char *what, int status)
{
    if (status != FNORM_OK) {
        fprintf(stderr, "%s: %s (%s)\n", what, fnorm_status_string(status), fnorm_last_error());
        exit(4);
    }
}

int main(int argc, char **argv)
{
    if (argc != 8) {
        fprintf(stderr, "usage: %s DIR ROWS WIDTH TOKENS Q_HEADS K_HEADS HEAD_DIM\n", argv[0]);
        return 1;
    }
    dir = argv[1];
    const int64_t rows = atoll(argv[2]), width = atoll(argv[3]), tokens = atoll(argv[4]);
    const int64_t qh = atoll(argv[5]), kh = atoll(argv[6]), hd = atoll(argv[7]);
    const size_t e = 2;   /* bf16 */
    const size_t xb = (size_t)(rows * width) * e, wb = (size_t)width * e;
    const size_t qb = (size_t)(tokens * qh * hd) * e, kb = (size_t)(tokens * kh * hd) * e;
    const size_t hb = (size_t)hd * e;

    void *x = read_to_device("x", xb), *g = read_to_device("g", xb);
    void *w = read_to_device("w", wb), *b = read_to_device("b", wb);
    void *q = read_to_device("q", qb), *k = read_to_device("k", kb);
    void *qw = read_to_device("qw", hb), *kw = read_to_device("kw", hb);
    void *y_rms = device_buffer(xb), *y_layer = device_buffer(xb), *y_gate = device_buffer(xb);
    void *qy = device_buffer(qb), *ky = device_buffer(kb);
    void *qr = device_buffer(qb), *kr = device_buffer(kb);

    check("fnorm_rms", fnorm_rms(x, w, y_rms, rows, width, 1e-5f, FNORM_BF16, NULL));
    check("fnorm_layer", fnorm_layer(x, w, b, y_layer, rows, width, 1e-5f, FNORM_BF16, NULL));
    check("fnorm_rms_swiglu",
          fnorm_rms_swiglu(x, g, w, y_gate, rows, width, 1e-5f, FNORM_BF16, NULL));
    check("fnorm_dual_head_rms", fnorm_dual_head_rms(q, k, qw, kw, qy, ky, tokens * qh,
                                                     tokens * kh, hd, 1e-6f, FNORM_BF16, NULL));
    check("fnorm_dual_head_rms_rope",
          fnorm_dual_head_rms_rope(q, k, qw, kw, qr, kr, tokens, qh, kh, hd, 1e-6f, hd, 0,
                                   10000.0f, 1.0f, 5, NULL, FNORM_BF16, NULL));
    if (hipDeviceSynchronize() != hipSuccess) { fprintf(stderr, "kernel failed\n"); return 5; }

    write_from_device("rms", y_rms, xb);
    write_from_device("layer", y_layer, xb);
    write_from_device("swiglu", y_gate, xb);
    write_from_device("qy", qy, qb);
    write_from_device("ky", ky, kb);
    write_from_device("qr", qr, qb);
    write_from_device("kr", kr, kb);
    printf("gpu_call ok\n");
    return 0;
}
