/*
 * fnorm: fused last-axis row normalizations for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfnorm.so.  Plain pointers and sizes only.
 *
 * Common conventions
 * ------------------
 *  - Tensors are row-major [rows, width], contiguous unless a call takes
 *    strides (the _strided forms below); the normalization runs
 *    over the last axis only (the fused kernels' contract in the
 *    Emily.Bumblebee.FastKernels docs, "What's not rewritten": norms over any
 *    other axis are not served).  rows is the product of the leading
 *    dimensions.
 *  - x, w, b and y are DEVICE pointers owned by the caller; they must stay
 *    valid until the work queued on `stream` has completed.  The library
 *    allocates nothing, frees nothing and never synchronizes.
 *  - All tensors of one call share one element type `dtype` (fnorm_dtype:
 *    fp32, bf16 or IEEE fp16); the output has the input's type.  Arithmetic
 *    is fp32; a bf16 or fp16 output is the fp32 result rounded once, to
 *    nearest even.
 *  - eps is fixed per call, must be finite and >= 0, and is added inside the
 *    square root.
 *  - `stream` is a hipStream_t; NULL means the null stream.  Calls return as
 *    soon as the kernel is queued.
 *  - y == x (in place) is allowed.  Any other overlap of an output with an
 *    input or with another output is rejected with FNORM_ERR_ALIAS.
 *  - Pointers that are not 16-byte aligned, and widths that are not a
 *    multiple of 16 bytes, are served (by a scalar-access kernel), not
 *    rejected.
 *  - rows == 0 is a no-op that returns FNORM_OK (pointers may then be NULL).
 *  - Every argument is validated before any HIP call; on an error nothing is
 *    launched, the status is returned and fnorm_last_error() describes it.
 *    Faults during execution surface on the stream, as for any kernel.
 *  - Thread safety: no mutable global state except read-only caches of
 *    device properties; the error text is per thread.
 */
#ifndef FNORM_H
#define FNORM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FNORM_F32 = 0, FNORM_BF16 = 1, FNORM_F16 = 2 } fnorm_dtype;

typedef enum {
    FNORM_OK = 0,
    FNORM_ERR_NULL = 1,        /* a required pointer is NULL while rows > 0 */
    FNORM_ERR_SHAPE = 2,       /* rows < 0, width <= 0, or sizes overflow */
    FNORM_ERR_EPS = 3,         /* eps negative, NaN or infinite */
    FNORM_ERR_DTYPE = 4,       /* dtype not an fnorm_dtype */
    FNORM_ERR_ALIAS = 5,       /* an output overlaps another buffer (other than y == x) */
    FNORM_ERR_UNSUPPORTED = 6, /* no kernel for the request, or variant out of range */
    FNORM_ERR_LAUNCH = 7,      /* the HIP launch failed; fnorm_last_error() has the text */
    FNORM_ERR_WORKSPACE = 8    /* workspace NULL, misaligned, too small or overlapping */
} fnorm_status;

/* Operation codes of the introspection calls (fnorm_variant_count,
 * fnorm_describe_shape, fnorm_describe).  LayerNorm with a bias and without
 * one run different kernels: FNORM_OP_LAYER names the first, except in
 * fnorm_describe, where the call's own b pointer decides. */
typedef enum {
    FNORM_OP_RMS = 0,
    FNORM_OP_LAYER = 1,
    FNORM_OP_DUAL = 2,
    FNORM_OP_RMS_SWIGLU = 3,
    FNORM_OP_LAYER_NOBIAS = 4
} fnorm_op;

/*
 * RMSNorm (Emily.Fast docs, section `rms_norm`; the composed form is the
 * Emily notebook's Part 1 RMSNorm cell):
 *     y[r, j] = x[r, j] * rsqrt(mean_j(x[r, :]^2) + eps) * w[j]
 * x, y: [rows, width]; w: [width], broadcast over rows.
 */
int fnorm_rms(const void* x, const void* w, void* y, int64_t rows, int64_t width, float eps,
              int dtype, void* stream);

/*
 * LayerNorm (Emily.Fast docs, section `layer_norm`):
 *     y[r, j] = (x[r, j] - mean) * rsqrt(var + eps) * w[j] + b[j]
 * mean and var over the row; var is the population variance (divides by
 * width).  b may be NULL, which means a zero bias (bitwise the same result).
 * x, y: [rows, width]; w, b: [width].
 */
int fnorm_layer(const void* x, const void* w, const void* b, void* y, int64_t rows,
                int64_t width, float eps, int dtype, void* stream);

/*
 * RMSNorm with a SiLU-gate epilogue, one pass (the output RMS normalization
 * of the gated-delta block chained into its SwiGLU epilogue, named in the
 * mlx-c-rust `compile/norm_fusion.rs` module docs, which rejected the fusion
 * for want of a pinned summation order):
 *     y[r, j] = RMSNorm(x, w, eps)[r, j] * SiLU(g[r, j]),
 *     SiLU(v) = v / (1 + exp(-v))
 * g (the gate) has x's shape and type.  The page does not define SwiGLU;
 * this is the gated form of the GLU variants (the gate through SiLU,
 * multiplying the normalized value), computed in fp32 and rounded once.
 * The row reduction is the one fnorm_rms uses (same kernel shapes, same
 * fixed tree), so the epilogue cannot change the summation order.
 * y may be x or g (in place); other overlaps are FNORM_ERR_ALIAS.  Gates
 * below about -87 give SiLU values under fp32's normal range.
 * The _strided form takes row strides (elements) for x, g and y as
 * fnorm_rms_strided does.
 */
int fnorm_rms_swiglu(const void* x, const void* g, const void* w, void* y, int64_t rows,
                     int64_t width, float eps, int dtype, void* stream);
int fnorm_rms_swiglu_v(const void* x, const void* g, const void* w, void* y, int64_t rows,
                       int64_t width, float eps, int dtype, void* stream, int variant);
int fnorm_rms_swiglu_strided(const void* x, int64_t x_stride, const void* g, int64_t g_stride,
                             const void* w, void* y, int64_t y_stride, int64_t rows,
                             int64_t width, float eps, int dtype, void* stream, int variant);

/*
 * Dual-output query/key head RMSNorm in ONE launch (mlx-c-rust
 * `compile/norm_fusion.rs`, module docs and the dual head-norm graph
 * builder: the per-head RMSNorms of queries and of keys, each with its own
 * scale weight and one shared eps, fused so a layer issues one launch for
 * both; the normalized queries are the first output, the keys the second).
 *     qy = RMSNorm(q, qw, eps) over head vectors of head_dim
 *     ky = RMSNorm(k, kw, eps)
 * q, qy: [q_rows, head_dim] with q_rows = tokens * query heads;
 * k, ky: [k_rows, head_dim]; qw, kw: [head_dim], shared by all heads.
 * Results are bitwise equal to fnorm_rms(q, qw, qy, ...) followed by
 * fnorm_rms(k, kw, ky, ...) with the same eps.  Either row count may be 0
 * (its pointers may then be NULL).  head_dim: any value up to 8192; above
 * that, 16-byte-aligned pointers and a multiple of the 16-byte pack (8
 * elements of bf16 / fp16, 4 of fp32), up to 65536 (bf16, fp16) or 32768
 * (fp32).  Other head sizes return FNORM_ERR_UNSUPPORTED (the row-wide
 * fnorm_rms serves any width).
 */
int fnorm_dual_head_rms(const void* q, const void* k, const void* qw, const void* kw, void* qy,
                        void* ky, int64_t q_rows, int64_t k_rows, int64_t head_dim, float eps,
                        int dtype, void* stream);

/*
 * Dual q/k head RMSNorm fused with the rotary position embedding (RoPE) of
 * both outputs, in one launch: qy = RoPE(RMSNorm(q, qw)), ky =
 * RoPE(RMSNorm(k, kw)), rounded once.  RoPE follows the Emily.Fast docs,
 * sections `rope` and `rope_with_freqs`: pair i of a head vector of token t
 * rotates by theta_i = (offset + t) * scale * inv_freq_i, with inv_freq_i =
 * base^(-2i / rope_dims), or freqs[i] when `freqs` (a DEVICE array of
 * rope_dims/2 fp32 inverse frequencies) is given; pairs are
 * (i, i + rope_dims/2) when traditional == 0 (split-half) and (2i, 2i + 1)
 * when traditional != 0 (interleaved); features at or past rope_dims pass
 * through.  Layout: q, qy [tokens, q_heads, head_dim]; k, ky
 * [tokens, k_heads, head_dim]; both share the positions.
 * rope_dims must be even, 2 <= rope_dims <= head_dim; base finite and > 0
 * (unless freqs), scale finite, offset >= 0; else FNORM_ERR_SHAPE.
 * Head shapes whose pair partners the kernel cannot reach (some partial
 * rope_dims on wide heads), and rope_dims above 4096 (the host's fp64
 * frequency tables, passed in the kernel arguments, cover 2048 pairs),
 * return FNORM_ERR_UNSUPPORTED.
 */
int fnorm_dual_head_rms_rope(const void* q, const void* k, const void* qw, const void* kw,
                             void* qy, void* ky, int64_t tokens, int64_t q_heads,
                             int64_t k_heads, int64_t head_dim, float eps, int64_t rope_dims,
                             int traditional, float base, float scale, int64_t offset,
                             const float* freqs, int dtype, void* stream);
int fnorm_dual_head_rms_rope_v(const void* q, const void* k, const void* qw, const void* kw,
                               void* qy, void* ky, int64_t tokens, int64_t q_heads,
                               int64_t k_heads, int64_t head_dim, float eps, int64_t rope_dims,
                               int traditional, float base, float scale, int64_t offset,
                               const float* freqs, int dtype, void* stream, int variant);

/*
 * Same calls with an explicit kernel variant: variant -1 is the default
 * choice (what the calls above use); 0 .. fnorm_variant_count()-1 force one
 * of the kernels able to serve the request (for testing every instance and
 * for A/B timing).  Out-of-range variants return FNORM_ERR_UNSUPPORTED.
 */
int fnorm_rms_v(const void* x, const void* w, void* y, int64_t rows, int64_t width, float eps,
                int dtype, void* stream, int variant);
int fnorm_layer_v(const void* x, const void* w, const void* b, void* y, int64_t rows,
                  int64_t width, float eps, int dtype, void* stream, int variant);
int fnorm_dual_head_rms_v(const void* q, const void* k, const void* qw, const void* kw, void* qy,
                          void* ky, int64_t q_rows, int64_t k_rows, int64_t head_dim, float eps,
                          int dtype, void* stream, int variant);

/*
 * Row-strided forms, for rows that are not packed back to back: views into a
 * wider buffer, such as the query and key parts of one packed QKV projection
 * output (the ffai-argus `kernel_micro_ab.rs` example, section 2, where the
 * packed QKV op writes the q and k buffers).  Strides count ELEMENTS of
 * `dtype`, not bytes.
 *   fnorm_rms_strided / fnorm_layer_strided: row r of x starts at
 *     x + r * x_stride, row r of y at y + r * y_stride; the rows are `width`
 *     contiguous elements.  Strides must be >= width when rows > 1.
 *   fnorm_dual_head_rms_strided / fnorm_dual_head_rms_rope_strided: q is
 *     [tokens, q_heads, head_dim] with the heads of one token contiguous and
 *     token t at q + t * q_stride (likewise k, qy, ky with their strides);
 *     every stride must be >= heads * head_dim of its tensor when
 *     tokens > 1.  The dual form computes per-head RMSNorm exactly as
 *     fnorm_dual_head_rms; the rope form exactly as fnorm_dual_head_rms_rope.
 * An output may be its own input (same pointer and stride); otherwise an
 * output must not share a byte with any other tensor of the call, which is
 * checked exactly for tensors of equal stride (interleaved q/k/v parts of one
 * buffer are accepted) and by overall extent otherwise.  The bytes between
 * rows are neither read nor written.  16-byte vector kernels are used when
 * the pointers are 16-byte aligned and every stride is a multiple of 16
 * bytes; otherwise the scalar-access kernels.  variant as for the _v calls
 * (-1 = default).  Other conventions as above.
 */
int fnorm_rms_strided(const void* x, int64_t x_stride, const void* w, void* y, int64_t y_stride,
                      int64_t rows, int64_t width, float eps, int dtype, void* stream,
                      int variant);
int fnorm_layer_strided(const void* x, int64_t x_stride, const void* w, const void* b, void* y,
                        int64_t y_stride, int64_t rows, int64_t width, float eps, int dtype,
                        void* stream, int variant);
int fnorm_dual_head_rms_strided(const void* q, int64_t q_stride, const void* k,
                                int64_t k_stride, const void* qw, const void* kw, void* qy,
                                int64_t qy_stride, void* ky, int64_t ky_stride, int64_t tokens,
                                int64_t q_heads, int64_t k_heads, int64_t head_dim, float eps,
                                int dtype, void* stream, int variant);
int fnorm_dual_head_rms_rope_strided(const void* q, int64_t q_stride, const void* k,
                                     int64_t k_stride, const void* qw, const void* kw, void* qy,
                                     int64_t qy_stride, void* ky, int64_t ky_stride,
                                     int64_t tokens, int64_t q_heads, int64_t k_heads,
                                     int64_t head_dim, float eps, int64_t rope_dims,
                                     int traditional, float base, float scale, int64_t offset,
                                     const float* freqs, int dtype, void* stream, int variant);

/*
 * Introspection: which kernel, and which launch form, a call takes.  A silent
 * slow path counts as a failure on the pages (the Emily notebook, Part 1,
 * compiles with native_fallback: :raise, so an op that cannot run natively
 * raises); these calls let a caller assert the path a concrete call takes.
 * Names look like "layer.bf16.vec8.vpt4.lpr128.blk256.exact.nt.persistent2":
 * operation, element type, elements per access (1 = the scalar-access kernel
 * taken for misaligned pointers, strides or widths), packs per thread,
 * threads per row, threads per workgroup, exact or masked width, cache
 * policy (".nt" non-temporal loads and stores, ".ntld" loads only, ".ntst"
 * stores only), and the launch: "persistent" (as many workgroups as fit),
 * "persistentK" (K per CU), "grid" (one workgroup per block of rows) or
 * "gridK" (the same, at most K resident per CU).  "wide" kernels make
 * several passes over rows wider than the register-resident capacity.
 * All of them are host-only: they make no HIP call.
 *
 * fnorm_describe, fnorm_describe_dual, fnorm_describe_dual_rope take the
 * arguments of the call they describe (strides in elements as in the
 * _strided forms; a contiguous call passes its width, or heads * head_dim,
 * and strides are ignored for a single row or token) and run that call's
 * validation and kernel choice without launching it: they return the status
 * the call would return (FNORM_ERR_* before any launch) and write the name
 * of the kernel it would launch, or "none" for a call that launches nothing
 * (no rows).  eps is not an argument (it does not affect the choice).
 *   fnorm_describe: op FNORM_OP_RMS (g and b ignored), FNORM_OP_LAYER (b may
 *     be NULL: the no-bias kernels), FNORM_OP_LAYER_NOBIAS (b ignored) or
 *     FNORM_OP_RMS_SWIGLU (g the gate, b ignored); other ops return
 *     FNORM_ERR_UNSUPPORTED.
 * fnorm_describe_shape names variant `variant` (-1 = default) for (op,
 * dtype, width) when every pointer and stride is 16-byte aligned
 * (aligned != 0) or not, and fnorm_variant_count counts those variants (0
 * for invalid arguments); variant as for the _v calls.
 * Each writes at most len bytes to buf (NUL-terminated); FNORM_ERR_NULL if
 * buf is NULL or len <= 0.
 */
int fnorm_variant_count(int op, int dtype, int64_t width, int aligned);
int fnorm_describe_shape(int op, int dtype, int64_t width, int aligned, int variant, char* buf,
                         int64_t len);
int fnorm_describe(int op, const void* x, int64_t x_stride, const void* g, int64_t g_stride,
                   const void* w, const void* b, const void* y, int64_t y_stride, int64_t rows,
                   int64_t width, int dtype, int variant, char* buf, int64_t len);
int fnorm_describe_dual(const void* q, int64_t q_stride, const void* k, int64_t k_stride,
                        const void* qw, const void* kw, const void* qy, int64_t qy_stride,
                        const void* ky, int64_t ky_stride, int64_t tokens, int64_t q_heads,
                        int64_t k_heads, int64_t head_dim, int dtype, int variant, char* buf,
                        int64_t len);
int fnorm_describe_dual_rope(const void* q, int64_t q_stride, const void* k, int64_t k_stride,
                             const void* qw, const void* kw, const void* qy, int64_t qy_stride,
                             const void* ky, int64_t ky_stride, int64_t tokens, int64_t q_heads,
                             int64_t k_heads, int64_t head_dim, int64_t rope_dims,
                             int traditional, float base, float scale, int64_t offset,
                             const float* freqs, int dtype, int variant, char* buf,
                             int64_t len);

/*
 * Composed (unfused) baselines: the same RMSNorm / LayerNorm computed one
 * primitive per launch, every intermediate going through HBM, the way a
 * framework runs the textbook formula op by op.
 *   RMSNorm (the composed cell of the Emily notebook, Part 1), 6 launches:
 *     square, row mean, + eps, sqrt, divide x by the root, multiply by w.
 *   LayerNorm (the `layer_norm` definition of the Emily.Fast docs), 9
 *   launches (8 without bias): row mean, subtract, square, row mean, + eps,
 *   sqrt, divide, multiply by w, add b.
 * Intermediates are fp32 in the caller's `workspace` (device memory, 16-byte
 * aligned, at least fnorm_composed_workspace_bytes(op, rows, width) bytes,
 * not overlapping any tensor); the output has the input's type.  They exist
 * to measure what fusion saves; they are checked against the same oracle.
 * Other conventions as above; in place (y == x) is allowed.
 */
int64_t fnorm_composed_workspace_bytes(int op, int64_t rows, int64_t width);
int fnorm_rms_composed(const void* x, const void* w, void* y, int64_t rows, int64_t width,
                       float eps, int dtype, void* workspace, int64_t workspace_bytes,
                       void* stream);
int fnorm_layer_composed(const void* x, const void* w, const void* b, void* y, int64_t rows,
                         int64_t width, float eps, int dtype, void* workspace,
                         int64_t workspace_bytes, void* stream);

/*
 * The composed RMSNorm (as fnorm_rms_composed) for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes no workspace and calls no allocating routine:
 * its fp32 intermediates live in a static device buffer of the library, 32
 * MiB per device (held by each device the library runs on until the process
 * ends), which serves rows * width up to about 8.38 million elements
 * (fnorm_composed_workspace_bytes(FNORM_OP_RMS, rows, width) <= 33554432);
 * larger calls return FNORM_ERR_WORKSPACE before any HIP call.  Every call
 * on one device shares that buffer: calls that overlap in time on one device
 * (two streams, or two threads) race and must be serialized by the caller.
 * The buffer keeps the last call's contents; the chain writes every
 * intermediate before reading it, so nothing needs clearing.  Results are
 * bitwise those of fnorm_rms_composed.  Other conventions as above.
 */
int fnorm_rms_composed_noalloc(const void* x, const void* w, void* y, int64_t rows,
                               int64_t width, float eps, int dtype, void* stream);

/* Variant count and kernel name of the fused dual norm + RoPE, as above. */
int fnorm_rope_variant_count(int dtype, int64_t head_dim, int64_t rope_dims, int traditional,
                             int aligned);
int fnorm_describe_rope(int dtype, int64_t head_dim, int64_t rope_dims, int traditional,
                        int aligned, int variant, char* buf, int64_t len);

/*
 * Errors follow the error type of mlx-c-rust `compile/norm_fusion.rs` (the
 * dual head-norm graph builder and its callers): a failed call reports an
 * operation name plus a description, and structural checks (input and output
 * counts there; pointers, sizes, overlaps here) run before any work.
 *
 * fnorm_status_string: static text of a status code ("unknown fnorm status"
 * for codes outside fnorm_status); never NULL.
 * fnorm_last_error: the text of the last error on the calling thread,
 * "operation: description" (e.g. "fnorm_rms: rows=-1 width=8 (need rows >=
 * 0, width > 0)"), or "" if the thread's last fnorm call succeeded.  The
 * storage is per thread and valid until that thread's next fnorm call.
 */
const char* fnorm_status_string(int status);
const char* fnorm_last_error(void);

/* Library version, as major * 10000 + minor * 100 + patch. */
int fnorm_version(void);

/*
 * Measurement aid, not a normalization: copies `bytes` bytes from src to dst
 * with 16-byte loads and stores (the practical HBM ceiling a one-pass norm
 * is compared with).  bytes must be a multiple of 16 and both pointers
 * 16-byte aligned, the ranges must not overlap; else FNORM_ERR_SHAPE /
 * FNORM_ERR_ALIAS.
 */
int fnorm_bench_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * Measurement aid: what the HIP runtime reports for the current device (the
 * one hipGetDevice names): its peak memory clock in kHz, its memory bus
 * width in bits and its compute-unit count.  Any output pointer may be
 * NULL.  FNORM_ERR_LAUNCH (with the runtime's text in fnorm_last_error())
 * when the runtime cannot be queried, e.g. with no device.
 */
int fnorm_device_memory(int* clock_khz, int* bus_bits, int* compute_units);

#ifdef __cplusplus
}
#endif

#endif /* FNORM_H */
