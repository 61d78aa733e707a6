// Row-normalization kernels for gfx950.
//
// Operations (definitions: Emily.Fast API docs, sections `rms_norm`,
// `layer_norm`, `rope`; dual form and the gated output norm: mlx-c-rust
// `compile/norm_fusion.rs`, module docs):
//   RMSNorm    y = x * rsqrt(mean(x^2) + eps) * w
//   LayerNorm  y = (x - mean) * rsqrt(var + eps) * w + b   (population var)
//   dual       RMSNorm of the query head vectors with the query weight and
//              of the key head vectors with the key weight, one launch.
//   gated      RMSNorm times SiLU(gate), the gate a second input of x's shape
//              (OP_RMS_GATED: the RMSNorm kernel with the gate read beside x).
//   dual+RoPE  the dual form with both outputs rotated before the store
//              (`dual_rope_rows`, in fnorm_rope.hpp).
//
// Resident kernel (`norm_rows`): a row of `width` elements is owned by LPR
// threads (a lane group inside a wavefront, one wavefront, or LPR/64
// wavefronts of a workgroup).  Thread `lane` holds VPT packs of VEC elements,
// pack v covering columns (v * LPR + lane) * VEC ...  + VEC - 1, so every
// load instruction of a row group reads LPR * 16 contiguous bytes.  The row
// is read from HBM once into registers, reduced, normalized and written
// once.  Weights (and bias) are loaded once per thread before the row loop
// and stay in registers for every row the block visits (grid-stride loop
// over block-rows, so the trip count is uniform inside a block and the
// barriers of multi-wave rows are never divergent).
//
// Arithmetic is fp32 throughout (bf16 and fp16 inputs widen exactly), with explicit
// fmaf where a fused multiply-add is meant; the library is compiled with
// -ffp-contract=off so no other contraction happens.  LayerNorm takes the
// mean first and then, from the registers (no second HBM read), the
// deviations d = x - mean: it uses the corrected two-pass form of Chan,
// Golub and LeVeque ("Algorithms for computing the sample variance", 1983):
// c = sum(d) / N is the rounding error of the fp32 mean, the centred values
// are d - c and var = (sum(d^2) - c * sum(d)) / N.  This stays accurate for
// rows with a large mean, with outliers, and with a variance far below eps,
// where an uncorrected fp32 mean error would be scaled by 1/sqrt(eps).
//
// Wide kernel (`norm_rows_wide`): rows wider than the resident capacity.  One
// workgroup per row; passes over the row accumulate the sums (re-reading x
// from memory) and a last pass normalizes.
#pragma once

#include "fnorm_device.hpp"

namespace fnorm {

struct NormArgs {
    const void* x;      // [rows1, width] (dual: queries)
    const void* w;      // [width]        (dual: query weight)
    const void* b;      // [width] or null (LayerNorm only)
    void* y;            // [rows1, width]
    const void* x2;     // dual only: keys [rows - rows1, width]
    const void* w2;     // dual only: key weight
    void* y2;           // dual only: normalized keys
    int64_t rows;       // rows to process (dual: query rows + key rows)
    int64_t rows1;      // rows of the first tensor (== rows unless dual)
    int64_t width;
    float eps;
    // Row addressing, in elements: row r of x starts at
    //   (r / xh) * xs + (r % xh) * width
    // (xh rows per token, xs the token stride; xh = 1 and xs = width for a
    // contiguous tensor) and its output row at the same with ys.  x2 / y2
    // likewise with x2h, x2s, y2s.
    int64_t xs, ys, xh;
    int64_t x2s, y2s, x2h;
    // OP_RMS_GATED only: the gate, row r at r * gs (one row per token).
    const void* g;
    int64_t gs;
    // Division by xh / x2h for rows < 2^31 (m == 0: not set, divide plainly).
    FastDiv xdiv, x2div;
    // 1 / width in fp32: the row means multiply by it (exact for power-of-two
    // widths; otherwise one more rounding than a division, ~6e-8 relative,
    // for a tenth of the instructions)
    float inv_width;
};

struct RowOff {
    int64_t x, y;
};

// Element offsets of row r's input and output (see NormArgs).  One-row
// tokens take no division; otherwise a multiply-high division by the
// invariant head count when the host prepared one and r fits in 32 bits.
__device__ __forceinline__ RowOff row_offsets(int64_t r, int64_t heads, const FastDiv& hd,
                                              int64_t xs, int64_t ys, int64_t width) {
    if (heads == 1) return RowOff{r * xs, r * ys};
    const int64_t t = (hd.m != 0 && r <= 0x7fffffff) ? int64_t(hd.div(uint32_t(r))) : r / heads;
    const int64_t h = r - t * heads;
    return RowOff{t * xs + h * width, t * ys + h * width};
}

template <int OP, int DT, int VEC, int VPT, int LPR, int BLOCK, bool MASKED, bool BIAS,
          bool DUAL, int NT>
__global__ __launch_bounds__(BLOCK) void norm_rows(NormArgs a) {
    constexpr bool NT_LD = (NT & NT_LOAD) != 0;
    constexpr bool NT_ST = (NT & NT_STORE) != 0;
    constexpr bool GATED = OP == OP_RMS_GATED;
    using R = typename Raw<DT, VEC>::type;
    static_assert(BLOCK % 64 == 0 && BLOCK % LPR == 0, "launch shape");
    static_assert(!(GATED && (DUAL || BIAS)), "the gate goes with plain RMSNorm");
    constexpr int RPB = BLOCK / LPR;                 // rows per block-row
    constexpr int WPR = LPR > 64 ? LPR / 64 : 1;     // waves per row
    constexpr int LDS_SLOTS = LPR > 64 ? RPB * WPR : 1;
    __shared__ float red[3][LDS_SLOTS];
    // Registers vs VALU work: with few elements per thread, let the compiler
    // keep the widened fp32 copies of x (across the passes) and of the
    // weights (across rows), saving a widening op per element per use; with
    // many, keep them as raw packs so the VGPR count (and so occupancy)
    // stays bounded.
    constexpr int E = VPT * VEC;
    constexpr bool PACK_X = E > 32;
    constexpr bool PACK_W = E > 16;

    const int tid = threadIdx.x;
    const int group = tid / LPR;
    const int lane = tid % LPR;
    const int64_t width = a.width;
    const float inv_width = a.inv_width;

    // Work units are block-rows of RPB rows.  A dual launch numbers the
    // first tensor's (queries) units before the second's (keys), so no unit
    // holds rows of both: the tensor of a unit is uniform over the
    // workgroup, its pointers and strides are scalars, and rows are counted
    // within the tensor.  One grid-stride loop covers all units, so the
    // work per workgroup stays as even as with a single tensor.
    const int64_t units1 = DUAL ? (a.rows1 + RPB - 1) / RPB : 0;
    const int64_t units = DUAL ? units1 + (a.rows - a.rows1 + RPB - 1) / RPB
                               : (a.rows + RPB - 1) / RPB;

    // Column of pack v of this thread, and whether it lies inside the row.
    auto col_of = [&](int v) { return int64_t(v * LPR + lane) * VEC; };
    auto in_row = [&](int v) { return !MASKED || col_of(v) < width; };
    // The same column as a byte offset: a row here spans at most 8192
    // 16-byte packs, so 32 bits hold it.
    auto col_b = [&](int v) { return uint32_t((v * LPR + lane) * VEC * Elem<DT>::bytes); };
    const char* const wb = static_cast<const char*>(a.w);
    const char* const bb = static_cast<const char*>(a.b);
    const char* const w2b = static_cast<const char*>(a.w2);

    R wv[VPT];
    R bv[BIAS ? VPT : 1];
    R wv2[DUAL ? VPT : 1];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        wv[v] = in_row(v) ? load_at<DT, VEC, false>(wb, col_b(v)) : raw_zero<DT, VEC>();
        if constexpr (BIAS)
            bv[v] = in_row(v) ? load_at<DT, VEC, false>(bb, col_b(v)) : raw_zero<DT, VEC>();
        if constexpr (DUAL)
            wv2[v] = in_row(v) ? load_at<DT, VEC, false>(w2b, col_b(v)) : raw_zero<DT, VEC>();
    }

    // Where block-row `base` of this thread's row group lives.  Row groups
    // past the end re-read the last row (in bounds, so the loads need no
    // predicate) and store nothing.  (Issuing the next block-row's loads
    // before this row's reductions measured slower on every bench shape.)
    struct Loc {
        bool valid, second;   // second: uniform over the workgroup
        const char* xr;       // first byte of the row, input and output
        char* yr;
        const char* gr;       // and of its gate row
    };
    auto locate = [&](int64_t unit) {
        Loc L;
        L.second = DUAL && unit >= units1;
        const int64_t base = (L.second ? unit - units1 : unit) * RPB;
        const int64_t last = (DUAL ? (L.second ? a.rows - a.rows1 : a.rows1) : a.rows) - 1;
        L.valid = base + group <= last;
        const int64_t r = L.valid ? base + group : last;   // row of this tensor
        const RowOff off = L.second ? row_offsets(r, a.x2h, a.x2div, a.x2s, a.y2s, width)
                                    : row_offsets(r, a.xh, a.xdiv, a.xs, a.ys, width);
        L.xr = static_cast<const char*>(L.second ? a.x2 : a.x) + off.x * Elem<DT>::bytes;
        L.yr = static_cast<char*>(L.second ? a.y2 : a.y) + off.y * Elem<DT>::bytes;
        L.gr = GATED ? static_cast<const char*>(a.g) + r * a.gs * Elem<DT>::bytes : nullptr;
        return L;
    };
    auto load_row = [&](const Loc& L, R* dst) {
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            dst[v] = in_row(v) ? load_at<DT, VEC, NT_LD>(L.xr, col_b(v)) : raw_zero<DT, VEC>();
    };
    auto load_gate = [&](const Loc& L, R* dst) {
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            dst[v] = in_row(v) ? load_at<DT, VEC, NT_LD>(L.gr, col_b(v)) : raw_zero<DT, VEC>();
    };

    int parity = 0;
    for (int64_t unit = xcd_major(blockIdx.x, gridDim.x, units); unit < units;
         unit += gridDim.x) {
        const Loc cur = locate(unit);
        R xv[VPT];
        load_row(cur, xv);
        R gv[GATED ? VPT : 1];
        if constexpr (GATED) load_gate(cur, gv);
        // Every load of the row is issued before any of its data is used.
        // Without this fence the scheduler may hold a load back to save a
        // few registers (for an occupancy the grid cap never uses), which
        // adds a second memory round trip per row: RMSNorm 16384x8192 ran
        // 13% slower that way.
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PACK_W) {
            keep_packed<VPT>(wv);
            if constexpr (BIAS) keep_packed<VPT>(bv);
            if constexpr (DUAL) keep_packed<VPT>(wv2);
        }

        // Row scalars, then out = (x - shift) * scale * w + bias.
        if constexpr (OP == OP_RMS || GATED) {
            float ss = 0.0f;
#pragma unroll
            for (int v = 0; v < VPT; ++v)
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const float f = elem<DT, VEC>(xv[v], i);
                    ss = __builtin_fmaf(f, f, ss);
                }
            ss = row_sum<LPR>(ss, red[parity], group, lane);
            parity ^= 1;
            const float scale = __builtin_amdgcn_rsqf(ss * inv_width + a.eps);
            if constexpr (PACK_X) keep_packed<VPT>(xv);
            if constexpr (GATED && PACK_X) keep_packed<VPT>(gv);
            if (cur.valid) {
                static_for<VPT>([&](auto vi) {
                    constexpr int v = decltype(vi)::value;
                    // a select of values: selecting between the two arrays'
                    // elements as lvalues makes a pointer select, which can
                    // push both weight arrays to scratch memory
                    const R w1 = wv[v];
                    R wr = w1;
                    if constexpr (DUAL) {
                        const R w2 = wv2[v];
                        wr = cur.second ? w2 : w1;
                    }
                    float o[VEC];
#pragma unroll
                    for (int i = 0; i < VEC; ++i)
                        o[i] = (elem<DT, VEC>(xv[v], i) * scale) * elem<DT, VEC>(wr, i);
                    if constexpr (GATED) {
#pragma unroll
                        for (int i = 0; i < VEC; ++i) o[i] *= silu(elem<DT, VEC>(gv[v], i));
                    }
                    if (in_row(v))
                        store_at<DT, VEC, NT_ST>(cur.yr, col_b(v), make_raw<DT, VEC>(o));
                });
            }
        } else {
            float sum = 0.0f;
#pragma unroll
            for (int v = 0; v < VPT; ++v)
#pragma unroll
                for (int i = 0; i < VEC; ++i) sum += elem<DT, VEC>(xv[v], i);
            sum = row_sum<LPR>(sum, red[0], group, lane);
            const float mean = sum * inv_width;
            if constexpr (PACK_X) keep_packed<VPT>(xv);
            float sd = 0.0f, sq = 0.0f;
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                if (in_row(v)) {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) {
                        const float d = elem<DT, VEC>(xv[v], i) - mean;
                        sd += d;
                        sq = __builtin_fmaf(d, d, sq);
                    }
                }
            }
            row_sum2<LPR>(sd, sq, red[1], red[2], group, lane);
            const float c = sd * inv_width;
            const float var = __builtin_fmaxf((sq - c * sd) * inv_width, 0.0f);
            const float scale = __builtin_amdgcn_rsqf(var + a.eps);
            if constexpr (PACK_X) keep_packed<VPT>(xv);
            // x - mean - c is evaluated as (x - mean) - c.
            if (cur.valid) {
                static_for<VPT>([&](auto vi) {
                    constexpr int v = decltype(vi)::value;
                    float o[VEC];
#pragma unroll
                    for (int i = 0; i < VEC; ++i) {
                        const float d = (elem<DT, VEC>(xv[v], i) - mean) - c;
                        const float bias = BIAS ? elem<DT, VEC>(bv[v], i) : 0.0f;
                        o[i] = __builtin_fmaf(d * scale, elem<DT, VEC>(wv[v], i), bias);
                    }
                    if (in_row(v))
                        store_at<DT, VEC, NT_ST>(cur.yr, col_b(v), make_raw<DT, VEC>(o));
                });
            }
        }
    }
}

// Rows wider than the resident capacity: one workgroup of BLOCK threads per
// row (grid-stride over rows), VEC elements per access, strided by
// BLOCK * VEC.  RMSNorm: one pass for sum(x^2), one to normalize.
// LayerNorm: one pass for the mean, one for the squared deviations, one to
// normalize (the same corrected two-pass as above).  The dual form is not
// offered here; rows are addressed with a plain row stride (xh = 1).  The
// gated RMSNorm reads its gate in the last pass.
template <int OP, int DT, int VEC, int BLOCK, bool BIAS>
__global__ __launch_bounds__(BLOCK) void norm_rows_wide(NormArgs a) {
    using R = typename Raw<DT, VEC>::type;
    __shared__ float red[3][BLOCK / 64];
    const int tid = threadIdx.x;
    const int64_t width = a.width;
    const float inv_width = a.inv_width;
    constexpr int64_t STEP = int64_t(BLOCK) * VEC;

    for (int64_t row = xcd_major(blockIdx.x, gridDim.x, a.rows); row < a.rows; row += gridDim.x) {
        const int64_t off = row * a.xs;
        const int64_t yoff = row * a.ys;
        float s, mean = 0.0f, c = 0.0f;
        if constexpr (OP == OP_RMS || OP == OP_RMS_GATED) {
            float ss = 0.0f;
            for (int64_t col = int64_t(tid) * VEC; col < width; col += STEP) {
                const R xr = load_raw<DT, VEC, false>(a.x, off + col);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const float f = elem<DT, VEC>(xr, i);
                    ss = __builtin_fmaf(f, f, ss);
                }
            }
            ss = row_sum<BLOCK>(ss, red[0], 0, tid);
            s = __builtin_amdgcn_rsqf(ss * inv_width + a.eps);
        } else {
            float sum = 0.0f;
            for (int64_t col = int64_t(tid) * VEC; col < width; col += STEP) {
                const R xr = load_raw<DT, VEC, false>(a.x, off + col);
#pragma unroll
                for (int i = 0; i < VEC; ++i) sum += elem<DT, VEC>(xr, i);
            }
            sum = row_sum<BLOCK>(sum, red[0], 0, tid);
            mean = sum * inv_width;
            float sd = 0.0f, sq = 0.0f;
            for (int64_t col = int64_t(tid) * VEC; col < width; col += STEP) {
                const R xr = load_raw<DT, VEC, false>(a.x, off + col);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const float d = elem<DT, VEC>(xr, i) - mean;
                    sd += d;
                    sq = __builtin_fmaf(d, d, sq);
                }
            }
            row_sum2<BLOCK>(sd, sq, red[1], red[2], 0, tid);
            c = sd * inv_width;
            const float var = __builtin_fmaxf((sq - c * sd) * inv_width, 0.0f);
            s = __builtin_amdgcn_rsqf(var + a.eps);
        }
        for (int64_t col = int64_t(tid) * VEC; col < width; col += STEP) {
            const R xr = load_raw<DT, VEC, false>(a.x, off + col);
            const R wr = load_raw<DT, VEC, false>(a.w, col);
            float o[VEC];
            if constexpr (OP == OP_RMS || OP == OP_RMS_GATED) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) o[i] = (elem<DT, VEC>(xr, i) * s) * elem<DT, VEC>(wr, i);
                if constexpr (OP == OP_RMS_GATED) {
                    const R gr = load_raw<DT, VEC, false>(a.g, row * a.gs + col);
#pragma unroll
                    for (int i = 0; i < VEC; ++i) o[i] *= silu(elem<DT, VEC>(gr, i));
                }
            } else {
                R br = raw_zero<DT, VEC>();
                if constexpr (BIAS) br = load_raw<DT, VEC, false>(a.b, col);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const float d = (elem<DT, VEC>(xr, i) - mean) - c;
                    o[i] = __builtin_fmaf(d * s, elem<DT, VEC>(wr, i), elem<DT, VEC>(br, i));
                }
            }
            store_raw<DT, VEC, false>(a.y, yoff + col, make_raw<DT, VEC>(o));
        }
        // The partial slots of this row are read above; make sure every wave
        // is past those reads before the next row overwrites them.
        __syncthreads();
    }
}

// Plain copy, the practical HBM ceiling the norms are measured against (it
// reads and writes the same bytes a one-pass norm does, with no
// arithmetic).  Each thread moves U 16-byte packs per step (all loads
// issued before the stores), with non-temporal accesses; `n16` = number of
// 16-byte packs.
template <int BLOCK, int U>
__global__ __launch_bounds__(BLOCK) void copy16(const u32x4* __restrict__ src,
                                                u32x4* __restrict__ dst, int64_t n16) {
    const int64_t step = int64_t(gridDim.x) * BLOCK * U;
    // hardware block order: with a full grid (one chunk per workgroup) the
    // XCD-major order spreads the chunks in flight over 8 distant regions
    // and measured 7% slower; it pays only for persistent grids
    for (int64_t base = int64_t(blockIdx.x) * BLOCK * U + threadIdx.x; base < n16;
         base += step) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + int64_t(u) * BLOCK;
            if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + int64_t(u) * BLOCK;
            if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

}  // namespace fnorm
