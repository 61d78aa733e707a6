// Row-normalization kernels for gfx950.
//
// Operations (definitions: Emily.Fast API docs, sections `rms_norm` and
// `layer_norm`; dual form: mlx-c-rust `compile/norm_fusion.rs`):
//   RMSNorm    y = x * rsqrt(mean(x^2) + eps) * w
//   LayerNorm  y = (x - mean) * rsqrt(var + eps) * w + b   (population var)
//   dual       RMSNorm of the query head vectors with the query weight and
//              of the key head vectors with the key weight, one launch.
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
// Arithmetic is fp32 throughout (bf16 inputs widen exactly), with explicit
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
};

template <int OP, int DT, int VEC, int VPT, int LPR, int BLOCK, bool MASKED, bool BIAS,
          bool DUAL, int NT>
__global__ __launch_bounds__(BLOCK) void norm_rows(NormArgs a) {
    constexpr bool NT_LD = (NT & NT_LOAD) != 0;
    constexpr bool NT_ST = (NT & NT_STORE) != 0;
    using R = typename Raw<DT, VEC>::type;
    static_assert(BLOCK % 64 == 0 && BLOCK % LPR == 0, "launch shape");
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
    const float fwidth = static_cast<float>(width);
    const int64_t last = a.rows - 1;

    // Column of pack v of this thread, and whether it lies inside the row.
    auto col_of = [&](int v) { return int64_t(v * LPR + lane) * VEC; };
    auto in_row = [&](int v) { return !MASKED || col_of(v) < width; };

    R wv[VPT];
    R bv[BIAS ? VPT : 1];
    R wv2[DUAL ? VPT : 1];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        wv[v] = in_row(v) ? load_raw<DT, VEC, false>(a.w, col_of(v)) : raw_zero<DT, VEC>();
        if constexpr (BIAS)
            bv[v] = in_row(v) ? load_raw<DT, VEC, false>(a.b, col_of(v)) : raw_zero<DT, VEC>();
        if constexpr (DUAL)
            wv2[v] = in_row(v) ? load_raw<DT, VEC, false>(a.w2, col_of(v)) : raw_zero<DT, VEC>();
    }

    int parity = 0;
    for (int64_t base = int64_t(blockIdx.x) * RPB; base < a.rows;
         base += int64_t(gridDim.x) * RPB) {
        // Row groups past the end re-read the last row (in bounds, so the
        // loads need no predicate) and store nothing.
        const bool valid = base + group <= last;
        const int64_t row = valid ? base + group : last;
        const void* xp = a.x;
        void* yp = a.y;
        int64_t r = row;
        bool second = false;
        if constexpr (DUAL) {
            second = row >= a.rows1;
            if (second) {
                xp = a.x2;
                yp = a.y2;
                r = row - a.rows1;
            }
        }
        const int64_t row_off = r * width;
        if constexpr (PACK_W) {
            keep_packed<VPT>(wv);
            if constexpr (BIAS) keep_packed<VPT>(bv);
            if constexpr (DUAL) keep_packed<VPT>(wv2);
        }

        R xv[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            xv[v] = in_row(v) ? load_raw<DT, VEC, NT_LD>(xp, row_off + col_of(v))
                              : raw_zero<DT, VEC>();

        // Row scalars: out = (x - shift) * scale * w + bias.
        float shift = 0.0f, scale;
        if constexpr (OP == OP_RMS) {
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
            scale = __builtin_amdgcn_rsqf(ss / fwidth + a.eps);
            if constexpr (PACK_X) keep_packed<VPT>(xv);
        } else {
            float sum = 0.0f;
#pragma unroll
            for (int v = 0; v < VPT; ++v)
#pragma unroll
                for (int i = 0; i < VEC; ++i) sum += elem<DT, VEC>(xv[v], i);
            sum = row_sum<LPR>(sum, red[0], group, lane);
            const float mean = sum / fwidth;
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
            const float c = sd / fwidth;
            const float var = __builtin_fmaxf((sq - c * sd) / fwidth, 0.0f);
            scale = __builtin_amdgcn_rsqf(var + a.eps);
            shift = mean;
            if constexpr (PACK_X) keep_packed<VPT>(xv);
            // x - mean - c is evaluated as (x - mean) - c below.
            if (valid) {
#pragma unroll
                for (int v = 0; v < VPT; ++v) {
                    float o[VEC];
#pragma unroll
                    for (int i = 0; i < VEC; ++i) {
                        const float d = (elem<DT, VEC>(xv[v], i) - shift) - c;
                        const float bias = BIAS ? elem<DT, VEC>(bv[v], i) : 0.0f;
                        o[i] = __builtin_fmaf(d * scale, elem<DT, VEC>(wv[v], i), bias);
                    }
                    if (in_row(v)) store_raw<DT, VEC, NT_ST>(yp, row_off + col_of(v), make_raw<DT, VEC>(o));
                }
            }
            continue;
        }
        if (valid) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                R wr = wv[v];
                if constexpr (DUAL) wr = second ? wv2[v] : wv[v];
                float o[VEC];
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    o[i] = (elem<DT, VEC>(xv[v], i) * scale) * elem<DT, VEC>(wr, i);
                if (in_row(v)) store_raw<DT, VEC, NT_ST>(yp, row_off + col_of(v), make_raw<DT, VEC>(o));
            }
        }
    }
}

// Rows wider than the resident capacity: one workgroup of BLOCK threads per
// row (grid-stride over rows), VEC elements per access, strided by
// BLOCK * VEC.  RMSNorm: one pass for sum(x^2), one to normalize.
// LayerNorm: one pass for the mean, one for the squared deviations, one to
// normalize (the same corrected two-pass as above).  The dual form is not
// offered here.
template <int OP, int DT, int VEC, int BLOCK, bool BIAS>
__global__ __launch_bounds__(BLOCK) void norm_rows_wide(NormArgs a) {
    using R = typename Raw<DT, VEC>::type;
    __shared__ float red[3][BLOCK / 64];
    const int tid = threadIdx.x;
    const int64_t width = a.width;
    const float fwidth = static_cast<float>(width);
    constexpr int64_t STEP = int64_t(BLOCK) * VEC;

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t off = row * width;
        float s, mean = 0.0f, c = 0.0f;
        if constexpr (OP == OP_RMS) {
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
            s = __builtin_amdgcn_rsqf(ss / fwidth + a.eps);
        } else {
            float sum = 0.0f;
            for (int64_t col = int64_t(tid) * VEC; col < width; col += STEP) {
                const R xr = load_raw<DT, VEC, false>(a.x, off + col);
#pragma unroll
                for (int i = 0; i < VEC; ++i) sum += elem<DT, VEC>(xr, i);
            }
            sum = row_sum<BLOCK>(sum, red[0], 0, tid);
            mean = sum / fwidth;
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
            c = sd / fwidth;
            const float var = __builtin_fmaxf((sq - c * sd) / fwidth, 0.0f);
            s = __builtin_amdgcn_rsqf(var + a.eps);
        }
        for (int64_t col = int64_t(tid) * VEC; col < width; col += STEP) {
            const R xr = load_raw<DT, VEC, false>(a.x, off + col);
            const R wr = load_raw<DT, VEC, false>(a.w, col);
            float o[VEC];
            if constexpr (OP == OP_RMS) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) o[i] = (elem<DT, VEC>(xr, i) * s) * elem<DT, VEC>(wr, i);
            } else {
                R br = raw_zero<DT, VEC>();
                if constexpr (BIAS) br = load_raw<DT, VEC, false>(a.b, col);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const float d = (elem<DT, VEC>(xr, i) - mean) - c;
                    o[i] = __builtin_fmaf(d * s, elem<DT, VEC>(wr, i), elem<DT, VEC>(br, i));
                }
            }
            store_raw<DT, VEC, false>(a.y, off + col, make_raw<DT, VEC>(o));
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
