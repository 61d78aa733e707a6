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
//              (`dual_rope_rows`, at the end of this file).
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

namespace fnorm {

// ---------------------------------------------------------------------------
// Dual q/k head RMSNorm fused with the rotary position embedding (RoPE) of
// both outputs, one launch.  Norm definition as above; RoPE (Emily.Fast
// docs, `rope` and `rope_with_freqs`): pair i of a head vector at position
// p = offset + token rotates by theta_i = p * scale * inv_freq_i, with
// inv_freq_i = base^(-2i/dims) or a given table; pairs are (i, i + dims/2)
// (split-half) or (2i, 2i + 1) (TRAD, interleaved); features past `dims`
// pass through.  The result is RoPE(RMSNorm(x)) rounded once.
//
// Rows are head vectors in [token][head] order, so the heads of one token
// are consecutive rows.  Each wavefront evaluates the (cos, sin) table once
// per token among its rows (the first slot of each token, found with one
// ballot) into its own LDS region, and every row of that token reads it;
// the table is private to the wavefront, and the inverse frequencies come
// in the kernel arguments, so the kernel has no workgroup barrier and no
// per-workgroup set-up beyond its weight loads.  The angle in turns,
// theta / (2 pi), is formed
// in fp64 and reduced exactly to its fractional part f in [-1/2, 1/2]; sin
// and cos of 2 pi f then come from the hardware v_sin_f32 / v_cos_f32 (which
// take turns), so large positions keep fp32-level accuracy at the cost of a
// few instructions.
// Split-half partners live in another lane (fetched with ds_bpermute, the
// pack layout puts pack p + dims/(2 VEC) in lane p + dims/(2 VEC) when a
// thread holds one pack) or in the same thread (when dims/(2 VEC) is a
// multiple of LPR); interleaved partners sit in the same 16-byte pack (in the
// neighbouring lane for scalar packs).  The host only launches shapes for
// which one of these holds.
struct RopeArgs {
    NormArgs n;          // x = q, w = qw, y = qy, x2 = k, w2 = kw, y2 = ky; xs / ys /
                         // x2s / y2s are token strides (heads taken from below)
    int64_t q_heads;     // >= 1 (1 when there are no query rows)
    int64_t k_heads;     // >= 1 (1 when there are no key rows)
    int64_t dims;        // rotated features, even, <= width
    int64_t offset;      // position of token 0
    float base;
    float scale;
    const float* freqs;  // dims/2 inverse frequencies, or null
    FastDiv qdiv, kdiv;  // division by q_heads / k_heads (rows < 2^31)
    uint32_t q_blocks;   // workgroups [0, q_blocks) serve the queries, the rest the keys
    // Inverse frequencies in turns per position, base^(-2i/dims) / (2 pi),
    // computed by the host in fp64 (unused with freqs): pair i's is
    // invf[i % kRopeTable] * invf_step[i / kRopeTable], where invf_step[j] =
    // base^(-2 j kRopeTable / dims), so dims/2 may reach kRopeTable *
    // kRopeSteps.  Kernel arguments, so a workgroup starts without a
    // prologue: its lanes read the entries they need straight from here.
    static constexpr int kRopeTable = 256;
    static constexpr int kRopeSteps = 8;
    double invf[kRopeTable];
    double invf_step[kRopeSteps];
};

template <int DT, int VEC, int VPT, int LPR, int BLOCK, bool MASKED, int NT, bool TRAD>
__global__ __launch_bounds__(BLOCK) void dual_rope_rows(RopeArgs ra) {
    using R = typename Raw<DT, VEC>::type;
    static_assert(LPR <= 64 && BLOCK % 64 == 0 && BLOCK % LPR == 0, "launch shape");
    constexpr int RPB = BLOCK / LPR;
    constexpr bool NT_LD = (NT & NT_LOAD) != 0;
    constexpr bool NT_ST = (NT & NT_STORE) != 0;
    extern __shared__ double rope_smem[];   // (cos, sin)[RPB][half]

    const NormArgs& a = ra.n;
    const int tid = threadIdx.x;
    const int group = tid / LPR;
    const int lane = tid % LPR;
    const int wave_lane = tid & 63;
    const int64_t width = a.width;
    const float inv_width = a.inv_width;
    const int64_t half = ra.dims / 2;

    // The grid is split in two segments: workgroups [0, q_blocks) serve the
    // query rows, the others the key rows.  A workgroup's tensor is then a
    // uniform choice, so its pointers, strides, head count and weight are
    // scalars, not per-lane selects, and rows are counted within the tensor.
    const bool second = blockIdx.x >= ra.q_blocks;
    const unsigned seg_block = second ? blockIdx.x - ra.q_blocks : blockIdx.x;
    const unsigned seg_grid = second ? gridDim.x - ra.q_blocks : ra.q_blocks;
    const int64_t seg_rows = second ? a.rows - a.rows1 : a.rows1;
    const int64_t last = seg_rows - 1;
    const void* const xp = second ? a.x2 : a.x;
    void* const yp = second ? a.y2 : a.y;
    const void* const wp = second ? a.w2 : a.w;
    const int64_t xs = second ? a.x2s : a.xs;
    const int64_t ys = second ? a.y2s : a.ys;
    const int64_t den = second ? ra.k_heads : ra.q_heads;
    const FastDiv hdiv = second ? ra.kdiv : ra.qdiv;
    float2* cs = reinterpret_cast<float2*>(rope_smem);

    // Inverse frequency of pair i in turns per position (inv_freq_i / (2 pi),
    // fp64): the caller's frequencies, else the host's table (relative error
    // ~1e-15 past its first kRopeTable pairs, which moves an angle by under
    // 1e-9 rad at a million positions).
    constexpr double kInvTwoPi = 0.15915494309189533577;
    auto inv_turns = [&](int i) -> double {
        if (ra.freqs) return kInvTwoPi * static_cast<double>(ra.freqs[i]);
        if (i < RopeArgs::kRopeTable) return ra.invf[i];
        return ra.invf[i % RopeArgs::kRopeTable] * ra.invf_step[i / RopeArgs::kRopeTable];
    };

    auto col_of = [&](int v) { return int64_t(v * LPR + lane) * VEC; };
    auto in_row = [&](int v) { return !MASKED || col_of(v) < width; };
    constexpr int W = 64 / LPR;                 // rows per wavefront
    const int wave = tid >> 6;
    const int wslot = wave_lane / LPR;          // this row's slot in the wave
    float2* wtab = cs + int64_t(wave) * W * half;
    const int ihalf = static_cast<int>(half);

    R wv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        wv[v] = in_row(v) ? load_raw<DT, VEC, false>(wp, col_of(v)) : raw_zero<DT, VEC>();

    const bool small = a.rows <= 0x7fffffff;
    for (int64_t base = xcd_major(seg_block, seg_grid, (seg_rows + RPB - 1) / RPB) * RPB;
         base < seg_rows;
         base += int64_t(seg_grid) * RPB) {
        // This row's loads are issued first, so their latency overlaps the
        // angle-table phase below.
        const bool valid = base + group <= last;
        // row of this tensor; its token (the heads of a token are
        // consecutive rows) and head
        const int64_t num = valid ? base + group : last;
        const int64_t tok = small ? int64_t(hdiv.div(uint32_t(num))) : num / den;
        const int64_t head = num - tok * den;
        const int64_t xo = tok * xs + head * width;
        const int64_t yo = tok * ys + head * width;
        R xv[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            xv[v] = in_row(v) ? load_raw<DT, VEC, NT_LD>(xp, xo + col_of(v))
                              : raw_zero<DT, VEC>();

        // Its position, and the first slot of this wavefront holding the
        // same token (the slot that owns the table).
        const int64_t first = tok * den;
        const int64_t wave_row0 = base + int64_t(wave) * W;
        const int leader = first > wave_row0 ? int(first - wave_row0) : 0;
        const double pos = static_cast<double>(ra.offset + tok) * static_cast<double>(ra.scale);

        // Angle table of the wavefront's leader slots: leader k's pair i is
        // work item k * half + i, spread round-robin over the 64 lanes.
        uint64_t leaders = __ballot(lane == 0 && leader == wslot);
        int k = 0;
        while (leaders) {                                   // uniform over the wave
            const int bit = __builtin_ctzll(leaders);
            leaders &= leaders - 1;
            const int g = bit / LPR;
            const int64_t pb = __builtin_bit_cast(int64_t, pos);
            const int lo = __builtin_amdgcn_readlane(int(pb & 0xffffffff), bit);
            const int hi = __builtin_amdgcn_readlane(int(pb >> 32), bit);
            const double pg = __builtin_bit_cast(double, (int64_t(hi) << 32) | uint32_t(lo));
            for (int i = (wave_lane - (k * ihalf) % 64 + 64) % 64; i < ihalf; i += 64) {
                // theta / (2 pi) in fp64, reduced to a fraction of a turn
                // exactly (t - rint(t)); the hardware sine and cosine take
                // their argument in turns (v_sin_f32 / v_cos_f32)
                const double t = pg * inv_turns(i);
                const float f = static_cast<float>(t - __builtin_rint(t));
                wtab[g * ihalf + i] =
                    make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
            }
            ++k;
        }
        // The table is written and read by this wavefront only, and a
        // wavefront's LDS operations execute in order: wavefront-scope
        // fences order them for the compiler and emit no wait (a
        // workgroup-scope release also waits for the row's HBM load).
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float2* tab = wtab + leader * ihalf;
        // Split-half, one pack per thread: this lane's (cos, sin) entries are
        // read now, while the row's loads are still in flight.
        const int64_t dp = half / VEC;     // partner distance in packs
        float2 tpre[(!TRAD && VPT == 1) ? VEC : 1];
        if constexpr (!TRAD && VPT == 1) {
            const int64_t p = lane;
            const int64_t t0 = p < 2 * dp ? (p < dp ? p : p - dp) * VEC : 0;
#pragma unroll
            for (int i = 0; i < VEC; ++i) tpre[i] = tab[t0 + i];
        }

        float ss = 0.0f;
#pragma unroll
        for (int v = 0; v < VPT; ++v)
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                const float f = elem<DT, VEC>(xv[v], i);
                ss = __builtin_fmaf(f, f, ss);
            }
        ss = lane_group_sum<LPR>(ss);
        const float scale = __builtin_amdgcn_rsqf(ss * inv_width + a.eps);

        float o[VPT][VEC];
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const R wr = wv[v];
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                o[v][i] = (elem<DT, VEC>(xv[v], i) * scale) * elem<DT, VEC>(wr, i);
        }

        // rotation of the normalized values
        float out[VPT][VEC];
#pragma unroll
        for (int v = 0; v < VPT; ++v)
#pragma unroll
            for (int i = 0; i < VEC; ++i) out[v][i] = o[v][i];
        if constexpr (TRAD) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                if constexpr (VEC >= 2) {
#pragma unroll
                    for (int i = 0; i < VEC; i += 2) {
                        const int64_t c = col_of(v) + i;
                        if (c < ra.dims) {
                            const float2 t = tab[c / 2];
                            out[v][i] = o[v][i] * t.x - o[v][i + 1] * t.y;
                            out[v][i + 1] = o[v][i + 1] * t.x + o[v][i] * t.y;
                        }
                    }
                } else {
                    // scalar packs: the pair partner is the neighbouring lane
                    const int src = (wave_lane ^ 1) << 2;
                    const float p = __builtin_bit_cast(
                        float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, o[v][0])));
                    const int64_t c = col_of(v);
                    if (c < ra.dims) {
                        const float2 t = tab[c / 2];
                        out[v][0] = (c & 1) ? o[v][0] * t.x + p * t.y : o[v][0] * t.x - p * t.y;
                    }
                }
            }
        } else {
            if constexpr (VPT == 1) {
                // one pack per thread: the partner pack is in lane lane +- dp.
                // All partner values and table entries are fetched before
                // any is used, so the LDS operations overlap.
                const int64_t p = lane;
                const bool rot = p < 2 * dp;
                const int64_t partner = p < dp ? p + dp : (rot ? p - dp : p);
                const int src = (wave_lane - lane + int(partner)) << 2;
                // power-of-two distances: the partner is lane ^ dp (DPP or
                // swizzle, no LDS traffic); others go through ds_bpermute
                const int d = (dp & (dp - 1)) == 0 ? int(dp) : 0;
                float q[VEC];
                const float2* t = tpre;
                with_partner_distance(d, [&](auto dc) {
                    constexpr int D = decltype(dc)::value;
#pragma unroll
                    for (int i = 0; i < VEC; ++i)
                        q[i] = lane_partner<D>(o[0][i], wave_lane, src);
                });
                if (rot) {
#pragma unroll
                    for (int i = 0; i < VEC; ++i)
                        out[0][i] = p < dp ? o[0][i] * t[i].x - q[i] * t[i].y
                                           : o[0][i] * t[i].x + q[i] * t[i].y;
                }
            } else {
                // the partner pack is in this thread, dv = dp / LPR packs
                // away (the host launches VPT > 1 only when dp % LPR == 0).
                // Pack v is rotated when v < 2 dv and pairs with pack v + dv
                // (v < dv) or v - dv: conditions on v alone, uniform.
                const int dv = int(dp / LPR);
                if (2 * dv == VPT) {
                    // every feature rotates: the pairing is known at compile time
                    static_for<VPT>([&](auto vi) {
                        constexpr int v = decltype(vi)::value;
                        constexpr bool first = v < VPT / 2;
                        constexpr int vp = first ? v + VPT / 2 : v - VPT / 2;
                        constexpr int tv = first ? v : vp;
#pragma unroll
                        for (int i = 0; i < VEC; ++i) {
                            const float2 t = tab[(tv * LPR + lane) * VEC + i];
                            out[v][i] = first ? o[v][i] * t.x - o[vp][i] * t.y
                                              : o[v][i] * t.x + o[vp][i] * t.y;
                        }
                    });
                } else {
#pragma unroll
                    for (int v = 0; v < VPT; ++v) {
                        if (v < 2 * dv) {
                            const bool first = v < dv;
                            const int vp = first ? v + dv : v - dv;
                            const int tv = first ? v : vp;
#pragma unroll
                            for (int i = 0; i < VEC; ++i) {
                                float q = 0.0f;
#pragma unroll
                                for (int u = 0; u < VPT; ++u)
                                    if (u == vp) q = o[u][i];
                                const float2 t = tab[(tv * LPR + lane) * VEC + i];
                                out[v][i] = first ? o[v][i] * t.x - q * t.y
                                                  : o[v][i] * t.x + q * t.y;
                            }
                        }
                    }
                }
            }
        }

        if (valid) {
            static_for<VPT>([&](auto vi) {
                constexpr int v = decltype(vi)::value;
                if (in_row(v))
                    store_raw<DT, VEC, NT_ST>(yp, yo + col_of(v), make_raw<DT, VEC>(out[v]));
            });
        }
        // every lane has read the table before the next block-row rewrites it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
}

}  // namespace fnorm
