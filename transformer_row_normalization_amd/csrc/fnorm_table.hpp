// The dispatch table: one entry per compiled kernel instance.
//
// An entry records the launch shape of a `norm_rows` / `norm_rows_wide`
// instance (element type, pack width VEC, packs per thread VPT, threads per
// row LPR, threads per block) and which operation kind it serves.  The host
// side (fnorm_api.hip) turns (op, dtype, width, alignment) into an ordered
// list of entries able to run it; the first is the default.
#pragma once

#include <stdint.h>

#include <vector>

namespace fnorm {

enum Kind : int {
    K_RMS = 0, K_LAYER = 1, K_LAYER_NOBIAS = 2, K_DUAL = 3, K_COPY = 4,
    K_ROPE_SPLIT = 5, K_ROPE_TRAD = 6,  // dual head RMSNorm + RoPE (split-half / interleaved)
    K_RMS_GATED = 7                     // RMSNorm times SiLU(gate)
};

struct Variant {
    const void* fn;     // host stub of the __global__ function
    int kind;           // Kind
    int dt;             // DT_F32 / DT_BF16
    int vec;            // elements per access
    int vpt;            // packs per thread (resident kernels)
    int lpr;            // threads per row
    int block;          // threads per workgroup
    bool masked;        // handles width < lpr*vpt*vec (per-pack predicate)
    int nt;             // NT_* mask: non-temporal loads of x / stores of y
    bool wide;          // non-resident multi-pass kernel
    int grid_cap;       // persistent grid: workgroups per CU (0 = as many as fit)
    bool grid_first;    // default launch is one workgroup per block-row, not persistent
    int grid_resident;  // plain grid: at most this many workgroups resident per CU (0 = as
                        // many as fit), held there by a reservation of dynamic LDS
    int64_t capacity() const { return wide ? INT64_MAX : int64_t(lpr) * vpt * vec; }
    int rows_per_block() const { return wide ? 1 : block / lpr; }
};

// Defined in fnorm_inst_f32.hip / fnorm_inst_bf16.hip: append every
// instance of that element type, in preference order.
void register_f32(std::vector<Variant>& table);
void register_bf16(std::vector<Variant>& table);
void register_f16(std::vector<Variant>& table);
// Defined in fnorm_inst_rope.hip: the fused dual norm + RoPE instances.
void register_rope(std::vector<Variant>& table);

}  // namespace fnorm
