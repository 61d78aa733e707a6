// Instantiation list shared by the two per-dtype translation units.
//
// Shapes are (VPT, LPR, BLOCK) for the 16-byte pack width of the element
// type (fp32x4 / bf16x8).  "exact" shapes have capacity lpr*vpt*vec equal to
// the width they serve and carry no column predicate; "masked" shapes serve
// every smaller width too.  Within one capacity the first registered shape
// is the default, so the order below is the preference order.
#pragma once

#include "fnorm_kernels.hpp"
#include "fnorm_table.hpp"

namespace fnorm {

template <int KIND>
constexpr int op_of() {
    return (KIND == K_LAYER || KIND == K_LAYER_NOBIAS) ? OP_LAYER
           : KIND == K_RMS_GATED                      ? OP_RMS_GATED
                                                      : OP_RMS;
}

// Grid-cap argument of an exact shape whose default launch is a plain grid
// (one workgroup per block-row); its persistent form is the other variant.
constexpr int GRID_FIRST = -1;

template <int KIND, int DT, int VEC, int VPT, int LPR, int BLOCK, bool MASKED, int NT>
inline Variant make_variant(int cap, int resident) {
    constexpr int OP = op_of<KIND>();
    constexpr bool BIAS = KIND == K_LAYER;
    constexpr bool DUAL = KIND == K_DUAL;
    Variant v{};
    v.fn = reinterpret_cast<const void*>(
        &norm_rows<OP, DT, VEC, VPT, LPR, BLOCK, MASKED, BIAS, DUAL, NT>);
    v.kind = KIND;
    v.dt = DT;
    v.vec = VEC;
    v.vpt = VPT;
    v.lpr = LPR;
    v.block = BLOCK;
    v.masked = MASKED;
    v.nt = NT;
    v.wide = false;
    v.grid_cap = cap > 0 ? cap : 0;
    v.grid_first = cap == GRID_FIRST;
    v.grid_resident = resident;
    return v;
}

// Sets of kinds one registration applies to (only those kernels are
// instantiated): a shape can then sit at a different place in the
// preference order of LayerNorm and of the RMSNorm family.
constexpr unsigned KM_LAYER_BIAS = 1u << K_LAYER;
constexpr unsigned KM_LAYER = KM_LAYER_BIAS | (1u << K_LAYER_NOBIAS);
constexpr unsigned KM_RMS_FAMILY = (1u << K_RMS) | (1u << K_DUAL) | (1u << K_RMS_GATED);
constexpr unsigned KM_ALL = KM_LAYER | KM_RMS_FAMILY;

template <int DT, int VEC, int VPT, int LPR, int BLOCK, bool MASKED, int NT, unsigned KINDS = KM_ALL>
inline void add_shape(std::vector<Variant>& t, int cap = 0, int resident = 0) {
    if constexpr ((KINDS >> K_RMS) & 1u)
        t.push_back(make_variant<K_RMS, DT, VEC, VPT, LPR, BLOCK, MASKED, NT>(cap, resident));
    if constexpr ((KINDS >> K_LAYER) & 1u)
        t.push_back(make_variant<K_LAYER, DT, VEC, VPT, LPR, BLOCK, MASKED, NT>(cap, resident));
    if constexpr ((KINDS >> K_LAYER_NOBIAS) & 1u)
        t.push_back(make_variant<K_LAYER_NOBIAS, DT, VEC, VPT, LPR, BLOCK, MASKED, NT>(cap, resident));
    if constexpr ((KINDS >> K_DUAL) & 1u)
        t.push_back(make_variant<K_DUAL, DT, VEC, VPT, LPR, BLOCK, MASKED, NT>(cap, resident));
    if constexpr ((KINDS >> K_RMS_GATED) & 1u)
        t.push_back(make_variant<K_RMS_GATED, DT, VEC, VPT, LPR, BLOCK, MASKED, NT>(cap, resident));
}

template <int KIND, int DT, int VEC, int BLOCK>
inline Variant make_wide() {
    constexpr int OP = op_of<KIND>();
    Variant v{};
    v.fn = reinterpret_cast<const void*>(&norm_rows_wide<OP, DT, VEC, BLOCK, KIND == K_LAYER>);
    v.kind = KIND;
    v.dt = DT;
    v.vec = VEC;
    v.vpt = 0;
    v.lpr = BLOCK;
    v.block = BLOCK;
    v.masked = true;
    v.nt = NT_NONE;
    v.wide = true;
    v.grid_cap = 0;
    v.grid_first = false;
    v.grid_resident = 0;
    return v;
}

template <int DT, int VEC>
inline void add_wide(std::vector<Variant>& t) {
    t.push_back(make_wide<K_RMS, DT, VEC, 1024>());
    t.push_back(make_wide<K_LAYER, DT, VEC, 1024>());
    t.push_back(make_wide<K_LAYER_NOBIAS, DT, VEC, 1024>());
    t.push_back(make_wide<K_RMS_GATED, DT, VEC, 1024>());
}

// Masked shapes for any width up to 8192 packs, used with pack width V
// (16-byte packs) and with V = 1 (scalar path for misaligned data or widths
// that are not a multiple of the pack).  The smallest capacity that holds
// the width serves it.  Rows of 16-byte packs with several packs per lane
// in 256-thread workgroups (the ragged hidden sizes 2560-12288) run 10-18%
// faster with non-temporal loads and stores on a plain grid than on a
// full-occupancy persistent grid (measured at bf16 2560-12288, fp16 3584 and
// 5120, fp32 2560-6144); 640 packs (bf16 5120) get a shape of their own, 6%
// faster for LayerNorm than the 1024-pack one, and 2049-3072 packs (bf16
// 18432, 24576) one of 512 threads, 10% faster for LayerNorm than the
// 1024-thread shape.  The 1024-thread shapes (one row per workgroup) stay
// persistent: a plain grid is 6-40% slower there.  LayerNorm with a bias at
// 4097-8192 packs runs 20% faster on 16 packs per lane in 512 threads than
// on 8 in 1024 (bf16 49152 and 65536, fp32 32768); without a bias, and for
// RMSNorm, the 1024-thread shape is as fast or faster.
//
// Plain grids keep few workgroups resident per CU, so that 64-96 KB of
// loads are in flight per CU: 3 for the shapes with 20-32 KB per workgroup,
// 4 for the 16 KB of one row of 4 packs per lane, 2 for the 48 KB of the
// 512-thread shape.  With as many as the registers allow they run 3-7%
// slower (LayerNorm at bf16 5120 and 12288, RMSNorm at 12288 and 18432), with
// fewer 5-30% slower.  The grids whose rows fit one wave with 2 or 4 packs
// per lane (8 and 16 KB per workgroup) run best unlimited.
template <int DT, int V>
inline void add_masked(std::vector<Variant>& t) {
    constexpr int WIDE_NT = V > 1 ? NT_BOTH : NT_NONE;
    constexpr int WIDE_CAP = V > 1 ? GRID_FIRST : 0;
    constexpr int R = V > 1 ? 1 : 0;   // resident limits for the 16-byte-pack grids
    add_shape<DT, V, 1, 1, 256, true, NT_NONE>(t);
    add_shape<DT, V, 1, 2, 256, true, NT_NONE>(t);
    add_shape<DT, V, 1, 4, 256, true, NT_NONE>(t);
    add_shape<DT, V, 1, 8, 256, true, NT_NONE>(t);
    // 9-16 packs (e.g. bf16 head_dim 96): non-temporal loads and stores,
    // 4-5% faster than ordinary ones (bf16 96 and 120)
    add_shape<DT, V, 1, 16, 256, true, (V > 1 ? NT_BOTH : NT_NONE)>(t);
    add_shape<DT, V, 1, 32, 256, true, NT_NONE>(t);
    // 33-64 packs: 2 packs per lane on a plain grid, 4-14% faster than one
    // pack per lane on a persistent grid (bf16 264-504, fp32 132-252).  The
    // same for 9-32 packs was 18-21% slower at bf16 120 (rows of 15 packs).
    if constexpr (V > 1) add_shape<DT, V, 2, 32, 256, true, NT_BOTH>(t, GRID_FIRST);
    add_shape<DT, V, 1, 64, 256, true, NT_NONE>(t);
    add_shape<DT, V, 2, 64, 256, true, WIDE_NT>(t, WIDE_CAP);
    add_shape<DT, V, 4, 64, 256, true, WIDE_NT>(t, WIDE_CAP);
    add_shape<DT, V, 8, 64, 256, true, WIDE_NT>(t, WIDE_CAP, 3 * R);
    if constexpr (V > 1) add_shape<DT, V, 5, 128, 256, true, WIDE_NT>(t, WIDE_CAP, 3);
    // LayerNorm with a bias at 641-896 packs: two rows of 7 packs per lane
    // per workgroup, 1-4% faster than one row of 4 (bf16 5632-7168, fp32
    // 3000-3072; bf16 7168: 91.2 against 94.8 us); without a bias, and for
    // RMSNorm, it gains nothing.
    if constexpr (V > 1) add_shape<DT, V, 7, 128, 256, true, WIDE_NT, KM_LAYER_BIAS>(t, WIDE_CAP, 3);
    add_shape<DT, V, 4, 256, 256, true, WIDE_NT>(t, WIDE_CAP, 4 * R);
    add_shape<DT, V, 8, 256, 256, true, WIDE_NT>(t, WIDE_CAP, 3 * R);
    if constexpr (V > 1) add_shape<DT, V, 6, 512, 512, true, WIDE_NT>(t, WIDE_CAP, 2);
    // one 1024-thread workgroup per CU: with 32-bit pack offsets the fp32
    // and fp16 RMSNorm kernels fit two, which took RMSNorm at fp32 16384
    // from 91.5 to 106.8 us
    add_shape<DT, V, 4, 1024, 1024, true, WIDE_NT>(t, V > 1 ? 1 : 0);
    if constexpr (V > 1) add_shape<DT, V, 16, 512, 512, true, WIDE_NT, KM_LAYER_BIAS>(t);
    add_shape<DT, V, 8, 1024, 1024, true, WIDE_NT>(t);
}

// EXACT(VPT, LPR, BLOCK, NT, CAP): an exact shape, its NT_* cache-policy
// mask, and its persistent-grid cap in workgroups per CU (0: as many as fit;
// GRID_FIRST: launch a plain grid by default).
#define FNORM_EXACT(VPT, LPR, BLOCK, NT, CAP) add_shape<DT, V, VPT, LPR, BLOCK, false, NT>(t, CAP);
// The same for one set of kinds only.
#define FNORM_EXACT_FOR(KINDS, VPT, LPR, BLOCK, NT, CAP) \
    add_shape<DT, V, VPT, LPR, BLOCK, false, NT, KINDS>(t, CAP);

// Preference order, measured on MI355X (cold HBM, 256 MiB inputs, bf16 and
// fp32): the first entry of each capacity is the default.  Rows of 128 packs
// and more win with a small persistent grid (2 workgroups per CU) and four
// to eight packs per lane, so that each wave keeps 4-8 KB of loads in
// flight: RMSNorm and LayerNorm agree on every shape there.  A grid cap of
// 3 or 4 is 10-15% slower than 2 at every width measured.  The RMSNorm
// default at 8192 (one 16 KB row per workgroup, ordinary stores) and the
// LayerNorm default at 4096 were chosen inside the three-kernel step, where
// the dirty lines one kernel leaves in the MALL are written back during the
// next.  Sub-wave rows (short head vectors) prefer a full-occupancy
// persistent grid, the 96-pack rows a plain grid.  Differences under about
// 3% between cache policies are within the run-to-run spread.
template <int DT>
inline void register_dtype(std::vector<Variant>& t) {
    constexpr int V = 16 / Elem<DT>::bytes;
    // Head-sized rows (8-64 packs) run on a plain grid: a persistent grid
    // caps the dual near 5.2 TB/s however many tokens there are, while the
    // plain grid reaches the copy kernel's rate from 8192 tokens on (bf16
    // head_dim 128, 32 query + 8 key heads: 32768 tokens 106 against 129 us,
    // 4096 tokens 17.8 against 18.2 us).
    // 8 packs (bf16 64 / f32 32): one 8-lane group per row (dual at head_dim
    // 64: 8-12% faster than the masked 8-lane shape with ordinary access)
    FNORM_EXACT(1, 8, 256, NT_BOTH, GRID_FIRST)
    FNORM_EXACT(1, 8, 256, NT_NONE, 0)
    // 16 packs (bf16 128 / f32 64): an 8-lane group per row, 2 packs per
    // lane (32 rows per workgroup)
    FNORM_EXACT(2, 8, 256, NT_BOTH, GRID_FIRST)
    FNORM_EXACT(1, 16, 256, NT_BOTH, 0)
    FNORM_EXACT(1, 16, 256, NT_LOAD, 0)
    FNORM_EXACT(1, 16, 256, NT_NONE, 0)
    // 24 packs (bf16 192 / f32 96): 3 packs in 8 lanes, 17-22% faster than
    // the masked 32-lane shape (bf16 192 RMSNorm 102.6 against 86.0 us per
    // 512 MiB, the copy kernel's rate; dual at head_dim 192 and 16384
    // tokens 97.3 against 81.5).  The same for 12 packs (3 in 4 lanes) was
    // 2-15% slower than the masked 16-lane shape.
    FNORM_EXACT(3, 8, 256, NT_BOTH, GRID_FIRST)
    // 32 packs (bf16 256 / f32 128): 2 packs in 16 lanes with non-temporal
    // loads and stores on a plain grid for RMSNorm, LayerNorm and the dual
    // (bf16 head_dim 256: the dual 30.2 -> 28.3 us at 4096 tokens, 112.9 ->
    // 104.5 at 16384; over 256 MiB LayerNorm 92.1 -> 84.3 us, RMSNorm 87.7 ->
    // 84.0; fp32 128 3-5%).  The gated form keeps one pack in 32 lanes
    // (121.6 against 126.9 us).  Non-temporal stores are 4-5% faster than
    // ordinary ones for the dual at these head sizes.
    FNORM_EXACT_FOR(KM_LAYER | (1u << K_RMS) | (1u << K_DUAL), 2, 16, 256, NT_BOTH, GRID_FIRST)
    FNORM_EXACT(1, 32, 256, NT_BOTH, GRID_FIRST)
    FNORM_EXACT(1, 32, 256, NT_LOAD, 0)
    FNORM_EXACT(2, 16, 256, NT_NONE, 0)
    FNORM_EXACT(1, 32, 256, NT_NONE, 0)
    FNORM_EXACT_FOR(1u << K_RMS_GATED, 2, 16, 256, NT_BOTH, GRID_FIRST)
    // 72 and 80 packs (bf16 576 and 640, fp32 288 and 320): 9 packs in 8
    // lanes and 5 in 16 on a plain grid, LayerNorm 7-16% faster than the
    // masked 64-lane shape the rows only partly fill (bf16 576: 102.9
    // against 91.6 us per 512 MiB), RMSNorm within 3%
    FNORM_EXACT(9, 8, 256, NT_BOTH, GRID_FIRST)
    FNORM_EXACT(5, 16, 256, NT_BOTH, GRID_FIRST)
    // 64 packs (bf16 512 / f32 256): a plain grid (dual at head_dim 512,
    // 16384 tokens: 218 against 264 us persistent)
    FNORM_EXACT(1, 64, 256, NT_LOAD, GRID_FIRST)
    FNORM_EXACT(1, 64, 256, NT_NONE, 0)
    // 96 packs (bf16 768)
    FNORM_EXACT(3, 32, 256, NT_BOTH, GRID_FIRST)
    FNORM_EXACT(3, 32, 256, NT_NONE, 0)
    // 128 packs (bf16 1024, f32 512)
    FNORM_EXACT(4, 32, 256, NT_BOTH, 2)
    FNORM_EXACT(2, 64, 256, NT_BOTH, 2)
    FNORM_EXACT(2, 64, 256, NT_NONE, 0)
    // 192 packs (f32 768, bf16 1536): non-temporal, 2 workgroups per CU,
    // 16-20% faster over 256 MiB than ordinary access at full occupancy
    FNORM_EXACT(3, 64, 256, NT_BOTH, 2)
    FNORM_EXACT(3, 64, 256, NT_NONE, 0)
    // 256 packs (f32 1024, bf16 2048)
    FNORM_EXACT(4, 64, 256, NT_BOTH, 2)
    FNORM_EXACT(2, 128, 256, NT_BOTH, 2)
    FNORM_EXACT(4, 64, 256, NT_NONE, 0)
    FNORM_EXACT(1, 256, 256, NT_LOAD, 2)
    // 512 packs (bf16 4096, f32 2048)
    FNORM_EXACT(4, 128, 256, NT_BOTH, 2)
    FNORM_EXACT(4, 128, 256, NT_NONE, 2)
    FNORM_EXACT(8, 64, 256, NT_BOTH, 0)
    FNORM_EXACT(2, 256, 256, NT_BOTH, 2)
    FNORM_EXACT(1, 512, 512, NT_LOAD, 2)
    FNORM_EXACT(1, 512, 1024, NT_LOAD, 2)
    // 1024 packs (bf16 8192, f32 4096): LayerNorm prefers non-temporal
    // stores (5-7% faster alone); RMSNorm, inside the three-kernel step,
    // ordinary ones (3% faster step), though non-temporal ones win alone.
    FNORM_EXACT_FOR(KM_LAYER, 4, 256, 256, NT_BOTH, 2)
    FNORM_EXACT(4, 256, 256, NT_LOAD, 2)
    FNORM_EXACT_FOR(KM_RMS_FAMILY, 4, 256, 256, NT_BOTH, 2)
    FNORM_EXACT(1, 1024, 1024, NT_LOAD, 2)
    FNORM_EXACT(1, 1024, 1024, NT_BOTH, 2)
    FNORM_EXACT(1, 1024, 1024, NT_NONE, 2)
    FNORM_EXACT(2, 512, 512, NT_LOAD, 2)
    FNORM_EXACT(8, 128, 256, NT_BOTH, 2)
    // 2048 packs (f32 8192, bf16 16384)
    FNORM_EXACT(8, 256, 256, NT_BOTH, 2)
    FNORM_EXACT(2, 1024, 1024, NT_BOTH, 2)
    FNORM_EXACT(4, 512, 512, NT_BOTH, 2)
    // LayerNorm with a bias at 2304 and 3072 packs (bf16 18432 and 24576):
    // 9 and 12 packs per lane on a plain grid, 3-6% faster than the masked
    // 512-thread shape (bf16 94.7 against 98.1 us, 90.6 against 96.1; fp32
    // 12288 90.8 against 93.6).  fp32 9216 was 4% slower with 9 packs.
    if constexpr (Elem<DT>::bytes == 2) FNORM_EXACT_FOR(KM_LAYER_BIAS, 9, 256, 256, NT_BOTH, GRID_FIRST)
    FNORM_EXACT_FOR(KM_LAYER_BIAS, 12, 256, 256, NT_BOTH, GRID_FIRST)
    add_masked<DT, V>(t);
    add_masked<DT, 1>(t);
    add_wide<DT, V>(t);
    add_wide<DT, 1>(t);
}

#undef FNORM_EXACT
#undef FNORM_EXACT_FOR

}  // namespace fnorm
