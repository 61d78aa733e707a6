// Kernel instances of the fused dual head RMSNorm + RoPE (head-vector
// shapes: one row per lane group of at most one wavefront).
#include "fnorm_kernels.hpp"
#include "fnorm_rope.hpp"
#include "fnorm_table.hpp"

namespace fnorm {
namespace {

template <int DT, int VEC, int VPT, int LPR, int BLOCK, bool MASKED, int NT, bool TRAD>
Variant make_rope(bool grid_first) {
    Variant v{};
    v.fn = reinterpret_cast<const void*>(&dual_rope_rows<DT, VEC, VPT, LPR, BLOCK, MASKED, NT, TRAD>);
    v.kind = TRAD ? K_ROPE_TRAD : K_ROPE_SPLIT;
    v.dt = DT;
    v.vec = VEC;
    v.vpt = VPT;
    v.lpr = LPR;
    v.block = BLOCK;
    v.masked = MASKED;
    v.nt = NT;
    v.wide = false;
    v.grid_cap = 0;
    v.grid_first = grid_first;
    return v;
}

// grid_first: the default launch is one workgroup per block of rows, the
// persistent grid the other variant.
template <int DT, int VEC, int VPT, int LPR, int BLOCK, bool MASKED, int NT>
void add_rope(std::vector<Variant>& t, bool grid_first = false) {
    t.push_back(make_rope<DT, VEC, VPT, LPR, BLOCK, MASKED, NT, false>(grid_first));
    t.push_back(make_rope<DT, VEC, VPT, LPR, BLOCK, MASKED, NT, true>(grid_first));
}

template <int DT, int V>
void add_rope_masked(std::vector<Variant>& t) {
    add_rope<DT, V, 1, 1, 256, true, NT_NONE>(t);
    add_rope<DT, V, 1, 2, 256, true, NT_NONE>(t);
    add_rope<DT, V, 1, 4, 256, true, NT_NONE>(t);
    add_rope<DT, V, 1, 8, 256, true, NT_NONE>(t);
    add_rope<DT, V, 1, 16, 256, true, NT_NONE>(t);
    add_rope<DT, V, 1, 32, 256, true, NT_NONE>(t);
    add_rope<DT, V, 1, 64, 256, true, NT_NONE>(t);
    add_rope<DT, V, 2, 64, 256, true, NT_NONE>(t);
    add_rope<DT, V, 4, 64, 256, true, NT_NONE>(t);
    add_rope<DT, V, 8, 64, 256, true, NT_NONE>(t);
}

template <int DT>
void register_rope_dtype(std::vector<Variant>& t) {
    constexpr int V = 16 / Elem<DT>::bytes;
    // exact head-vector shapes (bf16 head_dim 64/128/256/512, f32 32/64/128/256)
    // (preference order measured on MI355X, cold buffers, 32 query + 8 key
    // heads: 256-thread workgroups with non-temporal loads and stores; the
    // cache policy changes the full-size time by under 5%).  Rows of 16 and
    // 32 packs hold 2 packs per lane, so a split-half partner is in the same
    // thread, on a plain grid: at head_dim 128 (bf16) 19.6 against 19.9 us
    // for one pack per lane on a persistent grid at 4096 tokens, 58.7
    // against 62.6 at 16384, 110.8 against 124.2 at 32768.  With 2-byte
    // elements, rows of 32 and 64 packs take 4 packs per lane, so that a
    // wavefront holds 8 and 4 rows and builds fewer angle tables per row:
    // bf16 head_dim 256 at 16384 tokens 126.8 us against 151.4 with 2 packs
    // per lane and 186.0 with one; head_dim 512 at 4096 tokens 94.2 against
    // 110.7 with one.  fp32 head_dim 128 (32 packs of 4) is 3% faster with 2
    // packs per lane, and 4 packs in 4 lanes at bf16 head_dim 128 were
    // slower (22.6 us).  Rows of 8 packs keep one pack per lane on a
    // persistent grid (34.7 against 37.2 us at 16384 tokens).
    // With the split-half pairings of two- and four-pack rows fixed at
    // compile time (69-80 and 127 VGPRs), 4 packs in 8 lanes stays the
    // fastest for rows of 32 two-byte packs: bf16 head_dim 256 29.8 against
    // 30.4 us for 2 packs in 16 lanes at 4096 tokens, 105.6 against 108.4 at
    // 16384 (the plain dual: 30.2 and 113.0); head_dim 512 (4 in 16) 62.5
    // against 63.8 for 2 in 32 at 4096 tokens, 226.3 against 239.9 at 16384.
    add_rope<DT, V, 1, 8, 256, false, NT_BOTH>(t);
    add_rope<DT, V, 2, 8, 256, false, NT_BOTH>(t, true);
    if constexpr (Elem<DT>::bytes == 2) {
        add_rope<DT, V, 4, 8, 256, false, NT_BOTH>(t, true);
        add_rope<DT, V, 4, 16, 256, false, NT_BOTH>(t, true);
    }
    add_rope<DT, V, 2, 16, 256, false, NT_BOTH>(t, true);
    add_rope<DT, V, 1, 16, 256, false, NT_BOTH>(t);
    add_rope<DT, V, 1, 16, 512, false, NT_BOTH>(t);
    add_rope<DT, V, 1, 16, 1024, false, NT_BOTH>(t);
    add_rope<DT, V, 1, 32, 256, false, NT_BOTH>(t);
    add_rope<DT, V, 1, 64, 256, false, NT_BOTH>(t);
    add_rope<DT, V, 1, 16, 256, false, NT_NONE>(t);
    add_rope_masked<DT, V>(t);
    add_rope_masked<DT, 1>(t);
}

}  // namespace

void register_rope(std::vector<Variant>& table) {
    register_rope_dtype<DT_F32>(table);
    register_rope_dtype<DT_BF16>(table);
    register_rope_dtype<DT_F16>(table);
}

}  // namespace fnorm
