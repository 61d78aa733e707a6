// Kernel instances of the fused dual head RMSNorm + RoPE (head-vector
// shapes: one row per lane group of at most one wavefront).
#include "fnorm_kernels.hpp"
#include "fnorm_table.hpp"

namespace fnorm {
namespace {

template <int DT, int VEC, int VPT, int LPR, int BLOCK, bool MASKED, int NT, bool TRAD>
Variant make_rope() {
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
    return v;
}

template <int DT, int VEC, int VPT, int LPR, int BLOCK, bool MASKED, int NT>
void add_rope(std::vector<Variant>& t) {
    t.push_back(make_rope<DT, VEC, VPT, LPR, BLOCK, MASKED, NT, false>());
    t.push_back(make_rope<DT, VEC, VPT, LPR, BLOCK, MASKED, NT, true>());
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
    // (preference order measured on MI355X for head_dim 128 bf16, at 4096
    // tokens and at one decode token: 256-thread workgroups with
    // non-temporal loads and stores first; the cache policy changes the
    // full-size time by under 5%)
    add_rope<DT, V, 1, 8, 256, false, NT_BOTH>(t);
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
