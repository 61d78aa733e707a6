// Dual q/k head RMSNorm fused with the rotary position embedding, for
// gfx950: the kernel `dual_rope_rows` and its argument block.  It shares the
// norm's device helpers and argument layout with fnorm_kernels.hpp.
#pragma once

#include "fnorm_kernels.hpp"

namespace fnorm {

// DPP rotation by 8 within a 16-lane row, and ds_swizzle's bitmask mode
// for lane ^ 4 (and 0x1f, xor 0x04).
constexpr int DPP_ROW_ROR8 = 0x128;   // lane l <- lane l ^ 8 (rotate by 8 of 16)
constexpr int SWIZZLE_XOR4 = 0x101F;

// Value of `v` held by the lane at distance D within the row group (the
// split-half RoPE partner), D a compile-time distance: DPP for D = 1, 2, 8
// (inside a 16-lane row), ds_swizzle for D = 4 and 16, and ds_bpermute from
// `bperm_addr` (source lane * 4) for D = 0, meaning any other distance.  At
// D = 4 one swizzle replaces two row shifts and a select (three VALU
// instructions per element of a head_dim 64 row).
template <int D>
__device__ __forceinline__ float lane_partner(float v, int bperm_addr) {
    if constexpr (D == 1) {
        return dpp<DPP_QUAD_1032>(v);
    } else if constexpr (D == 2) {
        return dpp<DPP_QUAD_2301>(v);
    } else if constexpr (D == 4) {
        return __builtin_bit_cast(
            float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), SWIZZLE_XOR4));
    } else if constexpr (D == 8) {
        return dpp<DPP_ROW_ROR8>(v);
    } else if constexpr (D == 16) {
        return __builtin_bit_cast(
            float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), SWIZZLE_XOR16));
    } else {
        static_assert(D == 0, "partner distance");
        return __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(bperm_addr, __builtin_bit_cast(int, v)));
    }
}

// Calls f(std::integral_constant<int, D>) with D the compile-time form of
// the runtime partner distance d (0 for distances without a DPP/swizzle
// pattern), so that the choice is one uniform branch per row, not one per
// element.
template <class F>
__device__ __forceinline__ void with_partner_distance(int d, F&& f) {
    switch (d) {
        case 1: f(std::integral_constant<int, 1>{}); break;
        case 2: f(std::integral_constant<int, 2>{}); break;
        case 4: f(std::integral_constant<int, 4>{}); break;
        case 8: f(std::integral_constant<int, 8>{}); break;
        case 16: f(std::integral_constant<int, 16>{}); break;
        default: f(std::integral_constant<int, 0>{}); break;
    }
}

// ---------------------------------------------------------------------------
// Dual q/k head RMSNorm fused with the rotary position embedding (RoPE) of
// both outputs, one launch.  Norm definition as in fnorm_kernels.hpp; RoPE
// (Emily.Fast docs, `rope` and `rope_with_freqs`): pair i of a head vector
// at position p = offset + token rotates by theta_i = p * scale * inv_freq_i, with
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

    // Split-half rows of more than 128 features give a lane two or more
    // table entries per token.  In those kernels a lane's pairs are fixed
    // (L, L + 64, ...) and the inverse frequencies of the first two are
    // fetched once, before any row load; fetched inside the table phase, each
    // entry's load waited for the row's loads and for the entry before it.
    // Narrower rows (one entry per lane and token) keep the round-robin
    // spread, which holds no registers across the row loop.
    constexpr bool kHoist = !TRAD && !MASKED && VPT * LPR * VEC > 128;
    double inv0 = 0.0, inv1 = 0.0;
    if constexpr (kHoist) {
        inv0 = wave_lane < ihalf ? inv_turns(wave_lane) : 0.0;
        inv1 = wave_lane + 64 < ihalf ? inv_turns(wave_lane + 64) : 0.0;
    }

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
        // work item k * half + i, spread round-robin over the 64 lanes (or,
        // in the kernels above, pairs L, L + 64, ... of every leader).
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
            // theta / (2 pi) in fp64, reduced to a fraction of a turn exactly
            // (t - rint(t)); the hardware sine and cosine take their argument
            // in turns (v_sin_f32 / v_cos_f32)
            auto put = [&](int i, double inv) {
                const double t = pg * inv;
                const float f = static_cast<float>(t - __builtin_rint(t));
                wtab[g * ihalf + i] =
                    make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
            };
            if constexpr (kHoist) {
                if (wave_lane < ihalf) put(wave_lane, inv0);
                if (wave_lane + 64 < ihalf) put(wave_lane + 64, inv1);
                for (int i = wave_lane + 128; i < ihalf; i += 64) put(i, inv_turns(i));
            } else {
                for (int i = (wave_lane - (k * ihalf) % 64 + 64) % 64; i < ihalf; i += 64)
                    put(i, inv_turns(i));
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
                        q[i] = lane_partner<D>(o[0][i], src);
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
                // With two packs per lane the host's shape rule leaves only
                // full rotation (dv = 1), and with four only dv = 1 or 2, so
                // those kernels carry compile-time pairings and no code (or
                // registers) for the general case.
                if (VPT == 2 || 2 * dv == VPT) {
                    // every feature rotates: the pairing is known at compile
                    // time; pack v < VPT/2 pairs with pack v + VPT/2 and both
                    // rotate with the same table entries
                    static_for<VPT / 2>([&](auto vi) {
                        constexpr int v = decltype(vi)::value;
                        constexpr int vp = v + VPT / 2;
#pragma unroll
                        for (int i = 0; i < VEC; ++i) {
                            const float2 t = tab[(v * LPR + lane) * VEC + i];
                            out[v][i] = o[v][i] * t.x - o[vp][i] * t.y;
                            out[vp][i] = o[vp][i] * t.x + o[v][i] * t.y;
                        }
                    });
                } else if constexpr (VPT == 4) {
                    // four packs: the shape rule leaves dv = 2 (above) or
                    // dv = 1, where packs 0 and 1 rotate as a pair and packs
                    // 2 and 3 pass through
#pragma unroll
                    for (int i = 0; i < VEC; ++i) {
                        const float2 t = tab[lane * VEC + i];
                        out[0][i] = o[0][i] * t.x - o[1][i] * t.y;
                        out[1][i] = o[1][i] * t.x + o[0][i] * t.y;
                    }
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
