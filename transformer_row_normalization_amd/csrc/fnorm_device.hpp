// Device-side building blocks of the row-normalization kernels (gfx950).
//
//  * Raw element packs: 16-byte vectors (4 x fp32 or 8 x bf16) for the
//    coalesced path, single elements for the scalar path.  Rows stay in
//    registers as raw bits and are widened to fp32 at each use.
//  * bf16 / fp16 <-> fp32: bf16 widens by a shift (it is the high half of a
//    binary32), fp16 by v_cvt_f32_f16; narrowing is round-to-nearest-even
//    through gfx950's packed converts.
//  * Cross-lane sums with a fixed butterfly: after each step every lane of
//    the group holds the same bits (a + b computed in both lanes of a pair
//    is the same IEEE result), so row scalars are identical in every lane
//    and the reduction order depends only on the launch shape.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace fnorm {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
// OP_RMS_GATED: RMSNorm whose output is multiplied by SiLU(gate), the gate
// a second tensor of x's shape (the output norm's gate epilogue).
enum : int { OP_RMS = 0, OP_LAYER = 1, OP_RMS_GATED = 2 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- packs
template <int DT, int VEC> struct Raw;
template <> struct Raw<DT_F32, 4> { using type = u32x4; };
template <> struct Raw<DT_BF16, 8> { using type = u32x4; };
template <> struct Raw<DT_BF16, 4> { using type = u32x2; };
template <> struct Raw<DT_F32, 1> { using type = uint32_t; };
template <> struct Raw<DT_BF16, 1> { using type = uint16_t; };
template <> struct Raw<DT_F16, 8> { using type = u32x4; };
template <> struct Raw<DT_F16, 4> { using type = u32x2; };
template <> struct Raw<DT_F16, 1> { using type = uint16_t; };

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_F16> { static constexpr int bytes = 2; };

template <int DT, int VEC>
__device__ __forceinline__ typename Raw<DT, VEC>::type raw_zero() {
    return typename Raw<DT, VEC>::type(0);
}

// Cache policy of the row accesses: bit 0 = non-temporal (streaming) loads
// of x, bit 1 = non-temporal stores of y.
enum : int { NT_NONE = 0, NT_LOAD = 1, NT_STORE = 2, NT_BOTH = 3 };

// Load the pack that starts at element `idx` of `base`.  NT selects the
// non-temporal (streaming) cache policy.
template <int DT, int VEC, bool NT>
__device__ __forceinline__ typename Raw<DT, VEC>::type load_raw(const void* base, int64_t idx) {
    using R = typename Raw<DT, VEC>::type;
    const R* p = reinterpret_cast<const R*>(static_cast<const char*>(base) +
                                            idx * Elem<DT>::bytes);
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// Load the pack `off` bytes past `row`.  The 32-bit offset lets the compiler
// address each pack as one 64-bit row base plus a 32-bit lane offset (a
// scalar base when the row is uniform over the workgroup), so a lane keeps
// one register per pack offset instead of a 64-bit address per pack.
template <int DT, int VEC, bool NT>
__device__ __forceinline__ typename Raw<DT, VEC>::type load_at(const char* row, uint32_t off) {
    using R = typename Raw<DT, VEC>::type;
    const R* p = reinterpret_cast<const R*>(row + off);
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// SiLU(g) = g * sigmoid(g) in fp32, in a form that cannot overflow:
// e = exp(-|g|) lies in (0, 1], sigmoid(|g|) = 1 / (1 + e), and
// sigmoid(-|g|) = e / (1 + e).  e comes from the hardware base-2
// exponential (v_exp_f32) of -|g| log2(e); the product |g| log2(e) is
// carried as p + lo (lo from an fma remainder and the low part of log2(e)),
// so its rounding error does not grow with |g|, and exp2(-lo) is applied to
// first order (|lo| < 2^-17).  With the hardware reciprocal the result is
// within a few fp32 ulp; gates below about -87 give values under fp32's
// normal range.  (An expf and an IEEE division here made the gated kernel
// ALU-bound.)
__device__ __forceinline__ float silu(float g) {
    constexpr float kLog2e = 1.44269502163f;      // log2(e) rounded to fp32
    constexpr float kLog2eLo = 1.92596303e-08f;   // log2(e) - kLog2e
    constexpr float kLn2 = 0.693147182f;
    const float a = __builtin_fabsf(g);
    const float p = a * kLog2e;
    const float lo = __builtin_fmaf(a, kLog2e, -p) + a * kLog2eLo;
    const float e = __builtin_amdgcn_exp2f(-p) * __builtin_fmaf(-lo, kLn2, 1.0f);
    const float r = __builtin_amdgcn_rcpf(1.0f + e);
    return g * (g >= 0.0f ? r : e * r);
}

// Work order of workgroup b in a grid of g workgroups over `units` units of
// work (block-rows).  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup b runs on XCD b % 8, each XCD with its own L2 and address
// translation).  In a persistent grid (g < units: each workgroup loops over
// several units) numbering the workgroups XCD by XCD gives each XCD one
// contiguous share of every window of g units instead of every 8th unit;
// measured on the bench step: 1.5% faster, all three kernels.  A one-shot
// grid keeps the hardware order: there the same numbering sends the units
// in flight to 8 distant regions (1.5-4.5% slower for the norms, 7% for a
// copy).  A permutation of [0, g) in every case.
// Division of a 32-bit unsigned n by an invariant divisor d >= 1 with a
// multiply-high, two shifts and two adds (Granlund and Montgomery, "Division
// by invariant integers using multiplication", 1994, section 4): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, the quotient is
// (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0), t = mulhi(m, n), exact for
// every 32-bit n.  The host builds it with make_fast_div.
struct FastDiv {
    uint32_t m;
    uint32_t s1, s2;
    __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
        const uint32_t t = uint32_t((uint64_t(m) * n) >> 32);
        return (t + ((n - t) >> s1)) >> s2;
    }
};

inline FastDiv make_fast_div(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = (uint64_t(1) << 32) * ((uint64_t(1) << l) - d) / d + 1;
    return FastDiv{uint32_t(m), l < 1 ? l : 1u, l > 1 ? l - 1 : 0u};
}

constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_major(unsigned b, unsigned g, int64_t units) {
    return (g % kXcds == 0 && int64_t(g) < units) ? int64_t(b % kXcds) * (g / kXcds) + b / kXcds
                                                 : int64_t(b);
}

// f(0), f(1), ..., f(N-1) with compile-time indices and no loop in the IR.
// Used for the row stores: a `#pragma unroll` loop of one trip is still a
// loop when LICM runs, and its store promotion re-creates the store without
// the !nontemporal metadata.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int DT, int VEC, bool NT>
__device__ __forceinline__ void store_raw(void* base, int64_t idx, typename Raw<DT, VEC>::type v) {
    using R = typename Raw<DT, VEC>::type;
    R* p = reinterpret_cast<R*>(static_cast<char*>(base) + idx * Elem<DT>::bytes);
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Store counterpart of load_at.
template <int DT, int VEC, bool NT>
__device__ __forceinline__ void store_at(char* row, uint32_t off, typename Raw<DT, VEC>::type v) {
    using R = typename Raw<DT, VEC>::type;
    R* p = reinterpret_cast<R*>(row + off);
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }
__device__ __forceinline__ float f16_val(uint32_t h16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h16)));
}

// A 16-bit element (bf16 or fp16) widened to fp32, exactly.
template <int DT>
__device__ __forceinline__ float widen16(uint32_t bits16) {
    if constexpr (DT == DT_BF16) return __builtin_bit_cast(float, bits16 << 16);
    else return f16_val(bits16 & 0xFFFFu);
}

// Element i of a pack, widened to fp32 (exact).
template <int DT, int VEC>
__device__ __forceinline__ float elem(const typename Raw<DT, VEC>::type& r, int i) {
    if constexpr (VEC == 1) {
        if constexpr (DT == DT_F32) return __builtin_bit_cast(float, r);
        else return widen16<DT>(uint32_t(r));
    } else if constexpr (DT == DT_F32) {
        // Copy the component out first: bit_cast of a vector-component
        // lvalue reads component 0 whatever the index.
        const uint32_t u = r[i];
        return __builtin_bit_cast(float, u);
    } else {
        const uint32_t u = r[i >> 1];
        if constexpr (DT == DT_BF16) return (i & 1) ? bf16_hi(u) : bf16_lo(u);
        else return f16_val((i & 1) ? (u >> 16) : (u & 0xFFFFu));
    }
}

// Two fp32 values rounded (nearest, ties to even) to the 16-bit type,
// packed lo | hi << 16 (gfx950 packed converts).
template <int DT>
__device__ __forceinline__ uint32_t pack16x2(float lo, float hi) {
    if constexpr (DT == DT_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return pack16x2<DT_BF16>(lo, hi);
}

// VEC fp32 values stored into a pack of the element type.
template <int DT, int VEC>
__device__ __forceinline__ typename Raw<DT, VEC>::type make_raw(const float (&f)[VEC]) {
    if constexpr (VEC == 1) {
        if constexpr (DT == DT_F32) return __builtin_bit_cast(uint32_t, f[0]);
        else return uint16_t(pack16x2<DT>(f[0], 0.0f) & 0xFFFFu);
    } else if constexpr (DT == DT_F32) {
        return u32x4{__builtin_bit_cast(uint32_t, f[0]), __builtin_bit_cast(uint32_t, f[1]),
                     __builtin_bit_cast(uint32_t, f[2]), __builtin_bit_cast(uint32_t, f[3])};
    } else if constexpr (VEC == 4) {
        return u32x2{pack16x2<DT>(f[0], f[1]), pack16x2<DT>(f[2], f[3])};
    } else {
        return u32x4{pack16x2<DT>(f[0], f[1]), pack16x2<DT>(f[2], f[3]),
                     pack16x2<DT>(f[4], f[5]), pack16x2<DT>(f[6], f[7])};
    }
}

// Register-pressure control: an empty asm that "modifies" the packs makes
// their widened fp32 values non-invariant, so the compiler re-widens them at
// each use (one VALU op per element) instead of hoisting VPT*VEC fp32 copies
// out of the row loop and holding them in VGPRs for the whole kernel.
template <int N, typename R>
__device__ __forceinline__ void keep_packed(R (&p)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(p[i]));
}

// ---------------------------------------------------------------- reductions
// v moved across lanes by a DPP control.  A lane whose source lies outside
// its row reads 0 (bound_ctrl), so no register has to be cleared first.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// DPP controls (GFX9 encoding): quad permutes, and the in-row mirrors.
constexpr int DPP_QUAD_1032 = 0xB1;      // lane ^ 1
constexpr int DPP_QUAD_2301 = 0x4E;      // lane ^ 2
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <- lane 7 - i within 8
constexpr int DPP_ROW_MIRROR = 0x140;       // lane i <- lane 15 - i within 16
constexpr int SWIZZLE_XOR16 = 0x401F;       // bitmask mode: and 0x1f, xor 0x10

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64).
// Each step adds a value that is already uniform over the partner half, so
// the result is bitwise identical in every lane of the group.
template <int G>
__device__ __forceinline__ float lane_group_sum(float v) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "group size");
    if constexpr (G >= 2) v += dpp<DPP_QUAD_1032>(v);
    if constexpr (G >= 4) v += dpp<DPP_QUAD_2301>(v);
    if constexpr (G >= 8) v += dpp<DPP_ROW_HALF_MIRROR>(v);
    if constexpr (G >= 16) v += dpp<DPP_ROW_MIRROR>(v);
    if constexpr (G >= 32)
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                   SWIZZLE_XOR16));
    if constexpr (G >= 64) {
        const int lane = __lane_id();
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2,
                                                                    __builtin_bit_cast(int, v)));
    }
    return v;
}

// Sum over a group of LPR threads that owns one row.  LPR <= 64: lanes of one
// wavefront.  LPR > 64: LPR/64 whole wavefronts; each wave reduces, writes
// one partial to LDS, one barrier, then every thread adds the partials of
// its row in wave order.  `lds` has RPB * (LPR/64) slots for this call site;
// the caller keeps call sites apart so that a slot is never rewritten while
// a slower wave may still read it.
template <int LPR>
__device__ __forceinline__ float row_sum(float v, float* lds, int group, int lane_in_row) {
    if constexpr (LPR <= 64) {
        return lane_group_sum<LPR>(v);
    } else {
        constexpr int WPR = LPR / 64;
        v = lane_group_sum<64>(v);
        const int wave = lane_in_row >> 6;
        if ((lane_in_row & 63) == 0) lds[group * WPR + wave] = v;
        __syncthreads();
        float s = lds[group * WPR];
#pragma unroll
        for (int i = 1; i < WPR; ++i) s += lds[group * WPR + i];
        return s;
    }
}

// Two sums over the same row group at once (one barrier for both): `a` in
// slots lds_a, `b` in slots lds_b, each laid out like row_sum's.
template <int LPR>
__device__ __forceinline__ void row_sum2(float& a, float& b, float* lds_a, float* lds_b, int group,
                                         int lane_in_row) {
    if constexpr (LPR <= 64) {
        a = lane_group_sum<LPR>(a);
        b = lane_group_sum<LPR>(b);
    } else {
        constexpr int WPR = LPR / 64;
        a = lane_group_sum<64>(a);
        b = lane_group_sum<64>(b);
        const int wave = lane_in_row >> 6;
        if ((lane_in_row & 63) == 0) {
            lds_a[group * WPR + wave] = a;
            lds_b[group * WPR + wave] = b;
        }
        __syncthreads();
        float sa = lds_a[group * WPR], sb = lds_b[group * WPR];
#pragma unroll
        for (int i = 1; i < WPR; ++i) {
            sa += lds_a[group * WPR + i];
            sb += lds_b[group * WPR + i];
        }
        a = sa;
        b = sb;
    }
}

}  // namespace fnorm
