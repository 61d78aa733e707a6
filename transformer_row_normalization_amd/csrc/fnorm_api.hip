// C ABI of libfnorm: argument validation, kernel selection and launch.
//
// Validation runs first and makes no HIP call; only a valid request reaches
// the device-property queries and the launch.  Errors are reported as a
// status code plus a per-thread "operation: description" text, the
// convention of the error type in mlx-c-rust `compile/norm_fusion.rs`
// (operation name + description, structural checks before any work).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/fnorm.h"
#include "fnorm_composed.hpp"
#include "fnorm_kernels.hpp"
#include "fnorm_rope.hpp"
#include "fnorm_table.hpp"

namespace fnorm {

// Scratch of fnorm_rms_composed_noalloc: the fp32 intermediates of the
// composed chain, in device memory that belongs to the code object (each
// device holds its own copy from module load to process exit), so the call
// allocates nothing.  Host code never uses the name below as an address: the
// device address comes from hipGetSymbolAddress, once per device.
constexpr int64_t kNoAllocScratchBytes = int64_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kVersion = 201;  // 0.2.1: call-level describe, no-alloc composed RMSNorm

thread_local char g_err[512];

int fail(int status, const char* op, const char* fmt, ...) {
    int n = std::snprintf(g_err, sizeof g_err, "%s: ", op);
    if (n < 0 || n >= int(sizeof g_err)) n = 0;
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err + n, sizeof g_err - n, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return FNORM_OK;
}

// Device address of `scratch` on the current device, looked up on the first
// call there (with that device current) and kept per device.
int noalloc_scratch(const char* op, void** out) {
    constexpr int kMaxDevices = 64;
    static std::atomic<void*> addr[kMaxDevices];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(FNORM_ERR_LAUNCH, op, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(FNORM_ERR_UNSUPPORTED, op, "device %d beyond the %d this call serves", dev,
                    kMaxDevices);
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return fail(FNORM_ERR_LAUNCH, op, "hipGetSymbolAddress(scratch) failed: %s",
                            hipGetErrorString(e));
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return FNORM_OK;
}

struct Registry {
    std::vector<Variant> table;
    std::unique_ptr<std::atomic<int>[]> occupancy;  // blocks per CU, 0 = not yet queried
    std::unique_ptr<std::atomic<int>[]> grid_lds;   // resident-limit LDS, -1 = not yet set
};

const Registry& registry() {
    static const Registry r = [] {
        Registry reg;
        register_f32(reg.table);
        register_bf16(reg.table);
        register_f16(reg.table);
        register_rope(reg.table);
        reg.occupancy.reset(new std::atomic<int>[reg.table.size()]);
        reg.grid_lds.reset(new std::atomic<int>[reg.table.size()]);
        for (size_t i = 0; i < reg.table.size(); ++i) {
            reg.occupancy[i].store(0);
            reg.grid_lds[i].store(-1);
        }
        return reg;
    }();
    return r;
}

bool valid_dtype(int dtype) {
    return dtype == FNORM_F32 || dtype == FNORM_BF16 || dtype == FNORM_F16;
}
int elem_bytes(int dtype) { return dtype == FNORM_F32 ? 4 : 2; }
const char* dtype_name(int dtype) {
    return dtype == FNORM_F32 ? "f32" : dtype == FNORM_BF16 ? "bf16" : "f16";
}

// One runnable choice: a table entry plus the grid policy.
struct Choice {
    const Variant* v = nullptr;
    bool persistent = true;
};

constexpr int kMaxCandidates = 64;

const Variant* smallest_masked(int kind, int dt, int vec, int64_t width) {
    const Variant* best = nullptr;
    for (const Variant& v : registry().table) {
        if (v.kind != kind || v.dt != dt || v.vec != vec || !v.masked || v.wide) continue;
        if (v.capacity() < width) continue;
        if (!best || v.capacity() < best->capacity()) best = &v;
    }
    return best;
}

const Variant* find_wide(int kind, int dt, int vec) {
    for (const Variant& v : registry().table)
        if (v.kind == kind && v.dt == dt && v.vec == vec && v.wide) return &v;
    return nullptr;
}

// Kernels able to serve (kind, dtype, width, aligned), default first:
// exact-width resident shapes, then the smallest masked resident shape, then
// the scalar-access resident shape, then the multi-pass wide kernels.
int candidates(int kind, int dt, int64_t width, bool aligned, const Variant** out) {
    int n = 0;
    const int vec = 16 / elem_bytes(dt);
    const bool vec_ok = aligned && (width % vec == 0);
    if (vec_ok) {
        for (const Variant& v : registry().table)
            if (v.kind == kind && v.dt == dt && v.vec == vec && !v.masked && !v.wide &&
                v.capacity() == width && n < kMaxCandidates - 4)
                out[n++] = &v;
        if (const Variant* m = smallest_masked(kind, dt, vec, width)) out[n++] = m;
    }
    if (const Variant* s = smallest_masked(kind, dt, 1, width)) out[n++] = s;
    if (kind == K_RMS || kind == K_LAYER || kind == K_LAYER_NOBIAS || kind == K_RMS_GATED) {
        if (vec_ok)
            if (const Variant* w = find_wide(kind, dt, vec)) out[n++] = w;
        if (const Variant* w = find_wide(kind, dt, 1)) out[n++] = w;
    }
    return n;
}

// Whether a fused RoPE kernel shape can reach the pair partners of a
// rotation over the first `dims` features (see dual_rope_rows).
bool rope_ok(const Variant& v, int64_t dims) {
    if (v.kind == K_ROPE_TRAD) return v.vec >= 2 || v.lpr >= 2;
    const int64_t half = dims / 2;
    if (half % v.vec != 0) return false;
    const int64_t dp = half / v.vec;
    if (v.vpt == 1) return 2 * dp <= v.lpr;
    // two packs per lane: full rotation only (the kernel has no code for a
    // partial one there); more packs: whole packs of partners per lane
    if (v.vpt == 2) return dp == v.lpr;
    return dp % v.lpr == 0;
}

// LDS bytes of a fused RoPE launch: one (cos, sin) fp32 table per row slot.
int64_t rope_lds_bytes(const Variant& v, int64_t dims) {
    const int64_t half = dims / 2;
    return int64_t(v.rows_per_block()) * half * 8;
}

// The inverse-frequency tables of the kernel arguments for (base, dims), in
// turns per position: (1 / 2 pi) * exp2(-2i/dims * log2(base)) for the first
// kRopeTable pairs, and the factors exp2(-2 j kRopeTable / dims * log2(base))
// that carry them to the later pairs, fp64.  The last few tables are kept
// per thread, so a decode-size call copies one.
struct RopeTable {
    float base = 0.0f;
    int64_t dims = -1;
    double invf[RopeArgs::kRopeTable];
    double invf_step[RopeArgs::kRopeSteps];
};

const RopeTable& rope_table(float base, int64_t dims) {
    constexpr int kSlots = 4;
    thread_local RopeTable cache[kSlots];
    thread_local int next = 0;
    for (const RopeTable& e : cache)
        if (e.dims == dims && e.base == base) return e;
    RopeTable& e = cache[next];
    next = (next + 1) % kSlots;
    constexpr double kInvTwoPi = 0.15915494309189533577;
    const double lb = std::log2(static_cast<double>(base));
    const int64_t n = std::min<int64_t>(dims / 2, RopeArgs::kRopeTable);
    for (int64_t i = 0; i < RopeArgs::kRopeTable; ++i)
        e.invf[i] = i < n ? kInvTwoPi * std::exp2(-2.0 * static_cast<double>(i) /
                                                  static_cast<double>(dims) * lb)
                          : 0.0;
    for (int j = 0; j < RopeArgs::kRopeSteps; ++j)
        e.invf_step[j] = std::exp2(-2.0 * static_cast<double>(j * RopeArgs::kRopeTable) /
                                   static_cast<double>(dims) * lb);
    e.base = base;
    e.dims = dims;
    return e;
}

constexpr int64_t kMaxLds = 64 * 1024;

// Fused RoPE kernels able to serve the request, default first: exact
// shapes, the smallest masked 16-byte-pack shape, the smallest masked
// scalar shape; each only if it reaches the partners and fits in LDS.
int rope_candidates(int kind, int dt, int64_t width, bool aligned, int64_t dims,
                    const Variant** out) {
    int n = 0;
    const int vec = 16 / elem_bytes(dt);
    const bool vec_ok = aligned && (width % vec == 0);
    auto usable = [&](const Variant& v) {
        return v.kind == kind && v.dt == dt && rope_ok(v, dims) &&
               rope_lds_bytes(v, dims) <= kMaxLds && v.capacity() >= width;
    };
    if (vec_ok)
        for (const Variant& v : registry().table)
            if (usable(v) && v.vec == vec && !v.masked && v.capacity() == width &&
                n < kMaxCandidates - 2)
                out[n++] = &v;
    for (int pass_vec : {vec_ok ? vec : 0, 1}) {
        if (pass_vec == 0) continue;
        const Variant* best = nullptr;
        for (const Variant& v : registry().table)
            if (usable(v) && v.vec == pass_vec && v.masked &&
                (!best || v.capacity() < best->capacity()))
                best = &v;
        if (best) out[n++] = best;
    }
    return n;
}

// Candidate lists are a pure function of (kind, type, width, alignment,
// rotated dims) over an immutable table, so the last few lookups are kept
// per thread: a decode-size call would otherwise spend most of its host
// time scanning the table.
struct CandidateList {
    int kind = -1, dt = -1;
    int64_t width = -1, dims = -1;
    bool aligned = false;
    int n = 0;
    const Variant* list[kMaxCandidates];
};

const CandidateList& cached_candidates(int kind, int dt, int64_t width, bool aligned,
                                       int64_t dims) {
    constexpr int kSlots = 8;
    thread_local CandidateList cache[kSlots];
    thread_local int next = 0;
    for (const CandidateList& e : cache)
        if (e.kind == kind && e.dt == dt && e.width == width && e.aligned == aligned &&
            e.dims == dims)
            return e;
    CandidateList& e = cache[next];
    next = (next + 1) % kSlots;
    e.n = (kind == K_ROPE_SPLIT || kind == K_ROPE_TRAD)
              ? rope_candidates(kind, dt, width, aligned, dims, e.list)
              : candidates(kind, dt, width, aligned, e.list);
    e.kind = kind;
    e.dt = dt;
    e.width = width;
    e.aligned = aligned;
    e.dims = dims;
    return e;
}

// Variant index i -> candidate i / 2: its default launch (persistent grid,
// or a plain grid for grid-first shapes) when i is even, the other when odd.
bool pick(int kind, int dt, int64_t width, bool aligned, int variant, Choice* c) {
    const CandidateList& cl = cached_candidates(kind, dt, width, aligned, 0);
    const Variant* const* list = cl.list;
    const int n = cl.n;
    if (variant < 0) variant = 0;
    if (variant >= 2 * n) return false;
    c->v = list[variant / 2];
    c->persistent = ((variant % 2) == 0) != c->v->grid_first;
    return true;
}

int op_kind(int op, bool has_bias) {
    if (op == FNORM_OP_RMS) return K_RMS;
    if (op == FNORM_OP_LAYER) return has_bias ? K_LAYER : K_LAYER_NOBIAS;
    if (op == FNORM_OP_LAYER_NOBIAS) return K_LAYER_NOBIAS;
    if (op == FNORM_OP_RMS_SWIGLU) return K_RMS_GATED;
    return K_DUAL;
}

bool valid_op(int op) { return op >= FNORM_OP_RMS && op <= FNORM_OP_LAYER_NOBIAS; }

void describe_choice(const Choice& c, char* buf, size_t len) {
    const Variant& v = *c.v;
    static const char* nts[] = {"", ".ntst", ".ntld", ".nt"};
    const char* nt = nts[(v.nt & NT_LOAD ? 2 : 0) | (v.nt & NT_STORE ? 1 : 0)];
    static const char* kinds[] = {"rms",       "layer",     "layer",  "dual",
                                  "copy",      "ropesplit", "ropeinter", "rmsgate"};
    if (v.wide)
        std::snprintf(buf, len, "%s.%s.vec%d.wide.blk%d.%s", kinds[v.kind], dtype_name(v.dt),
                      v.vec, v.block, c.persistent ? "persistent" : "grid");
    else if (c.persistent && v.grid_cap > 0)
        std::snprintf(buf, len, "%s.%s.vec%d.vpt%d.lpr%d.blk%d.%s%s.persistent%d", kinds[v.kind],
                      dtype_name(v.dt), v.vec, v.vpt, v.lpr, v.block,
                      v.masked ? "masked" : "exact", nt, v.grid_cap);
    else if (!c.persistent && v.grid_resident > 0)
        std::snprintf(buf, len, "%s.%s.vec%d.vpt%d.lpr%d.blk%d.%s%s.grid%d", kinds[v.kind],
                      dtype_name(v.dt), v.vec, v.vpt, v.lpr, v.block,
                      v.masked ? "masked" : "exact", nt, v.grid_resident);
    else
        std::snprintf(buf, len, "%s.%s.vec%d.vpt%d.lpr%d.blk%d.%s%s.%s", kinds[v.kind],
                      dtype_name(v.dt), v.vec, v.vpt, v.lpr, v.block,
                      v.masked ? "masked" : "exact", nt, c.persistent ? "persistent" : "grid");
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b <= INT64_MAX / 8 for non-negative a, b; negative values pass (the
// checks that follow reject them with their own message).
bool product_fits(int64_t a, int64_t b) {
    if (a <= 0 || b <= 0) return true;
    return a <= (INT64_MAX / 8) / b;
}

bool overlap(const void* a, int64_t an, const void* b, int64_t bn) {
    if (!a || !b || an <= 0 || bn <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + uintptr_t(bn) && b0 < a0 + uintptr_t(an);
}

int check_scalars(const char* op, int dtype, int64_t rows, int64_t width, float eps) {
    if (!valid_dtype(dtype))
        return fail(FNORM_ERR_DTYPE, op, "dtype %d is not FNORM_F32 (0), FNORM_BF16 (1) or FNORM_F16 (2)",
                    dtype);
    if (rows < 0 || width <= 0)
        return fail(FNORM_ERR_SHAPE, op, "rows=%lld width=%lld (need rows >= 0, width > 0)",
                    (long long)rows, (long long)width);
    const int64_t limit = INT64_MAX / 8;
    if (rows > 0 && width > limit / rows)
        return fail(FNORM_ERR_SHAPE, op, "rows*width overflows (rows=%lld width=%lld)",
                    (long long)rows, (long long)width);
    if (!std::isfinite(eps) || eps < 0.0f)
        return fail(FNORM_ERR_EPS, op, "eps=%g must be finite and >= 0", double(eps));
    return FNORM_OK;
}

int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    std::atomic<int>& slot = cache[dev & 63];
    int n = slot.load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        slot.store(n, std::memory_order_relaxed);
    }
    return n;
}

int blocks_per_cu(const Variant* v) {
    const Registry& r = registry();
    std::atomic<int>& slot = r.occupancy[v - r.table.data()];
    int n = slot.load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, v->fn, v->block, 0) != hipSuccess ||
            n <= 0)
            n = 1;
        slot.store(n, std::memory_order_relaxed);
    }
    return n;
}

// Resident workgroups per CU of a variant launched with `lds` bytes of
// dynamic LDS, cached so that repeated calls (and calls recorded into a HIP
// graph) make no occupancy query.
int blocks_per_cu_lds(const Variant* v, int64_t lds) {
    static std::mutex mu;
    static std::unordered_map<uint64_t, int> cache;
    const uint64_t key = (uint64_t(v - registry().table.data()) << 32) | uint64_t(lds);
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, v->fn, v->block, size_t(lds)) !=
            hipSuccess || n <= 0)
        n = 1;
    cache.emplace(key, n);
    return n;
}

// Dynamic LDS per workgroup that holds a plain grid of `v` to at most
// k = v->grid_resident workgroups per CU: each reserves LDS_per_CU / (k + 1/2)
// bytes in all (its own LDS included), so k fit and k + 1 do not.  0 when the
// kernel's registers already hold it to k or fewer, or when the device cannot
// grant the reservation (then the grid runs unlimited).  Cached per variant.
int resident_lds(const Variant* v) {
    const Registry& r = registry();
    std::atomic<int>& slot = r.grid_lds[v - r.table.data()];
    int bytes = slot.load(std::memory_order_relaxed);
    if (bytes >= 0) return bytes;
    bytes = 0;
    const int k = v->grid_resident;
    int dev = 0, per_cu = 0, per_block = 0;
    hipFuncAttributes fa{};
    if (k > 0 && blocks_per_cu(v) > k && hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              dev) == hipSuccess &&
        hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
            hipSuccess &&
        hipFuncGetAttributes(&fa, v->fn) == hipSuccess) {
        const int64_t total = 2 * int64_t(per_cu) / (2 * k + 1);
        const int64_t dyn = total - int64_t(fa.sharedSizeBytes);
        if (dyn > 0 && total <= per_block && blocks_per_cu_lds(v, dyn) <= k)
            bytes = int(dyn);
    }
    slot.store(bytes, std::memory_order_relaxed);
    return bytes;
}

// Workgroups of a persistent grid over `units` block-rows when more than
// `cap` fit: the fewest that still give every workgroup the same number of
// turns (rounded up to a multiple of the XCD count, for the XCD-major
// order), so that the last turn does not run with part of the grid idle.
// The fused RoPE launch uses it (its persistent grids hold up to 8
// workgroups per CU, so a launch often has only a few turns: head_dim 64 at
// 4096 tokens 11.6 -> 11.0 us); the norms' persistent grids (2 workgroups
// per CU, tens of turns) measured the same or 0.5-1% slower with it.
int64_t balanced_grid(int64_t units, int64_t cap) {
    const int64_t turns = (units + cap - 1) / cap;
    int64_t g = (units + turns - 1) / turns;
    g = (g + kXcds - 1) / kXcds * kXcds;
    return g < cap ? g : cap;
}

// Workgroups of the query and key segments of a dual launch over qu and ku
// block-rows: one per block-row (a plain grid), or, when that is more than
// `cap` (> 0: a persistent grid), `cap` shared in proportion to the
// block-rows, the query share a multiple of 8 so that both segments keep the
// XCD-major order.  A segment with rows always gets a workgroup.
void split_grid(int64_t qu, int64_t ku, int64_t cap, int64_t* gq, int64_t* gk) {
    constexpr int64_t kMaxSegment = int64_t(1) << 29;   // grid-stride loops cover the rest
    int64_t q = qu, k = ku;
    if (cap > 0 && qu + ku > cap) {
        cap = balanced_grid(qu + ku, cap);
        q = ku > 0 ? cap * qu / (qu + ku) : cap;
        if (ku > 0 && q >= kXcds) q -= q % kXcds;
        if (qu > 0 && q < 1) q = 1;
        if (q > qu) q = qu;
        k = ku > 0 ? (cap - q > 1 ? cap - q : 1) : 0;
        if (k > ku) k = ku;
    }
    *gq = q < kMaxSegment ? q : kMaxSegment;
    *gk = k < kMaxSegment ? k : kMaxSegment;
}

int launch(const char* op, const Choice& c, NormArgs& a, void* stream) {
    const int64_t rpb = c.v->rows_per_block();
    int64_t cap = 0;
    if (c.persistent) {
        int per_cu = blocks_per_cu(c.v);
        if (c.v->grid_cap > 0 && c.v->grid_cap < per_cu) per_cu = c.v->grid_cap;
        cap = int64_t(device_cus()) * per_cu;
    }
    // work units: block-rows (a dual launch's two tensors do not share one)
    int64_t grid = c.v->kind == K_DUAL
                       ? (a.rows1 + rpb - 1) / rpb + (a.rows - a.rows1 + rpb - 1) / rpb
                       : (a.rows + rpb - 1) / rpb;
    if (cap > 0 && grid > cap) grid = cap;
    if (grid > (int64_t(1) << 30)) grid = int64_t(1) << 30;  // grid-stride covers the rest
    const int lds = !c.persistent && c.v->grid_resident > 0 ? resident_lds(c.v) : 0;
    void* args[] = {&a};
    // The launch's own status only: the thread's last-error slot may hold an
    // earlier, unrelated failure of the caller's, which is not this call's.
    const hipError_t e = hipLaunchKernel(c.v->fn, dim3(unsigned(grid)),
                                         dim3(unsigned(c.v->block)), args, size_t(lds),
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(FNORM_ERR_LAUNCH, op, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}


// A strided tensor in memory: `count` blocks of `len` bytes, the block i
// starting at base + i * stride bytes (one block per token or row).
struct Span {
    const void* base;
    int64_t stride, len, count;
};

Span span(const void* p, int64_t stride_elems, int64_t len_elems, int64_t count, int64_t eb) {
    return Span{p, stride_elems * eb, len_elems * eb, count};
}

// Whether two strided tensors share a byte.  Exact for two tensors with the
// same stride whose blocks interleave (e.g. the q and k parts of one packed
// QKV buffer); otherwise it compares the overall extents (conservative).
bool spans_overlap(const Span& a, const Span& b) {
    if (!a.base || !b.base || a.count <= 0 || b.count <= 0 || a.len <= 0 || b.len <= 0)
        return false;
    const int64_t a0 = int64_t(reinterpret_cast<uintptr_t>(a.base));
    const int64_t b0 = int64_t(reinterpret_cast<uintptr_t>(b.base));
    const int64_t a1 = a0 + (a.count - 1) * a.stride + a.len;
    const int64_t b1 = b0 + (b.count - 1) * b.stride + b.len;
    if (a1 <= b0 || b1 <= a0) return false;
    if (a.stride == b.stride && a.stride > 0 && a.len + b.len <= a.stride) {
        const int64_t s = a.stride;
        const int64_t dm = (((b0 - a0) % s) + s) % s;
        if (dm >= a.len && dm + b.len <= s) return false;
    }
    return true;
}

// y may be x itself (same base and stride); any other overlap is an error.
bool output_clashes(const Span& y, const Span& x) {
    if (y.base == x.base && y.stride == x.stride && y.len == x.len) return false;
    return spans_overlap(y, x);
}

bool stride_aligned(int64_t stride_elems, int64_t eb) { return (stride_elems * eb) % 16 == 0; }

// RMSNorm / LayerNorm over rows addressed with row strides (elements).
// With `plan` set, nothing is launched: the call is validated and its kernel
// choice returned there (plan->v == nullptr when the call launches nothing).
int rows_impl(const char* op, int fop, const void* x, int64_t xs, const void* g, int64_t gs,
              const void* w, const void* b, void* y, int64_t ys, int64_t rows, int64_t width,
              float eps, int dtype, void* stream, int variant, Choice* plan = nullptr) {
    if (plan) plan->v = nullptr;
    const bool gated = fop == FNORM_OP_RMS_SWIGLU;
    if (int s = check_scalars(op, dtype, rows, width, eps)) return s;
    if (rows > 1 && (xs < width || ys < width || (gated && gs < width)))
        return fail(FNORM_ERR_SHAPE, op, "row strides below width %lld", (long long)width);
    if (rows > 1 && (xs > (INT64_MAX / 8) / rows || ys > (INT64_MAX / 8) / rows ||
                     (gated && gs > (INT64_MAX / 8) / rows)))
        return fail(FNORM_ERR_SHAPE, op, "row strides overflow");
    if (rows == 0) return ok();
    if (!x || !w || !y) return fail(FNORM_ERR_NULL, op, "x, w and y must be non-NULL");
    if (gated && !g) return fail(FNORM_ERR_NULL, op, "the gate must be non-NULL");
    const int64_t eb = elem_bytes(dtype);
    const Span sx = span(x, xs, width, rows, eb), sy = span(y, ys, width, rows, eb);
    const Span sw = span(w, width, width, 1, eb), sb = span(b, width, width, 1, eb);
    const Span sg = span(g, gs, width, gated ? rows : 0, eb);
    if (output_clashes(sy, sx))
        return fail(FNORM_ERR_ALIAS, op, "y overlaps x without being x itself");
    if (output_clashes(sy, sg))
        return fail(FNORM_ERR_ALIAS, op, "y overlaps the gate without being the gate itself");
    if (spans_overlap(sy, sw)) return fail(FNORM_ERR_ALIAS, op, "y overlaps w");
    if (spans_overlap(sy, sb)) return fail(FNORM_ERR_ALIAS, op, "y overlaps b");
    const bool one = rows == 1;
    const bool al = aligned16(x) && aligned16(w) && aligned16(y) && (!b || aligned16(b)) &&
                    (!gated || aligned16(g)) &&
                    (one || (stride_aligned(xs, eb) && stride_aligned(ys, eb) &&
                             (!gated || stride_aligned(gs, eb))));
    Choice c;
    const int kind = op_kind(fop, b != nullptr);
    if (!pick(kind, dtype, width, al, variant, &c))
        return fail(FNORM_ERR_UNSUPPORTED, op, "no kernel variant %d for width %lld", variant,
                    (long long)width);
    if (plan) {
        *plan = c;
        return ok();
    }
    NormArgs a{x,    w,    b,     y,     nullptr, nullptr, nullptr, rows, rows, width,
               eps,  one ? width : xs, one ? width : ys, 1, width, width, 1,
               gated ? g : nullptr, one ? width : gs};
    a.inv_width = 1.0f / static_cast<float>(width);
    return launch(op, c, a, stream);
}

// Checks shared by the dual forms: q [tokens, q_heads, hd] and k [tokens,
// k_heads, hd] with token strides (elements) qs, ks, qys, kys.
int dual_checks(const char* op, const void* q, int64_t qs, const void* k, int64_t ks,
                const void* qw, const void* kw, const void* qy, int64_t qys, const void* ky,
                int64_t kys, int64_t tokens, int64_t q_heads, int64_t k_heads, int64_t head_dim,
                float eps, int dtype, const void* freqs, int64_t freq_count, bool* aligned) {
    if (tokens < 0 || q_heads < 0 || k_heads < 0)
        return fail(FNORM_ERR_SHAPE, op, "tokens=%lld q_heads=%lld k_heads=%lld must be >= 0",
                    (long long)tokens, (long long)q_heads, (long long)k_heads);
    if (q_heads > INT64_MAX / 4 - k_heads ||
        (tokens > 0 && (q_heads + k_heads) > (INT64_MAX / 16) / tokens))
        return fail(FNORM_ERR_SHAPE, op, "tokens * heads overflows");
    if (int s = check_scalars(op, dtype, tokens * (q_heads + k_heads), head_dim, eps)) return s;
    // with no tokens the row count above is 0 and bounds nothing
    if (!product_fits(q_heads, head_dim) || !product_fits(k_heads, head_dim))
        return fail(FNORM_ERR_SHAPE, op, "heads * head_dim overflows");
    const int64_t qext = q_heads * head_dim, kext = k_heads * head_dim;
    if (tokens > 1 && ((q_heads > 0 && (qs < qext || qys < qext)) ||
                       (k_heads > 0 && (ks < kext || kys < kext))))
        return fail(FNORM_ERR_SHAPE, op, "token strides below heads * head_dim");
    if (tokens > 1 && (qs > (INT64_MAX / 8) / tokens || ks > (INT64_MAX / 8) / tokens ||
                       qys > (INT64_MAX / 8) / tokens || kys > (INT64_MAX / 8) / tokens))
        return fail(FNORM_ERR_SHAPE, op, "token strides overflow");
    const int64_t q_rows = tokens * q_heads, k_rows = tokens * k_heads;
    if (q_rows + k_rows == 0) return FNORM_OK;
    if (q_rows > 0 && (!q || !qw || !qy))
        return fail(FNORM_ERR_NULL, op, "q, qw and qy must be non-NULL when q rows exist");
    if (k_rows > 0 && (!k || !kw || !ky))
        return fail(FNORM_ERR_NULL, op, "k, kw and ky must be non-NULL when k rows exist");
    const int64_t eb = elem_bytes(dtype);
    const int64_t nq = q_rows > 0 ? tokens : 0, nk = k_rows > 0 ? tokens : 0;
    const Span sq = span(q, qs, qext, nq, eb), sk = span(k, ks, kext, nk, eb);
    const Span sqy = span(qy, qys, qext, nq, eb), sky = span(ky, kys, kext, nk, eb);
    const Span sqw = span(qw, head_dim, head_dim, q_rows > 0 ? 1 : 0, eb);
    const Span skw = span(kw, head_dim, head_dim, k_rows > 0 ? 1 : 0, eb);
    const Span sfr = span(freqs, freq_count, freq_count, freqs ? 1 : 0, 4);
    if (output_clashes(sqy, sq)) return fail(FNORM_ERR_ALIAS, op, "qy overlaps q");
    if (output_clashes(sky, sk)) return fail(FNORM_ERR_ALIAS, op, "ky overlaps k");
    if (spans_overlap(sqy, sk) || spans_overlap(sky, sq))
        return fail(FNORM_ERR_ALIAS, op, "an output overlaps the other tensor's input");
    if (spans_overlap(sqy, sky)) return fail(FNORM_ERR_ALIAS, op, "qy overlaps ky");
    if (spans_overlap(sqy, sqw) || spans_overlap(sqy, skw) || spans_overlap(sky, sqw) ||
        spans_overlap(sky, skw) || spans_overlap(sqy, sfr) || spans_overlap(sky, sfr))
        return fail(FNORM_ERR_ALIAS, op, "an output overlaps a weight or the frequency table");
    const bool one = tokens == 1;
    *aligned = (q_rows == 0 || (aligned16(q) && aligned16(qw) && aligned16(qy) &&
                                (one || (stride_aligned(qs, eb) && stride_aligned(qys, eb))))) &&
               (k_rows == 0 || (aligned16(k) && aligned16(kw) && aligned16(ky) &&
                                (one || (stride_aligned(ks, eb) && stride_aligned(kys, eb)))));
    return FNORM_OK;
}

int dual_impl(const char* op, const void* q, int64_t qs, const void* k, int64_t ks,
              const void* qw, const void* kw, void* qy, int64_t qys, void* ky, int64_t kys,
              int64_t tokens, int64_t q_heads, int64_t k_heads, int64_t head_dim, float eps,
              int dtype, void* stream, int variant, Choice* plan = nullptr) {
    if (plan) plan->v = nullptr;
    bool al = false;
    if (int s = dual_checks(op, q, qs, k, ks, qw, kw, qy, qys, ky, kys, tokens, q_heads, k_heads,
                            head_dim, eps, dtype, nullptr, 0, &al))
        return s;
    const int64_t q_rows = tokens * q_heads, k_rows = tokens * k_heads;
    if (q_rows + k_rows == 0) return ok();
    Choice c;
    if (!pick(K_DUAL, dtype, head_dim, al, variant, &c))
        return fail(FNORM_ERR_UNSUPPORTED, op, "no kernel variant %d for head_dim %lld", variant,
                    (long long)head_dim);
    if (plan) {
        *plan = c;
        return ok();
    }
    // A side with no rows is never read; give the kernel the other side's
    // valid weight pointer so its register preload stays in bounds.
    const void* qw_eff = q_rows > 0 ? qw : kw;
    const void* kw_eff = k_rows > 0 ? kw : qw;
    // One-token tensors, and tokens packed back to back, address as plain rows.
    const bool qplain = tokens == 1 || (qs == q_heads * head_dim && qys == qs);
    const bool kplain = tokens == 1 || (ks == k_heads * head_dim && kys == ks);
    NormArgs a{q, qw_eff, nullptr, qy, k, kw_eff, ky, q_rows + k_rows, q_rows, head_dim, eps,
               qplain ? head_dim : qs, qplain ? head_dim : qys, qplain ? 1 : q_heads,
               kplain ? head_dim : ks, kplain ? head_dim : kys, kplain ? 1 : k_heads};
    // the kernel divides a row index by the head count only while rows < 2^31
    if (a.rows <= 0x7fffffff) {
        if (a.xh > 1) a.xdiv = make_fast_div(uint32_t(a.xh));
        if (a.x2h > 1) a.x2div = make_fast_div(uint32_t(a.x2h));
    }
    a.inv_width = 1.0f / static_cast<float>(head_dim);
    return launch(op, c, a, stream);
}

int rope_impl(const char* op, const void* q, int64_t qs, const void* k, int64_t ks,
              const void* qw, const void* kw, void* qy, int64_t qys, void* ky, int64_t kys,
              int64_t tokens, int64_t q_heads, int64_t k_heads, int64_t head_dim, float eps,
              int64_t rope_dims, int traditional, float base, float scale, int64_t offset,
              const float* freqs, int dtype, void* stream, int variant, Choice* plan = nullptr) {
    if (plan) plan->v = nullptr;
    if (rope_dims < 2 || rope_dims % 2 != 0 || rope_dims > head_dim)
        return fail(FNORM_ERR_SHAPE, op, "rope_dims=%lld must be even and in [2, head_dim=%lld]",
                    (long long)rope_dims, (long long)head_dim);
    if (rope_dims / 2 > int64_t(RopeArgs::kRopeTable) * RopeArgs::kRopeSteps)
        return fail(FNORM_ERR_UNSUPPORTED, op, "rope_dims=%lld above %lld", (long long)rope_dims,
                    2LL * RopeArgs::kRopeTable * RopeArgs::kRopeSteps);
    if (!std::isfinite(scale) || (!freqs && (!std::isfinite(base) || base <= 0.0f)))
        return fail(FNORM_ERR_SHAPE, op, "base must be finite and > 0, scale finite");
    if (offset < 0 || tokens < 0 || offset > (int64_t(1) << 52) - tokens)
        return fail(FNORM_ERR_SHAPE, op, "offset=%lld out of range", (long long)offset);
    bool al = false;
    if (int s = dual_checks(op, q, qs, k, ks, qw, kw, qy, qys, ky, kys, tokens, q_heads, k_heads,
                            head_dim, eps, dtype, freqs, rope_dims / 2, &al))
        return s;
    const int64_t q_rows = tokens * q_heads, k_rows = tokens * k_heads;
    if (q_rows + k_rows == 0) return ok();
    const int kind = traditional ? K_ROPE_TRAD : K_ROPE_SPLIT;
    const CandidateList& cl = cached_candidates(kind, dtype, head_dim, al, rope_dims);
    const Variant* const* list = cl.list;
    const int n = cl.n;
    if (variant < 0) variant = 0;
    if (variant >= 2 * n)
        return fail(FNORM_ERR_UNSUPPORTED, op,
                    "no fused kernel for head_dim %lld, rope_dims %lld (variant %d)",
                    (long long)head_dim, (long long)rope_dims, variant);
    const Variant* v = list[variant / 2];
    const bool persistent = (variant % 2 == 0) != v->grid_first;
    if (plan) {
        plan->v = v;
        plan->persistent = persistent;
        return ok();
    }
    const void* qw_eff = q_rows > 0 ? qw : kw;
    const void* kw_eff = k_rows > 0 ? kw : qw;
    RopeArgs ra{NormArgs{q, qw_eff, nullptr, qy, k, kw_eff, ky, q_rows + k_rows, q_rows,
                         head_dim, eps, qs, qys, q_heads > 0 ? q_heads : 1, ks, kys,
                         k_heads > 0 ? k_heads : 1},
                q_heads > 0 ? q_heads : 1, k_heads > 0 ? k_heads : 1, rope_dims, offset, base,
                scale, freqs, FastDiv{}, FastDiv{}, 0u};
    ra.n.inv_width = 1.0f / static_cast<float>(head_dim);
    if (!freqs) {
        const RopeTable& tab = rope_table(base, rope_dims);
        std::memcpy(ra.invf, tab.invf, sizeof(ra.invf));
        std::memcpy(ra.invf_step, tab.invf_step, sizeof(ra.invf_step));
    }
    // the kernel divides by the head counts only while rows < 2^31
    if (ra.n.rows <= 0x7fffffff) {
        ra.qdiv = make_fast_div(uint32_t(ra.q_heads));
        ra.kdiv = make_fast_div(uint32_t(ra.k_heads));
    }
    const int64_t lds = rope_lds_bytes(*v, rope_dims);
    const int64_t rpb = v->rows_per_block();
    const int64_t cap =
        persistent ? int64_t(device_cus()) * blocks_per_cu_lds(v, lds) : int64_t(0);
    int64_t gq = 0, gk = 0;
    split_grid((q_rows + rpb - 1) / rpb, (k_rows + rpb - 1) / rpb, cap, &gq, &gk);
    ra.q_blocks = uint32_t(gq);
    const int64_t grid = gq + gk;
    void* args[] = {&ra};
    const hipError_t e = hipLaunchKernel(v->fn, dim3(unsigned(grid)), dim3(unsigned(v->block)),
                                         args, size_t(lds), static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(FNORM_ERR_LAUNCH, op, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace
}  // namespace fnorm

using namespace fnorm;

extern "C" {

int fnorm_rms_v(const void* x, const void* w, void* y, int64_t rows, int64_t width, float eps,
                int dtype, void* stream, int variant) {
    return rows_impl("fnorm_rms", FNORM_OP_RMS, x, width, nullptr, 0, w, nullptr, y, width, rows,
                     width, eps, dtype, stream, variant);
}

int fnorm_rms(const void* x, const void* w, void* y, int64_t rows, int64_t width, float eps,
              int dtype, void* stream) {
    return fnorm_rms_v(x, w, y, rows, width, eps, dtype, stream, -1);
}

int fnorm_rms_strided(const void* x, int64_t x_stride, const void* w, void* y, int64_t y_stride,
                      int64_t rows, int64_t width, float eps, int dtype, void* stream,
                      int variant) {
    return rows_impl("fnorm_rms_strided", FNORM_OP_RMS, x, x_stride, nullptr, 0, w, nullptr, y,
                     y_stride, rows, width, eps, dtype, stream, variant);
}

int fnorm_layer_v(const void* x, const void* w, const void* b, void* y, int64_t rows,
                  int64_t width, float eps, int dtype, void* stream, int variant) {
    return rows_impl("fnorm_layer", FNORM_OP_LAYER, x, width, nullptr, 0, w, b, y, width, rows,
                     width, eps, dtype, stream, variant);
}

int fnorm_layer(const void* x, const void* w, const void* b, void* y, int64_t rows,
                int64_t width, float eps, int dtype, void* stream) {
    return fnorm_layer_v(x, w, b, y, rows, width, eps, dtype, stream, -1);
}

int fnorm_layer_strided(const void* x, int64_t x_stride, const void* w, const void* b, void* y,
                        int64_t y_stride, int64_t rows, int64_t width, float eps, int dtype,
                        void* stream, int variant) {
    return rows_impl("fnorm_layer_strided", FNORM_OP_LAYER, x, x_stride, nullptr, 0, w, b, y,
                     y_stride, rows, width, eps, dtype, stream, variant);
}

int fnorm_rms_swiglu_v(const void* x, const void* g, const void* w, void* y, int64_t rows,
                       int64_t width, float eps, int dtype, void* stream, int variant) {
    return rows_impl("fnorm_rms_swiglu", FNORM_OP_RMS_SWIGLU, x, width, g, width, w, nullptr, y,
                     width, rows, width, eps, dtype, stream, variant);
}

int fnorm_rms_swiglu(const void* x, const void* g, const void* w, void* y, int64_t rows,
                     int64_t width, float eps, int dtype, void* stream) {
    return fnorm_rms_swiglu_v(x, g, w, y, rows, width, eps, dtype, stream, -1);
}

int fnorm_rms_swiglu_strided(const void* x, int64_t x_stride, const void* g, int64_t g_stride,
                             const void* w, void* y, int64_t y_stride, int64_t rows,
                             int64_t width, float eps, int dtype, void* stream, int variant) {
    return rows_impl("fnorm_rms_swiglu_strided", FNORM_OP_RMS_SWIGLU, x, x_stride, g, g_stride,
                     w, nullptr, y, y_stride, rows, width, eps, dtype, stream, variant);
}

int fnorm_dual_head_rms_v(const void* q, const void* k, const void* qw, const void* kw, void* qy,
                          void* ky, int64_t q_rows, int64_t k_rows, int64_t head_dim, float eps,
                          int dtype, void* stream, int variant) {
    static const char* op = "fnorm_dual_head_rms";
    if (q_rows < 0 || k_rows < 0)
        return fail(FNORM_ERR_SHAPE, op, "q_rows=%lld k_rows=%lld must be >= 0",
                    (long long)q_rows, (long long)k_rows);
    // contiguous head vectors: one "token" whose heads are all the rows (a
    // single token's stride is never used, so none is formed: rows * head_dim
    // is only computed after the size checks)
    return dual_impl(op, q, 0, k, 0, qw, kw, qy, 0, ky, 0, 1, q_rows, k_rows, head_dim, eps,
                     dtype, stream, variant);
}

int fnorm_dual_head_rms(const void* q, const void* k, const void* qw, const void* kw, void* qy,
                        void* ky, int64_t q_rows, int64_t k_rows, int64_t head_dim, float eps,
                        int dtype, void* stream) {
    return fnorm_dual_head_rms_v(q, k, qw, kw, qy, ky, q_rows, k_rows, head_dim, eps, dtype,
                                 stream, -1);
}

int fnorm_dual_head_rms_strided(const void* q, int64_t q_stride, const void* k,
                                int64_t k_stride, const void* qw, const void* kw, void* qy,
                                int64_t qy_stride, void* ky, int64_t ky_stride, int64_t tokens,
                                int64_t q_heads, int64_t k_heads, int64_t head_dim, float eps,
                                int dtype, void* stream, int variant) {
    return dual_impl("fnorm_dual_head_rms_strided", q, q_stride, k, k_stride, qw, kw, qy,
                     qy_stride, ky, ky_stride, tokens, q_heads, k_heads, head_dim, eps, dtype,
                     stream, variant);
}

int fnorm_dual_head_rms_rope_v(const void* q, const void* k, const void* qw, const void* kw,
                               void* qy, void* ky, int64_t tokens, int64_t q_heads,
                               int64_t k_heads, int64_t head_dim, float eps, int64_t rope_dims,
                               int traditional, float base, float scale, int64_t offset,
                               const float* freqs, int dtype, void* stream, int variant) {
    static const char* op = "fnorm_dual_head_rms_rope";
    // token strides of the packed layout, formed only when they fit (negative
    // counts are reported by the shared checks)
    if (!product_fits(q_heads, head_dim) || !product_fits(k_heads, head_dim))
        return fail(FNORM_ERR_SHAPE, op, "heads * head_dim overflows");
    const int64_t qs = q_heads > 0 && head_dim > 0 ? q_heads * head_dim : 0;
    const int64_t ks = k_heads > 0 && head_dim > 0 ? k_heads * head_dim : 0;
    return rope_impl(op, q, qs, k, ks, qw, kw, qy, qs, ky, ks, tokens, q_heads, k_heads,
                     head_dim, eps, rope_dims, traditional, base, scale, offset, freqs, dtype,
                     stream, variant);
}

int fnorm_dual_head_rms_rope(const void* q, const void* k, const void* qw, const void* kw,
                             void* qy, void* ky, int64_t tokens, int64_t q_heads,
                             int64_t k_heads, int64_t head_dim, float eps, int64_t rope_dims,
                             int traditional, float base, float scale, int64_t offset,
                             const float* freqs, int dtype, void* stream) {
    return fnorm_dual_head_rms_rope_v(q, k, qw, kw, qy, ky, tokens, q_heads, k_heads, head_dim,
                                      eps, rope_dims, traditional, base, scale, offset, freqs,
                                      dtype, stream, -1);
}

int fnorm_dual_head_rms_rope_strided(const void* q, int64_t q_stride, const void* k,
                                     int64_t k_stride, const void* qw, const void* kw, void* qy,
                                     int64_t qy_stride, void* ky, int64_t ky_stride,
                                     int64_t tokens, int64_t q_heads, int64_t k_heads,
                                     int64_t head_dim, float eps, int64_t rope_dims,
                                     int traditional, float base, float scale, int64_t offset,
                                     const float* freqs, int dtype, void* stream, int variant) {
    return rope_impl("fnorm_dual_head_rms_rope_strided", q, q_stride, k, k_stride, qw, kw, qy,
                     qy_stride, ky, ky_stride, tokens, q_heads, k_heads, head_dim, eps,
                     rope_dims, traditional, base, scale, offset, freqs, dtype, stream, variant);
}

int fnorm_variant_count(int op, int dtype, int64_t width, int aligned) {
    if (!valid_dtype(dtype) || width <= 0 || !valid_op(op)) return 0;
    const Variant* list[kMaxCandidates];
    return 2 * candidates(op_kind(op, true), dtype, width, aligned != 0, list);
}

int fnorm_describe_shape(int op, int dtype, int64_t width, int aligned, int variant, char* buf,
                         int64_t len) {
    static const char* name = "fnorm_describe_shape";
    if (!buf || len <= 0) return fail(FNORM_ERR_NULL, name, "buf must be non-NULL, len > 0");
    buf[0] = '\0';
    if (!valid_dtype(dtype)) return fail(FNORM_ERR_DTYPE, name, "dtype %d", dtype);
    if (width <= 0) return fail(FNORM_ERR_SHAPE, name, "width %lld", (long long)width);
    if (!valid_op(op)) return fail(FNORM_ERR_UNSUPPORTED, name, "op %d", op);
    Choice c;
    if (!pick(op_kind(op, true), dtype, width, aligned != 0, variant, &c))
        return fail(FNORM_ERR_UNSUPPORTED, name, "no variant %d", variant);
    describe_choice(c, buf, size_t(len));
    return ok();
}

// The kernel name of a planned call, "none" when the call launches nothing.
static int describe_plan(int status, const Choice& c, char* buf, int64_t len) {
    if (status != FNORM_OK) return status;
    if (!c.v) std::snprintf(buf, size_t(len), "none");
    else describe_choice(c, buf, size_t(len));
    return ok();
}

int fnorm_describe(int op, const void* x, int64_t x_stride, const void* g, int64_t g_stride,
                   const void* w, const void* b, const void* y, int64_t y_stride, int64_t rows,
                   int64_t width, int dtype, int variant, char* buf, int64_t len) {
    static const char* name = "fnorm_describe";
    if (!buf || len <= 0) return fail(FNORM_ERR_NULL, name, "buf must be non-NULL, len > 0");
    buf[0] = '\0';
    if (op != FNORM_OP_RMS && op != FNORM_OP_LAYER && op != FNORM_OP_LAYER_NOBIAS &&
        op != FNORM_OP_RMS_SWIGLU)
        return fail(FNORM_ERR_UNSUPPORTED, name, "op %d is not a row operation", op);
    const int fop = op == FNORM_OP_LAYER_NOBIAS ? FNORM_OP_LAYER : op;
    const void* bias = op == FNORM_OP_LAYER ? b : nullptr;
    const void* gate = op == FNORM_OP_RMS_SWIGLU ? g : nullptr;
    Choice c;
    const int s = rows_impl(name, fop, x, x_stride, gate, g_stride, w, bias, const_cast<void*>(y),
                            y_stride, rows, width, 0.0f, dtype, nullptr, variant, &c);
    return describe_plan(s, c, buf, len);
}

int fnorm_describe_dual(const void* q, int64_t q_stride, const void* k, int64_t k_stride,
                        const void* qw, const void* kw, const void* qy, int64_t qy_stride,
                        const void* ky, int64_t ky_stride, int64_t tokens, int64_t q_heads,
                        int64_t k_heads, int64_t head_dim, int dtype, int variant, char* buf,
                        int64_t len) {
    static const char* name = "fnorm_describe_dual";
    if (!buf || len <= 0) return fail(FNORM_ERR_NULL, name, "buf must be non-NULL, len > 0");
    buf[0] = '\0';
    Choice c;
    const int s = dual_impl(name, q, q_stride, k, k_stride, qw, kw, const_cast<void*>(qy),
                            qy_stride, const_cast<void*>(ky), ky_stride, tokens, q_heads, k_heads,
                            head_dim, 0.0f, dtype, nullptr, variant, &c);
    return describe_plan(s, c, buf, len);
}

int fnorm_describe_dual_rope(const void* q, int64_t q_stride, const void* k, int64_t k_stride,
                             const void* qw, const void* kw, const void* qy, int64_t qy_stride,
                             const void* ky, int64_t ky_stride, int64_t tokens, int64_t q_heads,
                             int64_t k_heads, int64_t head_dim, int64_t rope_dims,
                             int traditional, float base, float scale, int64_t offset,
                             const float* freqs, int dtype, int variant, char* buf,
                             int64_t len) {
    static const char* name = "fnorm_describe_dual_rope";
    if (!buf || len <= 0) return fail(FNORM_ERR_NULL, name, "buf must be non-NULL, len > 0");
    buf[0] = '\0';
    Choice c;
    const int s = rope_impl(name, q, q_stride, k, k_stride, qw, kw, const_cast<void*>(qy),
                            qy_stride, const_cast<void*>(ky), ky_stride, tokens, q_heads, k_heads,
                            head_dim, 0.0f, rope_dims, traditional, base, scale, offset, freqs,
                            dtype, nullptr, variant, &c);
    return describe_plan(s, c, buf, len);
}

int fnorm_rope_variant_count(int dtype, int64_t head_dim, int64_t rope_dims, int traditional,
                             int aligned) {
    if (!valid_dtype(dtype) || head_dim <= 0 || rope_dims < 2 ||
        rope_dims % 2 != 0 || rope_dims > head_dim)
        return 0;
    const Variant* list[kMaxCandidates];
    return 2 * rope_candidates(traditional ? K_ROPE_TRAD : K_ROPE_SPLIT, dtype, head_dim,
                               aligned != 0, rope_dims, list);
}

int fnorm_describe_rope(int dtype, int64_t head_dim, int64_t rope_dims, int traditional,
                        int aligned, int variant, char* buf, int64_t len) {
    static const char* name = "fnorm_describe_rope";
    if (!buf || len <= 0) return fail(FNORM_ERR_NULL, name, "buf must be non-NULL, len > 0");
    buf[0] = '\0';
    const int n = fnorm_rope_variant_count(dtype, head_dim, rope_dims, traditional, aligned);
    if (variant < 0) variant = 0;
    if (variant >= n) return fail(FNORM_ERR_UNSUPPORTED, name, "no variant %d", variant);
    const Variant* list[kMaxCandidates];
    rope_candidates(traditional ? K_ROPE_TRAD : K_ROPE_SPLIT, dtype, head_dim, aligned != 0,
                    rope_dims, list);
    Choice c;
    c.v = list[variant / 2];
    c.persistent = (variant % 2 == 0) != c.v->grid_first;
    describe_choice(c, buf, size_t(len));
    return ok();
}

const char* fnorm_status_string(int status) {
    switch (status) {
        case FNORM_OK: return "FNORM_OK";
        case FNORM_ERR_NULL: return "FNORM_ERR_NULL: required pointer is NULL";
        case FNORM_ERR_SHAPE: return "FNORM_ERR_SHAPE: invalid rows/width";
        case FNORM_ERR_EPS: return "FNORM_ERR_EPS: eps must be finite and >= 0";
        case FNORM_ERR_DTYPE: return "FNORM_ERR_DTYPE: unknown dtype";
        case FNORM_ERR_ALIAS: return "FNORM_ERR_ALIAS: output overlaps another buffer";
        case FNORM_ERR_UNSUPPORTED: return "FNORM_ERR_UNSUPPORTED: no kernel for this request";
        case FNORM_ERR_LAUNCH: return "FNORM_ERR_LAUNCH: HIP launch failed";
        case FNORM_ERR_WORKSPACE: return "FNORM_ERR_WORKSPACE: workspace missing, small or overlapping";
        default: return "unknown fnorm status";
    }
}

int64_t fnorm_composed_workspace_bytes(int op, int64_t rows, int64_t width) {
    if ((op != FNORM_OP_RMS && op != FNORM_OP_LAYER) || rows < 0 || width <= 0) return -1;
    if (rows > 0 && width > (INT64_MAX / 16) / rows) return -1;
    return composed::workspace_bytes(op == FNORM_OP_LAYER, rows, width);
}

static int run_composed(const char* op, bool layer, const void* x, const void* w, const void* b,
                        void* y, int64_t rows, int64_t width, float eps, int dtype,
                        void* workspace, int64_t workspace_bytes, void* stream) {
    if (int s = check_scalars(op, dtype, rows, width, eps)) return s;
    if (rows == 0) return ok();
    if (!x || !w || !y) return fail(FNORM_ERR_NULL, op, "x, w and y must be non-NULL");
    const int64_t eb = elem_bytes(dtype);
    const int64_t xb = rows * width * eb;
    if (y != x && overlap(y, xb, x, xb))
        return fail(FNORM_ERR_ALIAS, op, "y overlaps x without being equal to it");
    if (overlap(y, xb, w, width * eb) || overlap(y, xb, b, width * eb))
        return fail(FNORM_ERR_ALIAS, op, "y overlaps a weight");
    const int64_t need = composed::workspace_bytes(layer, rows, width);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need)
        return fail(FNORM_ERR_WORKSPACE, op, "workspace must be 16-byte aligned and hold %lld bytes",
                    (long long)need);
    if (overlap(workspace, need, x, xb) || overlap(workspace, need, y, xb) ||
        overlap(workspace, need, w, width * eb) || overlap(workspace, need, b, width * eb))
        return fail(FNORM_ERR_WORKSPACE, op, "workspace overlaps a tensor");
    const bool vec4 = width % 4 == 0 && aligned16(x) && aligned16(w) && aligned16(y) &&
                      (!b || aligned16(b));
    hipError_t e = composed::run(layer, x, w, b, y, rows, width, eps, dtype, vec4, workspace,
                                 device_cus(), stream);
    if (e != hipSuccess)
        return fail(FNORM_ERR_LAUNCH, op, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int fnorm_rms_composed(const void* x, const void* w, void* y, int64_t rows, int64_t width,
                       float eps, int dtype, void* workspace, int64_t workspace_bytes,
                       void* stream) {
    return run_composed("fnorm_rms_composed", false, x, w, nullptr, y, rows, width, eps, dtype,
                        workspace, workspace_bytes, stream);
}

int fnorm_rms_composed_noalloc(const void* x, const void* w, void* y, int64_t rows,
                               int64_t width, float eps, int dtype, void* stream) {
    static const char* op = "fnorm_rms_composed_noalloc";
    if (int s = check_scalars(op, dtype, rows, width, eps)) return s;
    if (rows == 0) return ok();
    const int64_t need = composed::workspace_bytes(false, rows, width);
    if (need > kNoAllocScratchBytes)
        return fail(FNORM_ERR_WORKSPACE, op,
                    "rows=%lld width=%lld need %lld bytes of fp32 intermediates; the static "
                    "scratch holds %lld (rows * width up to about %lld elements)",
                    (long long)rows, (long long)width, (long long)need,
                    (long long)kNoAllocScratchBytes, (long long)(kNoAllocScratchBytes / 4 - 4096));
    void* ws = nullptr;
    if (int s = noalloc_scratch(op, &ws)) return s;
    return run_composed(op, false, x, w, nullptr, y, rows, width, eps, dtype, ws,
                        kNoAllocScratchBytes, stream);
}

int fnorm_layer_composed(const void* x, const void* w, const void* b, void* y, int64_t rows,
                         int64_t width, float eps, int dtype, void* workspace,
                         int64_t workspace_bytes, void* stream) {
    return run_composed("fnorm_layer_composed", true, x, w, b, y, rows, width, eps, dtype,
                        workspace, workspace_bytes, stream);
}

const char* fnorm_last_error(void) { return g_err; }

int fnorm_version(void) { return kVersion; }

int fnorm_device_memory(int* clock_khz, int* bus_bits, int* compute_units) {
    static const char* op = "fnorm_device_memory";
    int dev = 0, clock = 0, bus = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&clock, hipDeviceAttributeMemoryClockRate, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&bus, hipDeviceAttributeMemoryBusWidth, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return fail(FNORM_ERR_LAUNCH, op, "device query failed: %s", hipGetErrorString(e));
    if (clock_khz) *clock_khz = clock;
    if (bus_bits) *bus_bits = bus;
    if (compute_units) *compute_units = cus;
    return ok();
}

int fnorm_bench_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    static const char* op = "fnorm_bench_copy";
    if (!src || !dst) return fail(FNORM_ERR_NULL, op, "src and dst must be non-NULL");
    if (bytes < 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
        return fail(FNORM_ERR_SHAPE, op, "bytes must be a multiple of 16, pointers 16-B aligned");
    if (overlap(src, bytes, dst, bytes)) return fail(FNORM_ERR_ALIAS, op, "src overlaps dst");
    if (bytes == 0) return ok();
    // Full grid, 4 packs per thread: the best plain-copy shape measured on
    // MI355X.
    constexpr int kBlock = 256, kU = 4;
    const void* fn = reinterpret_cast<const void*>(&copy16<kBlock, kU>);
    const int64_t n16 = bytes / 16;
    int64_t grid = (n16 + kBlock * kU - 1) / (kBlock * kU);
    if (grid > (int64_t(1) << 30)) grid = int64_t(1) << 30;
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    int64_t n = n16;
    void* args[] = {&s, &d, &n};
    const hipError_t e = hipLaunchKernel(fn, dim3(unsigned(grid)), dim3(kBlock), args, 0,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FNORM_ERR_LAUNCH, op, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
