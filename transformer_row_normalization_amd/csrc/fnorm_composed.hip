// Composed (unfused) RMSNorm and LayerNorm: one primitive per launch, each
// launch reading its operands from HBM and writing its result back, the way
// a framework runs the textbook formula op by op.  This is the baseline the
// fused kernels are compared with, not a hot path.
//
//   RMSNorm (the composed cell of the Emily notebook, Part 1):
//     sq = x^2;  ms = mean_row(sq);  t = ms + eps;  r = sqrt(t);
//     q = x / r;  y = q * w                                  (6 launches)
//   LayerNorm (the definition in the Emily.Fast docs, `layer_norm`, one
//   primitive per launch):
//     m = mean_row(x);  xc = x - m;  s = xc^2;  v = mean_row(s);
//     t = v + eps;  r = sqrt(t);  xn = xc / r;  y = xn * w (+ b)
//                                                 (9 launches, 8 without b)
//
// Intermediates are fp32 (in a caller-provided workspace), so the chain
// computes the same function as the fused kernels, up to rounding; the
// output has the input's type.  Division and square root are IEEE
// correctly rounded (HIP's default for fp32).
#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

#include "fnorm_composed.hpp"
#include "fnorm_device.hpp"

namespace fnorm {
namespace composed {

enum : int { MAP_SQUARE = 0, MAP_SUB_ROW = 1, MAP_DIV_ROW = 2, MAP_MUL_COL = 3, MAP_ADD_COL = 4 };
enum : int { SC_ADD = 0, SC_SQRT = 1 };

constexpr int kBlock = 256;

template <int DT, int VEC>
__device__ __forceinline__ void load_f32(const void* base, int64_t idx, float (&f)[VEC]) {
    const auto r = load_raw<DT, VEC, false>(base, idx);
#pragma unroll
    for (int i = 0; i < VEC; ++i) f[i] = elem<DT, VEC>(r, i);
}

template <int DT, int VEC>
__device__ __forceinline__ void store_f32(void* base, int64_t idx, const float (&f)[VEC]) {
    store_raw<DT, VEC, false>(base, idx, make_raw<DT, VEC>(f));
}

// o[r, c] = f(a[r, c], rowv[r], colv[c]); one workgroup per row at a time.
template <int MAP, int DTA, int DTC, int DTO, int VEC>
__global__ __launch_bounds__(kBlock) void map_rows(const void* a, const float* rowv,
                                                   const void* colv, void* o, int64_t rows,
                                                   int64_t width) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const int64_t off = r * width;
        const float rv = (MAP == MAP_SUB_ROW || MAP == MAP_DIV_ROW) ? rowv[r] : 0.0f;
        for (int64_t c = int64_t(threadIdx.x) * VEC; c < width; c += int64_t(kBlock) * VEC) {
            float va[VEC], vc[VEC], vo[VEC];
            load_f32<DTA, VEC>(a, off + c, va);
            if constexpr (MAP == MAP_MUL_COL || MAP == MAP_ADD_COL) load_f32<DTC, VEC>(colv, c, vc);
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                if constexpr (MAP == MAP_SQUARE) vo[i] = va[i] * va[i];
                else if constexpr (MAP == MAP_SUB_ROW) vo[i] = va[i] - rv;
                else if constexpr (MAP == MAP_DIV_ROW) vo[i] = va[i] / rv;
                else if constexpr (MAP == MAP_MUL_COL) vo[i] = va[i] * vc[i];
                else vo[i] = va[i] + vc[i];
            }
            store_f32<DTO, VEC>(o, off + c, vo);
        }
    }
}

// out[r] = mean over the row of a; fixed-order per-thread sums, then an LDS
// tree, so the result is deterministic.
template <int DTA, int VEC>
__global__ __launch_bounds__(kBlock) void row_mean(const void* a, float* out, int64_t rows,
                                                   int64_t width) {
    __shared__ float part[kBlock];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const int64_t off = r * width;
        float s = 0.0f;
        for (int64_t c = int64_t(threadIdx.x) * VEC; c < width; c += int64_t(kBlock) * VEC) {
            float va[VEC];
            load_f32<DTA, VEC>(a, off + c, va);
#pragma unroll
            for (int i = 0; i < VEC; ++i) s += va[i];
        }
        part[threadIdx.x] = s;
        __syncthreads();
        for (int h = kBlock / 2; h > 0; h >>= 1) {
            if (int(threadIdx.x) < h) part[threadIdx.x] += part[threadIdx.x + h];
            __syncthreads();
        }
        if (threadIdx.x == 0) out[r] = part[0] / static_cast<float>(width);
        __syncthreads();
    }
}

// Per-row scalars: SC_ADD: o = v + eps;  SC_SQRT: o = sqrt(v).
template <int SC>
__global__ __launch_bounds__(kBlock) void row_scalar(const float* v, float* o, float eps,
                                                     int64_t rows) {
    for (int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x; i < rows;
         i += int64_t(gridDim.x) * kBlock)
        o[i] = SC == SC_ADD ? v[i] + eps : __builtin_sqrtf(v[i]);
}

}  // namespace composed
}  // namespace fnorm

// ------------------------------------------------------------------ host
namespace fnorm {
namespace composed {
namespace {

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

struct Launch {
    hipStream_t stream;
    int64_t rows, width;
    int grid_rows;      // workgroups for per-row kernels
    int grid_scalar;    // workgroups for per-row scalar kernels
    hipError_t err = hipSuccess;

    // The launch's own status (the thread's last-error slot may hold an
    // earlier, unrelated failure).  The arguments are converted to the
    // kernel's parameter types before their addresses are passed.
    template <typename... P, typename... A>
    void go(void (*kernel)(P...), int grid, A... args) {
        if (err != hipSuccess) return;
        launch(kernel, grid, std::tuple<P...>(args...), std::index_sequence_for<P...>{});
    }
    template <typename... P, size_t... I>
    void launch(void (*kernel)(P...), int grid, std::tuple<P...> t, std::index_sequence<I...>) {
        void* pa[] = {static_cast<void*>(&std::get<I>(t))...};
        err = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(unsigned(grid)),
                              dim3(kBlock), pa, 0, stream);
    }
};

template <int DT, int VEC>
hipError_t rms_chain(Launch& L, const void* x, const void* w, void* y, float eps, char* ws) {
    const int64_t n = L.rows * L.width;
    float* tmp = reinterpret_cast<float*>(ws);
    float* ms = reinterpret_cast<float*>(ws + align_up(n * 4));
    float* t = ms + align_up(L.rows * 4) / 4;
    float* r = t + align_up(L.rows * 4) / 4;
    L.go(map_rows<MAP_SQUARE, DT, DT, DT_F32, VEC>, L.grid_rows, x, (const float*)nullptr,
         (const void*)nullptr, (void*)tmp, L.rows, L.width);
    L.go(row_mean<DT_F32, VEC>, L.grid_rows, (const void*)tmp, ms, L.rows, L.width);
    L.go(row_scalar<SC_ADD>, L.grid_scalar, (const float*)ms, t, eps, L.rows);
    L.go(row_scalar<SC_SQRT>, L.grid_scalar, (const float*)t, r, 0.0f, L.rows);
    L.go(map_rows<MAP_DIV_ROW, DT, DT, DT_F32, VEC>, L.grid_rows, x, (const float*)r,
         (const void*)nullptr, (void*)tmp, L.rows, L.width);
    L.go(map_rows<MAP_MUL_COL, DT_F32, DT, DT, VEC>, L.grid_rows, (const void*)tmp,
         (const float*)nullptr, w, y, L.rows, L.width);
    return L.err;
}

template <int DT, int VEC>
hipError_t layer_chain(Launch& L, const void* x, const void* w, const void* b, void* y,
                       float eps, char* ws) {
    const int64_t n = L.rows * L.width;
    float* ta = reinterpret_cast<float*>(ws);
    float* tb = reinterpret_cast<float*>(ws + align_up(n * 4));
    float* m = reinterpret_cast<float*>(ws + 2 * align_up(n * 4));
    const int64_t rs = align_up(L.rows * 4) / 4;
    float* v = m + rs;
    float* t = v + rs;
    float* r = t + rs;
    const float* nil = nullptr;
    L.go(row_mean<DT, VEC>, L.grid_rows, x, m, L.rows, L.width);
    L.go(map_rows<MAP_SUB_ROW, DT, DT, DT_F32, VEC>, L.grid_rows, x, (const float*)m,
         (const void*)nullptr, (void*)ta, L.rows, L.width);
    L.go(map_rows<MAP_SQUARE, DT_F32, DT, DT_F32, VEC>, L.grid_rows, (const void*)ta, nil,
         (const void*)nullptr, (void*)tb, L.rows, L.width);
    L.go(row_mean<DT_F32, VEC>, L.grid_rows, (const void*)tb, v, L.rows, L.width);
    L.go(row_scalar<SC_ADD>, L.grid_scalar, (const float*)v, t, eps, L.rows);
    L.go(row_scalar<SC_SQRT>, L.grid_scalar, (const float*)t, r, 0.0f, L.rows);
    L.go(map_rows<MAP_DIV_ROW, DT_F32, DT, DT_F32, VEC>, L.grid_rows, (const void*)ta,
         (const float*)r, (const void*)nullptr, (void*)tb, L.rows, L.width);
    if (b) {
        L.go(map_rows<MAP_MUL_COL, DT_F32, DT, DT_F32, VEC>, L.grid_rows, (const void*)tb, nil,
             w, (void*)ta, L.rows, L.width);
        L.go(map_rows<MAP_ADD_COL, DT_F32, DT, DT, VEC>, L.grid_rows, (const void*)ta, nil, b,
             y, L.rows, L.width);
    } else {
        L.go(map_rows<MAP_MUL_COL, DT_F32, DT, DT, VEC>, L.grid_rows, (const void*)tb, nil, w,
             y, L.rows, L.width);
    }
    return L.err;
}

}  // namespace

int64_t workspace_bytes(bool layer, int64_t rows, int64_t width) {
    const int64_t n = rows * width;
    return (layer ? 2 : 1) * align_up(n * 4) + (layer ? 4 : 3) * align_up(rows * 4);
}

hipError_t run(bool layer, const void* x, const void* w, const void* b, void* y, int64_t rows,
               int64_t width, float eps, int dtype, bool vec4, void* workspace, int cus,
               void* stream) {
    Launch L{static_cast<hipStream_t>(stream), rows, width, 0, 0};
    L.grid_rows = int(rows < int64_t(cus) * 8 ? rows : int64_t(cus) * 8);
    const int64_t gs = (rows + kBlock - 1) / kBlock;
    L.grid_scalar = int(gs < int64_t(cus) * 4 ? gs : int64_t(cus) * 4);
    char* ws = static_cast<char*>(workspace);
    if (dtype == DT_F32) {
        if (layer) return vec4 ? layer_chain<DT_F32, 4>(L, x, w, b, y, eps, ws)
                               : layer_chain<DT_F32, 1>(L, x, w, b, y, eps, ws);
        return vec4 ? rms_chain<DT_F32, 4>(L, x, w, y, eps, ws) : rms_chain<DT_F32, 1>(L, x, w, y, eps, ws);
    }
    if (dtype == DT_F16) {
        if (layer) return vec4 ? layer_chain<DT_F16, 4>(L, x, w, b, y, eps, ws)
                               : layer_chain<DT_F16, 1>(L, x, w, b, y, eps, ws);
        return vec4 ? rms_chain<DT_F16, 4>(L, x, w, y, eps, ws)
                    : rms_chain<DT_F16, 1>(L, x, w, y, eps, ws);
    }
    if (layer) return vec4 ? layer_chain<DT_BF16, 4>(L, x, w, b, y, eps, ws)
                           : layer_chain<DT_BF16, 1>(L, x, w, b, y, eps, ws);
    return vec4 ? rms_chain<DT_BF16, 4>(L, x, w, y, eps, ws) : rms_chain<DT_BF16, 1>(L, x, w, y, eps, ws);
}

}  // namespace composed
}  // namespace fnorm
