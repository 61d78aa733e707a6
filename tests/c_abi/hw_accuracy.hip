// Accuracy of the gfx950 instructions the error bounds of the tests rely on,
// measured exhaustively on the device:
//   v_sin_f32 / v_cos_f32 (argument in turns): largest absolute error over
//     every fp32 argument in [-1/2, 1/2], against fp64 sinpi / cospi of 2f;
//   v_rsq_f32: largest relative error over every fp32 in [1, 4) (one period
//     of the exponent's parity; other binades scale by powers of two),
//     against fp64 1 / sqrt.
// Prints "sin <err>", "cos <err>", "rsq <err>" (one per line); exit status 0
// on success.  Each workgroup writes its maxima to its own slots of a
// device array sized to the grid.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

constexpr int kBlock = 256;
constexpr int kGrid = 2048;

__global__ __launch_bounds__(kBlock) void accuracy(double* out) {
    __shared__ double sm[3][kBlock];
    double es = 0.0, ec = 0.0, er = 0.0;
    const uint32_t npos = 0x3F000001u;   // fp32 bit patterns 0 .. 0.5
    const uint64_t total = 2ull * npos;  // and their negatives
    for (uint64_t i = uint64_t(blockIdx.x) * kBlock + threadIdx.x; i < total;
         i += uint64_t(kGrid) * kBlock) {
        const uint32_t bits = i < npos ? uint32_t(i) : (0x80000000u | uint32_t(i - npos));
        const float f = __builtin_bit_cast(float, bits);
        const double t = 2.0 * double(f);
        es = fmax(es, fabs(double(__builtin_amdgcn_sinf(f)) - sinpi(t)));
        ec = fmax(ec, fabs(double(__builtin_amdgcn_cosf(f)) - cospi(t)));
    }
    for (uint32_t b = 0x3F800000u + blockIdx.x * kBlock + threadIdx.x; b < 0x40800000u;
         b += kGrid * kBlock) {
        const float v = __builtin_bit_cast(float, b);
        const double ref = 1.0 / sqrt(double(v));
        er = fmax(er, fabs(double(__builtin_amdgcn_rsqf(v)) - ref) / ref);
    }
    sm[0][threadIdx.x] = es;
    sm[1][threadIdx.x] = ec;
    sm[2][threadIdx.x] = er;
    __syncthreads();
    if (threadIdx.x < 3) {
        double m = 0.0;
        for (int k = 0; k < kBlock; ++k) m = fmax(m, sm[threadIdx.x][k]);
        out[blockIdx.x * 3 + threadIdx.x] = m;
    }
}

int main() {
    double* d = nullptr;
    if (hipMalloc(&d, sizeof(double) * 3 * kGrid) != hipSuccess) return 1;
    hipLaunchKernelGGL(accuracy, dim3(kGrid), dim3(kBlock), 0, 0, d);
    if (hipDeviceSynchronize() != hipSuccess) return 2;
    static double h[3 * kGrid];
    if (hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return 3;
    double m[3] = {0.0, 0.0, 0.0};
    for (int i = 0; i < kGrid; ++i)
        for (int k = 0; k < 3; ++k) m[k] = fmax(m[k], h[i * 3 + k]);
    printf("sin %.9e\ncos %.9e\nrsq %.9e\n", m[0], m[1], m[2]);
    return hipFree(d) == hipSuccess ? 0 : 4;
}
