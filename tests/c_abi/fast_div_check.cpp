// Host check of the invariant-divisor division the fused RoPE kernel uses to
// find a row's token (FastDiv in fnorm_device.hpp, the same source the
// kernels compile): against plain integer division for every divisor up to
// 4096 and a spread of others, at the numerators around each multiple of the
// divisor, exhaustively below 2^20 for small divisors, and at the top of the
// 32-bit range.  Prints "ok" and exits 0, or the first mismatch and exits 1.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../transformer_row_normalization_amd/csrc/fnorm_device.hpp"

static int check(uint32_t d, uint32_t n) {
    const uint32_t q = fnorm::make_fast_div(d).div(n);
    if (q != n / d) {
        std::printf("mismatch: %u / %u = %u, fast %u\n", n, d, n / d, q);
        return 1;
    }
    return 0;
}

int main() {
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d <= 4096; ++d) ds.push_back(d);
    for (uint64_t d = 4097; d < (uint64_t(1) << 32); d = d * 3 + 7) ds.push_back(uint32_t(d));
    for (int k = 12; k < 32; ++k) {
        ds.push_back((1u << k) - 1);
        ds.push_back(1u << k);
        ds.push_back((1u << k) + 1);
    }
    uint64_t s = 0x9e3779b97f4a7c15ull;
    for (uint32_t d : ds) {
        const fnorm::FastDiv f = fnorm::make_fast_div(d);
        (void)f;
        // around multiples of d: k d - 1, k d, k d + 1 for spread-out k
        for (uint64_t k = 0; k * d <= 0xffffffffull; k = k < 64 ? k + 1 : k * 2 + 1) {
            const uint64_t b = k * d;
            for (int e = -1; e <= 1; ++e) {
                const int64_t n = int64_t(b) + e;
                if (n >= 0 && n <= 0xffffffffll && check(d, uint32_t(n))) return 1;
            }
        }
        for (int i = 0; i < 64; ++i) {   // pseudo-random numerators
            s = s * 6364136223846793005ull + 1442695040888963407ull;
            if (check(d, uint32_t(s >> 32))) return 1;
        }
        for (uint32_t n = 0xffffffffu - 64; n != 0; ++n)
            if (check(d, n)) return 1;
    }
    for (uint32_t d = 1; d <= 64; ++d)
        for (uint32_t n = 0; n < (1u << 20); ++n)
            if (check(d, n)) return 1;
    std::printf("ok\n");
    return 0;
}
