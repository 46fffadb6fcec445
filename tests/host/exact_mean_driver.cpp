// Host build of the library's exact-mean rounding (quantized_gemv_amd/csrc/
// exact_mean.h) for CPU tests: reads little-endian fp32 values from stdin
// (first a uint64 count of groups, then per group a uint64 length and the
// values) and prints, per group, the fp32 bit pattern of the mean of |x|.
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../quantized_gemv_amd/csrc/exact_mean.h"

int main() {
    uint64_t groups = 0;
    if (fread(&groups, 8, 1, stdin) != 1) return 2;
    for (uint64_t g = 0; g < groups; ++g) {
        uint64_t n = 0;
        if (fread(&n, 8, 1, stdin) != 1) return 2;
        std::vector<float> v(n);
        if (n && fread(v.data(), 4, n, stdin) != n) return 2;
        uint64_t hist[256];
        memset(hist, 0, sizeof(hist));
        for (float x : v) {
            uint32_t sh, m;
            qg::abs_binade(x, sh, m);
            hist[sh] += m;
        }
        const float r = qg::round_mean_from_binades(hist, n);
        uint32_t bits;
        memcpy(&bits, &r, 4);
        printf("%u\n", bits);
    }
    return 0;
}
