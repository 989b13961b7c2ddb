// Host check of libmrope's sincos_angle (canvas_rope_rotary_amd/csrc/mrope_math.h) against
// long-double libm: every angle fl32(fl32(pos) * inv_freq[j]) for pos in [-1, 65536) and the 32
// frequencies of theta = 1e7, plus pseudo-random positions up to 2^24.  Prints the max abs error
// of sin and of cos, and the angle of the worst sin.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "../../canvas_rope_rotary_amd/csrc/mrope_math.h"

int main(int argc, char **argv)
{
    double theta = argc > 1 ? atof(argv[1]) : 1e7;
    float inv[32];
    for (int j = 0; j < 32; ++j) inv[j] = 1.0f / (float)pow(theta, (2.0 * j) / 64.0);
    long double worst_s = 0, worst_c = 0;
    float worst_a = 0;
    auto check = [&](int32_t pos) {
        for (int j = 0; j < 32; ++j) {
            float a = (float)pos * inv[j];
            double s, c;
            mrope::sincos_angle(a, &s, &c);
            long double es = fabsl((long double)s - sinl((long double)a));
            long double ec = fabsl((long double)c - cosl((long double)a));
            if (es > worst_s) { worst_s = es; worst_a = a; }
            if (ec > worst_c) worst_c = ec;
        }
    };
    for (int32_t p = -1; p < 65536; ++p) check(p);
    uint64_t x = 0x9E3779B97F4A7C15ull;
    for (int i = 0; i < 200000; ++i) {
        x ^= x << 13; x ^= x >> 7; x ^= x << 17;
        check((int32_t)(x % (1u << 24)));
        check(-(int32_t)(x % 70000u));
    }
    printf("%.3Le %.3Le %.9g\n", worst_s, worst_c, worst_a);
    return 0;
}
