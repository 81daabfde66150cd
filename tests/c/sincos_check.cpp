// Host build of the device header qkv_sincos.h (sincos_rope), checked against
// the C library: for every angle, f32(sin((double)a)) and f32(cos((double)a))
// -- the values the oracle takes -- against sincos_rope's two results.
// Angle sets (argv[1]):
//   rope     f32(pos * inv[i]) for pos < 65536 and the inverse-frequency
//            tables of theta 1e6 (head_dim 128 and 64) and 1e4 (128);
//   random   4M angles uniform in (-2^20, 2^20), seeded;
//   quadrant the f32 values nearest k*pi/2 and their neighbours, k < 667544
//            (the arguments where the reduction cancels most).
// Prints: angles checked, mismatching values, largest difference in f32 ulps.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

#include "qkv_sincos.h"

using qkv_detail::sincos_rope;

static long long g_n, g_bad;
static int g_maxulp;

static int ulps(float x, float y)
{
    int32_t a, b;
    std::memcpy(&a, &x, 4);
    std::memcpy(&b, &y, 4);
    if (a < 0) a = INT32_MIN - a;
    if (b < 0) b = INT32_MIN - b;
    const long long d = (long long)a - (long long)b;
    return (int)(d < 0 ? -d : d);
}

static void check(float a)
{
    float s, c;
    sincos_rope(a, s, c);
    const float ws = (float)std::sin((double)a), wc = (float)std::cos((double)a);
    ++g_n;
    const int us = ulps(s, ws), uc = ulps(c, wc);
    if (us || uc) {
        ++g_bad;
        if (us > g_maxulp) g_maxulp = us;
        if (uc > g_maxulp) g_maxulp = uc;
    }
}

int main(int argc, char **argv)
{
    const char *mode = argc > 1 ? argv[1] : "rope";
    if (!std::strcmp(mode, "rope")) {
        const struct { double theta; int hd; } tabs[] = {{1e6, 128}, {1e6, 64}, {1e4, 128}};
        for (const auto &t : tabs) {
            for (int i = 0; i < t.hd / 2; ++i) {
                const float inv = (float)std::pow(t.theta, -(double)(2 * i) / (double)t.hd);
                for (int p = 0; p < 65536; ++p)
                    check((float)p * inv);
            }
        }
    } else if (!std::strcmp(mode, "random")) {
        std::mt19937_64 g(12345);
        std::uniform_real_distribution<float> u(-1048575.0f, 1048575.0f);
        for (int i = 0; i < 4000000; ++i)
            check(u(g));
    } else {
        const double half_pi = 1.5707963267948966;
        for (int k = 0; k < 667544; ++k) {
            const float a = (float)(k * half_pi);
            if (!(std::fabs(a) < 1048576.0f))
                break;
            check(a);
            check(std::nextafter(a, 0.0f));
            check(std::nextafter(a, 2e6f));
        }
    }
    std::printf("%s %lld %lld %d\n", mode, g_n, g_bad, g_maxulp);
    return 0;
}
