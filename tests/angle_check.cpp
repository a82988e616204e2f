// Host check of sr::angle_sincos (kv_cache_routing_amd/csrc/angle.h) against
// the C library's sin and cos, built and run by tests/test_host_sanitizers.py.
// Angles are those of a rotary embedding: positions up to 2^31 - 1 times
// frequencies base^(-2i/d) (fp32), plus random arguments up to 2^30 and up
// to 2^50 (the stated range) and the quadrant boundaries.  Prints the largest
// absolute error and fails above 4e-16 (sin and cos lie in [-1, 1]); checks
// that infinities and NaN give NaN.
#include <cmath>
#include <cstdio>
#include <random>

#include "angle.h"

int main() {
    double worst = 0.0, worst_x = 0.0;
    auto check = [&](double x) {
        double s, c;
        sr::angle_sincos(x, s, c);
        const double e = std::fmax(std::fabs(s - std::sin(x)), std::fabs(c - std::cos(x)));
        if (!(e <= worst)) {
            worst = e;
            worst_x = x;
        }
    };
    for (int d : {64, 128}) {
        for (int i = 0; i < d / 2; ++i) {
            const float f = static_cast<float>(std::pow(500000.0, -2.0 * i / d));
            for (long long pos = 0; pos < 600000; pos += 7) check(static_cast<double>(pos) * f);
            for (long long pos = 2147483647LL; pos > 2147000000LL; pos -= 997)
                check(static_cast<double>(pos) * f);
        }
    }
    std::mt19937_64 rng(7);
    std::uniform_real_distribution<double> u(-1073741823.0, 1073741823.0);
    for (int n = 0; n < 2000000; ++n) check(u(rng));
    for (long long k = -100000; k <= 100000; ++k) {  // near multiples of pi/4
        const double x = static_cast<double>(k) * 0.78539816339744830962;
        check(x);
        check(std::nextafter(x, 0.0));
        check(std::nextafter(x, 1e300));
    }
    std::uniform_real_distribution<double> wide(-0x1p50, 0x1p50);
    for (int n = 0; n < 200000; ++n) check(wide(rng));
    for (double x : {0.0, -0.0, 1e-300, 0x1p30, -0x1p30, 3e9, 1e15, 0x1p50 - 1.0}) check(x);
    for (double x : {INFINITY, -INFINITY, NAN}) {
        double s, c;
        sr::angle_sincos(x, s, c);
        if (!std::isnan(s) || !std::isnan(c)) {
            std::printf("angle_sincos: %g does not give NaN\n", x);
            return 1;
        }
    }
    std::printf("angle_sincos: max abs error %.3g at x = %.17g\n", worst, worst_x);
    return worst <= 4e-16 ? 0 : 1;
}
