// Sine and cosine of a rotary angle in fp64, without tables or calls.
//
// Cody and Waite's argument reduction (Software Manual for the Elementary
// Functions, 1980): k = nearest integer to x * 2/pi, r = x - k * pi/2 with
// pi/2 split into three pieces (the first two of 33 significant bits), each
// product taken exactly inside a fused multiply-add.  The first difference
// is then exact and r carries about one rounding; the split leaves 1e-37 of
// pi/2 unrepresented.  Then the Taylor series of sin and cos in r (truncation
// below 1e-17 for |r| < 1) and the quadrant k mod 4.  Valid for |x| < 2^50,
// where x * 2/pi is off by less than 1/4 and |r| < 1 (rotary angles are
// positions below 2^31 times frequencies of at most 1); infinities and NaN
// give NaN.  The library's sincos reduces large arguments through a table in
// memory and is a call, which costs a memory round trip and register saves in
// the decode launch that fuses the rotary step.
//
// Host and device code share it (tests/angle_check.cpp compares it with the
// C library over the angles a rotary embedding produces).
#pragma once

#include <math.h>

#include <hip/hip_runtime.h>

namespace sr {

// pi/2 = kPio2A + kPio2B + kPio2C (+ 1.0e-37); kPio2A and kPio2B are the first
// two 33-bit pieces of its binary expansion, kPio2C the rest rounded.
constexpr double kTwoOverPi = 0x1.45f306dc9c883p-1;
constexpr double kPio2A = 0x1.921fb544p+0;
constexpr double kPio2B = 0x1.0b4611a6p-34;
constexpr double kPio2C = 0x1.3198a2e037073p-69;

__host__ __device__ inline void angle_sincos(double x, double& s, double& c) {
    const double k = rint(x * kTwoOverPi);
    double r = fma(-k, kPio2A, x);
    r = fma(-k, kPio2B, r);
    r = fma(-k, kPio2C, r);
    const double z = r * r;
    // sin r = r (1 - z/3! + z^2/5! - ... + z^8/17!), cos r = 1 - z/2! + ... + z^9/18!
    double ps = 1.0 / 355687428096000.0;
    ps = fma(ps, z, -1.0 / 1307674368000.0);
    ps = fma(ps, z, 1.0 / 6227020800.0);
    ps = fma(ps, z, -1.0 / 39916800.0);
    ps = fma(ps, z, 1.0 / 362880.0);
    ps = fma(ps, z, -1.0 / 5040.0);
    ps = fma(ps, z, 1.0 / 120.0);
    ps = fma(ps, z, -1.0 / 6.0);
    ps = fma(ps * z, r, r);
    double pc = -1.0 / 6402373705728000.0;
    pc = fma(pc, z, 1.0 / 20922789888000.0);
    pc = fma(pc, z, -1.0 / 87178291200.0);
    pc = fma(pc, z, 1.0 / 479001600.0);
    pc = fma(pc, z, -1.0 / 3628800.0);
    pc = fma(pc, z, 1.0 / 40320.0);
    pc = fma(pc, z, -1.0 / 720.0);
    pc = fma(pc, z, 1.0 / 24.0);
    pc = fma(pc, z, -0.5);
    pc = fma(pc, z, 1.0);
    const int q = static_cast<int>(static_cast<long long>(k) & 3);
    s = q == 0 ? ps : (q == 1 ? pc : (q == 2 ? -ps : -pc));
    c = q == 0 ? pc : (q == 1 ? -ps : (q == 2 ? -pc : ps));
}

}  // namespace sr
