// Scalar math of the rotary step, shared by every kernel of libmrope.
//
// sincos of an fp32 angle, in double.  The rotary angle a = fl32(fl32(pos) * inv_freq[j]) reaches
// ~3.3e4 rad at the longest prompts (|pos| < 2^24 is supported), so the hardware's v_sin/v_cos
// (which scale by 1/(2*pi) in fp32 first) are far too coarse; and a rotated element can cancel to a
// value many orders of magnitude below its inputs, where only an absolute error near 1e-16 keeps the
// result within one bf16 ulp.  On this chip (packed fp32 disabled) a double FMA issues at the same
// per-lane rate as an fp32 one, so the whole rotation is done in double.
//
// Method: Cody & Waite argument reduction ("Software Manual for the Elementary Functions", 1980) --
// k = nearest integer to a * 2/pi, r = a - k*(pi/2) with pi/2 split into two doubles and fused
// multiply-adds, leaving r in [-pi/4, pi/4] with an error near 1e-16 -- then truncated Taylor series
// of sin (to r^15) and cos (to r^16), whose truncation error is below 5e-17 on that interval; the
// quadrant k mod 4 picks and signs the pair.
//
// The header also compiles as plain C++ on the host so the same function can be checked on the CPU
// against long-double libm over every angle the rotary produces.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define MROPE_HD __host__ __device__ __forceinline__
#else
#define MROPE_HD static inline
#endif

namespace mrope {

// pi/2 = kPio2Hi + kPio2Lo (kPio2Hi = pi/2 rounded to double, kPio2Lo = the rest rounded to double).
constexpr double kTwoOverPi = 0.63661977236758134307553505349006;
constexpr double kPio2Hi = 1.5707963267948966192313216916398;
constexpr double kPio2Lo = 6.1232339957367658e-17;

// Taylor coefficients (-1)^n / (2n+1)! and (-1)^n / (2n)!.
constexpr double kS3 = -1.0 / 6.0;
constexpr double kS5 = 1.0 / 120.0;
constexpr double kS7 = -1.0 / 5040.0;
constexpr double kS9 = 1.0 / 362880.0;
constexpr double kS11 = -1.0 / 39916800.0;
constexpr double kS13 = 1.0 / 6227020800.0;
constexpr double kS15 = -1.0 / 1307674368000.0;
constexpr double kC2 = -0.5;
constexpr double kC4 = 1.0 / 24.0;
constexpr double kC6 = -1.0 / 720.0;
constexpr double kC8 = 1.0 / 40320.0;
constexpr double kC10 = -1.0 / 3628800.0;
constexpr double kC12 = 1.0 / 479001600.0;
constexpr double kC14 = -1.0 / 87178291200.0;
constexpr double kC16 = 1.0 / 20922789888000.0;

MROPE_HD void sincos_angle(float a, double *s_out, double *c_out)
{
    const double ad = (double)a;
    const double kd = __builtin_rint(ad * kTwoOverPi);
    double r = __builtin_fma(-kd, kPio2Hi, ad);
    r = __builtin_fma(-kd, kPio2Lo, r);
    const int quad = (int)kd & 3;
    const double r2 = r * r;

    double sp = __builtin_fma(r2, kS15, kS13);
    sp = __builtin_fma(r2, sp, kS11);
    sp = __builtin_fma(r2, sp, kS9);
    sp = __builtin_fma(r2, sp, kS7);
    sp = __builtin_fma(r2, sp, kS5);
    sp = __builtin_fma(r2, sp, kS3);
    sp = __builtin_fma(r * r2, sp, r);

    double cp = __builtin_fma(r2, kC16, kC14);
    cp = __builtin_fma(r2, cp, kC12);
    cp = __builtin_fma(r2, cp, kC10);
    cp = __builtin_fma(r2, cp, kC8);
    cp = __builtin_fma(r2, cp, kC6);
    cp = __builtin_fma(r2, cp, kC4);
    cp = __builtin_fma(r2, cp, kC2);
    cp = __builtin_fma(r2, cp, 1.0);

    // a = r + k*pi/2:  k=0 (s, c)  k=1 (c, -s)  k=2 (-s, -c)  k=3 (-c, s)
    double sv = (quad & 1) ? cp : sp;
    double cv = (quad & 1) ? sp : cp;
    if (quad & 2) sv = -sv;
    if ((quad + 1) & 2) cv = -cv;
    *s_out = sv;
    *c_out = cv;
}

}  // namespace mrope
