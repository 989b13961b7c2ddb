// Scalar math of the rotary step, shared by every kernel of libmrope.
//
// sincos of an fp32 angle.  The rotary angle a = fl32(fl32(pos) * inv_freq[j]) reaches ~3.3e4 rad
// at the longest prompts (|pos| < 2^24 is supported), so the hardware's v_sin/v_cos (which scale by
// 1/(2*pi) in fp32 first) are far too coarse.  Method: Cody & Waite argument reduction ("Software
// Manual for the Elementary Functions", 1980) carried out in double -- k = nearest integer to
// a * 2/pi, r = a - k*(pi/2) with pi/2 split into two doubles and fused multiply-adds -- which leaves
// r in [-pi/4, pi/4] with an error near 1e-16; then truncated Taylor series for sin (to r^9) and
// cos (to r^10) in fp32 (truncation error below 2e-9 on that interval), and the quadrant k mod 4
// picks and signs the pair.  Result: within ~1.5 fp32 ulp of the exact sin/cos of the fp32 angle.
//
// The header also compiles as plain C++ on the host so the same function can be checked on the CPU
// against double libm over every angle the rotary produces.
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
constexpr float kS3 = (float)(-1.0 / 6.0);
constexpr float kS5 = (float)(1.0 / 120.0);
constexpr float kS7 = (float)(-1.0 / 5040.0);
constexpr float kS9 = (float)(1.0 / 362880.0);
constexpr float kC2 = -0.5f;
constexpr float kC4 = (float)(1.0 / 24.0);
constexpr float kC6 = (float)(-1.0 / 720.0);
constexpr float kC8 = (float)(1.0 / 40320.0);
constexpr float kC10 = (float)(-1.0 / 3628800.0);

MROPE_HD void sincos_angle(float a, float *s_out, float *c_out)
{
    const double ad = (double)a;
    const double kd = __builtin_rint(ad * kTwoOverPi);
    double rd = __builtin_fma(-kd, kPio2Hi, ad);
    rd = __builtin_fma(-kd, kPio2Lo, rd);
    const float r = (float)rd;
    const int quad = (int)kd & 3;
    const float r2 = r * r;

    float sp = __builtin_fmaf(r2, kS9, kS7);
    sp = __builtin_fmaf(r2, sp, kS5);
    sp = __builtin_fmaf(r2, sp, kS3);
    sp = __builtin_fmaf(r * r2, sp, r);

    float cp = __builtin_fmaf(r2, kC10, kC8);
    cp = __builtin_fmaf(r2, cp, kC6);
    cp = __builtin_fmaf(r2, cp, kC4);
    cp = __builtin_fmaf(r2, cp, kC2);
    cp = __builtin_fmaf(r2, cp, 1.0f);

    // a = r + k*pi/2:  k=0 (s, c)  k=1 (c, -s)  k=2 (-s, -c)  k=3 (-c, s)
    float sv = (quad & 1) ? cp : sp;
    float cv = (quad & 1) ? sp : cp;
    if (quad & 2) sv = -sv;
    if ((quad + 1) & 2) cv = -cv;
    *s_out = sv;
    *c_out = cv;
}

}  // namespace mrope
