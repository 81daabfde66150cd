// qkv_sincos.h -- sin and cos of an f32 rope angle, evaluated in double
// precision and rounded once to f32, for |angle| < 2^20.
//
// The rope angle pos * inv[i] (page "73 · D3-8 — G4 FusedQKV ported to CUDA",
// §3.2 Excerpt A) is an f32 value; cos and sin of it are taken in double and
// rounded to f32, so that they agree with the correctly rounded values except
// where the double result lies within its own error of an f32 rounding
// boundary (about 2^-28 of the values, a 1-ulp difference of c or s).  The
// general double-precision library routine spends most of its time on
// argument ranges and special cases a rope angle never reaches; this one
// covers |a| < 2^20 (positions below 2^20 at any frequency <= 1) in a short
// dependent chain, and the caller keeps the library routine for the rest.
//
//   reduction  a = k * pi/2 + r, k = nearest integer to a * 2/pi, with pi/2
//              split as P1 + P2 + P3 (P1, P2 of 33 significant bits): for
//              |a| < 2^20, |k| < 2^20, so k*P1 and k*P2 are exact in double
//              and r carries the rounding of two fused multiply-adds only;
//   series     the Taylor series of sin r to degree 15 and of cos r to degree
//              16: on |r| <= pi/4 the first omitted terms, r^17/17! and
//              r^18/18!, are below 2^-54 and 2^-58 of the result; each is a
//              polynomial in z = r^2 evaluated by Estrin's scheme (pairs of
//              coefficients combined with z, then z^2, then z^4), which keeps
//              the chain of dependent operations at four after z;
//   quadrant   k mod 4 selects (sin r, cos r), (cos r, -sin r), (-sin r,
//              -cos r) or (-cos r, sin r).
//
// The constants are the double values of pi/2's parts and of 1/n!, computed
// from a 60-digit pi and exact rationals.  Every operation is written out
// (fma calls, no contraction left to the compiler), so a host build computes
// the same bits as the device code; the CPU tests compare such a build with
// the C library's sin and cos over the angles the workloads use.

#ifndef QKV_SINCOS_H
#define QKV_SINCOS_H

#include <cmath>
#include <cstdint>

namespace qkv_detail {

constexpr float kSincosRange = 1048576.0f;  // 2^20

// pi/2 = kP1 + kP2 + kP3 (+ 1.0e-37)
constexpr double kP1 = 0x1.921fb54400000p+0;
constexpr double kP2 = 0x1.0b4611a600000p-34;
constexpr double kP3 = 0x1.3198a2e037073p-69;
constexpr double kTwoOverPi = 0x1.45f306dc9c883p-1;

// +-1/n!
constexpr double kS3 = -0x1.5555555555555p-3, kS5 = 0x1.1111111111111p-7,
                 kS7 = -0x1.a01a01a01a01ap-13, kS9 = 0x1.71de3a556c734p-19,
                 kS11 = -0x1.ae64567f544e4p-26, kS13 = 0x1.6124613a86d09p-33,
                 kS15 = -0x1.ae7f3e733b81fp-41;
constexpr double kC2 = -0x1.0000000000000p-1, kC4 = 0x1.5555555555555p-5,
                 kC6 = -0x1.6c16c16c16c17p-10, kC8 = 0x1.a01a01a01a01ap-16,
                 kC10 = -0x1.27e4fb7789f5cp-22, kC12 = 0x1.1eed8eff8d898p-29,
                 kC14 = -0x1.93974a8c07c9dp-37, kC16 = 0x1.ae7f3e733b81fp-45;

// Is a in the range sincos_rope covers?  (false for NaN)
__host__ __device__ inline bool sincos_rope_in_range(float a)
{
    return std::fabs(a) < kSincosRange;
}

// s = f32(sin a), c = f32(cos a), each evaluated in double, for |a| < 2^20.
__host__ __device__ inline void sincos_rope(float a, float &s, float &c)
{
    const double x = (double)a;
    const double kd = std::rint(x * kTwoOverPi);
    double r = std::fma(-kd, kP1, x);
    r = std::fma(-kd, kP2, r);
    r = std::fma(-kd, kP3, r);
    const double z = r * r;
    const double z2 = z * z;
    const double z4 = z2 * z2;
    // sin r = r + r z (S3 + S5 z + ... + S15 z^6)
    const double s01 = std::fma(kS5, z, kS3), s23 = std::fma(kS9, z, kS7),
                 s45 = std::fma(kS13, z, kS11);
    const double s03 = std::fma(s23, z2, s01), s46 = std::fma(kS15, z2, s45);
    const double ps = std::fma(s46, z4, s03);
    const double sn = std::fma(r * z, ps, r);
    // cos r = 1 + z (C2 + C4 z + ... + C16 z^7)
    const double c01 = std::fma(kC4, z, kC2), c23 = std::fma(kC8, z, kC6),
                 c45 = std::fma(kC12, z, kC10), c67 = std::fma(kC16, z, kC14);
    const double c03 = std::fma(c23, z2, c01), c47 = std::fma(c67, z2, c45);
    const double pc = std::fma(c47, z4, c03);
    const double cs = std::fma(pc, z, 1.0);
    const int q = (int)((int64_t)kd & 3);
    const double so = (q & 1) ? cs : sn;
    const double co = (q & 1) ? sn : cs;
    s = (float)((q & 2) ? -so : so);
    c = (float)(((q + 1) & 2) ? -co : co);
}

}  // namespace qkv_detail

#endif  // QKV_SINCOS_H
