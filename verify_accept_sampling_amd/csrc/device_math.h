// Float64 exponential for non-positive arguments, used by the float64 draw
// pass.  Tang's table-driven method (P. T. P. Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989), in base 2 with a 64-entry table:
//   t = x * 64/ln2 = 64 m + j + f,  |f| <= 1/2,
//   exp(x) = 2^m * 2^(j/64) * exp(f ln2/64),
// with exp(r), |r| <= ln2/128, from its degree-5 Taylor polynomial
// (truncation below 3.6e-17 relative) and 2^(j/64) from the table.
// Callers pass the scaled argument t directly (one fused multiply-add on the
// input); arguments whose result lies below the smallest subnormal, and
// -inf, give exactly 0.  Error about 2 ulp for an exact t.
#pragma once

#include <hip/hip_runtime.h>

namespace specv {

// 2^(j/64), j = 0..63, each rounded to the nearest double.
constexpr double kExp2Frac64[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0};

constexpr double kInvLn2x64 = 0x1.71547652b82fep+6;  // 64 / ln 2
constexpr double kLn2d64 = 0x1.62e42fefa39efp-7;     // ln 2 / 64
// Scaled arguments below this give results under half the smallest
// subnormal (x < -745.2).
constexpr double kTMin = -745.2 * 0x1.71547652b82fep+6;

// exp(t ln2/64) for t <= 0; `tab` points at the 64-entry table (a
// shared-memory copy on the device, kExp2Frac64 on the host).
__host__ __device__ inline double exp2_64(double t, const double* tab) {
  const double tc = fmax(t, kTMin);  // also maps -inf
  const double n = rint(tc);
  const double r = (tc - n) * kLn2d64;  // tc - n is exact
  double p = 1.0 / 120.0;
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int ni = static_cast<int>(n);
  const double v = ldexp(tab[ni & 63] * p, ni >> 6);
  return t >= kTMin ? v : 0.0;
}

// exp(x) for x <= 0 (x scaled here; the scaling adds |x| * 2^-53 of
// relative error, which matters only for results far below 1).
__host__ __device__ inline double exp_nonpos(double x, const double* tab) {
  return exp2_64(x * kInvLn2x64, tab);
}

}  // namespace specv
