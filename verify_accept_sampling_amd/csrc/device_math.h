// Float64 exponential for non-positive arguments, used by the float64 draw
// pass.  Tang's table-driven method (P. T. P. Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989):
//   x = (32 m + j) ln2/32 + r,  |r| <= ln2/64,
//   exp(x) = 2^m * 2^(j/32) * exp(r),
// with exp(r) from its degree-6 Taylor polynomial (truncation below 4e-18
// relative on |r| <= ln2/64) and 2^(j/32) from a 32-entry table.
// Arguments below -745.2 (results under the smallest subnormal) give 0;
// -inf gives 0.  Error: about 2 ulp.
#pragma once

#include <hip/hip_runtime.h>

namespace specv {

// 2^(j/32), j = 0..31, each rounded to the nearest double.
constexpr double kExp2Frac32[32] = {
    0x1.0000000000000p+0, 0x1.059b0d3158574p+0, 0x1.0b5586cf9890fp+0, 0x1.11301d0125b51p+0,
    0x1.172b83c7d517bp+0, 0x1.1d4873168b9aap+0, 0x1.2387a6e756238p+0, 0x1.29e9df51fdee1p+0,
    0x1.306fe0a31b715p+0, 0x1.371a7373aa9cbp+0, 0x1.3dea64c123422p+0, 0x1.44e086061892dp+0,
    0x1.4bfdad5362a27p+0, 0x1.5342b569d4f82p+0, 0x1.5ab07dd485429p+0, 0x1.6247eb03a5585p+0,
    0x1.6a09e667f3bcdp+0, 0x1.71f75e8ec5f74p+0, 0x1.7a11473eb0187p+0, 0x1.82589994cce13p+0,
    0x1.8ace5422aa0dbp+0, 0x1.93737b0cdc5e5p+0, 0x1.9c49182a3f090p+0, 0x1.a5503b23e255dp+0,
    0x1.ae89f995ad3adp+0, 0x1.b7f76f2fb5e47p+0, 0x1.c199bdd85529cp+0, 0x1.cb720dcef9069p+0,
    0x1.d5818dcfba487p+0, 0x1.dfc97337b9b5fp+0, 0x1.ea4afa2a490dap+0, 0x1.f50765b6e4540p+0};

constexpr double kInvLn2x32 = 0x1.71547652b82fep+5;  // 32 / ln 2
constexpr double kLn2d32Hi = 0x1.62e42fefa39efp-6;   // ln 2 / 32, leading part
constexpr double kLn2d32Lo = 0x1.abc9e3b39803fp-61;  // ln 2 / 32 - kLn2d32Hi

// exp(x) for x <= 0; `tab` points at the 32-entry table (a shared-memory
// copy on the device, kExp2Frac32 on the host).
__host__ __device__ inline double exp_nonpos(double x, const double* tab) {
  const double xc = x < -745.2 ? -745.2 : x;  // also maps -inf and keeps n finite
  const double n = rint(xc * kInvLn2x32);
  double r = fma(-n, kLn2d32Hi, xc);
  r = fma(-n, kLn2d32Lo, r);
  double p = 1.0 / 720.0;
  p = fma(p, r, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int ni = static_cast<int>(n);
  const double v = ldexp(tab[ni & 31] * p, ni >> 5);
  return x < -745.2 ? 0.0 : v;
}

}  // namespace specv
