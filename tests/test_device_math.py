"""Accuracy of the float64 exponential used by the draw pass (CPU build of
the same header): Tang's table-driven method, 2^(t/256), against the C
library's long double exp2l, over the whole range it serves (every table
entry, arguments down to the underflow clamp, and the positive arguments a
reference below the row maximum produces); and of its degree-3 variant for
summed terms against its truncation bound (ln2/512)^4 / 24."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "verify_accept_sampling_amd", "csrc")

DRIVER = r"""
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <random>
#include "device_math.h"
int main() {
  std::mt19937_64 g(12345);
  const double tmin = -745.0 * 256.0 / 0.6931471805599453;
  std::uniform_real_distribution<double> wide(tmin, 0.0), narrow(-16000.0, 0.0),
      above(0.0, 64.0 * 256.0);
  double worst = 0.0, worst_t = 0.0;
  long n = 0;
  for (int j = 0; j < 256; ++j) {  // table entries, correctly rounded
    const long double ref = exp2l((long double)j / 256.0L);
    if (specv::kExp2Frac256[j] != (double)ref) std::printf("BAD table %d\n", j);
  }
  auto check = [&](double t) {
    const double got = specv::exp2_256(t, specv::kExp2Frac256);
    const long double ref = exp2l((long double)t / 256.0L);
    if (ref < 2.2250738585072014e-308L) {  // subnormal results: absolute bound
      const long double err = fabsl((long double)got - ref) / 4.9406564584124654e-324L;
      if (err > 2.0) { std::printf("BAD subnormal t=%a got=%a\n", t, got); }
      return;
    }
    const long double ulp = (long double)std::nextafter((double)ref, 1e300) - (long double)(double)ref;
    const double e = (double)(fabsl((long double)got - ref) / ulp);
    if (e > worst) { worst = e; worst_t = t; }
    ++n;
  };
  for (int i = 0; i < 2000000; ++i) check(wide(g));
  for (int i = 0; i < 2000000; ++i) check(narrow(g));
  for (int i = 0; i < 500000; ++i) check(above(g));
  for (int i = 0; i < 100000; ++i) check(-std::ldexp((double)i, -14));
  const double specials[] = {0.0, -0.0, -1e-300, -1e-17, -0.5, -1.0, -256.0, -257.5, tmin, tmin + 1,
                             -1074.0 * 256.0, -1075.5 * 256.0};
  for (double t : specials) check(t);
  std::printf("checked %ld worst_ulp %.3f at %a\n", n, worst, worst_t);
  // the degree-3 variant for summed terms: relative error below 1.5e-13,
  // and never above the exact value by more than rounding (2^-51 relative)
  double worst3 = 0.0, above3 = 0.0;
  auto check3 = [&](double t) {
    const long double ref = exp2l((long double)t / 256.0L);
    if (ref < 2.2250738585072014e-308L) return;
    const long double got = specv::exp2_256_sum(t, specv::kExp2Frac256);
    const double rel = (double)((got - ref) / ref);
    if (-rel > worst3) worst3 = -rel;
    if (rel > above3) above3 = rel;
  };
  for (int i = 0; i < 2000000; ++i) check3(narrow(g));
  for (int i = 0; i < 1000000; ++i) check3(wide(g));
  for (int i = 0; i < 200000; ++i) check3(above(g));
  for (int j = -2000; j <= 2000; ++j) check3(j + 0.5), check3(j - 0.5);  // |f| = 1/2: the bound
  std::printf("deg3_below %.3e deg3_above %.3e zero3 %a\n", worst3, above3,
              specv::exp2_256_sum(0.0, specv::kExp2Frac256));
  std::printf("minus_inf %a below_range %a zero %a\n",
              specv::exp2_256(-INFINITY, specv::kExp2Frac256),
              specv::exp2_256(-1200.0 * 256.0, specv::kExp2Frac256),
              specv::exp2_256(0.0, specv::kExp2Frac256));
  return 0;
}
"""


def test_exp_nonpos_accuracy():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "drv.hip")
        exe = os.path.join(d, "drv")
        with open(src, "w") as f:
            f.write(DRIVER)
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", CSRC,
                        "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                       check=True, capture_output=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    assert "BAD" not in out, out
    words = out.split()
    worst = float(words[words.index("worst_ulp") + 1])
    assert worst < 3.0, out
    assert "minus_inf 0x0p+0" in out and "below_range 0x0p+0" in out and "zero 0x1p+0" in out, out
    below3 = float(words[words.index("deg3_below") + 1])
    above3 = float(words[words.index("deg3_above") + 1])
    assert below3 < 1.5e-13 and above3 < 2.0 ** -51, out
    assert "zero3 0x1p+0" in out, out
