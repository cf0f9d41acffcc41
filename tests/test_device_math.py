"""Accuracy of the float64 exponential used by the draw pass (CPU build of
the same header): Tang's table-driven method against the C library's long
double expl, over the whole non-positive range it serves."""
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
  std::uniform_real_distribution<double> wide(-745.0, 0.0), narrow(-40.0, 0.0);
  double worst = 0.0, worst_x = 0.0;
  long n = 0;
  auto check = [&](double x) {
    const double got = specv::exp_nonpos(x, specv::kExp2Frac32);
    const long double ref = expl((long double)x);
    if (ref < 2.2250738585072014e-308L) {  // subnormal results: absolute bound
      const long double err = fabsl((long double)got - ref) / 4.9406564584124654e-324L;
      if (err > 2.0) { std::printf("BAD subnormal x=%a got=%a\n", x, got); }
      return;
    }
    const long double ulp = (long double)std::nextafter((double)ref, 1e300) - (long double)(double)ref;
    const double e = (double)(fabsl((long double)got - ref) / ulp);
    if (e > worst) { worst = e; worst_x = x; }
    ++n;
  };
  for (int i = 0; i < 2000000; ++i) check(wide(g));
  for (int i = 0; i < 2000000; ++i) check(narrow(g));
  for (int i = 0; i < 100000; ++i) check(-std::ldexp((double)i, -20));
  const double specials[] = {0.0, -0.0, -1e-300, -1e-17, -0.5, -1.0, -700.0, -708.4, -744.0, -745.1};
  for (double x : specials) check(x);
  std::printf("checked %ld worst_ulp %.3f at %a\n", n, worst, worst_x);
  std::printf("minus_inf %a below_range %a zero %a\n",
              specv::exp_nonpos(-INFINITY, specv::kExp2Frac32),
              specv::exp_nonpos(-800.0, specv::kExp2Frac32),
              specv::exp_nonpos(0.0, specv::kExp2Frac32));
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
