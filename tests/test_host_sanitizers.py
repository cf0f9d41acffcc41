"""The host code of the C ABI (argument checks, workspace layout, timing
hooks) under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libspecverify_asan.so (host-only sources instrumented, device code
untouched) when it is missing or older than its sources, then runs the
C-ABI tests in a child process that loads it with the clang ASan runtime
preloaded; any sanitizer finding aborts the child and fails this test.
CPU only: no call reaches a kernel launch.
"""
import glob
import os
import subprocess
import sys

from verify_accept_sampling_amd import _build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib: str) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = glob.glob(os.path.join(B.CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*"))
    return any(os.path.getmtime(s) > t for s in srcs)


def test_abi_checks_are_clean_under_asan_and_ubsan():
    if _stale(B.ASAN_LIB):
        B.build(verbose=False, sanitize=True)
    env = B.sanitizer_env()
    code = ("import verify_accept_sampling_amd as S, os; "
            "S.load_library(); "
            "maps = open('/proc/self/maps').read(); "
            "assert 'libspecverify_asan.so' in maps and 'libclang_rt.asan' in maps")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_abi.py", "tests/test_zz_no_alloc.py"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
