"""Build libspecverify.so (the C-ABI verifier library) for gfx950 with hipcc.

Sources under csrc/ are compiled in parallel into _build/ and linked into
verify_accept_sampling_amd/libspecverify.so (in-tree, so it travels with the
repository snapshot).  Usable as `python -m verify_accept_sampling_amd._build`.

`python -m verify_accept_sampling_amd._build --sanitize` builds
libspecverify_asan.so instead: the host-only sources (the argument checks,
workspace layout and timing hooks, *.cpp) with AddressSanitizer and
UndefinedBehaviorSanitizer for the host pass (each -fsanitize is given with
-Xarch_host, so no device code is instrumented).  The CPU tests run against
it with SPEC_VERIFY_LIBRARY pointing at it and the clang ASan runtime
preloaded (see `sanitizer_env()`).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspecverify.so")
ASAN_LIB = os.path.join(PKG, "libspecverify_asan.so")
ARCH = os.environ.get("SPEC_VERIFY_ARCH", "gfx950")

# Packed fp32 arithmetic is disabled for all device code.
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


# Host-pass sanitizers for the host-only sources of the sanitized build.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-fno-omit-frame-pointer", "-g"]


def _compile(src: str, sanitize: bool = False) -> str:
    suffix = ".asan.o" if sanitize else ".o"
    obj = os.path.join(OBJ, os.path.basename(src) + suffix)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = SANITIZE if sanitize and src.endswith(".cpp") else []
    cmd = [hipcc(), *FLAGS, *extra, *lang, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if res.stderr.strip():
        # keep warnings visible, but the packed-fp32 host-pass notice is noise
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if any(l.strip() for l in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, sanitize), srcs))
    lib = ASAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libsan"] if sanitize else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def sanitizer_env() -> dict:
    """Environment for a Python process that loads the sanitized library:
    the clang ASan runtime preloaded (Python itself is not instrumented),
    leak reports off (the interpreter's own allocations), UBSan findings
    fatal."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    rt = res.stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        raise RuntimeError("clang ASan runtime not found")
    env = dict(os.environ)
    env.update({"LD_PRELOAD": rt, "SPEC_VERIFY_LIBRARY": ASAN_LIB,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    return env


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
