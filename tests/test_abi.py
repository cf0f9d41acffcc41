"""The C-ABI library loads, exports what its header declares, and rejects
bad arguments on the host without enqueuing work (CPU only: no call here
reaches a kernel launch)."""
import ctypes

import numpy as np
import pytest

import verify_accept_sampling_amd as S
import workloads as W

EINVAL, EDTYPE, EWORKSPACE, EHIP, ETREE = -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def lib():
    return S.load_library()


def test_exports_every_declared_symbol(lib):
    names = S.declared_symbols()
    assert {"spec_verify_greedy", "spec_verify_sample", "spec_verify_tree_greedy",
            "spec_fill_uniforms", "spec_workspace_bytes", "spec_strerror",
            "spec_tree_depth"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_strerror(lib):
    for code in (0, EINVAL, EDTYPE, EWORKSPACE, EHIP, ETREE, 12345):
        assert S.spec_strerror(code)
    assert "workspace" in S.spec_strerror(EWORKSPACE)


def test_workspace_bytes(lib):
    a = S.spec_workspace_bytes(64, 9, 128256)
    assert a > 0 and a % 256 == 0
    assert S.spec_workspace_bytes(128, 9, 128256) > a
    assert S.spec_workspace_bytes(0, 9, 128256) >= (2 << 20) + 256  # fixed counter region
    for bad in ((-1, 9, 10), (65537, 9, 10), (1, 0, 10), (1, 9, 0), (1, 2000, 10), (1, 9, 2 ** 30 + 1)):
        assert S.spec_workspace_bytes(*bad) == 0


def test_tree_depth(lib):
    assert S.spec_tree_depth(W.static_tree_parents()) == 5
    assert S.spec_tree_depth([-1]) == 0
    assert S.spec_tree_depth(list(range(-1, 9))) == 9
    for bad in ([0, 0], [-1, 1], [-1, 0, 3], [-1, -1]):
        with pytest.raises(S.SpecVerifyError) as e:
            S.spec_tree_depth(bad)
        assert e.value.code == ETREE
    with pytest.raises(S.SpecVerifyError):
        S.spec_tree_depth([-1] * 0)


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation


def test_greedy_rejects_bad_arguments(lib):
    g = lib.spec_verify_greedy
    ws = S.spec_workspace_bytes(2, 5, 100)
    assert g(FAKE, 7, 2, 4, 100, FAKE, FAKE, FAKE, FAKE, ws, None) == EDTYPE
    assert g(FAKE, 0, -1, 4, 100, FAKE, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert g(FAKE, 0, 2, -1, 100, FAKE, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert g(FAKE, 0, 2, 4, 0, FAKE, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert g(FAKE, 0, 2, 1024, 100, FAKE, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert g(None, 0, 2, 4, 100, FAKE, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert g(FAKE, 0, 2, 4, 100, None, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert g(FAKE, 0, 2, 4, 100, FAKE, None, FAKE, FAKE, ws, None) == EINVAL
    assert g(FAKE, 0, 2, 4, 100, FAKE, FAKE, None, FAKE, ws, None) == EINVAL
    assert g(FAKE, 0, 2, 4, 100, FAKE, FAKE, FAKE, None, ws, None) == EWORKSPACE
    assert g(FAKE, 0, 2, 4, 100, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == EWORKSPACE
    # B == 0 is a no-op
    assert g(None, 0, 0, 4, 100, None, None, None, None, 0, None) == 0


def test_sample_rejects_bad_arguments(lib):
    f = lib.spec_verify_sample
    ws = S.spec_workspace_bytes(2, 5, 100)

    def call(target=FAKE, draft=FAKE, dt=1, kind=0, B=2, k=4, V=100, toks=FAKE, u=None,
             T=1.0, flags=0, acc=FAKE, out=FAKE, probe=None, w=FAKE, wb=ws):
        return f(target, draft, dt, kind, B, k, V, toks, u, 0, 0, ctypes.c_float(T), flags, acc,
                 out, probe, w, wb, None)

    assert call(dt=3) == EDTYPE
    assert call(kind=2) == EDTYPE
    assert call(kind=1, dt=1) == EDTYPE          # probabilities must be float32
    assert call(kind=1, dt=0, T=0.5) == EINVAL   # probabilities take T = 1
    for T in (0.0, -1.0, float("nan"), float("inf"), 1e-39):
        assert call(T=T) == EINVAL, T
    assert call(B=-1) == EINVAL
    assert call(k=-1) == EINVAL
    assert call(V=0) == EINVAL
    assert call(target=None) == EINVAL
    assert call(draft=None) == EINVAL
    assert call(toks=None) == EINVAL
    assert call(acc=None) == EINVAL
    assert call(out=None) == EINVAL
    assert call(w=None) == EWORKSPACE
    assert call(wb=ws - 1) == EWORKSPACE
    # flags: a schedule (0..3), optionally the test bit; anything else is rejected
    for bad in (4, 15, 0x10, 0x200, -1, 0x100 | 7):
        assert call(flags=bad) == EINVAL, bad
    assert call(B=0, target=None, draft=None, toks=None, acc=None, out=None, w=None) == 0


def test_tree_rejects_bad_arguments(lib):
    f = lib.spec_verify_tree_greedy
    parent = (ctypes.c_int32 * 4)(-1, 0, 0, 1)
    badp = (ctypes.c_int32 * 4)(-1, 0, 3, 1)
    ws = S.spec_workspace_bytes(2, 4, 100)
    pp = ctypes.cast(parent, ctypes.c_void_p)
    assert f(FAKE, 5, 2, 4, 100, pp, FAKE, FAKE, FAKE, None, FAKE, ws, None) == EDTYPE
    assert f(FAKE, 1, 2, 4, 100, ctypes.cast(badp, ctypes.c_void_p), FAKE, FAKE, FAKE, None,
             FAKE, ws, None) == ETREE
    assert f(FAKE, 1, 2, 4, 100, None, FAKE, FAKE, FAKE, None, FAKE, ws, None) == EINVAL
    assert f(FAKE, 1, 2, 0, 100, pp, FAKE, FAKE, FAKE, None, FAKE, ws, None) == EINVAL
    assert f(FAKE, 1, 2, 1025, 100, pp, FAKE, FAKE, FAKE, None, FAKE, ws, None) == EINVAL
    assert f(None, 1, 2, 4, 100, pp, FAKE, FAKE, FAKE, None, FAKE, ws, None) == EINVAL
    assert f(FAKE, 1, 2, 4, 100, pp, None, FAKE, FAKE, None, FAKE, ws, None) == EINVAL
    assert f(FAKE, 1, 2, 4, 100, pp, FAKE, FAKE, FAKE, None, None, ws, None) == EWORKSPACE
    assert f(None, 1, 0, 4, 100, pp, None, None, None, None, None, 0, None) == 0


def test_tree_sample_rejects_bad_arguments(lib):
    f = lib.spec_verify_tree_sample
    parent = (ctypes.c_int32 * 4)(-1, 0, 0, 1)
    badp = (ctypes.c_int32 * 4)(-1, 0, 3, 1)
    ws = S.spec_workspace_bytes(2, 4, 100)
    pp = ctypes.cast(parent, ctypes.c_void_p)

    def call(target=FAKE, draft=FAKE, dtype=1, kind=0, B=2, N=4, V=100, par=pp, toks=FAKE,
             T=1.0, acc=FAKE, out=FAKE, w=FAKE, wb=ws):
        return f(target, draft, dtype, kind, B, N, V, par, toks, None, 1, 0, T, acc, out, None,
                 w, wb, None)

    assert call(dtype=5) == EDTYPE
    assert call(kind=1, dtype=1) == EDTYPE  # probability rows are float32
    assert call(kind=1, dtype=0, T=0.5) == EINVAL  # probabilities take T = 1
    assert call(T=0.0) == EINVAL
    assert call(T=float("inf")) == EINVAL
    assert call(par=ctypes.cast(badp, ctypes.c_void_p)) == ETREE
    assert call(par=None) == EINVAL
    assert call(N=0) == EINVAL
    assert call(N=1025) == EINVAL
    assert call(target=None) == EINVAL
    assert call(draft=None) == EINVAL
    assert call(toks=None) == EINVAL
    assert call(acc=None) == EINVAL
    assert call(w=None) == EWORKSPACE
    assert call(wb=ws - 1) == EWORKSPACE
    assert call(B=0, target=None, draft=None, toks=None, acc=None, out=None, w=None) == 0


def test_fill_uniforms_argument_checks(lib):
    assert lib.spec_fill_uniforms(1, 0, -1, FAKE, None) == EINVAL
    assert lib.spec_fill_uniforms(1, 0, 5, None, None) == EINVAL
    assert lib.spec_fill_uniforms(1, 0, 0, None, None) == 0


COUNTER_BYTES = (2097152 + 256)  # SPEC_WORKSPACE_COUNTER_BYTES


def test_workspace_status_and_reset_argument_checks(lib):
    ws = COUNTER_BYTES  # the two calls need the counter region only
    v = ctypes.c_uint32(0)
    assert lib.spec_workspace_status(None, ws, ctypes.byref(v), None) == EINVAL
    assert lib.spec_workspace_status(FAKE, ws, None, None) == EINVAL
    assert lib.spec_workspace_status(FAKE, ws - 1, ctypes.byref(v), None) == EWORKSPACE
    assert lib.spec_workspace_reset(None, ws, None) == EINVAL
    assert lib.spec_workspace_reset(FAKE, ws - 1, None) == EWORKSPACE


def test_status_word_sits_in_the_counter_region():
    import re

    with open(S._HEADER) as f:
        text = f.read()
    counter = int(re.search(r"SPEC_WORKSPACE_COUNTER_BYTES \((\d+) \+ 256\)", text).group(1)) + 256
    off = int(re.search(r"SPEC_WORKSPACE_STATUS_OFFSET (\d+)", text).group(1))
    assert off + 12 <= counter  # status word, then the 8-byte epoch
    assert S.spec_workspace_bytes(0, 1, 1) >= counter
