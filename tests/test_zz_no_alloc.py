"""spec_verify_sample_noalloc: the sampling verification on the library's
static per-GPU scratch array, for callers that cannot allocate.

Host side (no GPU): shapes beyond SPEC_NOALLOC_SCRATCH_BYTES return
SPEC_ESCRATCH, other bad arguments the codes of spec_verify_sample, and
nothing is enqueued.

GPU: through the C ABI, two calls in a row (the second on a smaller input)
must equal spec_verify_sample's outputs on a workspace, element by element
(both run the same kernels on the same inputs, so the integer outputs and
the probe values are identical); a call whose bounded wait is forced to give
up says so with -1 outputs, and the next call, with no reset, is exact
again (each call clears the counters it uses).
"""
import ctypes

import numpy as np
import pytest
import torch

import verify_accept_sampling_amd as S
import workloads as W
from parity_helpers import ints_to_device, to_device

EINVAL, ESCRATCH = -1, -6


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def lib():
    return S.load_library()


def _noalloc_raw(lib, B, k, V, dtype=1, kind=0, T=1.0, flags=0, ptr=0x1000):
    """Calls the entry point with stand-in (never dereferenced) pointers: only
    for argument checks that return before any launch."""
    p = ctypes.c_void_p(ptr)
    return lib.spec_verify_sample_noalloc(p, p, dtype, kind, B, k, V, p, None, 1, 0, T, flags,
                                          p, p, None, None)


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    limit = S.NOALLOC_SCRATCH_BYTES
    # B = 1024, k = 8, V = 128256 needs about 57 MiB; B = 4096 far more
    assert S.spec_workspace_bytes(1024, 9, 128256) <= limit
    assert S.spec_workspace_bytes(4096, 9, 128256) > limit
    assert _noalloc_raw(lib, 4096, 8, 128256) == ESCRATCH
    assert _noalloc_raw(lib, 2048, 8, 128256) == ESCRATCH  # about 112 MiB
    assert "SPEC_NOALLOC_SCRATCH_BYTES" in S.spec_strerror(ESCRATCH)


def test_noalloc_argument_checks(lib):
    assert _noalloc_raw(lib, 0, 8, 128256) == 0  # B = 0: nothing to do
    assert _noalloc_raw(lib, 4, 4, 1000, flags=0x40) == EINVAL
    assert _noalloc_raw(lib, 4, 4, 1000, T=0.0) == EINVAL
    assert _noalloc_raw(lib, 4, 4, 1000, dtype=1, kind=1) == -2  # probs need f32
    p = ctypes.c_void_p(0x1000)
    assert lib.spec_verify_sample_noalloc(None, p, 1, 0, 4, 4, 1000, p, None, 1, 0, 1.0, 0, p,
                                          p, None, None) == EINVAL


def _inputs(B, k, V, seed, dtype="bf16", T=1.0):
    wl = W.sample_chain(B, k, V, seed=seed, uniform_seed=seed + 1, target_std=2.0,
                        noise_std=1.0, temperature=T, dtype=dtype)
    return (wl, to_device(wl.target, dtype), to_device(wl.draft, dtype),
            ints_to_device(wl.draft_tokens))


def _both(wl, tgt, dft, toks, schedule, counter0=0, probe=True):
    ws = S.Workspace("cuda")
    ref = S.spec_verify_sample(tgt, dft, toks, wl.temperature, seed=wl.uniform_seed,
                               counter0=counter0, probe=probe, workspace=ws, schedule=schedule)
    got = S.spec_verify_sample_noalloc(tgt, dft, toks, wl.temperature, seed=wl.uniform_seed,
                                       counter0=counter0, probe=probe, schedule=schedule)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ref], [t.cpu().numpy() for t in got]


@pytest.mark.gpu
@pytest.mark.parametrize("schedule", ["auto", "two_launch", "early_exit"])
def test_noalloc_matches_the_workspace_entry_point(schedule):
    # call 1: the B=64, k=8, V=128256 shape; call 2: a smaller one (ragged V)
    for (B, k, V, seed, T) in ((64, 8, 128256, 71, 0.7), (5, 3, 32003, 73, 1.0)):
        _say(f"noalloc vs workspace entry point: schedule={schedule} B={B} k={k} V={V}")
        wl, tgt, dft, toks = _inputs(B, k, V, seed, T=T)
        ref, got = _both(wl, tgt, dft, toks, schedule)
        assert np.array_equal(ref[0], got[0]), (ref[0], got[0])
        assert np.array_equal(ref[1], got[1])
        assert np.array_equal(ref[2], got[2])  # probe values: same kernels, same inputs
        assert (got[0] >= 0).all()


@pytest.mark.gpu
def test_noalloc_probability_rows():
    _say("noalloc vs workspace entry point: probability rows B=16 k=4 V=50000")
    rng = np.random.default_rng(75)
    B, k, V = 16, 4, 50000
    p = rng.dirichlet(np.full(V, 0.05), size=(B, k + 1)).astype(np.float32)
    q = rng.dirichlet(np.full(V, 0.05), size=(B, k)).astype(np.float32)
    toks = rng.integers(0, V, size=(B, k)).astype(np.int32)
    tgt, dft, tk = (torch.from_numpy(p).cuda(), torch.from_numpy(q).cuda(),
                    torch.from_numpy(toks).cuda())
    ws = S.Workspace("cuda")
    for counter0 in (0, 1000):
        ref = S.spec_verify_sample(tgt, dft, tk, 1.0, seed=9, counter0=counter0, kind="probs",
                                   workspace=ws)
        got = S.spec_verify_sample_noalloc(tgt, dft, tk, 1.0, seed=9, counter0=counter0,
                                           kind="probs")
        torch.cuda.synchronize()
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])


@pytest.mark.gpu
def test_noalloc_give_up_does_not_outlive_its_call():
    _say("noalloc: forced give-up, then a normal call without reset")
    wl, tgt, dft, toks = _inputs(8, 4, 32000, 77)
    # the one-launch schedule: its bounded waits are what the flag makes give up
    acc, out = S.spec_verify_sample_noalloc(tgt, dft, toks, wl.temperature,
                                            seed=wl.uniform_seed, test_give_up=True,
                                            schedule="one_launch")
    torch.cuda.synchronize()
    acc = acc.cpu().numpy()
    out = out.cpu().numpy()
    assert acc[0] == -1 and (out[0] == -1).all()
    ref, got = _both(wl, tgt, dft, toks, "auto", probe=False)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])
    assert (got[0] >= 0).all()


@pytest.mark.gpu
def test_noalloc_preallocated_outputs_two_calls():
    # the allocation-free way to call it from Python: outputs passed in
    wl1, t1, d1, k1 = _inputs(32, 6, 65536, 79)
    wl2, t2, d2, k2 = _inputs(3, 2, 4097, 81)
    acc = torch.full((32,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((32, 7), -7, dtype=torch.int32, device="cuda")
    for wl, t, d, k in ((wl1, t1, d1, k1), (wl2, t2, d2, k2)):
        _say(f"noalloc with preallocated outputs: B={wl.B} k={wl.k} V={wl.V}")
        a, o = acc[: wl.B], out[: wl.B, : wl.k + 1]
        if not o.is_contiguous():
            o = torch.empty((wl.B, wl.k + 1), dtype=torch.int32, device="cuda")
        r = S.spec_verify_sample_noalloc(t, d, k, wl.temperature, seed=wl.uniform_seed,
                                         out=(a, o))
        assert r[0].data_ptr() == a.data_ptr()
        ref = S.spec_verify_sample(t, d, k, wl.temperature, seed=wl.uniform_seed)
        torch.cuda.synchronize()
        assert torch.equal(ref[0], a) and torch.equal(ref[1], o)
