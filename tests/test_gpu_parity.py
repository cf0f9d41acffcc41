"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Integer outputs must match bit-exactly, except that a disagreement is
allowed when its first differing decision lies within 1e-5 of its boundary
in the oracle (flagged); unflagged mismatches must be zero.  Probabilities
reported by the probe must agree within 1e-5 absolute.
"""
import numpy as np
import pytest
import torch

import oracle.rng as R
import oracle.verify as O
import verify_accept_sampling_amd as S
import workloads as W
from parity_helpers import (PROB_TOL, check_chain_structure, check_probe, compare_sample,
                            ints_to_device, to_device)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


# Schedule of the sampling calls in _run_sample, and whether it asks for
# probe values (set per schedule by the fixture below).
_SCHED = {"value": "auto", "probe": True}


@pytest.fixture(params=["one_launch", "two_launch", "early_exit"])
def sample_path(request):
    """Run a sampling test through the one-launch kernel, the two-launch
    kernels and the early-exit kernel (the call's schedule argument).  Early
    exit reads every row when probe values are asked for, so there the probe
    is left out and the outputs alone are compared."""
    _SCHED["value"] = request.param
    _SCHED["probe"] = request.param != "early_exit"
    yield request.param
    _SCHED["value"] = "auto"
    _SCHED["probe"] = True


# ---------------------------------------------------------------------------
# uniforms
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("seed,ctr,n", [(0, 0, 1000), (2003, 0, 64 * 9 * 2),
                                        (12345678901234567, 2 ** 63 + 11, 4097),
                                        (7, 2 ** 64 - 5, 300), (99, 5, 1)])
def test_uniforms_bit_exact(seed, ctr, n):
    g = S.spec_fill_uniforms(seed, ctr, n).cpu().numpy().astype(np.float64)
    assert np.array_equal(g, R.uniforms(seed, ctr, n))


# ---------------------------------------------------------------------------
# greedy chain
# ---------------------------------------------------------------------------


def _run_greedy(wl):
    acc_o, out_o, _ = O.verify_greedy(wl.target, wl.draft_tokens, wl.dtype)
    acc_g, out_g = S.spec_verify_greedy(to_device(wl.target, wl.dtype),
                                        ints_to_device(wl.draft_tokens))
    torch.cuda.synchronize()
    acc_g, out_g = acc_g.cpu().numpy(), out_g.cpu().numpy()
    assert np.array_equal(acc_g, acc_o)
    assert np.array_equal(out_g, out_o)
    check_chain_structure(acc_g, out_g, wl.draft_tokens, wl.V)


def test_greedy_chain_v1000_full():
    _say("greedy chain B=1 k=4 V=1000 f32")
    _run_greedy(W.greedy_chain())


@pytest.mark.parametrize("B,k,V,dtype", [(37, 6, 50_000, "bf16"), (5, 8, 128256, "bf16"),
                                         (9, 3, 1001, "f32"), (9, 3, 1001, "bf16"),
                                         (3, 2, 7, "f32"), (4, 0, 300, "bf16"),
                                         (2, 1, 1, "f32"), (1, 200, 64, "f32"),
                                         (64, 8, 32768, "f32")])
def test_greedy_chain_shapes(B, k, V, dtype):
    _say(f"greedy chain B={B} k={k} V={V} {dtype}")
    _run_greedy(W.greedy_chain(B=B, k=k, V=V, seed=B * 1000 + V, dtype=dtype))


@pytest.mark.parametrize("V", [3000, 2000])  # chunked kernel; one work-group per request
def test_greedy_chain_ties_masks_and_bad_tokens(V):
    rng = np.random.default_rng(5)
    B, k = 40, 5
    z = np.round(rng.standard_normal((B, k + 1, V)) * 1.2).astype(np.float32)  # many ties
    z[rng.random(z.shape) < 0.3] = -np.inf
    z[3, 1] = -np.inf  # a wholly masked row: its argmax is index 0
    amax = np.argmax(z[:, :k], axis=-1)
    toks = np.where(rng.random((B, k)) < 0.8, amax, rng.integers(0, V, (B, k))).astype(np.int32)
    toks[0, 0] = -1
    toks[1, 2] = V
    toks[2, 1] = 2 ** 31 - 1
    wl = W.ChainWorkload("ties", z, None, toks, "logits", "f32", 1.0, 0)
    _run_greedy(wl)
    wl_bf = W.ChainWorkload("ties_bf16", W.f32_to_bf16_bits(z), None, toks, "logits", "bf16",
                            1.0, 0)
    _run_greedy(wl_bf)


# ---------------------------------------------------------------------------
# tree greedy
# ---------------------------------------------------------------------------


def _run_tree(wl):
    acc_o, out_o, path_o, _ = O.verify_tree_greedy(wl.target, wl.parent, wl.node_tokens,
                                                   wl.dtype)
    acc_g, out_g, path_g = S.spec_verify_tree_greedy(to_device(wl.target, wl.dtype), wl.parent,
                                                     ints_to_device(wl.node_tokens))
    torch.cuda.synchronize()
    assert np.array_equal(acc_g.cpu().numpy(), acc_o)
    assert np.array_equal(out_g.cpu().numpy(), out_o)
    assert np.array_equal(path_g.cpu().numpy(), path_o)


def test_tree_greedy_v128256_full():
    _say("tree greedy B=16 N=61 V=128256 bf16")
    _run_tree(W.tree_greedy())


@pytest.mark.parametrize("B,V,dtype,p", [(64, 12, "f32", 0.8), (32, 1000, "bf16", 0.9),
                                         (8, 30001, "bf16", 0.9), (5, 4096, "f32", 1.0)])
def test_tree_greedy_small(B, V, dtype, p):
    _say(f"tree greedy B={B} V={V} {dtype}")
    _run_tree(W.tree_greedy(B=B, V=V, seed=V, p_match=p, dtype=dtype))


def test_tree_shapes_chain_single_and_deep():
    # chain-shaped tree equals chain greedy
    wl = W.greedy_chain(B=20, k=7, V=500, seed=3, p_match=0.85)
    parent = np.arange(-1, wl.k, dtype=np.int32)
    nt = np.concatenate([np.zeros((wl.B, 1), np.int32), wl.draft_tokens], axis=1)
    tw = W.TreeWorkload("chain", wl.target, parent, nt, "f32")
    _run_tree(tw)
    acc_c, out_c = S.spec_verify_greedy(to_device(wl.target, "f32"),
                                        ints_to_device(wl.draft_tokens))
    acc_t, out_t, _ = S.spec_verify_tree_greedy(to_device(wl.target, "f32"), parent,
                                                ints_to_device(nt))
    assert torch.equal(acc_c, acc_t) and torch.equal(out_c, out_t)
    # root only
    _run_tree(W.tree_greedy(B=3, V=100, seed=4, parent=np.array([-1], np.int32)))
    # deep chain of 1024 nodes, every draft correct
    deep = W.tree_greedy(B=2, V=16, seed=6, parent=np.arange(-1, 1023, dtype=np.int32),
                         p_match=1.0, dtype="f32")
    _run_tree(deep)
    # wide star with duplicate siblings
    star = np.array([-1] + [0] * 300 + list(range(1, 301)), dtype=np.int32)
    _run_tree(W.tree_greedy(B=4, V=8, seed=7, parent=star, p_match=0.5, dtype="f32"))


# ---------------------------------------------------------------------------
# sampling chain
# ---------------------------------------------------------------------------


def _run_sample(wl, seed=None, counter0=0, requests=None, use_array=True, max_mismatch=0,
                probe=None):
    probe = _SCHED["probe"] if probe is None else probe
    sched = _SCHED["value"]
    seed = wl.uniform_seed if seed is None else seed
    u = R.chain_uniforms(seed, wl.B, wl.k, counter0)
    tgt = to_device(wl.target, wl.dtype)
    dft = to_device(wl.draft, wl.dtype) if wl.k > 0 else None
    toks = ints_to_device(wl.draft_tokens)
    if use_array:
        ug = S.spec_fill_uniforms(seed, counter0, wl.B * (wl.k + 1) * 2).view(wl.B, wl.k + 1, 2)
        res_g = S.spec_verify_sample(tgt, dft, toks, wl.temperature, uniforms=ug, kind=wl.kind,
                                     probe=probe, schedule=sched)
    else:
        res_g = S.spec_verify_sample(tgt, dft, toks, wl.temperature, seed=seed,
                                     counter0=counter0, kind=wl.kind, probe=probe,
                                     schedule=sched)
    torch.cuda.synchronize()
    acc_g, out_g = res_g[0].cpu().numpy(), res_g[1].cpu().numpy()
    check_chain_structure(acc_g, out_g, wl.draft_tokens, wl.V)
    reqs = list(range(wl.B)) if requests is None else list(requests)
    acc_o, out_o, res = O.verify_sample(wl.target, wl.draft, wl.draft_tokens, u,
                                        wl.temperature, wl.kind, wl.dtype, requests=reqs)
    st = compare_sample(acc_g, out_g, acc_o, out_o, res, reqs)
    if probe:
        where = []
        worst = check_probe(res_g[2].cpu().numpy(), wl, acc_g, acc_o, res, reqs, where)
        _say(f"  {wl.name}: {st} probe_max_abs_err={worst:.3g} at "
             f"(b, i, field, gpu, oracle)={where[0]}")
        assert worst <= PROB_TOL
    else:
        _say(f"  {wl.name}: {st} (no probe)")
    assert st["unflagged"] == 0, st["unflagged_requests"]
    assert st["mismatches"] <= max_mismatch, st
    return acc_g, out_g


def test_sample_chain_v32000_full(sample_path):
    _say("sample chain B=8 k=4 V=32000 bf16 T=1")
    _run_sample(W.sample_chain_v32000())


def test_sample_chain_llama3_full(llama3_full, sample_path):
    _say("sample chain B=64 k=8 V=128256 bf16 T=0.7")
    wl = llama3_full
    a1, o1 = _run_sample(wl, use_array=False)
    # the inline counter uniforms and an explicit uniform array agree exactly
    a2, o2 = _run_sample(wl, use_array=True)
    assert np.array_equal(a1, a2) and np.array_equal(o1, o2)


@pytest.mark.parametrize("B,k,V,dtype,T", [(50, 3, 1001, "f32", 1.0), (40, 5, 4000, "bf16", 0.3),
                                           (30, 4, 32000, "f32", 2.5), (16, 0, 5000, "bf16", 1.0),
                                           (20, 1, 17, "bf16", 0.8), (8, 12, 65536, "bf16", 1.0),
                                           # more draw chunks than threads of a work-group:
                                           # the draw's tiled tail
                                           (4, 3, 152064, "bf16", 1.0), (3, 2, 262400, "f32", 0.6)])
def test_sample_chain_shapes(B, k, V, dtype, T, sample_path):
    _say(f"sample chain B={B} k={k} V={V} {dtype} T={T} path={sample_path}")
    wl = W.sample_chain(B, k, V, seed=B + k + V, uniform_seed=77 + V, target_std=2.0,
                        noise_std=1.0, temperature=T, dtype=dtype)
    _run_sample(wl)


def test_sample_identical_draft_accepts_everything(sample_path):
    wl = W.sample_chain(24, 6, 3000, seed=1, uniform_seed=2, target_std=2.0, noise_std=1.0,
                        temperature=0.9, dtype="bf16")
    wl.draft = wl.target[:, : wl.k].copy()
    acc, _ = _run_sample(wl)
    assert np.all(acc == wl.k)


def test_sample_requests_decided_after_early_positions(sample_path):
    """Rows of only the first few positions precede the one-launch kernel's
    early acceptance tests when B x row chunks is large (here 48 requests x 3
    chunks of V = 140000).  A request that accepts all of them is finished
    by its first draw work-group from the later rows: every draft accepted
    (identical draft rows), and drafts that match for four positions, then
    differ."""
    wl = W.sample_chain(48, 5, 140000, seed=5, uniform_seed=6, target_std=2.0, noise_std=1.0,
                        temperature=1.0, dtype="bf16")
    same = wl.draft.copy()
    same[:] = wl.target[:, : wl.k]
    wl_all = W.ChainWorkload("identical_draft_wide", wl.target, same, wl.draft_tokens, "logits",
                             wl.dtype, wl.temperature, wl.uniform_seed)
    acc, _ = _run_sample(wl_all)
    assert np.all(acc == wl.k)
    part = wl.draft.copy()
    part[:, :4] = wl.target[:, :4]
    wl_part = W.ChainWorkload("late_rejections", wl.target, part, wl.draft_tokens, "logits",
                              wl.dtype, wl.temperature, wl.uniform_seed)
    acc, _ = _run_sample(wl_part)
    assert np.all(acc >= 4) and (acc < wl.k).any()


def test_sample_long_chain(sample_path):
    """k = 130 draft positions: the acceptance tests run in rounds of 64
    positions per wave (and the probe values of the positions after a stop
    in batches of 64)."""
    # drafts close to the target: the oracle stops these four at 130, 101,
    # 130 and 99 (the second and third rounds of 64)
    wl = W.sample_chain(4, 130, 512, seed=23, uniform_seed=24, target_std=1.0, noise_std=0.01,
                        temperature=1.0, dtype="f32")
    acc, _ = _run_sample(wl)
    assert acc.min() >= 64
    same = wl.draft.copy()
    same[:] = wl.target[:, : wl.k]
    wl_all = W.ChainWorkload("long_identical", wl.target, same, wl.draft_tokens, "logits",
                             wl.dtype, wl.temperature, wl.uniform_seed)
    acc_all, _ = _run_sample(wl_all)
    assert np.all(acc_all == wl.k)


def test_sample_masks_and_bad_tokens(sample_path):
    rng = np.random.default_rng(11)
    wl = W.sample_chain(32, 4, 2048, seed=9, uniform_seed=10, target_std=2.0, noise_std=1.0,
                        temperature=1.0, dtype="f32")
    t = wl.target.copy()
    d = wl.draft.copy()
    t[rng.random(t.shape) < 0.2] = -np.inf
    d[rng.random(d.shape) < 0.2] = -np.inf
    wl.target, wl.draft = t, d
    toks = wl.draft_tokens.copy()
    toks[0, 0] = -5
    toks[1, 1] = 2048
    toks[2, 3] = 2 ** 31 - 1
    wl.draft_tokens = toks
    _run_sample(wl)


def test_sample_early_exit_matches_full_sweep(llama3_full):
    """Early exit stops reading rows past each request's first rejection;
    with and without probe values its outputs equal the full sweep's, bit
    for bit, over several uniform draws."""
    wl = llama3_full
    tgt, dft = to_device(wl.target, wl.dtype), to_device(wl.draft, wl.dtype)
    toks = ints_to_device(wl.draft_tokens)
    for c in range(4):
        ctr = c * wl.B * (wl.k + 1) * 2
        outs = []
        for path, probe in (("one_launch", False), ("early_exit", False), ("early_exit", True),
                            ("two_launch", False)):
            r = S.spec_verify_sample(tgt, dft, toks, wl.temperature, seed=wl.uniform_seed,
                                     counter0=ctr, probe=probe, schedule=path)
            torch.cuda.synchronize()
            outs.append((r[0].cpu().numpy(), r[1].cpu().numpy()))
        for a, o in outs[1:]:
            assert np.array_equal(a, outs[0][0]) and np.array_equal(o, outs[0][1])


def test_sample_probs_small_and_empty_residual():
    wl = W.controlled_acceptance(B=90, k=4, V=1000, seed=21, uniform_seed=22, logit_std=1.0)
    _run_sample(wl)
    # q >= p elementwise (q carries extra mass): rejections have an empty residual
    rng = np.random.default_rng(3)
    B, k, V = 16, 2, 64
    p = rng.dirichlet(np.ones(V), size=(B, k + 1)).astype(np.float32)
    q = (p[:, :k] * np.float32(1.5)).astype(np.float32)
    toks = rng.integers(0, V, size=(B, k)).astype(np.int32)
    wl2 = W.ChainWorkload("empty_residual", p, q, toks, "probs", "f32", 1.0, 5)
    acc, out = _run_sample(wl2)
    assert (acc < k).any()


def test_sample_probs_wide_vocabulary():
    # probability rows wider than one tile of draw chunks
    wl = W.controlled_acceptance(B=6, k=3, V=200003, seed=31, uniform_seed=32, logit_std=1.0)
    _run_sample(wl)


def test_sample_probs_many_chunks():
    # more draw chunks per row than a work-group has threads, so the chunk
    # search runs over several tiles; 16-byte aligned rows and element loads
    for V in (600000, 600001):
        wl = W.controlled_acceptance(B=3, k=2, V=V, seed=33, uniform_seed=34, logit_std=1.0)
        _run_sample(wl)


def test_sample_controlled_acceptance_full(controlled_full):
    _say("sample probs B=512 k=8 V=128256")
    _run_sample(controlled_full)


COUNTER_BYTES = (2 << 20) + 256  # SPEC_WORKSPACE_COUNTER_BYTES: fixed region at the start
PER_REQUEST_BYTES = 2 << 20      # its per-request words; then the status word, the epoch


def test_workspace_reuse_with_stale_partials(sample_path):
    """A workspace whose scratch holds garbage (as left by calls of other
    shapes) gives the same results: only the counter region must start at
    zero, and every completed call leaves it zero again."""
    ws = S.Workspace(DEV)
    buf = ws.get(S.spec_workspace_bytes(64, 9, 128256))
    buf[COUNTER_BYTES:].fill_(0xA5)
    wl = W.sample_chain(12, 5, 20000, seed=4, uniform_seed=5, target_std=2.0, noise_std=1.0,
                        temperature=0.8, dtype="bf16")
    tgt, dft = to_device(wl.target, "bf16"), to_device(wl.draft, "bf16")
    toks = ints_to_device(wl.draft_tokens)
    ref = S.spec_verify_sample(tgt, dft, toks, wl.temperature, seed=5, schedule=sample_path)
    g = W.greedy_chain(B=7, k=3, V=999, seed=3)
    gref = S.spec_verify_greedy(to_device(g.target, "f32"), ints_to_device(g.draft_tokens))
    for _ in range(3):
        got = S.spec_verify_sample(tgt, dft, toks, wl.temperature, seed=5, workspace=ws,
                                   schedule=sample_path)
        assert all(torch.equal(a, b) for a, b in zip(ref, got))
        ggot = S.spec_verify_greedy(to_device(g.target, "f32"), ints_to_device(g.draft_tokens),
                                    workspace=ws)
        assert all(torch.equal(a, b) for a, b in zip(gref, ggot))
        torch.cuda.synchronize()
        # every per-request word back to zero; the status word stays zero
        assert int(buf[:PER_REQUEST_BYTES + 8].count_nonzero()) == 0
        assert S.spec_workspace_status(ws) == 0
        buf[COUNTER_BYTES:].fill_(0x5A)


def test_greedy_bindings_write_preallocated_outputs():
    """out= hands in the output tensors: they are written in place, returned,
    and hold what freshly allocated outputs would."""
    wl = W.greedy_chain(B=6, k=3, V=5000, seed=12, dtype="bf16")
    t, tk = to_device(wl.target, "bf16"), ints_to_device(wl.draft_tokens)
    ref = S.spec_verify_greedy(t, tk)
    outs = (torch.full((6,), -9, dtype=torch.int32, device="cuda"),
            torch.full((6, 4), -9, dtype=torch.int32, device="cuda"))
    got = S.spec_verify_greedy(t, tk, out=outs)
    assert got[0] is outs[0] and got[1] is outs[1]
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    tw = W.tree_greedy(B=5, V=3000, seed=13)
    tt, tn = to_device(tw.target, tw.dtype), ints_to_device(tw.node_tokens)
    D = int(W.tree_depths(tw.parent).max())
    ref = S.spec_verify_tree_greedy(tt, tw.parent.tolist(), tn)
    outs = tuple(torch.full(shape, -9, dtype=torch.int32, device="cuda")
                 for shape in ((5,), (5, D + 1), (5, D + 1)))
    got = S.spec_verify_tree_greedy(tt, tw.parent.tolist(), tn, out=outs)
    assert all(g is o for g, o in zip(got, outs))
    assert all(torch.equal(r, g) for r, g in zip(ref, got))
    with pytest.raises(ValueError):
        S.spec_verify_greedy(t, tk, out=(outs[0], outs[1][:, :2]))


def test_empty_batches_through_every_entry_point():
    """B = 0 through the binding: every call returns empty outputs and
    launches nothing."""
    dev = "cuda"
    k, V = 3, 1000
    t = torch.zeros(0, k + 1, V, dtype=torch.bfloat16, device=dev)
    d = torch.zeros(0, k, V, dtype=torch.bfloat16, device=dev)
    tk = torch.zeros(0, k, dtype=torch.int32, device=dev)
    acc, out = S.spec_verify_sample(t, d, tk, 0.8, seed=1)
    assert acc.shape == (0,) and out.shape == (0, k + 1)
    acc, out = S.spec_verify_greedy(t, tk)
    assert acc.shape == (0,) and out.shape == (0, k + 1)
    parent = [-1, 0, 0, 1]
    tt = torch.zeros(0, 4, V, dtype=torch.bfloat16, device=dev)
    nt = torch.zeros(0, 4, dtype=torch.int32, device=dev)
    acc, out, path = S.spec_verify_tree_greedy(tt, parent, nt)
    assert acc.shape == (0,) and out.shape == (0, 3)
    acc, out, path = S.spec_verify_tree_sample(tt, tt.clone(), parent, nt, 0.8, seed=1)
    assert acc.shape == (0,) and out.shape == (0, 3)
    torch.cuda.synchronize()
