"""GPU parity of spec_verify_tree_sample against the float64 oracle, through
the C ABI.

* The static 60-node tree (branching 4, 3, 2, 2, 1) with draft logits, at
  B = 16, V = 128256, bf16, T = 0.7: every request element by element by
  the first-differing-decision rule (a disagreement must sit within 1e-5 of
  its boundary in the oracle), with explicit uniforms and with the seeded
  counter.
* Shapes that span the kernels' cases: float32 and bfloat16 logits, ragged V
  (the scalar loads), probability rows, a 20-deep chain, a 9-child star, a
  random 300-node tree (the full-size table setup), a root with no
  children, a 100-child star (children in two tiles of the walk),
  out-of-range node tokens, a root whose draft row equals its target row
  so the residual after a rejection is empty, and masked (-inf) logits
  with logits spread wide at a low temperature (the float64 statistics'
  reference handling); a call captured into a HIP graph and replayed on
  new inputs, with eager calls of another shape in between; V = 300000
  (more statistic chunks and draw chunks than the kernels keep at once).
* Statistics: with every child's token drawn from the draft at its parent,
  the first emitted token follows the target's root distribution
  (chi-square over 40000 requests).
"""
import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle.rng as R
import oracle.verify as O
import verify_accept_sampling_amd as S
import workloads as W
from parity_helpers import compare_tree_sample, ints_to_device, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _run_gpu(wl, u=None, counter0=0, kind=None, ws=None):
    dt = wl.dtype
    tgt = to_device(wl.target, dt)
    dft = to_device(wl.draft, dt)
    toks = ints_to_device(wl.node_tokens)
    uu = None if u is None else torch.from_numpy(np.ascontiguousarray(u, np.float32)).cuda()
    acc, out, path = S.spec_verify_tree_sample(tgt, dft, wl.parent.tolist(), toks,
                                               wl.temperature, uniforms=uu,
                                               seed=wl.uniform_seed, counter0=counter0,
                                               kind=kind or wl.kind, workspace=ws)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy(), path.cpu().numpy()


def _check(wl, acc, out, path, counter0=0, kind=None):
    u = R.tree_uniforms(wl.uniform_seed, wl.B, wl.n_nodes, counter0)
    acc_o, out_o, path_o, res = O.verify_tree_sample(wl.target, wl.draft, wl.parent,
                                                     wl.node_tokens, u, wl.temperature,
                                                     kind or wl.kind, wl.dtype)
    st = compare_tree_sample(acc, out, path, res, wl.parent, range(wl.B))
    assert st["unflagged"] == 0, st["unflagged_requests"][:5]
    # structure of every output
    D = out.shape[1] - 1
    for b in range(wl.B):
        n = int(acc[b])
        assert 0 <= n <= D
        assert path[b, 0] == 0 and all(wl.parent[path[b, i + 1]] == path[b, i] for i in range(n))
        assert list(out[b, :n]) == [int(wl.node_tokens[b, j]) for j in path[b, 1: n + 1]]
        assert (out[b, n + 1:] == -1).all() and (path[b, n + 1:] == -1).all()
        assert -1 <= out[b, n] < wl.V
    return st


def test_static_tree_full_size():
    _say("tree sampling: static 60-node tree, B=16 V=128256 bf16 T=0.7")
    wl = W.tree_sample()
    u = R.tree_uniforms(wl.uniform_seed, wl.B, wl.n_nodes)
    acc, out, path = _run_gpu(wl, u=u)
    st = _check(wl, acc, out, path)
    _say(f"  {st}")
    assert st["mismatches"] <= 1
    # the seeded counter gives the same outputs as the same uniforms passed in
    acc2, out2, path2 = _run_gpu(wl)
    assert np.array_equal(acc, acc2) and np.array_equal(out, out2) and np.array_equal(path, path2)
    # a later call on the same workspace with another counter
    ws = S.Workspace("cuda")
    for c0 in (0, 10 ** 6):
        acc3, out3, path3 = _run_gpu(wl, counter0=c0, ws=ws)
        _check(wl, acc3, out3, path3, counter0=c0)


def _random_tree(N, rng, max_children=None):
    parent = [-1]
    kids = [0]
    for j in range(1, N):
        while True:
            p = int(rng.integers(0, j))
            if max_children is None or kids[p] < max_children:
                break
        parent.append(p)
        kids[p] += 1
        kids.append(0)
    return np.array(parent, dtype=np.int32)


def _shape_cases():
    rng = np.random.default_rng(5)
    chain = np.arange(-1, 20, dtype=np.int32)
    star = np.array([-1] + [0] * 9, dtype=np.int32)
    big = _random_tree(300, rng, max_children=6)
    mid = _random_tree(40, rng)
    return [
        ("chain20_f32_V1000", chain, 24, 1000, "f32", 1.0, 11),
        ("star9_bf16_V4097", star, 32, 4097, "bf16", 0.8, 12),
        ("mid40_bf16_V32000", mid, 16, 32000, "bf16", 1.0, 13),
        ("mid40_f32_V3001", mid, 16, 3001, "f32", 1.3, 14),
        ("big300_bf16_V2048", big, 4, 2048, "bf16", 1.0, 15),
        ("root_only_bf16_V5000", np.array([-1], np.int32), 8, 5000, "bf16", 1.0, 16),
    ]


@pytest.mark.parametrize("case", _shape_cases(), ids=lambda c: c[0])
def test_tree_shapes(case):
    name, parent, B, V, dt, T, seed = case
    _say(f"tree sampling: {name}")
    wl = W.tree_sample(B=B, V=V, seed=seed, uniform_seed=77, parent=parent,
                       target_std=2.0, noise_std=1.0, temperature=T, n_peaks=0, dtype=dt)
    acc, out, path = _run_gpu(wl)
    _check(wl, acc, out, path)


def test_out_of_range_tokens_and_empty_residual():
    _say("tree sampling: out-of-range node tokens, empty residual at the root")
    parent = np.array([-1, 0, 0, 0, 1, 1], dtype=np.int32)
    wl = W.tree_sample(B=64, V=3000, seed=9, uniform_seed=10, parent=parent, target_std=2.0,
                       noise_std=1.0, temperature=1.0, n_peaks=0, dtype="f32")
    wl.node_tokens[::2, 1] = wl.V + 5      # out of range: rejected, residual taken
    wl.node_tokens[1::4, 2] = -3
    wl.draft[::2, 0] = wl.target[::2, 0]   # q = p at the root: the residual is empty
    acc, out, path = _run_gpu(wl)
    st = _check(wl, acc, out, path)
    # the even requests: node 1 rejected, p kept, node 2 (ratio 1) accepted
    u = R.tree_uniforms(wl.uniform_seed, wl.B, wl.n_nodes)
    _, _, _, res = O.verify_tree_sample(wl.target, wl.draft, wl.parent, wl.node_tokens, u,
                                        wl.temperature, "logits", "f32")
    kept = sum(1 for b in range(0, wl.B, 2)
               if any(d.kind == "residual" and d.outcome == 0 for d in res[b].decisions))
    assert kept > 0
    assert st["mismatches"] == 0


def test_wide_star_children_past_one_wave():
    # 100 children at the root: the walk takes them in tiles of 64; the
    # first 70 are made to fail (out-of-range tokens) in even requests, so
    # the tests reach the second tile through 70 residual updates
    _say("tree sampling: a 100-child star, 70 forced rejections")
    parent = np.array([-1] + [0] * 100, dtype=np.int32)
    wl = W.tree_sample(B=8, V=1024, seed=21, uniform_seed=22, parent=parent, target_std=2.0,
                       noise_std=1.0, temperature=1.0, n_peaks=0, dtype="bf16")
    wl.node_tokens[::2, 1:71] = wl.V + 1
    acc, out, path = _run_gpu(wl)
    st = _check(wl, acc, out, path)
    assert st["mismatches"] == 0
    assert all(path[b, 1] > 70 or acc[b] == 0 for b in range(0, wl.B, 2))


@pytest.mark.parametrize("n_children", [63, 64])
def test_star_at_the_lane_limit(n_children):
    # 64 nodes (one per lane: the walk holds every node in registers) and
    # 65 (tables in shared memory); the first 40 children are made to fail
    # in even requests, so the walk applies 40 residual updates before the
    # first child it can accept
    _say(f"tree sampling: a {n_children}-child star, 40 forced rejections")
    parent = np.array([-1] + [0] * n_children, dtype=np.int32)
    wl = W.tree_sample(B=8, V=1024, seed=23, uniform_seed=24, parent=parent, target_std=2.0,
                       noise_std=1.0, temperature=1.0, n_peaks=0, dtype="bf16")
    wl.node_tokens[::2, 1:41] = wl.V + 1
    acc, out, path = _run_gpu(wl)
    st = _check(wl, acc, out, path)
    assert st["mismatches"] == 0
    assert all(path[b, 1] > 40 or acc[b] == 0 for b in range(0, wl.B, 2))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_masked_and_wide_low_temperature_logits(dt):
    """The float64 row statistics' reference: rows whose first element is
    masked (-inf), a first 16384-element chunk wholly masked, about 30% of
    every row masked, and logits spread so wide at T = 0.1 that elements
    exceed a row's first element by far more than 400 binades of the
    scaled exponent (the reference moves up, and chunks with different
    references merge by rescaling).  Masked tokens are never emitted."""
    _say(f"tree sampling: masked and wide low-temperature logits, {dt}")
    rng = np.random.default_rng(31)
    parent = np.array([-1, 0, 0, 0, 1, 1, 2, 4, 4, 6], dtype=np.int32)
    B, V = 12, 40000
    wl = W.tree_sample(B=B, V=V, seed=33, uniform_seed=34, parent=parent, target_std=20.0,
                       noise_std=4.0, temperature=0.1, n_peaks=0, dtype=dt)
    N = wl.n_nodes
    mask = rng.random((B, N, V)) < 0.3
    mask[::2, :, 0] = True             # the first element of every other request's rows
    mask[1::3, :3, :16384] = True      # a whole first statistics chunk
    neg = np.uint16(0xFF80) if dt == "bf16" else np.float32(-np.inf)
    for arr in (wl.target, wl.draft):
        arr[mask] = neg
    # node tokens: drawn again from the masked draft at the parent
    yq = W.logits_as_f32(wl.draft, dt).astype(np.float64) / wl.temperature
    for j in range(1, N):
        for b in range(B):
            row = yq[b, parent[j]]
            pr = np.exp(row - row.max())
            wl.node_tokens[b, j] = rng.choice(V, p=pr / pr.sum())
    acc, out, path = _run_gpu(wl)
    st = _check(wl, acc, out, path)
    assert st["mismatches"] == 0
    zt = W.logits_as_f32(wl.target, dt)
    for b in range(B):
        n = int(acc[b])
        node = int(path[b, n])
        tok = int(out[b, n])
        assert tok >= 0 and np.isfinite(zt[b, node, tok]), (b, node, tok)


def test_large_vocabulary():
    """V = 300000: more than 8 statistic chunks per row (the merges' second
    batch) and more than 512 draw chunks (the pick's tiles past those it
    keeps in registers)."""
    _say("tree sampling: V=300000")
    parent = np.array([-1, 0, 0, 1, 1], dtype=np.int32)
    wl = W.tree_sample(B=6, V=300000, seed=61, uniform_seed=62, parent=parent, target_std=2.0,
                       noise_std=1.0, temperature=1.0, n_peaks=0, dtype="bf16")
    wl.node_tokens[::2, 1] = wl.V + 1  # rejected: draws from residuals over the whole row
    acc, out, path = _run_gpu(wl)
    st = _check(wl, acc, out, path)
    assert st["mismatches"] == 0


def test_graph_capture_and_replay():
    """A tree-sampling call captured into a HIP graph and replayed on new
    inputs (copied into the captured tensors), with an eager call of another
    tree and shape on the same workspace between replays: every replay and
    every eager call matches the oracle (the draw's completion tickets and
    the tables leave the workspace ready for the next call)."""
    _say("tree sampling: graph capture and replay")
    parent = np.array([-1, 0, 0, 0, 1, 1, 2, 4, 4, 5], dtype=np.int32)
    B, V, T = 8, 20000, 0.9
    wls = [W.tree_sample(B=B, V=V, seed=80 + r, uniform_seed=90 + r, parent=parent,
                         target_std=2.0, noise_std=1.0, temperature=T, n_peaks=0, dtype="bf16")
           for r in range(3)]
    N = len(parent)
    dev = torch.device("cuda")
    tgt = to_device(wls[0].target, "bf16")
    dft = to_device(wls[0].draft, "bf16")
    toks = ints_to_device(wls[0].node_tokens)
    ug = torch.empty(B, N, 2, dtype=torch.float32, device=dev)
    D = int(W.tree_depths(parent).max())
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty(B, D + 1, dtype=torch.int32, device=dev)
    path = torch.empty(B, D + 1, dtype=torch.int32, device=dev)
    ws = S.Workspace(dev)
    ws.get(S.spec_workspace_bytes(16, 61, 128256))

    def call():
        S.spec_verify_tree_sample(tgt, dft, parent.tolist(), toks, T, uniforms=ug,
                                  workspace=ws, out=(acc, out, path))

    u0 = R.tree_uniforms(wls[0].uniform_seed, B, N, 0)
    ug.copy_(torch.from_numpy(np.ascontiguousarray(u0, np.float32)))
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    other = W.tree_sample(B=5, V=3001, seed=95, uniform_seed=96,
                          parent=np.array([-1, 0, 0, 1, 1, 1, 2], np.int32), target_std=2.0,
                          noise_std=1.0, temperature=1.0, n_peaks=0, dtype="f32")
    for r, wl in enumerate(wls):
        u = R.tree_uniforms(wl.uniform_seed, B, N, 0)
        tgt.copy_(to_device(wl.target, "bf16"))
        dft.copy_(to_device(wl.draft, "bf16"))
        toks.copy_(ints_to_device(wl.node_tokens))
        ug.copy_(torch.from_numpy(np.ascontiguousarray(u, np.float32)))
        acc.fill_(-7)
        out.fill_(-7)
        path.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        st = _check(wl, acc.cpu().numpy(), out.cpu().numpy(), path.cpu().numpy())
        _say(f"  replay {r}: {st['mismatches']} mismatches")
        a2, o2, p2 = _run_gpu(other, ws=ws)
        _check(other, a2, o2, p2)
    assert S.spec_workspace_status(ws) == 0


def test_probability_rows():
    _say("tree sampling: probability rows, mid tree, V=20000")
    rng = np.random.default_rng(3)
    parent = _random_tree(30, rng, max_children=4)
    B, V = 12, 20000
    N = len(parent)
    target = rng.dirichlet(np.full(V, 0.05), size=(B, N)).astype(np.float32)
    draft = (0.5 * target + 0.5 * rng.dirichlet(np.full(V, 0.05), size=(B, N))).astype(
        np.float32)
    toks = np.zeros((B, N), np.int32)
    for j in range(1, N):
        for b in range(B):
            q = draft[b, parent[j]].astype(np.float64)
            toks[b, j] = rng.choice(V, p=q / q.sum())
    wl = W.TreeSampleWorkload("tree_probs", target, draft, parent, toks, "probs", "f32", 1.0,
                              55)
    acc, out, path = _run_gpu(wl)
    _check(wl, acc, out, path)


def test_first_token_law_chi_square():
    """Children drawn from the draft at the root: the first emitted token
    follows p_root (losslessness), over requests with independent node
    tokens and uniforms."""
    _say("tree sampling: first-token law, 40000 requests, V=16")
    rng = np.random.default_rng(21)
    B, V, T = 40000, 16, 1.0
    parent = np.array([-1, 0, 0, 0, 1, 1, 2], dtype=np.int32)
    N = len(parent)
    zp = (rng.standard_normal(V) * 1.5).astype(np.float32)
    zq = (zp + rng.standard_normal(V).astype(np.float32) * 1.2).astype(np.float32)
    target = np.broadcast_to(zp, (B, N, V)).copy()
    draft = np.broadcast_to(zq, (B, N, V)).copy()
    q = special.softmax(zq.astype(np.float64) / T)
    toks = rng.choice(V, size=(B, N), p=q).astype(np.int32)
    wl = W.TreeSampleWorkload("tree_law", target, draft, parent, toks, "logits", "f32", T, 123)
    acc, out, path = _run_gpu(wl)
    first = out[:, 0]
    counts = np.bincount(first, minlength=V)
    p = special.softmax(zp.astype(np.float64) / T)
    pval = stats.chisquare(counts, p * B).pvalue
    _say(f"  chi-square p-value {pval:.3g}")
    assert pval > 1e-4
