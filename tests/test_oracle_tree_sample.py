"""Pins of the float64 tree-sampling oracle (oracle.verify.verify_tree_sample*).

The reading (multi-step speculative sampling over siblings) is pinned by
what it must satisfy, with the oracle as a black box:
  * losslessness, exactly: with each node's children drawn independently
    from the draft's distribution there, the first emitted token follows the
    target's distribution at the root, integrated over node tokens and
    uniforms (bisection on each uniform the walk consumes);
  * two tokens deep, exactly: on a tree over a toy Markov model, the first
    two tokens -- the round's second token, or a fresh target sample when
    the round emitted one -- follow p(a | s) p(b | a);
  * a chain-shaped tree gives the chain oracle's outputs (uniforms mapped
    node j <-> position j - 1 for the tests, j for the draw);
  * hand-worked cases fix what the law cannot see: siblings in increasing
    node index, the residual carried from one sibling to the next, the draw
    from the residual after the last rejection, an empty residual keeping p;
  * planted mistakes (modified copies of the oracle) fail the law tests.
"""
import inspect
import itertools
import math

import numpy as np
import pytest
from scipy import special

import oracle.rng as R
import oracle.verify as O

U_TOP = 1.0 - 2.0 ** -53


def _boundary(pred, lo=0.0, hi=U_TOP, iters=64):
    """pred is True on [0, b) and False on [b, 1): return b."""
    if not pred(lo):
        return 0.0
    if pred(hi):
        return 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if pred(mid):
            lo = mid
        else:
            hi = mid
    return hi


def tree_law(fn, target, draft, parent, toks, T, kind, dtype):
    """Exact law of the emitted sequence for fixed node tokens, over the
    uniforms: the walk is steered (u = 0 accepts a child whose test can
    pass, u = 1 - 2^-53 rejects it) and each branch's probability is the
    boundary found by bisection on the one uniform deciding it."""
    N, V = target.shape
    kids = [[] for _ in range(N)]
    for j in range(1, N):
        kids[int(parent[j])].append(j)
    law = {}

    def run(steer):
        u = np.full((N, 2), 0.5)
        for (j, s), v in steer.items():
            u[j, s] = v
        return fn(target, draft, parent, toks, u, T, kind, dtype)

    def explore(node, i, steer, prob):
        if i < len(kids[node]):
            c = kids[node][i]
            b = _boundary(lambda v: c in run({**steer, (c, 0): v}).path)
            if b > 0.0:
                explore(c, 0, {**steer, (c, 0): 0.0}, prob * b)
            if b < 1.0:
                explore(node, i + 1, {**steer, (c, 0): U_TOP}, prob * (1.0 - b))
            return
        prev = 0.0
        for t in range(V):
            bt = _boundary(lambda v: run({**steer, (node, 1): v}).tokens[-1] <= t)
            if bt > prev:
                seq = tuple(run({**steer, (node, 1): 0.5 * (prev + bt)}).tokens)
                law[seq] = law.get(seq, 0.0) + prob * (bt - prev)
            prev = bt

    explore(0, 0, {}, 1.0)
    return law


def _planted(old, new):
    src = inspect.getsource(O.verify_tree_sample_request)
    assert old in src
    ns = dict(O.__dict__)
    exec(src.replace(old, new), ns)
    return ns["verify_tree_sample_request"]


def _star_first_token_law(fn, p_logits, q_logits, m, T):
    """Root with m children, each child's token drawn from q: the law of the
    first emitted token, integrated over the m-tuples of tokens."""
    V = p_logits.shape[0]
    q = special.softmax(q_logits.astype(np.float64) / T)
    parent = [-1] + [0] * m
    target = np.stack([p_logits] * (m + 1)).astype(np.float32)
    draft = np.stack([q_logits] * (m + 1)).astype(np.float32)
    first = np.zeros(V)
    for tup in itertools.product(range(V), repeat=m):
        w = float(np.prod([q[x] for x in tup]))
        toks = np.array([0] + list(tup), dtype=np.int32)
        for seq, pr in tree_law(fn, target, draft, parent, toks, T, "logits", "f32").items():
            first[seq[0]] += w * pr
    return first


@pytest.mark.parametrize("m,T,seed", [(1, 1.0, 1), (2, 1.0, 2), (3, 0.8, 3), (4, 1.3, 4)])
def test_star_first_token_law_is_target(m, T, seed):
    V = 3
    rng = np.random.default_rng(seed)
    zp = (rng.standard_normal(V) * 1.5).astype(np.float32)
    zq = (zp + rng.standard_normal(V).astype(np.float32) * 1.2).astype(np.float32)
    law = _star_first_token_law(O.verify_tree_sample_request, zp, zq, m, T)
    p = special.softmax(zp.astype(np.float64) / T)
    np.testing.assert_allclose(law, p, atol=1e-12, rtol=0)


class ToyMarkov:
    """Target and draft next-token logits depending on the last token."""

    def __init__(self, V, seed, noise=1.2):
        rng = np.random.default_rng(seed)
        self.V = V
        self.tp = (rng.standard_normal((V, V)) * 1.3).astype(np.float32)
        self.tq = (self.tp + rng.standard_normal((V, V)).astype(np.float32) * noise).astype(
            np.float32)


def _two_token_law(fn, model, parent, s, T):
    """Completed law of the first two tokens after context token s."""
    V = model.V
    P = special.softmax(model.tp.astype(np.float64) / T, axis=1)
    Q = special.softmax(model.tq.astype(np.float64) / T, axis=1)
    N = len(parent)
    joint = np.zeros((V, V))
    for tup in itertools.product(range(V), repeat=N - 1):
        tok = [s] + list(tup)
        w = 1.0
        for j in range(1, N):  # child tokens drawn from the draft at the parent
            w *= Q[tok[parent[j]], tok[j]]
        if w == 0.0:
            continue
        target = model.tp[tok]
        draft = model.tq[tok]
        law = tree_law(fn, target, draft, parent, np.array(tok, dtype=np.int32), T, "logits",
                       "f32")
        for seq, pr in law.items():
            if len(seq) >= 2:
                joint[seq[0], seq[1]] += w * pr
            else:
                joint[seq[0], :] += w * pr * P[seq[0]]
    return joint, P[s][:, None] * P


@pytest.mark.parametrize("parent,seed", [([-1, 0, 0, 1], 11), ([-1, 0, 1, 1], 12),
                                         ([-1, 0, 0, 0], 13)])
def test_two_token_completed_law_is_target(parent, seed):
    m = ToyMarkov(3, seed)
    joint, want = _two_token_law(O.verify_tree_sample_request, m, parent, 1, 1.0)
    np.testing.assert_allclose(joint, want, atol=1e-12, rtol=0)


@pytest.mark.parametrize("old,new", [
    ("                p = w / mass\n", "                pass\n"),   # no residual carry
    ("w = np.maximum(0.0, p - q)", "w = np.maximum(0.0, q - p)"),   # sign flip
    ("t, m2, total = inverse_cdf(p, float(u[cur, 1]))",
     "t, m2, total = inverse_cdf(dist(target, cur), float(u[cur, 1]))"),  # draw from p
    ("accept = u[c, 0] * qx < px", "accept = u[c, 0] * px < qx"),  # u < q/p
])
def test_planted_mistakes_break_the_root_law(old, new):
    bad = _planted(old, new)
    rng = np.random.default_rng(2)
    V = 3
    zp = (rng.standard_normal(V) * 1.5).astype(np.float32)
    zq = (zp + rng.standard_normal(V).astype(np.float32) * 1.2).astype(np.float32)
    law = _star_first_token_law(bad, zp, zq, 3, 1.0)
    p = special.softmax(zp.astype(np.float64))
    assert np.max(np.abs(law - p)) > 1e-3


def test_planted_wrong_draft_row_breaks_the_two_token_law():
    bad = _planted("q = dist(draft, cur) if kids[cur] else None",
                   "q = dist(draft, 0) if kids[cur] else None")
    m = ToyMarkov(3, 11)
    joint, want = _two_token_law(bad, m, [-1, 0, 0, 1], 1, 1.0)
    assert np.max(np.abs(joint - want)) > 1e-3


def test_planted_no_reset_of_p_at_the_child_breaks_the_two_token_law():
    # keep the parent's (residual) distribution after moving to a child
    bad = _planted("        p = dist(target, cur)\n",
                   "        p = dist(target, cur) if cur == 0 else p\n")
    m = ToyMarkov(3, 12)
    joint, want = _two_token_law(bad, m, [-1, 0, 1, 1], 1, 1.0)
    assert np.max(np.abs(joint - want)) > 1e-3


# ---------------------------------------------------------------------------
# Chain-shaped trees
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("kind,dtype,T,seed", [("logits", "f32", 1.0, 3), ("logits", "bf16", 0.7, 4),
                                               ("probs", "f32", 1.0, 5)])
def test_chain_shaped_tree_equals_the_chain(kind, dtype, T, seed):
    import workloads as W

    B, k, V = 24, 5, 300
    if kind == "logits":
        wl = W.sample_chain(B, k, V, seed=seed, uniform_seed=seed + 1, target_std=2.0,
                            noise_std=1.0, temperature=T, dtype=dtype)
        target, draft, toks = wl.target, wl.draft, wl.draft_tokens
        T = wl.temperature
    else:
        rng = np.random.default_rng(seed)
        target = rng.dirichlet(np.full(V, 0.3), size=(B, k + 1)).astype(np.float32)
        draft = rng.dirichlet(np.full(V, 0.3), size=(B, k)).astype(np.float32)
        toks = rng.integers(0, V, size=(B, k)).astype(np.int32)
    u = R.chain_uniforms(seed, B, k)
    acc_c, out_c, _ = O.verify_sample(target, draft, toks, u, T, kind, dtype)
    parent = np.arange(-1, k, dtype=np.int32)  # node j's parent is j - 1
    node_toks = np.concatenate([np.zeros((B, 1), np.int32), toks], axis=1)
    # draft row j of the tree is the draft's distribution after node j (the
    # chain's draft row j); the leaf's row is never read
    tdraft = np.concatenate([draft, draft[:, :1]], axis=1)
    tu = np.empty((B, k + 1, 2))
    tu[:, 1:, 0] = u[:, :k, 0]
    tu[:, 0, 0] = 0.5
    tu[:, :, 1] = u[:, :, 1]
    acc_t, out_t, path_t, _ = O.verify_tree_sample(target, tdraft, parent, node_toks, tu, T,
                                                   kind, dtype)
    assert np.array_equal(acc_t, acc_c)
    assert np.array_equal(out_t, out_c)
    for b in range(B):
        assert list(path_t[b, : acc_t[b] + 1]) == list(range(acc_t[b] + 1))


# ---------------------------------------------------------------------------
# Hand-worked cases (probability rows, V = 3, values chosen so every ratio
# and residual can be checked by hand)
# ---------------------------------------------------------------------------

P0 = np.array([0.5, 0.3, 0.2], np.float32)
Q0 = np.array([0.25, 0.5, 0.25], np.float32)
P_LEAF = np.array([0.1, 0.1, 0.8], np.float32)


def _run(parent, toks, u, rows=None):
    N = len(parent)
    target = np.stack([P0] + [P_LEAF] * (N - 1)) if rows is None else rows[0]
    draft = np.stack([Q0] * N) if rows is None else rows[1]
    return O.verify_tree_sample_request(target, draft, parent, np.array(toks, np.int32),
                                        np.asarray(u, np.float64), 1.0, "probs", "f32")


def test_siblings_are_tried_in_increasing_node_index():
    # children 1 (token 1: ratio 0.3/0.5 = 0.6) and 2 (token 0: ratio 2);
    # u = 0.1 accepts node 1 first; the reverse order would take node 2
    r = _run([-1, 0, 0], [0, 1, 0], [[0.5, 0.5], [0.1, 0.5], [0.1, 0.3]])
    assert r.path == [0, 1] and r.tokens[0] == 1
    # drawn from P_LEAF at node 1 with u = 0.5: cumulative 0.1, 0.2, 1.0 -> token 2
    assert r.tokens == [1, 2] and r.accepted == 1


def test_residual_carries_to_the_next_sibling():
    # node 1 (token 1) rejected at u = 0.7 >= 0.6; residual
    # max(0, P0 - Q0) = [0.25, 0, 0] -> [1, 0, 0]; node 2 (token 2) then has
    # ratio 0 / 0.25 = 0 and is rejected for every u (against P0 it would be
    # 0.2 / 0.25 = 0.8 and u = 0.1 would accept it); node 3 (token 0) has
    # ratio 1 / 0.25 = 4: accepted
    r = _run([-1, 0, 0, 0], [0, 1, 2, 0], [[0.5, 0.5], [0.7, 0.5], [0.1, 0.5], [0.99, 0.5]])
    kinds = [(d.kind, d.position, d.outcome) for d in r.decisions]
    assert kinds[:5] == [("accept", 1, 0), ("residual", 1, 1), ("accept", 2, 0),
                         ("residual", 2, 1), ("accept", 3, 1)]
    assert r.path == [0, 3] and r.tokens[0] == 0
    resid1 = [d for d in r.decisions if d.kind == "residual"][0]
    assert abs(resid1.margin - 0.25) < 1e-7


def test_draw_after_the_last_rejection_is_from_the_residual():
    # both children rejected (token 1 at u = 0.9; then token 1 again:
    # residual [1, 0, 0] gives ratio 0); residual after the second rejection
    # max(0, [1, 0, 0] - Q0) = [0.75, 0, 0] -> [1, 0, 0]: token 0 for any u
    for ud in (0.0, 0.5, 0.999):
        r = _run([-1, 0, 0], [0, 1, 1], [[0.5, ud], [0.9, 0.5], [0.0, 0.5]])
        assert r.accepted == 0 and r.path == [0] and r.tokens == [0]
    # with P0 itself (no residual) u = 0.999 would give token 2


def test_empty_residual_keeps_p():
    # draft = target at the root: an out-of-range first child is rejected,
    # max(0, p - q) is all zero, so p stays; the second child (ratio 1) is
    # accepted for any u < 1
    rows = (np.stack([P0, P_LEAF, P_LEAF]), np.stack([P0, P0, P0]))
    r = _run([-1, 0, 0], [0, 7, 2], [[0.5, 0.5], [0.0, 0.5], [0.999, 0.5]], rows)
    kinds = [(d.kind, d.position, d.outcome) for d in r.decisions]
    assert kinds[:3] == [("accept", 1, 0), ("residual", 1, 0), ("accept", 2, 1)]
    assert r.path == [0, 2] and r.tokens[0] == 2


def test_leaf_draws_the_bonus_from_its_target_row():
    # a single child accepted (q = p at the root: ratio 1), then the leaf's
    # draw from P_LEAF: cumulative 0.1, 0.2, 1.0
    rows = (np.stack([P0, P_LEAF]), np.stack([P0, P0]))
    for ud, want in ((0.05, 0), (0.15, 1), (0.2, 2), (0.9, 2)):
        r = _run([-1, 0], [0, 1], [[0.5, 0.5], [0.3, ud]], rows)
        assert r.path == [0, 1] and r.tokens == [1, want]


def test_tree_uniform_layout():
    u = R.tree_uniforms(99, 3, 7, counter0=5)
    flat = R.uniforms_loop(99, 5, 3 * 7 * 2)
    for b in range(3):
        for j in range(7):
            for s in range(2):
                assert u[b, j, s] == flat[(b * 7 + j) * 2 + s]
    assert np.array_equal(R.tree_uniforms(3, 2, 5), R.chain_uniforms(3, 2, 4))


def test_stop_structure_on_the_static_tree():
    import workloads as W

    parent = W.static_tree_parents()
    N, V = len(parent), 50
    rng = np.random.default_rng(7)
    B = 40
    target = (rng.standard_normal((B, N, V)) * 2).astype(np.float32)
    draft = (target + rng.standard_normal((B, N, V)).astype(np.float32)).astype(np.float32)
    toks = rng.integers(0, V, size=(B, N)).astype(np.int32)
    u = R.tree_uniforms(8, B, N)
    acc, out, path, res = O.verify_tree_sample(target, draft, parent, toks, u, 1.0, "logits",
                                               "f32")
    depth = np.zeros(N, np.int64)
    for j in range(1, N):
        depth[j] = depth[parent[j]] + 1
    for b in range(B):
        n = int(acc[b])
        pth = list(path[b, : n + 1])
        assert pth[0] == 0 and all(parent[pth[i + 1]] == pth[i] for i in range(n))
        assert depth[pth[-1]] == n
        assert list(out[b, :n]) == [int(toks[b, j]) for j in pth[1:]]
        assert 0 <= out[b, n] < V and (out[b, n + 1:] == -1).all() and (path[b, n + 1:] == -1).all()
        # margins of every accept decision bound |u - ratio|
        for d in res[b].decisions:
            if d.kind == "accept" and math.isfinite(d.margin):
                assert d.margin >= 0.0
