"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself:
  * published SplitMix64 outputs (golden file);
  * the printed expected-tokens table (golden file) and its closed form;
  * losslessness: the exact law of an emitted token equals the target
    distribution p, integrated over the uniforms with the oracle as a black
    box (bisection on u), for logits and probability inputs;
  * end-to-end: speculative decoding of a toy Markov "target model" with the
    oracle as verifier reproduces plain greedy decoding exactly, and plain
    ancestral sampling in law (chi-square);
  * special cases (q = p; q one-hot on a token p gives no mass);
  * tree greedy against brute-force path enumeration and against the chain
    rule on a chain-shaped tree;
  * planted mistakes (a modified copy of the oracle) must fail the law tests.
"""
import inspect
import math
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle.rng as R
import oracle.verify as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------
# SplitMix64
# ---------------------------------------------------------------------------


def test_splitmix64_published_outputs():
    rows = _read_golden("splitmix64_seed0.txt")
    want = [int(h, 16) for _, h in rows]
    assert R.splitmix64_stream(0, len(want)) == want
    # counter form = stream form
    assert [R.splitmix64_output(0, i) for i in range(len(want))] == want


def test_uniform_grid_and_law():
    u = R.uniforms(7, 0, 200_000)
    assert np.array_equal(u[:2000], R.uniforms_loop(7, 0, 2000))
    scaled = u * 2.0 ** 24
    assert np.all(scaled == np.floor(scaled))
    assert u.min() >= 0.0 and u.max() <= 1.0 - 2.0 ** -24
    hist = np.histogram(u, bins=32, range=(0, 1))[0]
    assert stats.chisquare(hist).pvalue > 1e-4
    # counter offsets address the same stream
    assert np.array_equal(R.uniforms(7, 1000, 50), u[1000:1050])
    # wrap-around of the 64-bit counter
    big = (1 << 64) - 3
    assert np.array_equal(R.uniforms(11, big, 6), R.uniforms_loop(11, big, 6))


def test_chain_uniform_layout():
    u = R.chain_uniforms(5, 3, 4, counter0=17)
    flat = R.uniforms(5, 17, 3 * 5 * 2)
    assert u.shape == (3, 5, 2)
    for b in range(3):
        for i in range(5):
            for s in range(2):
                assert u[b, i, s] == flat[(b * 5 + i) * 2 + s]


# ---------------------------------------------------------------------------
# Black-box integration over the uniforms
# ---------------------------------------------------------------------------

U_TOP = 1.0 - 2.0 ** -53


def _boundary(pred, lo=0.0, hi=U_TOP, iters=64):
    """pred is True on [0, b) and False on [b, 1): return b (bisection)."""
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


def first_token_law(fn, target, draft, T, kind, dtype):
    """Exact law of the first emitted token of a k=1 chain with draft token
    x ~ q, u_acc, u_res ~ U[0, 1), using `fn` (an oracle request function)
    as a black box.  target [2, V], draft [1, V]."""
    V = target.shape[1]
    if kind == "logits":
        q = special.softmax(W.logits_as_f32(draft[0], dtype).astype(np.float64) / T)
    else:
        q = draft[0].astype(np.float64)
        q = q / q.sum()
    law = np.zeros(V)
    for x in range(V):
        if q[x] == 0.0:
            continue
        toks = np.array([x])

        def run(ua, ur):
            u = np.array([[ua, ur], [0.5, 0.5]])
            return fn(target, draft, toks, u, T, kind, dtype)

        p_acc = _boundary(lambda ua: run(ua, 0.5).accepted == 1)
        law[x] += q[x] * p_acc
        if p_acc >= 1.0:
            continue
        # rejection: token as a nondecreasing function of u_res
        prev = 0.0
        for j in range(V):
            b = _boundary(lambda ur: run(U_TOP, ur).tokens[0] <= j)
            law[j] += q[x] * (1.0 - p_acc) * (b - prev)
            prev = b
    return law


def _planted(old, new):
    src = inspect.getsource(O.verify_sample_request)
    assert old in src
    ns = dict(O.__dict__)
    exec(src.replace(old, new), ns)
    return ns["verify_sample_request"]


def _tiny_rows(seed, V, kind):
    rng = np.random.default_rng(seed)
    if kind == "logits":
        t = (rng.standard_normal((2, V)) * 1.5).astype(np.float32)
        d = (t[:1] + rng.standard_normal((1, V)).astype(np.float32)).astype(np.float32)
        return t, d
    p = rng.dirichlet(np.ones(V), size=2).astype(np.float32)
    q = rng.dirichlet(np.ones(V), size=1).astype(np.float32)
    return p, q


@pytest.mark.parametrize("kind,T,seed", [("logits", 1.0, 1), ("logits", 0.7, 2),
                                         ("logits", 1.9, 3), ("probs", 1.0, 4),
                                         ("probs", 1.0, 5)])
def test_emitted_token_law_equals_target(kind, T, seed):
    """Losslessness: min(p,q) + max(0,p-q) = p, so the emitted token ~ p."""
    V = 5
    t, d = _tiny_rows(seed, V, kind)
    law = first_token_law(O.verify_sample_request, t, d, T, kind, "f32")
    if kind == "logits":
        p = special.softmax(t[0].astype(np.float64) / T)
    else:
        p = t[0].astype(np.float64)
        q = d[0].astype(np.float64)
        # unnormalised rows: the law is p up to the float32 normalisation error
        p = p  # used as given
        assert abs(p.sum() - 1) < 1e-6 and abs(q.sum() - 1) < 1e-6
    tol = 1e-12 if kind == "logits" else 2e-6
    np.testing.assert_allclose(law, p, atol=tol, rtol=0)


def test_emitted_token_law_bf16_inputs():
    V = 6
    rng = np.random.default_rng(9)
    t = W.f32_to_bf16_bits((rng.standard_normal((2, V)) * 2).astype(np.float32))
    d = W.f32_to_bf16_bits((rng.standard_normal((1, V)) * 2).astype(np.float32))
    law = first_token_law(O.verify_sample_request, t, d, 0.8, "logits", "bf16")
    p = special.softmax(W.bf16_bits_as_f32(t[0]).astype(np.float64) / 0.8)
    np.testing.assert_allclose(law, p, atol=1e-12, rtol=0)


@pytest.mark.parametrize("old,new", [
    ("w = np.maximum(0.0, p - q)", "w = p.copy()"),            # resample from p
    ("w = np.maximum(0.0, p - q)", "w = np.maximum(0.0, q - p)"),  # sign flip
    ("accept = u[i, 0] * qx < px", "accept = u[i, 0] * px < qx"),  # u < q/p
    ("accept = u[i, 0] * qx < px", "accept = u[i, 0] < px"),       # u < p
])
def test_planted_mistakes_break_the_law(old, new):
    bad = _planted(old, new)
    V = 5
    t, d = _tiny_rows(1, V, "logits")
    law = first_token_law(bad, t, d, 1.0, "logits", "f32")
    p = special.softmax(t[0].astype(np.float64))
    assert np.max(np.abs(law - p)) > 1e-3


def test_residual_mass_is_total_variation():
    rng = np.random.default_rng(3)
    V = 40
    for trial in range(20):
        t = (rng.standard_normal((2, V)) * 2).astype(np.float32)
        d = (t[:1] + rng.standard_normal((1, V)) * 1.5).astype(np.float32)
        T = 0.9
        p = special.softmax(t[0].astype(np.float64) / T)
        q = special.softmax(d[0].astype(np.float64) / T)
        # find a rejecting uniform for the draft token with the largest q/p
        x = int(np.argmax(q / p))
        u = np.array([[U_TOP, 0.3], [0.5, 0.5]])
        r = O.verify_sample_request(t, d, np.array([x]), u, T, "logits", "f32")
        assert r.accepted == 0
        tv = 0.5 * np.abs(p - q).sum()
        assert abs(r.residual_mass - tv) < 1e-12
        assert abs(r.residual_mass - (1.0 - np.minimum(p, q).sum())) < 1e-12


# ---------------------------------------------------------------------------
# Special cases
# ---------------------------------------------------------------------------


def test_identical_draft_always_accepts_and_bonus_follows_p():
    rng = np.random.default_rng(4)
    V, k = 7, 3
    t = (rng.standard_normal((k + 1, V)) * 2).astype(np.float32)
    d = t[:k].copy()
    for trial in range(200):
        toks = rng.integers(0, V, size=k)
        u = rng.random((k + 1, 2))
        r = O.verify_sample_request(t, d, toks, u, 1.3, "logits", "f32")
        assert r.accepted == k
        assert r.tokens[:k] == [int(x) for x in toks]
    # law of the bonus token over u_res is p_k
    pk = special.softmax(t[k].astype(np.float64) / 1.3)
    prev, law = 0.0, np.zeros(V)
    toks = np.zeros(k, dtype=np.int64)
    for j in range(V):
        b = _boundary(lambda ur: O.verify_sample_request(
            t, d, toks, np.array([[0.5, 0.5]] * k + [[0.5, ur]]), 1.3,
            "logits", "f32").tokens[k] <= j)
        law[j] = b - prev
        prev = b
    np.testing.assert_allclose(law, pk, atol=1e-12)


def test_one_hot_draft_on_zero_mass_token_always_rejects():
    V = 6
    p = np.array([[0.1, 0.2, 0.0, 0.3, 0.25, 0.15], [1, 0, 0, 0, 0, 0]], dtype=np.float32)
    q = np.zeros((1, V), dtype=np.float32)
    q[0, 2] = 1.0
    law = first_token_law(O.verify_sample_request, p, q, 1.0, "probs", "f32")
    np.testing.assert_allclose(law, p[0].astype(np.float64), atol=1e-12)
    for ua in (0.0, 0.5, U_TOP):
        r = O.verify_sample_request(p, q, np.array([2]), np.array([[ua, 0.4], [0.5, 0.5]]),
                                    1.0, "probs", "f32")
        assert r.accepted == 0 and r.tokens[0] != 2


def test_out_of_range_draft_token_is_a_rejection():
    V = 5
    t, d = _tiny_rows(2, V, "logits")
    for x in (-1, V, 10 ** 6):
        r = O.verify_sample_request(t, d, np.array([x]), np.array([[0.0, 0.3], [0.5, 0.5]]),
                                    1.0, "logits", "f32")
        assert r.accepted == 0 and 0 <= r.tokens[0] < V
    acc, out, _ = O.verify_greedy(t[None], np.array([[V]]), "f32")
    assert acc[0] == 0 and out[0, 0] == int(np.argmax(t[0]))


def test_empty_residual_falls_back_to_p():
    # p <= q everywhere (q carries extra mass): any rejection has zero residual
    p = np.array([[0.2, 0.3, 0.5], [0.3, 0.3, 0.4]], dtype=np.float32)
    q = np.array([[0.2, 0.35, 0.5]], dtype=np.float32)
    u = np.array([[U_TOP, 0.1], [0.5, 0.5]])
    r = O.verify_sample_request(p, q, np.array([1]), u, 1.0, "probs", "f32")
    assert r.accepted == 0
    assert r.tokens[0] == 0  # first bin of p: 0.1 * 1.0 < 0.2
    assert any(dc.kind == "empty_residual" for dc in r.decisions)


def test_stop_bounds_and_padding():
    wl = W.sample_chain(5, 6, 300, seed=3, uniform_seed=4, target_std=2.0,
                        noise_std=1.0, temperature=1.0, dtype="f32")
    u = R.chain_uniforms(4, wl.B, wl.k)
    acc, out, res = O.verify_sample(wl.target, wl.draft, wl.draft_tokens, u,
                                    wl.temperature, wl.kind, wl.dtype)
    for b in range(wl.B):
        n = acc[b]
        assert 0 <= n <= wl.k
        assert np.all(out[b, : n] == wl.draft_tokens[b, : n])
        assert 0 <= out[b, n] < wl.V
        assert np.all(out[b, n + 1:] == -1)


# ---------------------------------------------------------------------------
# Decision margins
# ---------------------------------------------------------------------------


def test_margins_bound_the_decision_boundary():
    """Moving u by less than the recorded margin keeps the outcome; moving it
    past the margin on the side of the nearer boundary changes it."""
    rng = np.random.default_rng(12)
    V = 30
    for trial in range(40):
        t, d = _tiny_rows(100 + trial, V, "logits")
        x = int(rng.integers(0, V))
        u = rng.random((2, 2))
        r = O.verify_sample_request(t, d, np.array([x]), u, 1.0, "logits", "f32")
        acc_dec = r.decisions[0]
        m = acc_dec.margin
        if math.isfinite(m) and m > 1e-9:
            for s in (-0.5, 0.5):
                u2 = u.copy()
                u2[0, 0] = min(max(u[0, 0] + s * m, 0.0), U_TOP)
                r2 = O.verify_sample_request(t, d, np.array([x]), u2, 1.0, "logits", "f32")
                assert r2.accepted == r.accepted
        if r.accepted == 0:
            res = [dc for dc in r.decisions if dc.kind == "resample"][0]
            m = res.margin
            for s in (-0.5, 0.5):
                u2 = u.copy()
                u2[0, 1] = u[0, 1] + s * m
                r2 = O.verify_sample_request(t, d, np.array([x]), u2, 1.0, "logits", "f32")
                assert r2.tokens == r.tokens
            u2 = u.copy()
            lo_side = True
            # find which side is nearer by probing just past the margin
            changed = False
            for s in (-1.0001, 1.0001):
                u2[0, 1] = u[0, 1] + s * m
                if 0.0 <= u2[0, 1] < 1.0:
                    r2 = O.verify_sample_request(t, d, np.array([x]), u2, 1.0, "logits", "f32")
                    changed |= r2.tokens != r.tokens
            assert changed


# ---------------------------------------------------------------------------
# Expected tokens per iteration (printed table)
# ---------------------------------------------------------------------------


def _expected(alpha, k):
    return (1.0 - alpha ** (k + 1)) / (1.0 - alpha)


def test_printed_table_matches_closed_form():
    rows = _read_golden("expected_tokens_table.txt")
    for a, *vals in rows:
        for k, v in zip((2, 4, 8), vals):
            assert abs(_expected(float(a), k) - float(v)) <= 0.005 + 1e-12


@pytest.mark.parametrize("alpha", [0.6, 0.8, 0.9])
def test_per_position_acceptance_is_overlap(alpha):
    """P(accept) = sum_x q(x) min(1, p/q) = sum min(p, q) = 1 - TV(p, q)."""
    wl = W.controlled_acceptance(B=2, k=2, V=48, seed=77, alphas=(alpha,), logit_std=1.0)
    for b in range(wl.B):
        for i in range(wl.k):
            p = wl.target[b, i].astype(np.float64)
            q = wl.draft[b, i].astype(np.float64)
            tot = 0.0
            for x in range(wl.V):
                def acc(ua):
                    u = np.array([[ua, 0.5], [0.5, 0.5]])
                    return O.verify_sample_request(wl.target[b, i:i + 2], wl.draft[b, i:i + 1],
                                                   np.array([x]), u, 1.0, "probs",
                                                   "f32").accepted == 1
                tot += q[x] / q.sum() * _boundary(acc)
            assert abs(tot - alpha) < 2e-6


@pytest.mark.parametrize("alpha", [0.6, 0.8, 0.9])
@pytest.mark.parametrize("k", [2, 4, 8])
def test_mean_tokens_per_iteration_matches_table(alpha, k):
    rows = {float(r[0]): dict(zip((2, 4, 8), map(float, r[1:])))
            for r in _read_golden("expected_tokens_table.txt")}
    N = 3000
    wl = W.controlled_acceptance(B=N, k=k, V=32, seed=500 + k, alphas=(alpha,),
                                 logit_std=0.5, one_hot_mass=0.95)
    u = R.chain_uniforms(900 + k, N, k)
    acc, out, _ = O.verify_sample(wl.target, wl.draft, wl.draft_tokens, u, 1.0,
                                  "probs", "f32")
    emitted = acc.astype(np.float64) + 1.0
    se = emitted.std(ddof=1) / math.sqrt(N)
    assert abs(emitted.mean() - _expected(alpha, k)) < 4 * se
    assert abs(emitted.mean() - rows[alpha][k]) < 4 * se + 0.005


# ---------------------------------------------------------------------------
# End to end with a toy Markov target: greedy and sampling
# ---------------------------------------------------------------------------


class ToyMarkov:
    """Next-token logits depend on the previous token only: table[prev]."""

    def __init__(self, V, seed, scale=2.0):
        rng = np.random.default_rng(seed)
        self.V = V
        self.table = (rng.standard_normal((V, V)) * scale).astype(np.float32)

    def greedy(self, start, n):
        seq = [start]
        for _ in range(n):
            seq.append(int(np.argmax(self.table[seq[-1]])))
        return seq[1:]


def test_greedy_speculation_reproduces_greedy_decoding():
    m = ToyMarkov(50, 1)
    rng = np.random.default_rng(2)
    want = m.greedy(3, 60)
    for k in (1, 3, 6):
        seq = [3]
        while len(seq) < 61:
            drafts, prev = [], seq[-1]
            for _ in range(k):
                nxt = int(np.argmax(m.table[prev])) if rng.random() < 0.6 else int(rng.integers(0, m.V))
                drafts.append(nxt)
                prev = nxt
            ctx = [seq[-1]] + drafts
            target = m.table[ctx][None]  # [1, k+1, V]
            acc, out, _ = O.verify_greedy(target, np.array([drafts]), "f32")
            seq.extend(int(t) for t in out[0, : acc[0] + 1])
        assert seq[1:61] == want


def test_tree_greedy_reproduces_greedy_decoding():
    m = ToyMarkov(40, 5)
    rng = np.random.default_rng(6)
    parent = W.static_tree_parents((3, 2, 2), 12)
    want = m.greedy(7, 50)
    seq = [7]
    while len(seq) < 51:
        N = len(parent)
        tok = np.zeros(N, dtype=np.int64)
        tok[0] = seq[-1]
        for j in range(1, N):
            pa = int(tok[parent[j]])
            tok[j] = int(np.argmax(m.table[pa])) if rng.random() < 0.5 else int(rng.integers(0, m.V))
        target = m.table[tok][None]  # row j = next-token logits after node j
        acc, out, path, _ = O.verify_tree_greedy(target, parent, tok[None].astype(np.int32), "f32")
        seq.extend(int(t) for t in out[0, : acc[0] + 1])
    assert seq[1:51] == want


def test_sampling_speculation_preserves_joint_law():
    """Two-token sequences from speculative sampling with an autoregressive
    draft follow the target's joint law p(t1|s) p(t2|t1)."""
    V, T, k, N = 4, 1.0, 2, 6000
    rng = np.random.default_rng(8)
    tp = (rng.standard_normal((V, V)) * 1.2).astype(np.float32)
    tq = (tp + rng.standard_normal((V, V)).astype(np.float32) * 1.5).astype(np.float32)
    P = special.softmax(tp.astype(np.float64) / T, axis=1)
    Q = special.softmax(tq.astype(np.float64) / T, axis=1)
    s = 1
    joint = P[s][:, None] * P  # joint[t1, t2]
    counts = np.zeros((V, V))
    ctr = 0
    for n in range(N):
        seq = [s]
        while len(seq) < 3:
            drafts, prev = [], seq[-1]
            for _ in range(k):
                nxt = int(rng.choice(V, p=Q[prev]))
                drafts.append(nxt)
                prev = nxt
            ctx = [seq[-1]] + drafts
            u = R.uniforms(31, ctr, (k + 1) * 2).reshape(k + 1, 2)
            ctr += (k + 1) * 2
            r = O.verify_sample_request(tp[ctx], tq[ctx[:-1]], np.array(drafts), u, T,
                                        "logits", "f32")
            seq.extend(r.tokens)
        counts[seq[1], seq[2]] += 1
    pval = stats.chisquare(counts.ravel(), joint.ravel() * N).pvalue
    assert pval > 1e-4


# ---------------------------------------------------------------------------
# Tree greedy: brute force and chain equivalence
# ---------------------------------------------------------------------------


def _brute_tree(target, parent, tok):
    N = len(parent)
    best = (0, 0)
    for j in range(N):
        path = [j]
        while path[-1] != 0:
            path.append(int(parent[path[-1]]))
        path.reverse()
        ok = all(int(tok[path[d]]) == int(np.argmax(target[path[d - 1]]))
                 for d in range(1, len(path)))
        if ok:
            cand = (len(path) - 1, -j)
            if cand > best:
                best = cand
    node = -best[1]
    path = [node]
    while path[-1] != 0:
        path.append(int(parent[path[-1]]))
    path.reverse()
    return best[0], [int(tok[n]) for n in path[1:]] + [int(np.argmax(target[node]))], path


def test_tree_against_brute_force():
    wl = W.tree_greedy(B=40, V=12, seed=9, p_match=0.7, dtype="f32")
    # many exact ties in argmax and duplicate siblings at V=12
    acc, out, path, _ = O.verify_tree_greedy(wl.target, wl.parent, wl.node_tokens, "f32")
    for b in range(wl.B):
        n, toks, pth = _brute_tree(wl.target[b].astype(np.float64), wl.parent, wl.node_tokens[b])
        assert acc[b] == n
        assert list(out[b, : n + 1]) == toks
        assert list(path[b, : n + 1]) == pth


def test_chain_shaped_tree_equals_chain_greedy():
    wl = W.greedy_chain(B=30, k=6, V=20, seed=10, p_match=0.8)
    parent = np.arange(-1, wl.k, dtype=np.int32)  # parent[j] = j - 1
    node_tokens = np.concatenate([np.full((wl.B, 1), -7, np.int32), wl.draft_tokens], axis=1)
    acc_c, out_c, _ = O.verify_greedy(wl.target, wl.draft_tokens, "f32")
    acc_t, out_t, _, _ = O.verify_tree_greedy(wl.target, parent, node_tokens, "f32")
    assert np.array_equal(acc_c, acc_t)
    assert np.array_equal(out_c, out_t)


def test_greedy_ties_take_lowest_index():
    V = 8
    t = np.zeros((1, 2, V), dtype=np.float32)
    t[0, 0, [2, 5]] = 3.0
    t[0, 1, [1, 6]] = -1.0
    t[0, 1, [0, 2, 3, 4, 5, 7]] = -2.0
    acc, out, _ = O.verify_greedy(t, np.array([[2]]), "f32")
    assert acc[0] == 1 and list(out[0]) == [2, 1]
    acc, out, _ = O.verify_greedy(t, np.array([[5]]), "f32")
    assert acc[0] == 0 and out[0, 0] == 2


def test_planted_no_stop_at_first_reject_breaks_the_mean():
    """Ignoring the stop-at-first-rejection rule inflates the mean far past
    the printed value (alpha = 0.6, k = 8: 2.47)."""
    src = inspect.getsource(O.verify_sample_request)
    old = "        if accept:\n            continue\n"
    assert old in src
    ns = dict(O.__dict__)
    exec(src.replace(old, "        if accept or i < k - 1:\n            continue\n"), ns)
    bad = ns["verify_sample_request"]
    k, N = 8, 400
    wl = W.controlled_acceptance(B=N, k=k, V=32, seed=501, alphas=(0.6,), logit_std=0.5,
                                 one_hot_mass=0.95)
    u = R.chain_uniforms(901, N, k)
    em = [bad(wl.target[b], wl.draft[b], wl.draft_tokens[b], u[b], 1.0, "probs",
              "f32").accepted + 1 for b in range(N)]
    assert np.mean(em) > 2.47 + 1.0


@pytest.mark.parametrize("kind,dtype,T", [("logits", "f32", 0.9), ("logits", "bf16", 1.4),
                                          ("probs", "f32", 1.0)])
def test_fixed_rows_sampler_takes_the_same_decisions(kind, dtype, T):
    """The batched evaluator used for decision-rate runs reproduces
    verify_sample_request decision for decision (tokens, stop positions and
    margins identical), including an empty residual (probability rows with
    q = 1.5 p) and out-of-range draft tokens."""
    rng = np.random.default_rng(31)
    B, k, V, N = 5, 3, 40, 150
    if kind == "logits":
        t = (rng.standard_normal((B, k + 1, V)) * 2).astype(np.float32)
        d = (t[:, :k] + rng.standard_normal((B, k, V)).astype(np.float32)).astype(np.float32)
        if dtype == "bf16":
            t, d = W.f32_to_bf16_bits(t), W.f32_to_bf16_bits(d)
    else:
        t = rng.dirichlet(np.ones(V), size=(B, k + 1)).astype(np.float32)
        d = rng.dirichlet(np.ones(V), size=(B, k)).astype(np.float32)
        d[1] = (t[1, :k] * np.float32(1.5)).astype(np.float32)  # residual is empty
    toks = rng.integers(0, V, size=(B, k)).astype(np.int32)
    toks[2, 1] = V      # out of range: a rejection
    toks[3, 0] = -1
    fr = O.FixedRowsSampler(t, d, toks, T, kind, dtype)
    u = R.uniforms(77, 0, N * B * (k + 1) * 2).reshape(N, B, k + 1, 2)
    first, token, am, dm = fr.run(u)
    saw_fallback = False
    for c in range(N):
        for b in range(B):
            r = O.verify_sample_request(t[b], d[b], toks[b], u[c, b], T, kind, dtype)
            assert first[c, b] == r.accepted and token[c, b] == r.tokens[-1]
            acc_m = [x.margin for x in r.decisions if x.kind == "accept"]
            assert np.array_equal(am[c, b, :len(acc_m)], np.asarray(acc_m))
            draw = [x for x in r.decisions if x.kind == "resample"]
            assert dm[c, b] == draw[0].margin
            saw_fallback |= any(x.kind == "empty_residual" for x in r.decisions)
    assert saw_fallback == (kind == "probs")


def test_fixed_rows_sampler_without_drafts():
    rng = np.random.default_rng(5)
    t = (rng.standard_normal((3, 1, 17))).astype(np.float32)
    fr = O.FixedRowsSampler(t, np.zeros((3, 0, 17), np.float32), np.zeros((3, 0), np.int32),
                            1.0, "logits", "f32")
    u = R.uniforms(3, 0, 20 * 3 * 2).reshape(20, 3, 1, 2)
    first, token, _, _ = fr.run(u)
    assert np.all(first == 0)
    for c in range(20):
        for b in range(3):
            r = O.verify_sample_request(t[b], None, np.zeros(0, np.int32), u[c, b], 1.0,
                                        "logits", "f32")
            assert token[c, b] == r.tokens[-1]


# ---------------------------------------------------------------------------
# Probe values: p_i(x_i), q_i(x_i) and the mass drawn from at the stop
# ---------------------------------------------------------------------------
#
# The probe is what the 1e-5 probability tolerance is checked on, so the
# oracle's probe_values is pinned against the decision function (itself pinned
# by the law tests above) and against properties any softmax of z/T has:
#   * the acceptance boundary in u that verify_sample_request exhibits at
#     position i (found by bisection, the oracle used as a black box) equals
#     min(1, p_i(x_i)/q_i(x_i)) from the probe;
#   * summed over every token x, the probe's p_i(x) is 1 (logits);
#   * ratios p_i(x)/p_i(y) = exp((z_x - z_y)/T): the temperature is applied;
#   * the value at (b, i) depends on target row (b, i) and draft row (b, i)
#     only: perturbing any other row, position or request leaves it unchanged;
#   * probability rows are returned as given, bit for bit.
# Planted mistakes (wrong position, wrong request, no temperature, target and
# draft swapped) must each fail one of these.


def _probe_rows(seed, B, k, V, dtype, T):
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((B, k + 1, V)) * 1.7).astype(np.float32)
    y = (z[:, :k] + rng.standard_normal((B, k, V)) * 0.8).astype(np.float32)
    toks = rng.integers(0, V, size=(B, k)).astype(np.int32)
    if dtype == "bf16":
        return W.f32_to_bf16_bits(z), W.f32_to_bf16_bits(y), toks
    return z, y, toks


def _probe_pins_hold(fn, dtype, T, seed=31):
    """True when probe function `fn` (signature of O.probe_values) satisfies
    every property listed above on a small batch."""
    B, k, V = 3, 3, 7
    z, y, toks = _probe_rows(seed, B, k, V, dtype, T)
    zf = W.logits_as_f32(z, dtype).astype(np.float64)
    ok = True
    for b in range(B):
        pv, qv = fn(z, y, toks, T, "logits", dtype, b)
        for i in range(k):
            # acceptance boundary of the (pinned) decision function at position i
            x = int(toks[b, i])

            def accepts(ua, b=b, i=i):
                u = np.full((k + 1, 2), 0.5)
                u[:i, 0] = 0.0  # earlier positions: u = 0 accepts unless p = 0
                u[i, 0] = ua
                r = O.verify_sample_request(z[b], y[b], toks[b], u, T, "logits", dtype)
                return r.accepted > i

            # every earlier position must accept at u = 0 for the boundary at
            # i to be visible; softmax values are never 0 here
            want = _boundary(accepts)
            got = min(1.0, pv[i] / qv[i])
            ok &= abs(got - want) < 1e-12
            # normalisation and temperature, over every token of the row
            all_p = []
            for xx in range(V):
                t2 = toks.copy()
                t2[b, i] = xx
                all_p.append(fn(z, y, t2, T, "logits", dtype, b)[0][i])
            all_p = np.array(all_p)
            ok &= abs(all_p.sum() - 1.0) < 1e-12
            ratio = all_p / all_p[0]
            ok &= np.allclose(ratio, np.exp((zf[b, i] - zf[b, i, 0]) / T), rtol=1e-12, atol=0)
    # locality: perturb every row but (b, i) of target and draft
    b, i = 1, 2
    pv, qv = fn(z, y, toks, T, "logits", dtype, b)
    z2, y2 = z.copy(), y.copy()
    rng = np.random.default_rng(seed + 1)
    for bb in range(B):
        for ii in range(k + 1):
            if (bb, ii) != (b, i):
                z2[bb, ii] = rng.permutation(z2[bb, ii])
                if ii < k:
                    y2[bb, ii] = rng.permutation(y2[bb, ii])
    pv2, qv2 = fn(z2, y2, toks, T, "logits", dtype, b)
    ok &= pv2[i] == pv[i] and qv2[i] == qv[i]
    return bool(ok)


@pytest.mark.parametrize("dtype,T", [("f32", 1.0), ("f32", 0.6), ("bf16", 0.8), ("bf16", 1.7)])
def test_probe_values_pins(dtype, T):
    assert _probe_pins_hold(O.probe_values, dtype, T)


def test_probe_values_probability_rows_as_given():
    rng = np.random.default_rng(8)
    B, k, V = 2, 3, 9
    p = rng.dirichlet(np.ones(V), size=(B, k + 1)).astype(np.float32)
    q = rng.dirichlet(np.ones(V), size=(B, k)).astype(np.float32)
    toks = rng.integers(0, V, size=(B, k)).astype(np.int32)
    toks[1, 1] = V  # out of range: 0 by definition
    for b in range(B):
        pv, qv = O.probe_values(p, q, toks, 1.0, "probs", "f32", b)
        for i in range(k):
            x = int(toks[b, i])
            if 0 <= x < V:
                assert pv[i] == float(p[b, i, x]) and qv[i] == float(q[b, i, x])
            else:
                assert pv[i] == 0.0 and qv[i] == 0.0


def _planted_probe(old, new):
    src = inspect.getsource(O.probe_values)
    assert old in src, old
    ns = dict(O.__dict__)
    exec(src.replace(old, new), ns)
    return ns["probe_values"]


@pytest.mark.parametrize("old,new", [
    ("zp = decode(target[b, i], dtype)", "zp = decode(target[b, (i + 1) % (k + 1)], dtype)"),
    ("zq = decode(draft[b, i], dtype)", "zq = decode(draft[b, (i + 1) % k], dtype)"),
    ("zp = decode(target[b, i], dtype)",
     "zp = decode(target[(b + 1) % target.shape[0], i], dtype)"),
    ("pv[i] = tempered_softmax(zp, temperature)[x]", "pv[i] = tempered_softmax(zp, 1.0)[x]"),
    ("qv[i] = tempered_softmax(zq, temperature)[x]", "qv[i] = tempered_softmax(zp, temperature)[x]"),
])
def test_planted_probe_mistakes_fail(old, new):
    assert not _probe_pins_hold(_planted_probe(old, new), "f32", 0.6)


def test_bonus_mass_is_the_total_of_p():
    """At the bonus position the draw is from p_k itself, so the mass drawn
    from is sum_x p_k(x): 1 for logits (a softmax), and the sum of the given
    values for probability rows (used as given, not renormalised)."""
    rng = np.random.default_rng(14)
    k, V = 2, 11
    for T in (0.5, 1.0, 2.3):
        z = (rng.standard_normal((k + 1, V)) * 2).astype(np.float32)
        r = O.verify_sample_request(z, z[:k].copy(), np.array([1, 4]), np.full((k + 1, 2), 0.5),
                                    T, "logits", "f32")
        assert r.accepted == k
        assert abs(r.residual_mass - 1.0) < 1e-12
    p = rng.dirichlet(np.ones(V), size=k + 1).astype(np.float32)
    p[k] *= np.float32(0.75)  # an unnormalised bonus row
    r = O.verify_sample_request(p, p[:k].copy(), np.array([2, 3]), np.full((k + 1, 2), 0.5), 1.0,
                                "probs", "f32")
    assert r.accepted == k
    want = math.fsum(float(v) for v in p[k])
    assert abs(r.residual_mass - want) < 1e-15
    assert abs(r.residual_mass - 0.75) < 1e-6
