"""Mean emitted tokens of the greedy workloads against closed forms.

A greedy draft token is accepted exactly when it equals the target's argmax.
In the greedy workloads each draft (chain position, or tree node) is the
argmax with probability p_match and otherwise uniform over V tokens, so it
is accepted with probability a = p_match + (1 - p_match) / V, independently.

* Chain: the number of emitted tokens per step is 1 + the accepted prefix,
  whose mean is (1 - a^(k+1)) / (1 - a) -- the expected-token formula of the
  serving chapter's expected-token section (pinned against its printed table
  elsewhere).  For B=1, k=4, V=1000, p_match=0.7: 2.7747.
* Tree: 1 + the depth of the deepest accepted node.  tree_expected_emitted
  computes it exactly by a recursion over the tree (pinned here by brute
  force over every acceptance pattern of small trees); for the static
  61-node tree at V=128256, p_match=0.6: 5.0911.

CPU: the oracle's mean over many generated requests matches.  GPU: the
kernels' mean over many generated requests matches (5 standard errors).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle.verify as O
import verify_accept_sampling_amd as S
import workloads as W
from parity_helpers import ints_to_device, to_device


def chain_expected_emitted(a: float, k: int) -> float:
    return (1.0 - a ** (k + 1)) / (1.0 - a)


def tree_expected_emitted(parent, a: float) -> float:
    """1 + E[depth of the deepest accepted node], every non-root node accepted
    with probability a given its parent is.  f_u(d) = P(no accepted node
    below u deeper than d | u accepted) = prod over children c of
    (1 - a) + a f_c(d) for d >= depth(u)."""
    N = len(parent)
    depth = [0] * N
    kids = [[] for _ in range(N)]
    for j in range(1, N):
        depth[j] = depth[parent[j]] + 1
        kids[parent[j]].append(j)
    D = max(depth)
    f = np.zeros((N, D + 1))
    for u in range(N - 1, -1, -1):  # children have larger indices
        for d in range(D + 1):
            if d < depth[u]:
                continue
            v = 1.0
            for c in kids[u]:
                v *= (1.0 - a) + a * f[c, d]
            f[u, d] = v
    return 1.0 + sum(1.0 - f[0, d] for d in range(D))


def _brute_tree(parent, a):
    N = len(parent)
    depth = [0] * N
    for j in range(1, N):
        depth[j] = depth[parent[j]] + 1
    e = 0.0
    for bits in itertools.product((0, 1), repeat=N - 1):
        acc = [True] + [False] * (N - 1)
        pr = 1.0
        for j in range(1, N):
            pr *= a if bits[j - 1] else 1.0 - a
            acc[j] = acc[parent[j]] and bool(bits[j - 1])
        e += pr * (1 + max(depth[j] for j in range(N) if acc[j]))
    return e


@pytest.mark.parametrize("parent", [[-1, 0, 0, 1, 1, 2], [-1, 0, 1, 2, 3], [-1, 0, 0, 0, 0],
                                    [-1, 0, 1, 1, 0, 4, 2, 2]])
def test_tree_recursion_matches_brute_force(parent):
    for a in (0.3, 0.6, 0.95):
        assert abs(tree_expected_emitted(parent, a) - _brute_tree(parent, a)) < 1e-12


def test_chain_shaped_tree_gives_the_chain_formula():
    for k in (1, 4, 8):
        parent = list(range(-1, k))
        assert abs(tree_expected_emitted(parent, 0.7) - chain_expected_emitted(0.7, k)) < 1e-12


def test_workload_values():
    a1 = 0.7 + 0.3 / 1000
    assert abs(chain_expected_emitted(a1, 4) - 2.7747) < 5e-5
    a4 = 0.6 + 0.4 / 128256
    assert abs(tree_expected_emitted(W.static_tree_parents(), a4) - 5.0911) < 5e-5


def test_oracle_greedy_chain_mean():
    B, k, V = 20000, 4, 1000
    g = W.greedy_chain(B=B, k=k, V=V, seed=41)
    acc, _, _ = O.verify_greedy(g.target, g.draft_tokens, "f32")
    emitted = acc.astype(np.float64) + 1
    want = chain_expected_emitted(0.7 + 0.3 / V, k)
    se = emitted.std() / np.sqrt(B)
    assert abs(emitted.mean() - want) < 5 * se, (emitted.mean(), want, se)


def test_oracle_tree_greedy_mean():
    B, V = 3000, 64
    t = W.tree_greedy(B=B, V=V, seed=43, dtype="f32")
    acc, _, _, _ = O.verify_tree_greedy(t.target, t.parent, t.node_tokens, "f32")
    emitted = acc.astype(np.float64) + 1
    want = tree_expected_emitted(list(t.parent), 0.6 + 0.4 / V)
    se = emitted.std() / np.sqrt(B)
    assert abs(emitted.mean() - want) < 5 * se, (emitted.mean(), want, se)


@pytest.mark.gpu
def test_gpu_greedy_chain_mean():
    B, k, V = 65536, 4, 1000
    g = W.greedy_chain(B=B, k=k, V=V, seed=45)
    acc, _ = S.spec_verify_greedy(to_device(g.target, "f32"), ints_to_device(g.draft_tokens))
    torch.cuda.synchronize()
    emitted = acc.cpu().numpy().astype(np.float64) + 1
    want = chain_expected_emitted(0.7 + 0.3 / V, k)  # 2.7747
    se = emitted.std() / np.sqrt(B)
    assert abs(emitted.mean() - want) < 5 * se, (emitted.mean(), want, se)


@pytest.mark.gpu
def test_gpu_tree_greedy_mean():
    # the static 61-node tree; V = 1024 keeps the generated rows small
    B, V = 4096, 1024
    t = W.tree_greedy(B=B, V=V, seed=47)
    acc, _, _ = S.spec_verify_tree_greedy(to_device(t.target, "bf16"), t.parent.tolist(),
                                          ints_to_device(t.node_tokens))
    torch.cuda.synchronize()
    emitted = acc.cpu().numpy().astype(np.float64) + 1
    want = tree_expected_emitted(list(t.parent), 0.6 + 0.4 / V)
    se = emitted.std() / np.sqrt(B)
    assert abs(emitted.mean() - want) < 5 * se, (emitted.mean(), want, se)
