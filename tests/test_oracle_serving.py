"""Serving outputs on the CPU: the oracle's rejected-draft masks and
tree-choices converter against hand-worked cases, brute force and
invariants; the library's host-only converter and argument checks of the
mask entry points (no kernel is launched here)."""
import ctypes
import itertools

import numpy as np
import pytest

import oracle.serving as OS
import oracle.verify as O
import verify_accept_sampling_amd as S
import workloads as W

EINVAL, ETREE = -1, -5

# A five-node tree worked by hand:   0 -> 1 -> 3
#                                      |    `-> 4
#                                      `-> 2 -> 5
HAND_CHOICES = [(0,), (1,), (0, 0), (0, 1), (1, 0)]
HAND_PARENT = [-1, 0, 0, 1, 1, 2]


def test_chain_mask_hand_worked():
    got = OS.rejected_mask_chain([0, 2, 4, 7, -1], 4)
    want = np.array([[1, 1, 1, 1], [0, 0, 1, 1], [0, 0, 0, 0], [0, 0, 0, 0], [1, 1, 1, 1]],
                    dtype=bool)
    assert np.array_equal(got, want)
    assert OS.rejected_mask_chain([3], 0).shape == (1, 0)


def test_chain_mask_counts_and_prefix():
    rng = np.random.default_rng(5)
    k = 8
    n = rng.integers(0, k + 1, size=200)
    m = OS.rejected_mask_chain(n, k)
    assert np.array_equal(m.sum(axis=1), k - n)  # k - n drafts dropped
    # the kept entries form a prefix: no kept entry after a dropped one
    assert not np.any(m[:, :-1] & ~m[:, 1:])


def test_tree_mask_hand_worked():
    got = OS.rejected_mask_tree(HAND_PARENT, [3, 0, 5, 2])
    want = np.array([[0, 0, 1, 0, 1, 1],   # path 0-1-3
                     [0, 1, 1, 1, 1, 1],   # root only
                     [0, 1, 0, 1, 1, 0],   # path 0-2-5
                     [0, 1, 0, 1, 1, 1]],  # path 0-2
                    dtype=bool)
    assert np.array_equal(got, want)


def _root_paths(parent):
    paths = []
    for j in range(len(parent)):
        p, v = [], j
        while v >= 0:
            p.append(v)
            v = parent[v]
        paths.append(tuple(reversed(p)))
    return paths


@pytest.mark.parametrize("seed", range(6))
def test_tree_mask_brute_force(seed):
    # node j is kept iff its root path is a prefix of the deepest node's
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    parent = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
    paths = _root_paths(parent)
    for d in range(n):
        m = OS.rejected_mask_tree(parent, [d])[0]
        for j in range(n):
            kept = paths[d][:len(paths[j])] == paths[j]
            assert m[j] == (not kept)
        assert (~m).sum() == len(paths[d])  # depth(d) + 1 nodes stay
        assert not m[0]


def test_tree_mask_matches_oracle_tree_outputs():
    # the kept non-root nodes, by depth, carry the accepted tokens
    wl = W.tree_greedy(B=12, V=50, seed=11, p_match=0.7, dtype="f32")
    acc, out, path, _ = O.verify_tree_greedy(wl.target, wl.parent, wl.node_tokens, wl.dtype)
    deepest = [int(path[b, acc[b]]) for b in range(wl.B)]
    m = OS.rejected_mask_tree(wl.parent, deepest)
    depth = W.tree_depths(wl.parent)
    for b in range(wl.B):
        kept = sorted((int(depth[j]), j) for j in range(len(wl.parent)) if not m[b, j])
        assert [j for _, j in kept] == [int(v) for v in path[b, :acc[b] + 1]]
        assert [int(wl.node_tokens[b, j]) for _, j in kept[1:]] == list(out[b, :acc[b]])


def test_padding():
    slots = np.arange(12, dtype=np.int64).reshape(3, 4) + 100
    m = OS.rejected_mask_chain([1, 4, 0], 4)
    got = OS.apply_padding(slots, m, -7)
    assert got.tolist() == [[100, -7, -7, -7], [104, 105, 106, 107], [-7, -7, -7, -7]]
    assert slots[0, 1] == 101  # the input is left alone


def _choices_from_parent(parent):
    # sibling rank = order among the node's siblings in node order
    rank, seen, ch = {}, {}, {0: ()}
    for j in range(1, len(parent)):
        p = parent[j]
        rank[j] = seen.get(p, 0)
        seen[p] = rank[j] + 1
        ch[j] = ch[p] + (rank[j],)
    return [ch[j] for j in range(1, len(parent))]


def test_choices_hand_worked_and_round_trip():
    assert OS.parent_from_choices(HAND_CHOICES) == HAND_PARENT
    assert OS.parent_from_choices([]) == [-1]
    rng = np.random.default_rng(2)
    for _ in range(20):
        n = int(rng.integers(1, 80))
        parent = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
        assert OS.parent_from_choices(_choices_from_parent(parent)) == parent


def test_choices_level_counts():
    # drafts per level, counted from the tuples' lengths as the serving code
    # does, equal the node counts per depth of the parent array
    choices = W.static_tree_choices()
    parent = OS.parent_from_choices(choices)
    depth = W.tree_depths(np.asarray(parent))
    D = len(choices[-1])
    per_level = [0] * D
    for c in choices:
        per_level[len(c) - 1] += 1
    assert per_level == [int((depth == d).sum()) for d in range(1, D + 1)]
    assert parent == W.static_tree_parents().tolist()


@pytest.mark.parametrize("bad", [[(0,), (0,)], [(0, 0)], [(1, 0), (1,)], [(0,), (-1,)], [()]])
def test_choices_errors(bad):
    with pytest.raises(OS.TreeChoicesError):
        OS.parent_from_choices(bad)


# ---- the library's host-only converter and argument checks ----------------

@pytest.fixture(scope="module")
def lib():
    return S.load_library()


def test_library_converter_matches_oracle(lib):
    assert S.spec_tree_from_choices(HAND_CHOICES) == HAND_PARENT
    assert S.spec_tree_from_choices([]) == [-1]
    cs = W.static_tree_choices()
    assert S.spec_tree_from_choices(cs) == OS.parent_from_choices(cs)
    chain = [tuple([0] * d) for d in range(1, 1024)]  # deepest tree the verifier takes
    assert S.spec_tree_from_choices(chain) == OS.parent_from_choices(chain)
    rng = np.random.default_rng(9)
    for _ in range(10):
        n = int(rng.integers(1, 300))
        parent = [-1] + [int(rng.integers(0, j)) for j in range(1, n)]
        cs = _choices_from_parent(parent)
        assert S.spec_tree_from_choices(cs) == parent


@pytest.mark.parametrize("bad,code", [([(0,), (0,)], ETREE), ([(0, 0)], ETREE),
                                      ([(1, 0), (1,)], ETREE), ([(0,), (-1,)], ETREE),
                                      ([()], EINVAL), ([(0,)] + [(0, i) for i in range(1023)], EINVAL)])
def test_library_converter_errors(lib, bad, code):
    with pytest.raises(S.SpecVerifyError) as e:
        S.spec_tree_from_choices(bad)
    assert e.value.code == code


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation


def test_mask_argument_checks(lib):
    assert lib.spec_rejected_mask(FAKE, -1, 4, FAKE, None, -1, None) == EINVAL
    assert lib.spec_rejected_mask(FAKE, 65537, 4, FAKE, None, -1, None) == EINVAL
    assert lib.spec_rejected_mask(FAKE, 2, 1024, FAKE, None, -1, None) == EINVAL
    assert lib.spec_rejected_mask(None, 2, 4, FAKE, None, -1, None) == EINVAL
    assert lib.spec_rejected_mask(FAKE, 2, 4, None, None, -1, None) == EINVAL
    assert lib.spec_rejected_mask(None, 0, 4, None, None, -1, None) == 0  # nothing to do
    assert lib.spec_rejected_mask(None, 3, 0, None, None, -1, None) == 0
    assert lib.spec_tree_rejected_mask(FAKE, 2, 0, 0, FAKE, None, -1, None) == EINVAL
    assert lib.spec_tree_rejected_mask(FAKE, 2, 1025, 3, FAKE, None, -1, None) == EINVAL
    assert lib.spec_tree_rejected_mask(FAKE, 2, 5, 5, FAKE, None, -1, None) == EINVAL
    assert lib.spec_tree_rejected_mask(FAKE, 2, 5, -1, FAKE, None, -1, None) == EINVAL
    assert lib.spec_tree_rejected_mask(None, 2, 5, 2, FAKE, None, -1, None) == EINVAL
    assert lib.spec_tree_rejected_mask(FAKE, 2, 5, 2, None, None, -1, None) == EINVAL
    assert lib.spec_tree_rejected_mask(None, 0, 5, 2, None, None, -1, None) == 0
