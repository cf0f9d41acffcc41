"""GPU parity of the rejected-draft masks (KV-cache trimming) against the
oracle, on masks computed from the verifier's own outputs and on direct
inputs including out-of-range lengths, with the slot-mapping update."""
import numpy as np
import pytest
import torch

import oracle.rng as R
import oracle.serving as OS
import oracle.verify as O
import verify_accept_sampling_amd as S
import workloads as W
from parity_helpers import ints_to_device, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("B,k", [(1, 1), (700, 8), (3, 1023), (64, 0)])
def test_chain_mask_direct(B, k):
    _say(f"chain mask B={B} k={k}")
    rng = np.random.default_rng(B + k)
    n = rng.integers(-2, k + 3, size=B).astype(np.int32)
    slots = rng.integers(0, 1 << 40, size=(B, k)).astype(np.int64)
    slots_g = torch.from_numpy(slots).cuda()
    m = S.spec_rejected_mask(ints_to_device(n), k, slot_mapping=slots_g, pad_slot=-3)
    torch.cuda.synchronize()
    want = OS.rejected_mask_chain(n, k)
    assert np.array_equal(m.cpu().numpy(), want)
    assert np.array_equal(slots_g.cpu().numpy(), OS.apply_padding(slots, want, -3))
    m2 = S.spec_rejected_mask(ints_to_device(n), k)  # mask only
    torch.cuda.synchronize()
    assert np.array_equal(m2.cpu().numpy(), want)


def test_chain_mask_after_sampling():
    _say("chain mask after spec_verify_sample B=24 k=6 V=3000")
    wl = W.sample_chain(24, 6, 3000, seed=31, uniform_seed=32, target_std=2.0, noise_std=1.0,
                        temperature=0.8)
    u = R.chain_uniforms(wl.uniform_seed, wl.B, wl.k)
    acc_o = O.verify_sample(wl.target, wl.draft, wl.draft_tokens, u, wl.temperature, wl.kind,
                            wl.dtype)[0]
    acc_g, _ = S.spec_verify_sample(to_device(wl.target, wl.dtype), to_device(wl.draft, wl.dtype),
                                    ints_to_device(wl.draft_tokens), wl.temperature,
                                    seed=wl.uniform_seed)
    m = S.spec_rejected_mask(acc_g, wl.k)
    torch.cuda.synchronize()
    assert np.array_equal(acc_g.cpu().numpy(), acc_o)
    assert np.array_equal(m.cpu().numpy(), OS.rejected_mask_chain(acc_o, wl.k))


def _tree_case(wl):
    acc_o, _, path_o, _ = O.verify_tree_greedy(wl.target, wl.parent, wl.node_tokens, wl.dtype)
    _, _, path_g = S.spec_verify_tree_greedy(to_device(wl.target, wl.dtype), wl.parent,
                                             ints_to_device(wl.node_tokens))
    N = len(wl.parent)
    rng = np.random.default_rng(N)
    slots = rng.integers(0, 1 << 30, size=(wl.B, N)).astype(np.int64)
    slots_g = torch.from_numpy(slots).cuda()
    m = S.spec_tree_rejected_mask(path_g, N, slot_mapping=slots_g, pad_slot=-1)
    torch.cuda.synchronize()
    deepest = [int(path_o[b, acc_o[b]]) for b in range(wl.B)]
    want = OS.rejected_mask_tree(wl.parent, deepest)
    assert np.array_equal(m.cpu().numpy(), want)
    assert np.array_equal(slots_g.cpu().numpy(), OS.apply_padding(slots, want, -1))


def test_tree_mask_static_tree():
    _say("tree mask, 61-node tree, B=16 V=2000")
    _tree_case(W.tree_greedy(B=16, V=2000, seed=41, p_match=0.7, dtype="bf16"))


def test_tree_mask_shapes():
    _say("tree mask: root only, deep chain, wide star")
    _tree_case(W.tree_greedy(B=3, V=100, seed=4, parent=np.array([-1], np.int32)))
    _tree_case(W.tree_greedy(B=2, V=16, seed=6, parent=np.arange(-1, 1023, dtype=np.int32),
                             p_match=0.995, dtype="f32"))
    star = np.array([-1] + [0] * 300 + list(range(1, 301)), dtype=np.int32)
    _tree_case(W.tree_greedy(B=4, V=8, seed=7, parent=star, p_match=0.5, dtype="f32"))


def test_tree_mask_from_choices():
    _say("tree mask, tree built from choices")
    parent = np.asarray(S.spec_tree_from_choices(W.static_tree_choices()), dtype=np.int32)
    _tree_case(W.tree_greedy(B=8, V=500, seed=43, parent=parent, p_match=0.8, dtype="f32"))
