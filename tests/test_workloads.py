"""Sanity of the seeded synthetic inputs (CPU)."""
import numpy as np
import pytest
import torch
from scipy import special, stats

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 50,
                        np.array([0.0, -0.0, 1.0, -3.5, 1e-40, 3.0e38], dtype=np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_as_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_gumbel_max_draws_follow_softmax():
    rng = np.random.default_rng(1)
    lw = np.array([0.3, -1.0, 2.0, 0.0, 1.1])
    draws = W.gumbel_max_draw(rng, np.tile(lw, (40_000, 1)))
    counts = np.bincount(draws, minlength=5)
    assert stats.chisquare(counts, special.softmax(lw) * len(draws)).pvalue > 1e-4


def test_static_tree_shape():
    parent = W.static_tree_parents()
    assert len(parent) == 61 and parent[0] == -1
    assert all(0 <= parent[j] < j for j in range(1, 61))
    depth = W.tree_depths(parent)
    assert depth.max() == 5
    assert [int((depth == d).sum()) for d in range(1, 6)] == [4, 9, 15, 19, 13]
    # the first chain (first child at every level) branches 4, 3, 2, 2, 1
    node, widths = 0, []
    while True:
        kids = [j for j in range(61) if parent[j] == node]
        if not kids:
            break
        widths.append(len(kids))
        node = kids[0]
    assert widths == [4, 3, 2, 2, 1]


def test_controlled_acceptance_overlap():
    wl = W.controlled_acceptance(B=6, k=3, V=4096, seed=3)
    alphas = W.request_alpha(6)
    for b in range(6):
        for i in range(3):
            p = wl.target[b, i].astype(np.float64)
            q = wl.draft[b, i].astype(np.float64)
            assert abs(np.minimum(p, q).sum() - alphas[b]) < 1e-6
            assert abs(p.sum() - 1) < 1e-5 and abs(q.sum() - 1) < 1e-5


def test_greedy_chain_draft_matches_argmax_often():
    wl = W.greedy_chain(B=200, k=4, V=1000, seed=5)
    amax = np.argmax(wl.target[:, :4], axis=-1)
    rate = (amax == wl.draft_tokens).mean()
    assert 0.65 < rate < 0.75
    assert wl.target.dtype == np.float32 and wl.target.shape == (200, 5, 1000)


def test_sample_chain_shapes_and_peaks():
    wl = W.sample_chain(8, 3, 200, seed=9, uniform_seed=1, target_std=3.0, noise_std=1.5,
                        temperature=0.7, n_peaks=20, peak_boost=8.0)
    assert wl.target.dtype == np.uint16 and wl.target.shape == (8, 4, 200)
    assert wl.draft.shape == (8, 3, 200) and wl.draft_tokens.shape == (8, 3)
    z = W.bf16_bits_as_f32(wl.target).astype(np.float64)
    # 20 of 200 entries per row carry +8: the grand mean is 0.8 (sd 0.075)
    assert abs(z.mean() - 0.8) < 0.3
    assert abs(z.std() - np.sqrt(9 + 64 * 0.1 * 0.9)) < 0.3
    assert wl.temperature == float(np.float32(0.7))
