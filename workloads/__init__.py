"""Seeded synthetic inputs for batched speculative-decoding verification.

This module is the only code shared by the oracle side (tests, CPU baseline)
and the HIP side (parity tests, bench).  It builds inputs and nothing else:
logit rows, draft tokens, tree shapes and the controlled-acceptance rows.  It
holds none of the verification arithmetic (no acceptance test, no residual,
no inverse-CDF search, no uniform generator): draft tokens are drawn with the
Gumbel-max trick (Gumbel 1954) so that no softmax or CDF is evaluated here.

The five workloads follow the verification step described on the pages
"EAGLE-3 speculative decoding review" (section "Speculative Decoding", the
Draft / Verification / Accept-or-Reject cycle) and the LLM-serving chapter on
speculative decoding (section on how it works): per request, target logits at
k+1 positions, draft logits at k positions and the k draft tokens.

Every array is numpy; bf16 tensors are carried as their uint16 bit patterns
(round-to-nearest-even from float32).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# ---------------------------------------------------------------------------
# bf16 helpers (input construction only)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _gumbel(rng: np.random.Generator, shape) -> np.ndarray:
    u = rng.random(shape)
    # rng.random is in [0, 1); map 0 to the smallest positive double.
    u = np.where(u == 0.0, np.finfo(np.float64).tiny, u)
    return -np.log(-np.log(u))


def gumbel_max_draw(rng: np.random.Generator, log_weights: np.ndarray) -> np.ndarray:
    """Draw one index per row with P(j) proportional to exp(log_weights[..., j]).

    Gumbel-max trick: argmax_j (log w_j + G_j) with G_j i.i.d. standard Gumbel.
    Rows are processed one leading index at a time to bound memory.
    """
    lw = np.asarray(log_weights, dtype=np.float64)
    lead = lw.shape[:-1]
    flat = lw.reshape(-1, lw.shape[-1])
    out = np.empty(flat.shape[0], dtype=np.int64)
    for r in range(flat.shape[0]):
        out[r] = int(np.argmax(flat[r] + _gumbel(rng, flat.shape[1])))
    return out.reshape(lead)


# ---------------------------------------------------------------------------
# Containers
# ---------------------------------------------------------------------------


@dataclass
class ChainWorkload:
    """Chain verification inputs: B requests, k drafts, vocabulary V.

    target        [B, k+1, V]  f32 values, or uint16 bf16 bits, or f32 probs
    draft         [B, k, V]    same dtype as target (None for greedy)
    draft_tokens  [B, k]       int32
    kind          "logits" or "probs"
    dtype         "f32" or "bf16"
    temperature   sampling temperature (logits kind only; 1.0 for probs)
    uniform_seed  seed for the per-position uniforms
    """

    name: str
    target: np.ndarray
    draft: Optional[np.ndarray]
    draft_tokens: np.ndarray
    kind: str
    dtype: str
    temperature: float
    uniform_seed: int
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.target.shape[0])

    @property
    def k(self) -> int:
        return int(self.target.shape[1]) - 1

    @property
    def V(self) -> int:
        return int(self.target.shape[2])


@dataclass
class TreeWorkload:
    """Tree verification inputs.

    target       [B, N, V] logits at the root and every tree node
    parent       [N] int32, parent[0] = -1, parent[j] < j
    node_tokens  [B, N] int32 (column 0, the root, is ignored)
    """

    name: str
    target: np.ndarray
    parent: np.ndarray
    node_tokens: np.ndarray
    dtype: str
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.target.shape[0])

    @property
    def n_nodes(self) -> int:
        return int(self.target.shape[1])

    @property
    def V(self) -> int:
        return int(self.target.shape[2])


def logits_as_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Input-side view of a logit tensor as float32 (used by the generators)."""
    if dtype == "bf16":
        return bf16_bits_as_f32(arr)
    return np.asarray(arr, dtype=np.float32)


# ---------------------------------------------------------------------------
# Workload 1: greedy chain, B=1, k=4, V=1000, fp32 N(0, 2^2)
# ---------------------------------------------------------------------------


def greedy_chain(B: int = 1, k: int = 4, V: int = 1000, seed: int = 1001,
                 p_match: float = 0.7, std: float = 2.0,
                 dtype: str = "f32") -> ChainWorkload:
    """Target logits N(0, std^2); each draft token equals the target row's
    argmax with probability p_match, else a uniform token (which may coincide)."""
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((B, k + 1, V), dtype=np.float32) * np.float32(std))
    target = f32_to_bf16_bits(z) if dtype == "bf16" else z.astype(np.float32)
    zf = logits_as_f32(target, dtype)
    amax = np.argmax(zf[:, :k, :], axis=-1)
    rand = rng.integers(0, V, size=(B, k))
    pick = rng.random((B, k)) < p_match
    toks = np.where(pick, amax, rand).astype(np.int32)
    return ChainWorkload("greedy_chain", target, None, toks, "logits", dtype,
                         1.0, 0, meta=dict(seed=seed, p_match=p_match, std=std))


# ---------------------------------------------------------------------------
# Workloads 2 and 3: sampling chains with a noisy draft
# ---------------------------------------------------------------------------


def sample_chain(B: int, k: int, V: int, seed: int, uniform_seed: int,
                 target_std: float, noise_std: float, temperature: float,
                 n_peaks: int = 0, peak_boost: float = 0.0,
                 dtype: str = "bf16", name: str = "sample_chain") -> ChainWorkload:
    """Target z ~ N(0, target_std^2) (+peak_boost on n_peaks distinct ids per
    row), draft y = z + N(0, noise_std^2), both rounded to dtype; draft token
    i of request b drawn from softmax(y[b, i] / T) by Gumbel-max."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, k + 1, V), dtype=np.float32) * np.float32(target_std)
    if n_peaks > 0:
        for b in range(B):
            for i in range(k + 1):
                ids = rng.choice(V, size=n_peaks, replace=False)
                z[b, i, ids] += np.float32(peak_boost)
    target = f32_to_bf16_bits(z) if dtype == "bf16" else z
    zt = logits_as_f32(target, dtype)[:, :k, :]
    y = zt + rng.standard_normal((B, k, V), dtype=np.float32) * np.float32(noise_std)
    draft = f32_to_bf16_bits(y) if dtype == "bf16" else y.astype(np.float32)
    yq = logits_as_f32(draft, dtype).astype(np.float64) / float(np.float32(temperature))
    toks = gumbel_max_draw(rng, yq).astype(np.int32)
    return ChainWorkload(name, target, draft, toks, "logits", dtype,
                         float(np.float32(temperature)), uniform_seed,
                         meta=dict(seed=seed, target_std=target_std,
                                   noise_std=noise_std, n_peaks=n_peaks,
                                   peak_boost=peak_boost))


def sample_chain_v32000(B: int = 8, k: int = 4, V: int = 32000,
                        seed: int = 1002, uniform_seed: int = 2002) -> ChainWorkload:
    """B=8, k=4, V=32000 bf16; z ~ N(0, 2^2); y = z + N(0, 1); T = 1."""
    return sample_chain(B, k, V, seed, uniform_seed, 2.0, 1.0, 1.0,
                        name="sample_chain_v32000")


def sample_chain_llama3(B: int = 64, k: int = 8, V: int = 128256,
                        seed: int = 1003, uniform_seed: int = 2003) -> ChainWorkload:
    """B=64, k=8, V=128256 bf16; z ~ N(0, 3^2) with 20 distinct peak ids per
    row boosted by +8; y = z + N(0, 1.5^2); T = 0.7."""
    return sample_chain(B, k, V, seed, uniform_seed, 3.0, 1.5, 0.7,
                        n_peaks=min(20, V), peak_boost=8.0,
                        name="sample_chain_llama3")


# ---------------------------------------------------------------------------
# Workload 4: static EAGLE-style tree, greedy verification
# ---------------------------------------------------------------------------


def static_tree_choices(branching=(4, 3, 2, 2, 1), n_keep: int = 60) -> list:
    """The nodes of a static draft tree as choices: tuples of 0-based
    sibling ranks from the root, listed level by level.

    The full tree with per-depth branching `branching` is built.  Nodes are
    ranked by (sum of the ranks on the path, depth, path) and the first n_keep
    are kept, which is closed under taking parents because a parent ranks
    strictly before each of its children.  They are listed in (depth, path)
    order.
    """
    paths = []

    def grow(path):
        d = len(path)
        if d == len(branching):
            return
        for r in range(branching[d]):
            child = path + (r,)
            paths.append(child)
            grow(child)

    grow(())
    kept = sorted(paths, key=lambda p: (sum(p), len(p), p))[:n_keep]
    return sorted(kept, key=lambda p: (len(p), p))


def static_tree_parents(branching=(4, 3, 2, 2, 1), n_keep: int = 60) -> np.ndarray:
    """Parent array of the static draft tree of static_tree_choices (root =
    node 0, node i + 1 = choice i)."""
    kept = static_tree_choices(branching, n_keep)
    ids = {(): 0}
    for i, p in enumerate(kept):
        ids[p] = i + 1
    parent = [-1] + [ids[p[:-1]] for p in kept]
    return np.asarray(parent, dtype=np.int32)


def tree_depths(parent: np.ndarray) -> np.ndarray:
    depth = np.zeros(len(parent), dtype=np.int32)
    for j in range(1, len(parent)):
        depth[j] = depth[parent[j]] + 1
    return depth


def tree_greedy(B: int = 16, V: int = 128256, seed: int = 1004,
                parent: Optional[np.ndarray] = None, p_match: float = 0.6,
                std: float = 2.0, dtype: str = "bf16") -> TreeWorkload:
    """Target logits N(0, std^2) at every node row; node j's token equals the
    argmax of its parent's row with probability p_match, else a uniform token."""
    if parent is None:
        parent = static_tree_parents()
    parent = np.asarray(parent, dtype=np.int32)
    N = len(parent)
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, N, V), dtype=np.float32) * np.float32(std)
    target = f32_to_bf16_bits(z) if dtype == "bf16" else z
    zf = logits_as_f32(target, dtype)
    amax = np.argmax(zf, axis=-1)
    toks = np.zeros((B, N), dtype=np.int32)
    for j in range(1, N):
        rand = rng.integers(0, V, size=B)
        pick = rng.random(B) < p_match
        toks[:, j] = np.where(pick, amax[:, parent[j]], rand)
    toks[:, 0] = -7  # root column is ignored by the verifier
    return TreeWorkload("tree_greedy", target, parent, toks, dtype,
                        meta=dict(seed=seed, p_match=p_match, std=std))


@dataclass
class TreeSampleWorkload:
    """Tree sampling inputs.

    target, draft  [B, N, V] logits after every node's prefix (node j's
                   children were drawn from the draft's row j)
    parent         [N] int32, parent[0] = -1, parent[j] < j
    node_tokens    [B, N] int32 (column 0, the root, is ignored)
    """

    name: str
    target: np.ndarray
    draft: np.ndarray
    parent: np.ndarray
    node_tokens: np.ndarray
    kind: str
    dtype: str
    temperature: float
    uniform_seed: int
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.target.shape[0])

    @property
    def n_nodes(self) -> int:
        return int(self.target.shape[1])

    @property
    def V(self) -> int:
        return int(self.target.shape[2])


def tree_sample(B: int = 16, V: int = 128256, seed: int = 1006, uniform_seed: int = 2006,
                parent: Optional[np.ndarray] = None, target_std: float = 3.0,
                noise_std: float = 1.5, temperature: float = 0.7, n_peaks: int = 20,
                peak_boost: float = 8.0, dtype: str = "bf16") -> TreeSampleWorkload:
    """The static tree (60 nodes, branching 4, 3, 2, 2, 1 by default) with
    draft logits: target z ~ N(0, target_std^2) (+peak_boost on n_peaks
    distinct ids per row), draft y = z + N(0, noise_std^2), both rounded to
    dtype; every child of node j draws its token independently from
    softmax(y[b, j] / T) by Gumbel-max."""
    if parent is None:
        parent = static_tree_parents()
    parent = np.asarray(parent, dtype=np.int32)
    N = len(parent)
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, N, V), dtype=np.float32) * np.float32(target_std)
    if n_peaks > 0:
        for b in range(B):
            for j in range(N):
                ids = rng.choice(V, size=min(n_peaks, V), replace=False)
                z[b, j, ids] += np.float32(peak_boost)
    target = f32_to_bf16_bits(z) if dtype == "bf16" else z
    zt = logits_as_f32(target, dtype)
    y = zt + rng.standard_normal((B, N, V), dtype=np.float32) * np.float32(noise_std)
    draft = f32_to_bf16_bits(y) if dtype == "bf16" else y.astype(np.float32)
    yq = logits_as_f32(draft, dtype)
    T = float(np.float32(temperature))
    toks = np.zeros((B, N), dtype=np.int32)
    for j in range(1, N):
        toks[:, j] = gumbel_max_draw(rng, yq[:, parent[j], :].astype(np.float64) / T)
    toks[:, 0] = -7  # root column is ignored by the verifier
    return TreeSampleWorkload("tree_sample", target, draft, parent, toks, "logits", dtype, T,
                              uniform_seed, meta=dict(seed=seed, target_std=target_std,
                                                      noise_std=noise_std, n_peaks=n_peaks,
                                                      peak_boost=peak_boost))


# ---------------------------------------------------------------------------
# Workload 5: controlled acceptance, fp32 probabilities
# ---------------------------------------------------------------------------

ALPHAS = (0.6, 0.8, 0.9)


def controlled_acceptance(B: int = 512, k: int = 8, V: int = 128256,
                          seed: int = 1005, uniform_seed: int = 2005,
                          alphas=ALPHAS, logit_std: float = 2.0,
                          one_hot_mass: float = 0.9) -> ChainWorkload:
    """Rows with a prescribed overlap alpha = 1 - TV(p, q).

    p = softmax(N(0, logit_std^2) logits); r = one_hot_mass * e_j +
    (1 - one_hot_mass) / V with j uniform per (b, i);
    q = (1 - beta) p + beta r.  Because q - p = beta (r - p), TV(p, q) =
    beta TV(p, r), so beta = (1 - alpha) / TV(p, r).  Request b uses
    alpha = alphas[b mod len(alphas)] at every position.  p and q are stored
    as float32; draft tokens are drawn from q by Gumbel-max.
    """
    rng = np.random.default_rng(seed)
    p_out = np.empty((B, k + 1, V), dtype=np.float32)
    q_out = np.empty((B, k, V), dtype=np.float32)
    toks = np.empty((B, k), dtype=np.int32)
    realised = np.empty((B, k), dtype=np.float64)
    for b in range(B):
        alpha = alphas[b % len(alphas)]
        z = rng.standard_normal((k + 1, V)) * logit_std
        e = np.exp(z - z.max(axis=-1, keepdims=True))
        p = e / e.sum(axis=-1, keepdims=True)
        p_out[b] = p
        for i in range(k):
            j = int(rng.integers(0, V))
            r = np.full(V, (1.0 - one_hot_mass) / V)
            r[j] += one_hot_mass
            tv_pr = 0.5 * np.abs(p[i] - r).sum()
            beta = (1.0 - alpha) / tv_pr
            if not (0.0 < beta <= 1.0):
                raise ValueError(f"alpha={alpha} not reachable (beta={beta})")
            q = (1.0 - beta) * p[i] + beta * r
            q_out[b, i] = q
            realised[b, i] = 1.0 - 0.5 * np.abs(p[i] - q).sum()
        with np.errstate(divide="ignore"):
            lq = np.log(q_out[b].astype(np.float64))
        toks[b] = gumbel_max_draw(rng, lq).astype(np.int32)
    return ChainWorkload("controlled_acceptance", p_out, q_out, toks, "probs",
                         "f32", 1.0, uniform_seed,
                         meta=dict(seed=seed, alphas=tuple(alphas),
                                   realised_alpha=realised,
                                   one_hot_mass=one_hot_mass))


def request_alpha(B: int, alphas=ALPHAS) -> np.ndarray:
    return np.asarray([alphas[b % len(alphas)] for b in range(B)])


# ---------------------------------------------------------------------------
# Registry of the five workloads at full size
# ---------------------------------------------------------------------------

WORKLOADS = {
    1: ("greedy_chain_b1_k4_v1000_f32", lambda: greedy_chain()),
    2: ("sample_chain_b8_k4_v32000_bf16", lambda: sample_chain_v32000()),
    3: ("sample_chain_b64_k8_v128256_bf16_t0.7", lambda: sample_chain_llama3()),
    4: ("tree_greedy_b16_n61_v128256_bf16", lambda: tree_greedy()),
    5: ("controlled_acceptance_b512_k8_v128256_f32probs",
        lambda: controlled_acceptance()),
}
