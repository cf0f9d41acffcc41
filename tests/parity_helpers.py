"""Shared helpers of the GPU parity tests: device transfer and the
oracle-vs-HIP comparison with decision margins."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.verify as O

# A deciding comparison within this distance of its boundary is "flagged":
# the HIP path (float32 row statistics) and the float64 oracle may then
# legitimately disagree.
FLAG_BAND = 1e-5
PROB_TOL = 1e-5


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def ints_to_device(arr: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).to(device)


def check_chain_structure(acc, out, draft_tokens, V):
    """Invariants of any chain output: 0 <= n <= k, prefix = drafts, one
    emitted token in [0, V), then -1 padding."""
    B, kp1 = out.shape
    k = kp1 - 1
    for b in range(B):
        n = int(acc[b])
        assert 0 <= n <= k, (b, n)
        assert np.array_equal(out[b, :n], draft_tokens[b, :n]), b
        assert 0 <= out[b, n] < V, (b, out[b, n])
        assert np.all(out[b, n + 1:] == -1), b


def compare_sample(acc_g, out_g, acc_o, out_o, results, requests):
    """Classify GPU/oracle disagreements by the first differing decision.

    Returns a dict with counts of decisions, flagged decisions (oracle
    margin < FLAG_BAND), mismatching requests and unflagged mismatches (a
    disagreement whose first differing decision was not near its boundary).
    """
    st = dict(requests=0, accept_decisions=0, draw_decisions=0, flagged=0, mismatches=0,
              unflagged=0, unflagged_requests=[])
    for b in requests:
        r = results[b]
        st["requests"] += 1
        acc_dec = [d for d in r.decisions if d.kind == "accept"]
        draw_dec = [d for d in r.decisions if d.kind == "resample"]
        st["accept_decisions"] += len(acc_dec)
        st["draw_decisions"] += len(draw_dec)
        st["flagged"] += sum(1 for d in r.decisions if d.margin < FLAG_BAND)
        if int(acc_g[b]) == int(acc_o[b]) and np.array_equal(out_g[b], out_o[b]):
            continue
        st["mismatches"] += 1
        n_g, n_o = int(acc_g[b]), int(acc_o[b])
        if n_g != n_o:
            pos = min(n_g, n_o)
            d = [x for x in acc_dec if x.position == pos][0]
        else:
            d = draw_dec[0]
        if not d.margin < FLAG_BAND:
            st["unflagged"] += 1
            st["unflagged_requests"].append((b, d.kind, d.position, d.margin))
    return st


def check_probe(probe_g, wl, acc_g, acc_o, results, requests, detail=None):
    """p_i(x_i), q_i(x_i) within PROB_TOL of the oracle's float64 values, and
    the mass of the drawn-from distribution at the stop position.  Returns the
    largest absolute difference; `detail` (a list) receives where it is."""
    worst = 0.0
    where = None
    for b in requests:
        pv, qv = O.probe_values(wl.target, wl.draft, wl.draft_tokens, wl.temperature,
                                wl.kind, wl.dtype, b)
        k = wl.k
        for i in range(k):
            for f, ref in ((0, pv[i]), (1, qv[i])):
                d = abs(float(probe_g[b, i, f]) - ref)
                if d > worst:
                    worst, where = d, (b, i, f, float(probe_g[b, i, f]), ref)
        n = int(acc_o[b])
        m = results[b].residual_mass
        if math.isfinite(m) and int(acc_g[b]) == n:
            d = abs(float(probe_g[b, n, 2]) - m)
            if d > worst:
                worst, where = d, (b, n, 2, float(probe_g[b, n, 2]), m)
    if detail is not None:
        detail.append(where)
    return worst


def compare_tree_sample(acc_g, out_g, path_g, results, parent, requests):
    """Classify tree-sampling disagreements by the first differing decision.

    Where the GPU's and the oracle's paths part, the first child of the
    parting node that one side accepted and the other rejected decides; the
    disagreement is flagged when that test, or a residual mass at that node
    before it, lies within FLAG_BAND of its boundary in the oracle.  Equal
    paths with different tokens are classified by the draw (and the stop
    node's residual masses)."""
    kids = [[] for _ in range(len(parent))]
    for j in range(1, len(parent)):
        kids[int(parent[j])].append(j)
    st = dict(requests=0, accept_decisions=0, draw_decisions=0, flagged=0, mismatches=0,
              unflagged=0, unflagged_requests=[])
    for b in requests:
        r = results[b]
        st["requests"] += 1
        st["accept_decisions"] += sum(1 for d in r.decisions if d.kind == "accept")
        st["draw_decisions"] += 1
        st["flagged"] += sum(1 for d in r.decisions if d.margin < FLAG_BAND)
        n_g = int(acc_g[b])
        pg = [int(v) for v in path_g[b, : n_g + 1]] if n_g >= 0 else []
        tg = [int(v) for v in out_g[b, : n_g + 1]] if n_g >= 0 else []
        if n_g == r.accepted and pg == r.path and tg == r.tokens:
            continue
        st["mismatches"] += 1
        if n_g < 0 or not pg or pg[0] != 0:
            st["unflagged"] += 1
            st["unflagged_requests"].append((b, "invalid", n_g, None))
            continue
        d = 1
        while d < len(pg) and d < len(r.path) and pg[d] == r.path[d]:
            d += 1
        node = r.path[d - 1]
        at_node = [x for x in r.decisions if x.position in kids[node]]
        if d == len(pg) and d == len(r.path):  # same stop node: the draw
            cand = [x for x in r.decisions if x.kind == "resample"]
            cand += [x for x in at_node if x.kind == "residual"]
        else:
            g_child = pg[d] if d < len(pg) else None
            o_child = r.path[d] if d < len(r.path) else None
            order = kids[node]
            idx = [order.index(c) for c in (g_child, o_child) if c is not None]
            first = order[min(idx)]
            cand = [x for x in at_node if x.kind == "accept" and x.position == first]
            cand += [x for x in at_node if x.kind == "residual" and order.index(x.position)
                     < order.index(first)]
        if not any(x.margin < FLAG_BAND for x in cand):
            st["unflagged"] += 1
            st["unflagged_requests"].append((b, node, pg, r.path))
    return st
