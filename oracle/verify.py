"""fp64 oracle: greedy, sampling and tree-greedy verification.

TEST INFRASTRUCTURE (see the package header): only tests/, smoke() and the
bench's cpu_baseline leg use it.

What is computed, and where the pages define it
-----------------------------------------------
Pages: "EAGLE-3 speculative decoding review" (6unoyunr.github.io) and the
speculative-decoding chapter of an LLM-serving book (froggydisk.github.io).

* Chain cycle: drafts are checked front to back, the first rejection ends the
  check and everything after it is dropped, the rejected position is
  resampled, and when every draft passes one extra token comes from the
  target's last distribution.  (EAGLE-3 review, section "Speculative
  Decoding", step 3 "Accept or Reject"; serving chapter, section on how it
  works, the "accept" step and the paragraph after it: one token in the worst
  case, k+1 in the best.)
* Greedy rule: a draft token is kept exactly when it equals the target's
  argmax; at the first mismatch the target's argmax is emitted.  (EAGLE-3
  review, section asking whether a small draft hurts quality, greedy bullets;
  serving chapter, acceptance-rule section, last sentence on temperature 0.)
* Sampling rule: draft token x is kept with probability A(x) = min(1,
  p(x)/q(x)); on rejection a token is drawn from the normalised residual
  max(0, p - q).  (EAGLE-3 review, same section, equations A(x) and
  p_residual; serving chapter, acceptance-rule section.)
* Tree greedy: the longest root-to-node prefix whose every token equals the
  target's choice at its parent is kept, then the target's choice after it.
  (EAGLE-3 review, section on the full inference loop, steps 3 "Tree
  Attention" and 4 "Strict Acceptance".)

Readings where the pages are silent (each listed in the design notes):
* Temperature T scales both target and draft logits: p = softmax(z/T),
  q = softmax(y/T).  "probs" inputs are used as given (no temperature, not
  renormalised for the ratio).
* Acceptance is the strict comparison u < p/q, evaluated as u*q < p so that
  q = 0 is well defined (p > 0: accept; p = 0: reject).
* Uniforms: u[i, 0] decides draft i, u[i, 1] drives the one inverse-CDF draw
  at the position where the request stops.
* Inverse CDF: token = min{ j : C_j > u * C_{V-1} } with C the running sum
  of the weights in ascending token id (never picks a zero-weight token).
* Empty residual (C_{V-1} == 0 after a rejection, possible only through
  rounding or unnormalised probability rows): draw from p with the same u.
* Argmax ties resolve to the lowest token id; tree ties resolve to the
  deepest accepted node, then the lowest node index.
* A draft or node token outside [0, V) is a rejection / mismatch.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# Input decoding (the oracle's own; exact widening to float64)
# ---------------------------------------------------------------------------


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Widen a logit/probability array to float64 exactly.

    dtype "bf16": arr holds uint16 bit patterns; the float32 with the same
    top 16 bits is the value.  dtype "f32": arr is float32.
    """
    if dtype == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def tempered_softmax(z: np.ndarray, T: float) -> np.ndarray:
    """p = softmax(z / T) in float64, with the row maximum subtracted."""
    a = np.asarray(z, dtype=np.float64) / float(T)
    m = np.max(a)
    e = np.exp(a - m)
    return e / np.sum(e)


# ---------------------------------------------------------------------------
# Decisions
# ---------------------------------------------------------------------------


@dataclass
class Decision:
    """One decision and its distance to the nearest boundary.

    kind     "accept" (u vs p/q), "resample" (inverse-CDF draw),
             "argmax" (greedy compare; margin = top1 - top2, informational)
    position chain position i (or node index for trees)
    margin   |u - r| for accept; min(u - F_{t-1}, F_t - u) for resample
    """

    kind: str
    position: int
    margin: float
    outcome: int


@dataclass
class RequestResult:
    accepted: int
    tokens: list
    decisions: list = field(default_factory=list)
    # total weight of the distribution the final token was drawn from, in
    # probability units: sum max(0, p_n - q_n) after a rejection, sum p_k for
    # the bonus draw
    residual_mass: float = float("nan")
    path: list = field(default_factory=list)


def inverse_cdf(w: np.ndarray, u: float):
    """Draw from weights w (not necessarily normalised) with uniform u.

    C = cumulative sum in ascending token id; result t = min{ j : C_j > u C_{V-1} }.
    Returns (t, margin, C_{V-1}); t = -1 when the total is zero.
    """
    C = np.cumsum(w)
    total = float(C[-1])
    if not total > 0.0:
        return -1, 0.0, total
    thr = u * total
    t = int(np.searchsorted(C, thr, side="right"))
    lo = float(C[t - 1]) / total if t > 0 else 0.0
    hi = float(C[t]) / total
    return t, min(u - lo, hi - u), total


# ---------------------------------------------------------------------------
# Greedy chain
# ---------------------------------------------------------------------------


def _argmax_with_margin(row: np.ndarray):
    j = int(np.argmax(row))
    if row.shape[0] > 1:
        top2 = np.partition(row, -2)[-2]
        margin = float(row[j] - top2)
    else:
        margin = math.inf
    return j, margin


def verify_greedy_request(target: np.ndarray, draft_tokens: np.ndarray) -> RequestResult:
    """One request: target [k+1, V] (float64), draft_tokens [k]."""
    k = target.shape[0] - 1
    decisions = []
    out = []
    for i in range(k + 1):
        a, margin = _argmax_with_margin(target[i])
        if i == k:
            out.append(a)
            decisions.append(Decision("argmax", i, margin, a))
            return RequestResult(k, out, decisions)
        x = int(draft_tokens[i])
        decisions.append(Decision("argmax", i, margin, a))
        if x == a:
            out.append(x)
            continue
        out.append(a)
        return RequestResult(i, out, decisions)
    raise AssertionError("unreachable")


def verify_greedy(target: np.ndarray, draft_tokens: np.ndarray, dtype: str):
    """Batch greedy chain verification.

    target [B, k+1, V] (f32 or bf16 bits), draft_tokens [B, k].
    Returns (accepted_len [B], out_tokens [B, k+1] padded with -1, results).
    """
    B, kp1, _ = target.shape
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, kp1), -1, dtype=np.int32)
    results = []
    for b in range(B):
        r = verify_greedy_request(decode(target[b], dtype), draft_tokens[b])
        acc[b] = r.accepted
        out[b, : len(r.tokens)] = r.tokens
        results.append(r)
    return acc, out, results


# ---------------------------------------------------------------------------
# Sampling chain
# ---------------------------------------------------------------------------


def verify_sample_request(target: np.ndarray, draft: np.ndarray,
                          draft_tokens: np.ndarray, u: np.ndarray,
                          temperature: float, kind: str, dtype: str) -> RequestResult:
    """One request, positions visited in order and stopped at the first reject.

    target [k+1, V] and draft [k, V] raw rows (logits or probabilities in
    `dtype`), draft_tokens [k], u [k+1, 2] uniforms.
    """
    k = target.shape[0] - 1
    V = target.shape[1]

    def dist(rows, i):
        row = decode(rows[i], dtype)
        if kind == "logits":
            return tempered_softmax(row, temperature)
        return row  # probabilities, used as given

    decisions = []
    for i in range(k):
        p = dist(target, i)
        q = dist(draft, i)
        x = int(draft_tokens[i])
        if 0 <= x < V:
            px, qx = float(p[x]), float(q[x])
            accept = u[i, 0] * qx < px
            ratio = px / qx if qx > 0.0 else math.inf
            margin = abs(float(u[i, 0]) - ratio)
        else:
            accept = False
            margin = math.inf
        decisions.append(Decision("accept", i, margin, int(accept)))
        if accept:
            continue
        w = np.maximum(0.0, p - q)
        t, m2, total = inverse_cdf(w, float(u[i, 1]))
        mass = total
        if t < 0:
            t, m2, _ = inverse_cdf(p, float(u[i, 1]))
            decisions.append(Decision("empty_residual", i, 0.0, t))
        decisions.append(Decision("resample", i, m2, t))
        toks = [int(v) for v in draft_tokens[:i]] + [t]
        return RequestResult(i, toks, decisions, residual_mass=mass)
    p = dist(target, k)
    t, m2, total = inverse_cdf(p, float(u[k, 1]))
    decisions.append(Decision("resample", k, m2, t))
    toks = [int(v) for v in draft_tokens[:k]] + [t]
    return RequestResult(k, toks, decisions, residual_mass=total)


def verify_sample(target: np.ndarray, draft: np.ndarray, draft_tokens: np.ndarray,
                  uniforms: np.ndarray, temperature: float, kind: str, dtype: str,
                  requests=None):
    """Batch sampling chain verification.

    target [B, k+1, V], draft [B, k, V], draft_tokens [B, k], uniforms
    [B, k+1, 2].  `requests` optionally restricts the work to a subset of
    request indices (other rows of the outputs stay -1).
    Returns (accepted_len [B], out_tokens [B, k+1], results dict b -> result).
    """
    B, kp1, _ = target.shape
    acc = np.full(B, -1, dtype=np.int32)
    out = np.full((B, kp1), -1, dtype=np.int32)
    results = {}
    idx = range(B) if requests is None else requests
    for b in idx:
        r = verify_sample_request(target[b], draft[b] if draft is not None else None,
                                  draft_tokens[b], uniforms[b], temperature, kind, dtype)
        acc[b] = r.accepted
        out[b, : len(r.tokens)] = r.tokens
        results[b] = r
    return acc, out, results


class FixedRowsSampler:
    """Many verification calls over the same rows and draft tokens, each with
    its own uniforms, for decision-rate runs.

    Every decision is the one verify_sample_request takes: the acceptance
    test u * q(x) < p(x) on the same float64 p(x), q(x), and inverse_cdf on
    the same weight vector (max(0, p - q) after a rejection, falling back to
    p when its total is zero; p at the bonus position).  The distributions
    and cumulative sums of a request are computed once and reused; nothing
    else differs.
    """

    def __init__(self, target, draft, draft_tokens, temperature, kind, dtype):
        self.target, self.draft = target, draft
        self.tokens = np.asarray(draft_tokens)
        self.T, self.kind, self.dtype = temperature, kind, dtype
        self.B, kp1, self.V = target.shape
        self.k = kp1 - 1
        self.px = np.zeros((self.B, self.k))
        self.qx = np.zeros((self.B, self.k))
        self.valid = np.zeros((self.B, self.k), dtype=bool)
        for b in range(self.B):
            for i in range(self.k):
                x = int(self.tokens[b, i])
                if 0 <= x < self.V:
                    self.valid[b, i] = True
                    self.px[b, i] = float(self._dist(target, b, i)[x])
                    self.qx[b, i] = float(self._dist(draft, b, i)[x])
        with np.errstate(divide="ignore"):
            ratio = np.where(self.qx > 0.0, self.px / np.where(self.qx > 0.0, self.qx, 1.0),
                             np.inf)
        self.ratio = np.where(self.valid, ratio, np.nan)
        self._cdf = {}

    def _dist(self, rows, b, i):
        row = decode(rows[b, i], self.dtype)
        if self.kind == "logits":
            return tempered_softmax(row, self.T)
        return row

    def cdf(self, b, n):
        """Cumulative weights and their total for a request stopping at n."""
        key = (b, n)
        if key not in self._cdf:
            p = self._dist(self.target, b, n)
            if n < self.k:
                C = np.cumsum(np.maximum(0.0, p - self._dist(self.draft, b, n)))
                if not float(C[-1]) > 0.0:
                    C = np.cumsum(p)
            else:
                C = np.cumsum(p)
            self._cdf[key] = (C, float(C[-1]))
        return self._cdf[key]

    def run(self, u):
        """u [N, B, k+1, 2] (float64).  Returns accepted [N, B], the drawn
        token [N, B], the acceptance margins |u - p/q| [N, B, k] (inf for an
        invalid token) and the draw margin [N, B]."""
        N = u.shape[0]
        k = self.k
        ua = u[:, :, :k, 0]
        accept = (ua * self.qx[None]) < self.px[None]
        accept &= self.valid[None]
        with np.errstate(invalid="ignore"):
            amargin = np.where(self.valid[None], np.abs(ua - self.ratio[None]), np.inf)
        rej = ~accept
        first = np.where(rej.any(axis=2), rej.argmax(axis=2), k) if k > 0 else np.zeros(
            (N, self.B), dtype=np.int64)
        token = np.zeros((N, self.B), dtype=np.int64)
        dmargin = np.zeros((N, self.B))
        ures = np.take_along_axis(u[:, :, :, 1], first[:, :, None], axis=2)[:, :, 0]
        for b in range(self.B):
            for n in np.unique(first[:, b]):
                sel = first[:, b] == n
                C, total = self.cdf(b, int(n))
                uu = ures[sel, b]
                t = np.searchsorted(C, uu * total, side="right")
                lo = np.where(t > 0, C[np.maximum(t - 1, 0)] / total, 0.0)
                hi = C[t] / total
                token[sel, b] = t
                dmargin[sel, b] = np.minimum(uu - lo, hi - uu)
        return first, token, amargin, dmargin


def probe_values(target: np.ndarray, draft: np.ndarray, draft_tokens: np.ndarray,
                 temperature: float, kind: str, dtype: str, b: int):
    """p_i(x_i) and q_i(x_i) for every draft position i of request b (float64)."""
    k = target.shape[1] - 1
    V = target.shape[2]
    pv = np.zeros(k)
    qv = np.zeros(k)
    for i in range(k):
        x = int(draft_tokens[b, i])
        if not 0 <= x < V:
            continue
        zp = decode(target[b, i], dtype)
        zq = decode(draft[b, i], dtype)
        if kind == "logits":
            pv[i] = tempered_softmax(zp, temperature)[x]
            qv[i] = tempered_softmax(zq, temperature)[x]
        else:
            pv[i] = zp[x]
            qv[i] = zq[x]
    return pv, qv


# ---------------------------------------------------------------------------
# Tree greedy
# ---------------------------------------------------------------------------


def verify_tree_request(target: np.ndarray, parent: np.ndarray,
                        node_tokens: np.ndarray) -> RequestResult:
    """One request: target [N, V] float64 rows (row j = the target's
    distribution after node j's prefix), parent [N], node_tokens [N]."""
    N = len(parent)
    amax = {}

    def choice(j):
        if j not in amax:
            amax[j] = int(np.argmax(target[j]))
        return amax[j]

    depth = [0] * N
    accepted = [False] * N
    accepted[0] = True
    for j in range(1, N):
        pa = int(parent[j])
        depth[j] = depth[pa] + 1
        if accepted[pa]:
            accepted[j] = int(node_tokens[j]) == choice(pa)
    best = 0
    for j in range(1, N):
        if accepted[j] and depth[j] > depth[best]:
            best = j  # strict '>' keeps the lowest index among equal depths
    path = [best]
    while path[-1] != 0:
        path.append(int(parent[path[-1]]))
    path.reverse()
    toks = [int(node_tokens[n]) for n in path[1:]] + [choice(best)]
    return RequestResult(depth[best], toks, [], path=path)


def verify_tree_greedy(target: np.ndarray, parent: np.ndarray,
                       node_tokens: np.ndarray, dtype: str):
    """Batch tree-greedy verification.

    target [B, N, V], parent [N], node_tokens [B, N].  Returns
    (accepted_len [B], out_tokens [B, D+1], out_path [B, D+1], results) with
    D the tree depth; out_path lists node ids from the root, padded with -1.
    """
    B, N, _ = target.shape
    depth = np.zeros(N, dtype=np.int64)
    for j in range(1, N):
        depth[j] = depth[parent[j]] + 1
    D = int(depth.max()) if N else 0
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, D + 1), -1, dtype=np.int32)
    path = np.full((B, D + 1), -1, dtype=np.int32)
    results = []
    for b in range(B):
        r = verify_tree_request(decode(target[b], dtype), parent, node_tokens[b])
        acc[b] = r.accepted
        out[b, : len(r.tokens)] = r.tokens
        path[b, : len(r.path)] = r.path
        results.append(r)
    return acc, out, path, results


# ---------------------------------------------------------------------------
# Tree sampling
# ---------------------------------------------------------------------------
#
# The EAGLE-3 review (section on the full inference loop, step 4 "Strict
# Acceptance") says only that sampling over the tree applies the min(1, p/q)
# test with residual correction so that the target distribution is kept.
# The order over siblings is not on the pages; the reading taken is
# SpecInfer's multi-step speculative sampling (Miao et al., ASPLOS 2024):
# at the current node the children are tried in increasing node index, each
# with the test u < p(x)/q(x) against the current target distribution p;
# after a rejection p becomes normalise(max(0, p - q)) (q, the draft's
# distribution at the node, is the one every child there was drawn from);
# the first accepted child becomes the current node, with p reset to the
# target's distribution there; when no child is accepted (or the node has
# none) one token is drawn from the current p by inverse CDF.


def _children(parent) -> list:
    N = len(parent)
    kids = [[] for _ in range(N)]
    for j in range(1, N):
        kids[int(parent[j])].append(j)
    return kids


def verify_tree_sample_request(target: np.ndarray, draft: np.ndarray, parent,
                               node_tokens: np.ndarray, u: np.ndarray,
                               temperature: float, kind: str, dtype: str) -> RequestResult:
    """One request.  target [N, V] and draft [N, V] raw rows (row j: the
    target's / the draft's distribution after node j's prefix; node j's
    children were drawn from draft row j), parent [N] (parent[0] = -1,
    parent[j] < j), node_tokens [N] (entry 0 unused), u [N, 2]: u[j, 0]
    decides node j's test, u[j, 1] drives the draw if the request stops at
    node j.

    Decisions: "accept" (node j: margin |u - p(x)/q(x)|), "residual" (after
    each rejection: margin = the mass of max(0, p - q), outcome 1 if p was
    replaced, 0 if that mass is zero and p is kept), "resample" (the draw at
    the stop node)."""
    V = target.shape[1]
    kids = _children(parent)

    def dist(rows, j):
        row = decode(rows[j], dtype)
        if kind == "logits":
            return tempered_softmax(row, temperature)
        return row  # probabilities, used as given

    decisions = []
    path = [0]
    cur = 0
    while True:
        p = dist(target, cur)
        q = dist(draft, cur) if kids[cur] else None
        nxt = None
        for c in kids[cur]:
            x = int(node_tokens[c])
            if 0 <= x < V:
                px, qx = float(p[x]), float(q[x])
                accept = u[c, 0] * qx < px
                ratio = px / qx if qx > 0.0 else math.inf
                margin = abs(float(u[c, 0]) - ratio)
            else:
                accept, margin = False, math.inf
            decisions.append(Decision("accept", c, margin, int(accept)))
            if accept:
                nxt = c
                break
            w = np.maximum(0.0, p - q)
            mass = float(np.sum(w))
            if mass > 0.0:
                p = w / mass
            decisions.append(Decision("residual", c, mass, int(mass > 0.0)))
        if nxt is None:
            t, m2, total = inverse_cdf(p, float(u[cur, 1]))
            decisions.append(Decision("resample", cur, m2, t))
            toks = [int(node_tokens[j]) for j in path[1:]] + [t]
            return RequestResult(len(path) - 1, toks, decisions, residual_mass=total, path=path)
        path.append(nxt)
        cur = nxt


def verify_tree_sample(target: np.ndarray, draft: np.ndarray, parent, node_tokens: np.ndarray,
                       uniforms: np.ndarray, temperature: float, kind: str, dtype: str,
                       requests=None):
    """Batch tree sampling verification.

    target [B, N, V], draft [B, N, V], parent [N], node_tokens [B, N],
    uniforms [B, N, 2].  Returns (accepted_len [B], out_tokens [B, D+1],
    out_path [B, D+1], results dict b -> result), D the tree depth; rows of
    requests outside `requests` stay -1."""
    B, N, _ = target.shape
    depth = np.zeros(N, dtype=np.int64)
    for j in range(1, N):
        depth[j] = depth[parent[j]] + 1
    D = int(depth.max()) if N else 0
    acc = np.full(B, -1, dtype=np.int32)
    out = np.full((B, D + 1), -1, dtype=np.int32)
    path = np.full((B, D + 1), -1, dtype=np.int32)
    results = {}
    for b in (range(B) if requests is None else requests):
        r = verify_tree_sample_request(target[b], draft[b], parent, node_tokens[b], uniforms[b],
                                       temperature, kind, dtype)
        acc[b] = r.accepted
        out[b, : len(r.tokens)] = r.tokens
        path[b, : len(r.path)] = r.path
        results[b] = r
    return acc, out, path, results
