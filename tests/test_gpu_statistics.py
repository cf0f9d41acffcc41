"""Statistical checks of the HIP path against what the pages fix, and the
decision-rate run behind the "mismatches below 1e-6 of decisions" bar.

* Law of the emitted tokens: speculative sampling emits tokens distributed
  exactly as the target distribution ("EAGLE-3 speculative decoding review",
  section asking whether a small draft hurts quality, and the sections on
  interpreting losslessness).  Checked by chi-square over 10^6 GPU draws on a
  tiny vocabulary, at every position: the first token follows p_0, the token
  after an accepted first draft follows p_1, the bonus token follows p_k.
* Expected tokens per step: with a per-position acceptance rate alpha the
  mean number of emitted tokens is (1 - alpha^(k+1)) / (1 - alpha) (the
  serving chapter's expected-token-count section).  Checked on the
  controlled-acceptance workload with fresh draft tokens and uniforms per
  call.
* Decision rate: over 10^6+ decisions on fixed rows with fresh uniforms,
  every GPU/oracle disagreement must be flagged (its first differing
  decision within 1e-5 of the boundary in the oracle) and disagreements
  must stay below 1e-6 of decisions.
"""
import math

import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle.rng as R
import oracle.verify as O
import verify_accept_sampling_amd as S
import workloads as W
from parity_helpers import FLAG_BAND, ints_to_device, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _gumbel_tokens(rng, logq, n):
    """n independent draws from each row of logq [k, V] (float64 log
    weights): int32 [n, k]."""
    g = rng.gumbel(size=(n,) + logq.shape)
    return np.argmax(logq[None] + g, axis=2).astype(np.int32)


def _chi2_pvalue(counts, probs):
    n = counts.sum()
    exp = n * probs
    assert exp.min() >= 5.0, exp.min()
    return float(stats.chi2.sf(((counts - exp) ** 2 / exp).sum(), len(probs) - 1))


# ---------------------------------------------------------------------------
# law of the emitted tokens
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("kind,dtype,T,seed", [("logits", "f32", 0.8, 41),
                                               ("logits", "bf16", 1.3, 42),
                                               ("probs", "f32", 1.0, 43)])
def test_emitted_token_law_chi_square(kind, dtype, T, seed):
    V, k, B, calls = 6, 2, 65536, 16
    rng = np.random.default_rng(seed)
    if kind == "logits":
        t = (rng.standard_normal((k + 1, V)) * 1.5).astype(np.float32)
        d = (t[:k] + rng.standard_normal((k, V)).astype(np.float32) * 1.2).astype(np.float32)
        if dtype == "bf16":
            t, d = W.f32_to_bf16_bits(t), W.f32_to_bf16_bits(d)
        tf = W.logits_as_f32(t, dtype).astype(np.float64)
        df = W.logits_as_f32(d, dtype).astype(np.float64)
        p = special.softmax(tf / T, axis=1)
        q = special.softmax(df / T, axis=1)
    else:
        t = rng.dirichlet(np.ones(V) * 2, size=k + 1).astype(np.float32)
        d = rng.dirichlet(np.ones(V) * 2, size=k).astype(np.float32)
        p = t.astype(np.float64) / t.astype(np.float64).sum(axis=1, keepdims=True)
        q = d.astype(np.float64) / d.astype(np.float64).sum(axis=1, keepdims=True)
    assert 0.5 * np.abs(p[0] - q[0]).sum() > 0.05  # the draft is visibly wrong
    tgt = to_device(np.broadcast_to(t, (B,) + t.shape), dtype)
    dft = to_device(np.broadcast_to(d, (B,) + d.shape), dtype)
    ws = S.Workspace(DEV)
    accs, outs = [], []
    for c in range(calls):
        toks = ints_to_device(_gumbel_tokens(rng, np.log(q), B))
        a, o = S.spec_verify_sample(tgt, dft, toks, T, seed=seed, counter0=c * B * (k + 1) * 2,
                                    kind=kind, workspace=ws)
        accs.append(a)
        outs.append(o)
    acc = torch.cat(accs).cpu().numpy()
    out = torch.cat(outs).cpu().numpy()
    n = acc.shape[0]
    _say(f"{kind} {dtype}: {n} draws, P(n=0,1,2) = "
         f"{[round(float(np.mean(acc == j)), 4) for j in range(k + 1)]}")
    assert np.all((out >= 0) & (out < V) | (out == -1))
    pv = []
    for i in range(k + 1):
        sel = acc >= i if i < k else acc == k
        counts = np.bincount(out[sel, i], minlength=V).astype(np.float64)
        pv.append(_chi2_pvalue(counts, p[i]))
        if i == 0:
            # power: the same counts are far from the draft's law
            assert _chi2_pvalue(counts, q[0]) < 1e-12
    _say(f"chi-square p-values by position: {pv}")
    assert min(pv) > 1e-4, pv


# ---------------------------------------------------------------------------
# expected tokens per step
# ---------------------------------------------------------------------------


def test_mean_emitted_tokens_controlled_acceptance(controlled_full):
    wl = controlled_full
    B, k, V = wl.B, wl.k, wl.V
    calls = 600
    tgt, dft = to_device(wl.target, "f32"), to_device(wl.draft, "f32")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1234)
    ws = S.Workspace(DEV)
    q2 = dft.view(B * k, V)
    accs = []
    for c in range(calls):
        toks = torch.multinomial(q2, 1, generator=gen).view(B, k).to(torch.int32)
        a, _ = S.spec_verify_sample(tgt, dft, toks, 1.0, seed=wl.uniform_seed + 17,
                                    counter0=c * B * (k + 1) * 2, kind="probs", workspace=ws)
        accs.append(a)
    emitted = torch.stack(accs).cpu().numpy().astype(np.float64) + 1.0  # [calls, B]
    # expected emitted tokens per request from its realised per-position
    # acceptance rates: 1 + a_0 + a_0 a_1 + ... (= (1 - a^(k+1)) / (1 - a) for
    # constant a)
    ra = wl.meta["realised_alpha"]
    expect = 1.0 + np.cumprod(ra, axis=1).sum(axis=1)
    alpha = W.request_alpha(B)
    for a in sorted(set(alpha.tolist())):
        cols = alpha == a
        x = emitted[:, cols].ravel()
        mean, se = x.mean(), x.std(ddof=1) / math.sqrt(x.size)
        closed = (1 - a ** (k + 1)) / (1 - a)
        e = float(expect[cols].mean())
        _say(f"alpha={a}: mean emitted {mean:.4f} +- {se:.4f} over {x.size} requests; "
             f"expected {e:.4f} (closed form {closed:.4f})")
        assert abs(e - closed) < 1e-6
        assert abs(mean - e) < 5 * se, (a, mean, e, se)


# ---------------------------------------------------------------------------
# decision rate
# ---------------------------------------------------------------------------


def _decision_rate(wl, calls, chunk):
    B, k, V = wl.B, wl.k, wl.V
    tgt, dft = to_device(wl.target, wl.dtype), to_device(wl.draft, wl.dtype)
    toks_d = ints_to_device(wl.draft_tokens)
    ws = S.Workspace(DEV)
    fr = O.FixedRowsSampler(wl.target, wl.draft, wl.draft_tokens, wl.temperature, wl.kind,
                            wl.dtype)
    per_call = B * (k + 1) * 2
    seed = wl.uniform_seed + 1
    st = dict(requests=0, accept_decisions=0, draw_decisions=0, flagged=0, mismatches=0,
              unflagged=0)
    for c0 in range(0, calls, chunk):
        n = min(chunk, calls - c0)
        accs, outs = [], []
        for c in range(c0, c0 + n):
            a, o = S.spec_verify_sample(tgt, dft, toks_d, wl.temperature, seed=seed,
                                        counter0=c * per_call, kind=wl.kind, workspace=ws)
            accs.append(a)
            outs.append(o)
        acc_g = torch.stack(accs).cpu().numpy()
        out_g = torch.stack(outs).cpu().numpy()
        u = R.uniforms(seed, c0 * per_call, n * per_call).reshape(n, B, k + 1, 2)
        first, token, am, dm = fr.run(u)
        # structure: accepted prefix = draft tokens, then the token, then -1
        pos = np.arange(k + 1)[None, None, :]
        pre = np.broadcast_to(np.concatenate([wl.draft_tokens, np.zeros((B, 1), np.int32)],
                                             axis=1)[None], out_g.shape)
        assert np.all(np.where(pos < acc_g[..., None], out_g == pre, True))
        assert np.all(np.where(pos > acc_g[..., None], out_g == -1, True))
        tok_g = np.take_along_axis(out_g, acc_g[..., None].astype(np.int64), axis=2)[..., 0]
        n_acc = np.minimum(first + 1, k) if k > 0 else np.zeros_like(first)
        st["requests"] += first.size
        st["accept_decisions"] += int(n_acc.sum())
        st["draw_decisions"] += first.size
        in_play = np.arange(k)[None, None, :] < n_acc[..., None]
        st["flagged"] += int(((am < FLAG_BAND) & in_play).sum() + (dm < FLAG_BAND).sum())
        bad = (acc_g != first) | (tok_g != token)
        if bad.any():
            cs, bs = np.nonzero(bad)
            for c, b in zip(cs, bs):
                st["mismatches"] += 1
                if acc_g[c, b] != first[c, b]:
                    m = am[c, b, min(acc_g[c, b], first[c, b])]
                else:
                    m = dm[c, b]
                if not m < FLAG_BAND:
                    st["unflagged"] += 1
                    _say(f"UNFLAGGED call {c0 + c} request {b}: gpu ({acc_g[c, b]}, "
                         f"{tok_g[c, b]}) oracle ({first[c, b]}, {token[c, b]}) margin {m}")
    return st


@pytest.mark.parametrize("name,calls,chunk", [("v32000", 100000, 20000),
                                              ("llama3", 20000, 2500)])
def test_decision_rate(name, calls, chunk, request):
    wl = W.sample_chain_v32000() if name == "v32000" else request.getfixturevalue("llama3_full")
    st = _decision_rate(wl, calls, chunk)
    dec = st["accept_decisions"] + st["draw_decisions"]
    _say(f"decision rate {name}: {st}; decisions {dec}, mismatch rate "
         f"{st['mismatches'] / dec:.3g}, flagged share {st['flagged'] / dec:.3g}")
    assert st["unflagged"] == 0
    assert st["mismatches"] < 1e-6 * dec
