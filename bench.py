#!/usr/bin/env python3
"""Benchmark of the batched sampling verification step on one MI355X.

Workload: B=64 requests, k=8 drafts, V=128256 (Llama-3 vocabulary), bf16
target logits N(0, 3^2) with 20 peak tokens per row boosted by +8, draft =
target + N(0, 1.5^2), temperature 0.7, draft tokens drawn from the draft
distribution, uniforms from the SplitMix64 counter (fresh per step).

One step = one spec_verify_sample call: the float32 row-statistics pass, the
float64 min(1, p/q) tests, and the float64 residual / bonus draw, in one
launch (k_sample_one).  The default schedule exits early: a row whose
request is known to stop before its position is not read further (identical
outputs).  --path one_launch reads every row; --path two_launch runs the row
pass then the draw.  Inputs are resident in HBM; `--copies` input copies are
rotated so the 256 MB Infinity Cache cannot serve a step from the previous
one.

Prints one JSON line: verified positions per second (B * (k+1) target
positions per step) and, for the dominant kernel, the workload's algorithmic
HBM bytes per launch (every logit row once, plus the rows each request draws
from and the searched chunk) over its average duration, timed with events
that each launch stamps from its own dispatch, against the 8 TB/s peak; the
bytes a call must read; the other one-launch schedule on the same steps; the
float64 oracle on the host, whose outputs gate the timed steps' outputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
# Float64 vector issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (one
# fp64 add, multiply, fma, max, round or scale per lane per clock; the
# published 78.6 TFLOP/s counts an fma as two flops).
PEAK_FP64_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# fp64 operations per element of a float64 row statistic: the scaled
# argument (fma), the clamp (max), the split into n and f (round, subtract),
# the degree-3 polynomial (3 fma), the table product (mul), the scaling by
# 2^(n/256 integer part) (ldexp) and the accumulation (add).
TREE_STAT_OPS_PER_ELEM = 10
METRIC = "verified positions/sec + achieved HBM GB/s (% of peak), B=64 k=8 V=128256"
# Dominant kernel of each path, and the committed rocprofv3 counter summary of
# its HBM traffic at this workload.
KERNELS = {"auto": "k_sample_one", "one_launch": "k_sample_one", "two_launch": "k_row_stats",
           "early_exit": "k_sample_one"}
# The schedule each --path asks for (auto: the library picks by shape; at the
# headline shape it picks early exit).
SCHEDULE_OF = {"auto": "auto", "one_launch": "one_launch", "two_launch": "two_launch",
               "early_exit": "early_exit"}


# Kernel sources each traffic summary is keyed to.
COMMON_SOURCES = ["verify_accept_sampling_amd/csrc/device_common.h",
                  "verify_accept_sampling_amd/csrc/device_math.h",
                  "verify_accept_sampling_amd/csrc/internal.h"]
SAMPLE_SOURCES = ["verify_accept_sampling_amd/csrc/sample.hip",
                  "verify_accept_sampling_amd/csrc/sample_device.h"] + COMMON_SOURCES
PROBS_SOURCES = ["verify_accept_sampling_amd/csrc/probs.hip",
                 "verify_accept_sampling_amd/csrc/sample_device.h"] + COMMON_SOURCES
# Traffic summaries: key (a --path of the headline workload, or "probs") ->
# (dominant kernel, file tag, workload, sources).
TRAFFIC = {
    "auto": ("k_sample_one", "b64_k8_v128256_early_exit", "B=64 k=8 V=128256 bf16",
             SAMPLE_SOURCES),
    "early_exit": ("k_sample_one", "b64_k8_v128256_early_exit", "B=64 k=8 V=128256 bf16",
                   SAMPLE_SOURCES),
    "one_launch": ("k_sample_one", "b64_k8_v128256", "B=64 k=8 V=128256 bf16", SAMPLE_SOURCES),
    "two_launch": ("k_row_stats", "b64_k8_v128256", "B=64 k=8 V=128256 bf16", SAMPLE_SOURCES),
    "probs": ("k_probs_rows", "b512_k8_v128256", "B=512 k=8 V=128256 fp32 probabilities",
              PROBS_SOURCES),
}


def traffic_file(key: str) -> str:
    kernel, tag, _, _ = TRAFFIC[key]
    return os.path.join(ROOT, "profiles", f"{kernel}_{tag}_traffic.json")


# Algorithmic bytes of the row pass at this workload: every logit of the
# 2k+1 = 17 rows of all 64 requests read once (bf16).
ALGO_ROW_BYTES = 64 * 17 * 128256 * 2
# Elements of the chunk the inverse-CDF search reads again.
DRAW_CHUNK = 512
PROBS_PICK_CHUNK = 2048  # elements of the chunk the probability-row draw searches


def kernel_source_sha(sources) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch of the dominant kernel of `key` (a headline
    path, or "probs") from the committed rocprofv3 counter summary, or None
    if absent or taken on other kernel sources."""
    try:
        with open(traffic_file(key)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha(TRAFFIC[key][3]):
        return None
    return t.get("hbm_bytes_per_launch")


def _pmc_means(csv_path: str, counter: str, kernel: str):
    """Mean per-dispatch value of `counter` for `kernel` and for the
    calibration copy (torch's elementwise negation kernel), from a rocprofv3
    --pmc CSV."""
    import csv

    acc = {"row": [], "copy": []}
    with open(csv_path, newline="") as f:
        for rec in csv.DictReader(f):
            if rec["Counter_Name"] != counter:
                continue
            name = rec["Kernel_Name"]
            key = "row" if kernel in name else "copy" if "neg_kernel" in name else None
            if key:
                acc[key].append(float(rec["Counter_Value"]))
    if not acc["row"] or not acc["copy"]:
        raise SystemExit(f"{csv_path}: no {counter} rows for {kernel} and the copy kernel")
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def summarize_pmc(fetch_csv: str, write_csv: str, copy_mib: int, command: str, key: str):
    """Turn the FETCH_SIZE and WRITE_SIZE passes (KiB per dispatch) into HBM
    bytes per launch of `kernel`.  Each counter is scaled by what it reads
    for a plain elementwise copy of copy_mib MiB (which reads and writes
    exactly that many bytes), and the result is written next to the
    kernel-source hash it was taken on."""
    nbytes = copy_mib * 1024 * 1024
    kernel, _, workload, sources = TRAFFIC[key]
    fetch, nf = _pmc_means(fetch_csv, "FETCH_SIZE", kernel)
    write, nw = _pmc_means(write_csv, "WRITE_SIZE", kernel)
    f_scale = nbytes / (fetch["copy"] * 1024.0)
    w_scale = nbytes / (write["copy"] * 1024.0)
    rd = fetch["row"] * 1024.0 * f_scale
    wr = write["row"] * 1024.0 * w_scale
    out = {
        "kernel": kernel, "path": key, "workload": workload,
        "kernel_source_sha": kernel_source_sha(sources),
        "fetch_kib_per_dispatch": fetch["row"], "write_kib_per_dispatch": write["row"],
        "copy_bytes": nbytes, "copy_fetch_kib": fetch["copy"], "copy_write_kib": write["copy"],
        "fetch_scale": f_scale, "write_scale": w_scale,
        "dispatches": {"fetch_pass": nf, "write_pass": nw},
        "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
        "hbm_bytes_per_launch": rd + wr,
        "command": command,
    }
    with open(traffic_file(key), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


# ---------------------------------------------------------------------------
# cpu_baseline leg: the float64 oracle on the timed steps' own inputs
# ---------------------------------------------------------------------------
#
# Step i of the timed GPU pass verifies the workload with the uniforms at
# counter0 = i * B * (k+1) * 2.  The oracle legs run the same steps (their
# requests one by one, as the oracle stands), so their outputs double as the
# correctness gate of the GPU pass.  They run before anything touches the GPU
# (the all-cores leg forks a process pool).

_LEG = {}  # the workload, shared with forked workers (copy-on-write)


def _oracle_request(step: int, b: int):
    """Oracle outputs of request b at timed step `step`, with what the gate
    needs to classify a disagreement: (accepted, tokens, accept margins by
    position, draw margin)."""
    import oracle.rng as R
    import oracle.verify as O

    wl, n_u = _LEG["wl"], _LEG["n_u"]
    u = R.uniforms(wl.uniform_seed, step * n_u + b * (wl.k + 1) * 2, (wl.k + 1) * 2)
    r = O.verify_sample_request(wl.target[b], wl.draft[b] if wl.k > 0 else None,
                                wl.draft_tokens[b], u.reshape(wl.k + 1, 2), wl.temperature,
                                wl.kind, wl.dtype)
    acc_m = {d.position: d.margin for d in r.decisions if d.kind == "accept"}
    draw_m = [d.margin for d in r.decisions if d.kind == "resample"][0]
    return r.accepted, list(r.tokens), acc_m, draw_m


def _oracle_steps(steps, budget_s: float, t0=None):
    """Whole steps (every request) in order until the budget is spent."""
    t0 = time.perf_counter() if t0 is None else t0
    out = {}
    wl = _LEG["wl"]
    for st in steps:
        if time.perf_counter() - t0 >= budget_s:
            break
        out[st] = [_oracle_request(st, b) for b in range(wl.B)]
    return out


def _pool_worker(args):
    steps, budget_s = args
    return _oracle_steps(steps, budget_s)


def oracle_legs(wl, first_step: int, n_steps: int, budget_s: float, label: str):
    """(1-core leg, all-cores leg, oracle outputs by step).  Each leg runs
    whole timed steps for about budget_s seconds."""
    import multiprocessing as mp

    _LEG["wl"] = wl
    _LEG["n_u"] = wl.B * (wl.k + 1) * 2
    steps = list(range(first_step, first_step + n_steps))
    print(f"bench: cpu baseline, 1 core ({budget_s:.0f} s)", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    res1 = _oracle_steps(steps, budget_s, t0)
    dt1 = time.perf_counter() - t0
    pos1 = len(res1) * wl.B * (wl.k + 1)
    one = {"value": pos1 / dt1, "unit": "verified positions/s", "cores": 1, "kind": "oracle",
           "sample": f"{len(res1)} timed steps ({len(res1) * wl.B} requests) of the {label} "
                     f"workload, {dt1:.1f} s on 1 host thread"}
    cores = min(16, len(os.sched_getaffinity(0)))
    # the steps the 1-core leg did not reach first, then the others again
    rest = steps[len(res1):] + steps[:len(res1)]
    print(f"bench: cpu baseline, {cores} processes ({budget_s:.0f} s)", file=sys.stderr,
          flush=True)
    chunks = [(rest[w::cores], budget_s) for w in range(cores)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        parts = pool.map(_pool_worker, chunks)
    dtn = time.perf_counter() - t0
    resn = {}
    for p_ in parts:
        resn.update(p_)
    posn = len(resn) * wl.B * (wl.k + 1)
    allc = {"value": posn / dtn, "unit": "verified positions/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(resn)} timed steps ({len(resn) * wl.B} requests) of the {label} "
                      f"workload, {dtn:.1f} s in {cores} processes (one request at a time "
                      f"each)"}
    res = dict(res1)
    res.update(resn)
    return one, allc, res


FLAG_BAND = 1e-5


def correctness_gate(acc_steps, out_steps, first_step: int, oracle_res):
    """Compare the GPU outputs of the timed steps the oracle legs covered.
    A disagreement is allowed only when its first differing decision (the
    acceptance test at the earlier stop, else the draw) lies within 1e-5 of
    its boundary in the oracle."""
    g = dict(steps=0, requests=0, decisions=0, accept_decisions=0, draw_decisions=0, flagged=0,
             mismatches=0, unflagged=0)
    for st, reqs in sorted(oracle_res.items()):
        i = st - first_step
        g["steps"] += 1
        for b, (n_o, toks_o, acc_m, draw_m) in enumerate(reqs):
            g["requests"] += 1
            g["accept_decisions"] += len(acc_m)
            g["draw_decisions"] += 1
            g["flagged"] += sum(1 for m in acc_m.values() if m < FLAG_BAND)
            g["flagged"] += int(draw_m < FLAG_BAND)
            n_g = int(acc_steps[i, b])
            toks_g = [int(t) for t in out_steps[i, b, : n_g + 1]] if 0 <= n_g else []
            if n_g == n_o and toks_g == toks_o:
                continue
            g["mismatches"] += 1
            m = acc_m.get(min(n_g, n_o), 0.0) if n_g != n_o else draw_m
            if not (0 <= n_g and m < FLAG_BAND):
                g["unflagged"] += 1
    g["decisions"] = g["accept_decisions"] + g["draw_decisions"]
    return g


def probe_and_emitted_check(wl, acc_steps, probe_np):
    """Two more checks of the timed outputs against the oracle on the same
    inputs.  (i) The probe of one call, p_i(x_i) and q_i(x_i) for every draft
    position, against the oracle's float64 values: the largest absolute
    difference (the pages' softmax probabilities, 1e-5 at most).  (ii) The
    mean emitted tokens over the timed steps against its expectation: every
    step sees the same rows and draft tokens with fresh uniforms, so request
    b accepts position i with probability a_i = min(1, p_i(x_i)/q_i(x_i))
    while the ones before it were accepted, and emits 1 + sum over n = 1..k
    of prod_{i<n} a_i tokens on average (the expected-token formula with
    these per-position rates).  Reported with the standard error of the
    per-step means and its z score."""
    import numpy as np

    import oracle.verify as O

    B, k = wl.B, wl.k
    pv = np.zeros((B, k))
    qv = np.zeros((B, k))
    for b in range(B):
        pv[b], qv[b] = O.probe_values(wl.target, wl.draft, wl.draft_tokens, wl.temperature,
                                      wl.kind, wl.dtype, b)
    dp = float(max(np.abs(probe_np[:, :k, 0] - pv).max(), np.abs(probe_np[:, :k, 1] - qv).max()))
    with np.errstate(divide="ignore", invalid="ignore"):
        a = np.where(qv > 0, np.minimum(1.0, pv / np.where(qv > 0, qv, 1.0)), 0.0)
    expect = 1.0 + np.cumprod(a, axis=1).sum(axis=1)  # per request
    emitted = acc_steps.astype(np.float64) + 1.0
    per_step = emitted.mean(axis=1)
    se = float(per_step.std(ddof=1) / np.sqrt(len(per_step))) if len(per_step) > 1 else None
    mean = float(per_step.mean())
    e = float(expect.mean())
    return ({"max_abs_dp": dp, "positions": int(B * k), "tolerance": 1e-5},
            {"mean": mean, "expected": e, "se": se,
             "z": (mean - e) / se if se else None, "steps": int(len(per_step))})


# Extra workloads (not the headline line): greedy chain and tree greedy.
GREEDY_WORKLOADS = {
    "tree": "tree greedy, B=16, 61 nodes (1 root + 60, depth 5), V=128256, bf16",
    "greedy_b64": "greedy chain, B=64, k=8, V=128256, bf16",
    "greedy_b1": "greedy chain, B=1, k=4, V=1000, fp32 (latency)",
}
GREEDY_KERNELS = {"tree": "k_tree_greedy", "greedy_b64": "k_greedy_chain",
                  "greedy_b1": "k_greedy_chain"}


def copy_calibration(mib: int, dev):
    """A plain elementwise copy (negation) of `mib` MiB of float32, three
    times: the reference kernel that scales the HBM counters."""
    if mib <= 0:
        return
    import torch

    nb = mib * 1024 * 1024
    src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)  # one elementwise kernel: reads nb bytes, writes nb
    torch.cuda.synchronize()
    del src, dst
    print(f"bench: copy calibration, 3 x {mib} MiB", file=sys.stderr, flush=True)


def timed_steps(step, first, steps, profile, keep=None):
    """Run `steps` steps between two events and return ms per step.  With
    profile, every launch also carries dispatch-stamped start/stop events
    (read afterwards with spec_profile_read); those add host work per launch,
    so the step rate comes from an uninstrumented pass."""
    import torch

    import verify_accept_sampling_amd as S

    S.spec_profile_enable(profile)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        out = step(first + i)
        if keep is not None:
            keep.append(out[0])
    end.record()
    torch.cuda.synchronize()
    if profile:
        S.spec_profile_enable(False)
    return start.elapsed_time(end) / steps


def bench_greedy(args):
    """One JSON line for a greedy workload: the kernel reads every logit row
    once (B * rows * V * elem bytes), so its roofline is HBM at that size."""
    import numpy as np

    import oracle.verify as O
    import workloads as W

    name = args.workload
    print(f"bench: generating {GREEDY_WORKLOADS[name]}", file=sys.stderr, flush=True)
    if name == "tree":
        wl = W.tree_greedy()
        rows, dtype = len(wl.parent), wl.dtype
        parent = wl.parent.tolist()
    elif name == "greedy_b64":
        wl = W.greedy_chain(B=64, k=8, V=128256, seed=1003, dtype="bf16")
        rows, dtype = wl.k + 1, wl.dtype
    else:
        wl = W.greedy_chain()
        rows, dtype = wl.k + 1, wl.dtype
    B, V = wl.target.shape[0], wl.target.shape[-1]
    # The oracle first, before anything touches the GPU (the all-cores leg
    # forks): once on one host thread (its outputs are the gate's), then the
    # requests split over the host cores.
    t_cpu = time.perf_counter()
    if name == "tree":
        want = O.verify_tree_greedy(wl.target, wl.parent, wl.node_tokens, dtype)[:2]
    else:
        want = O.verify_greedy(wl.target, wl.draft_tokens, dtype)[:2]
    dt_cpu = time.perf_counter() - t_cpu
    cores = max(1, min(16, len(os.sched_getaffinity(0)), B))
    dt_all = dt_cpu
    if cores > 1:
        import multiprocessing as mp

        _LEG["wl"] = wl
        bounds = np.linspace(0, B, cores + 1).astype(int)
        t_all = time.perf_counter()
        with mp.get_context("fork").Pool(cores) as pool:
            pool.map(_greedy_oracle_leg,
                     [(name, int(bounds[i]), int(bounds[i + 1])) for i in range(cores)])
        dt_all = time.perf_counter() - t_all

    import torch

    import verify_accept_sampling_amd as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    toks = torch.from_numpy(wl.node_tokens if name == "tree" else wl.draft_tokens).to(dev)

    def to_dev(a):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t0 = to_dev(wl.target)
    copies = [t0] + [t0.clone() for _ in range(args.copies - 1)]
    ws = S.Workspace(dev)
    # preallocated outputs, as a serving loop keeps them
    n_out = (int(W.tree_depths(np.asarray(parent)).max()) + 1) if name == "tree" else rows
    outs = (torch.empty(B, dtype=torch.int32, device=dev),
            torch.empty(B, n_out, dtype=torch.int32, device=dev))

    def step(i):
        t = copies[i % len(copies)]
        if name == "tree":
            return S.spec_verify_tree_greedy(t, parent, toks, want_path=False, workspace=ws,
                                             out=outs)
        return S.spec_verify_greedy(t, toks, workspace=ws, out=outs)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step = timed_steps(step, args.warmup, args.steps, profile=False)
    timed_steps(step, args.warmup + args.steps, args.steps, profile=True)
    n, ms = S.spec_profile_read("row_pass")
    kern_us = ms / n * 1e3
    elem = 2 if dtype == "bf16" else 4
    nbytes = float(B * rows * V * elem)
    achieved = nbytes / (kern_us * 1e-6) / 1e9
    positions = B * rows
    result = {
        "metric": f"verified positions/s ({GREEDY_WORKLOADS[name]})",
        "value": positions / (ms_step * 1e-3),
        "unit": "verified positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "B": B, "rows_per_request": rows, "V": V, "logits": dtype,
                   "input_copies": len(copies)},
        "roofline": {"bound": "hbm", "kernel": GREEDY_KERNELS[name], "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": None, "algorithmic_bytes_per_launch": nbytes},
        "kernels_avg_us": {GREEDY_KERNELS[name]: kern_us},
    }
    # Gate: the outputs on every input copy against the oracle, which must
    # agree exactly (argmax and integer comparisons only).  The oracle's
    # times on the same workload are the CPU baselines.
    mism = 0
    for i in range(len(copies)):
        got = step(i)
        mism += int((got[0].cpu().numpy() != want[0]).sum())
        mism += int((got[1].cpu().numpy() != want[1]).sum())
    result["correctness_gate"] = {"input_copies": len(copies), "requests": B * len(copies),
                                  "mismatched_outputs": mism}
    result["cpu_baseline"] = {"value": positions / dt_all, "unit": "verified positions/s",
                              "cores": cores, "kind": "oracle",
                              "sample": f"the whole workload ({B} requests) once, {dt_all:.2f} s "
                                        f"in {cores} processes (requests split evenly)"}
    result["cpu_baseline_1core"] = {"value": positions / dt_cpu, "unit": "verified positions/s",
                                    "cores": 1, "kind": "oracle",
                                    "sample": f"the whole workload ({B} requests) once, "
                                              f"{dt_cpu:.2f} s on 1 host thread"}
    print(json.dumps(result), flush=True)
    if mism:
        print("bench: FAILED: greedy outputs differ from the oracle", file=sys.stderr, flush=True)
        sys.exit(1)


def bench_serving(args):
    """One JSON line for the rejected-draft mask after a chain verification
    at the headline shape (B=64, k=8), with the slot mapping padded in
    place.  Bytes per launch: accepted_len read, the mask written, and the
    rejected entries' 8-byte slots written; the launch is bound by its own
    latency, not by HBM, and the line says so."""
    import numpy as np
    import torch

    import verify_accept_sampling_amd as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, k = 64, 8
    rng = np.random.default_rng(2024)
    acc = torch.from_numpy(rng.integers(0, k + 1, size=B).astype(np.int32)).to(dev)
    slots = torch.arange(B * k, dtype=torch.int64, device=dev).view(B, k)

    def step(i):
        return S.spec_rejected_mask(acc, k, slot_mapping=slots, pad_slot=-1)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step = timed_steps(step, args.warmup, args.steps, profile=False)
    timed_steps(step, args.warmup + args.steps, args.steps, profile=True)
    n, ms = S.spec_profile_read("serving")
    kern_us = ms / n * 1e3
    rejected = int((k - acc.clamp(0, k)).sum().item())
    nbytes = float(B * 4 + B * k + rejected * 8)
    achieved = nbytes / (kern_us * 1e-6) / 1e9
    result = {
        "metric": "rejected-draft masks per second (chain, B=64, k=8, slot mapping padded)",
        "value": 1.0 / (ms_step * 1e-3), "unit": "calls/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic",
        "config": {"workload": "rejected_mask_b64_k8", "B": B, "k": k},
        "roofline": {"bound": "hbm", "kernel": "k_rejected_mask", "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": None, "algorithmic_bytes_per_launch": nbytes,
                     "note": "launch-latency bound: a few KB per launch"},
        "kernels_avg_us": {"k_rejected_mask": kern_us},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def _greedy_oracle_leg(args_tuple):
    """Worker of the greedy lines' all-cores leg: the oracle over requests
    [b0, b1) of the shared workload (argmax and integer rules only)."""
    import oracle.verify as O

    name, b0, b1 = args_tuple
    wl = _LEG["wl"]
    if name == "tree":
        O.verify_tree_greedy(wl.target[b0:b1], wl.parent, wl.node_tokens[b0:b1], wl.dtype)
    else:
        O.verify_greedy(wl.target[b0:b1], wl.draft_tokens[b0:b1], wl.dtype)
    return b1 - b0


def _tree_oracle_steps(args_tuple):
    """Oracle outputs of whole timed steps of the tree workload (shared
    through _LEG) until the budget is spent."""
    steps, budget_s = args_tuple
    import oracle.rng as R
    import oracle.verify as O

    wl = _LEG["wl"]
    t0 = time.perf_counter()
    out = {}
    for st in steps:
        if time.perf_counter() - t0 >= budget_s:
            break
        u = R.tree_uniforms(wl.uniform_seed, wl.B, wl.n_nodes, st * wl.B * wl.n_nodes * 2)
        _, _, _, res = O.verify_tree_sample(wl.target, wl.draft, wl.parent, wl.node_tokens, u,
                                            wl.temperature, wl.kind, wl.dtype)
        out[st] = res
    return out


def bench_tree_sample(args):
    """One JSON line for tree sampling verification: the static tree (1 root
    + 60 nodes, branching 4, 3, 2, 2, 1) with draft logits, B=16,
    V=128256, bf16, T=0.7.  Algorithmic bytes of a call: both rows of the
    nodes with children once (their float64 statistics), the leaves' target
    rows once (float32 statistics), both rows of a node once per
    sibling-rank mass pass, and the stop node's rows drawn from.  The
    dominant kernel, k_tree_stats, is bound by float64 arithmetic (one exp
    term per element): its roofline is fp64 operations against the vector
    issue rate."""
    import numpy as np

    import workloads as W

    print("bench: generating the tree sampling workload", file=sys.stderr, flush=True)
    wl = W.tree_sample()
    B, N, V = wl.B, wl.n_nodes, wl.V
    first = args.warmup
    n_u = B * N * 2
    res_cpu = None
    one = None
    if not args.no_cpu_baseline:
        import multiprocessing as mp

        _LEG["wl"] = wl
        steps = list(range(first, first + args.steps))
        print(f"bench: cpu baseline, 1 core ({args.cpu_seconds:.0f} s)", file=sys.stderr,
              flush=True)
        t0 = time.perf_counter()
        res1 = _tree_oracle_steps((steps, args.cpu_seconds))
        dt1 = time.perf_counter() - t0
        one = {"value": len(res1) * B / dt1, "unit": "verified requests/s", "cores": 1,
               "kind": "oracle", "sample": f"{len(res1)} timed steps ({len(res1) * B} requests), "
                                           f"{dt1:.1f} s on 1 host thread"}
        cores = min(16, len(os.sched_getaffinity(0)))
        rest = steps[len(res1):] + steps[:len(res1)]
        t0 = time.perf_counter()
        with mp.get_context("fork").Pool(cores) as pool:
            parts = pool.map(_tree_oracle_steps,
                             [(rest[w::cores], args.cpu_seconds) for w in range(cores)])
        dtn = time.perf_counter() - t0
        res_cpu = dict(res1)
        n_all = 0
        for p_ in parts:
            n_all += len(p_)
            res_cpu.update(p_)
        allc = {"value": n_all * B / dtn, "unit": "verified requests/s", "cores": cores,
                "kind": "oracle", "sample": f"{n_all} timed steps ({n_all * B} requests), "
                                            f"{dtn:.1f} s in {cores} processes"}

    import torch

    import verify_accept_sampling_amd as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    t0d, d0d = dev_bf16(wl.target), dev_bf16(wl.draft)
    n_copies = max(args.copies, 2)  # 0.5 GB per copy
    copies = [(t0d, d0d)] + [(t0d.clone(), d0d.clone()) for _ in range(n_copies - 1)]
    toks = torch.from_numpy(wl.node_tokens).to(dev)
    parent = wl.parent.tolist()
    ws = S.Workspace(dev)
    D = int(W.tree_depths(wl.parent).max())
    acc_all = torch.empty((args.steps, B), dtype=torch.int32, device=dev)
    out_all = torch.empty((args.steps, B, D + 1), dtype=torch.int32, device=dev)
    path_all = torch.empty((args.steps, B, D + 1), dtype=torch.int32, device=dev)
    scratch = (torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B, D + 1), dtype=torch.int32, device=dev),
               torch.empty((B, D + 1), dtype=torch.int32, device=dev))

    def run(i, out):
        t, d = copies[i % len(copies)]
        S.spec_verify_tree_sample(t, d, parent, toks, wl.temperature, seed=wl.uniform_seed,
                                  counter0=i * n_u, workspace=ws, out=out)

    for i in range(args.warmup):
        run(i, scratch)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for j in range(args.steps):
        run(first + j, (acc_all[j], out_all[j], path_all[j]))
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    S.spec_profile_enable(True)
    for j in range(args.steps):
        run(first + j, scratch)
    torch.cuda.synchronize()
    S.spec_profile_enable(False)
    kinds = ("tree_stats", "tree_mass", "tree_walk", "tree_leaf", "tree_draw")
    kern = {}
    for kk in kinds:
        d = S.spec_profile_durations(kk)
        if d:
            kern[kk] = {"launches": len(d), "avg_us": sum(d) / len(d) * 1e3,
                        "p10_us": _pct(d, 10) * 1e3, "p90_us": _pct(d, 90) * 1e3}
    # bytes
    kids = [[] for _ in range(N)]
    for j in range(1, N):
        kids[parent[j]].append(j)
    n_int = sum(1 for k_ in kids if k_)
    mass_units = sum(max(0, len(k_) - 1) for k_ in kids)
    row = V * 2
    stats_bytes = float(B * 2 * n_int * row)
    stats_ops = float(B * 2 * n_int * V * TREE_STAT_OPS_PER_ELEM)
    acc_np = acc_all.cpu().numpy()
    path_np = path_all.cpu().numpy()
    out_np = out_all.cpu().numpy()
    # draw: the stop node's target row, and its draft row after a rejection;
    # a stop leaf's target row is also read once before, for its statistic
    drawn = leaves = 0
    for jj in range(args.steps):
        for b in range(B):
            s_node = int(path_np[jj, b, acc_np[jj, b]])
            drawn += 2 if kids[s_node] else 1
            leaves += 0 if kids[s_node] else 1
    draw_bytes = drawn / args.steps * row
    leaf_bytes = leaves / args.steps * row
    mass_bytes = float(B * mass_units * 2 * row)
    step_bytes = stats_bytes + leaf_bytes + mass_bytes + draw_bytes
    st_us = kern["tree_stats"]["avg_us"]
    achieved = stats_ops / (st_us * 1e-6) / 1e12
    gate = None
    if res_cpu is not None:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from parity_helpers import compare_tree_sample

        gate = dict(steps=0, requests=0, flagged=0, mismatches=0, unflagged=0)
        for st, res in sorted(res_cpu.items()):
            j = st - first
            g = compare_tree_sample(acc_np[j], out_np[j], path_np[j], res, wl.parent, range(B))
            gate["steps"] += 1
            for key in ("requests", "flagged", "mismatches", "unflagged"):
                gate[key] += g[key]
    result = {
        "metric": "verified requests/s (tree sampling, 61-node tree, B=16, V=128256, bf16, T=0.7)",
        "value": B / (ms_step * 1e-3), "unit": "verified requests/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": "tree_sample_b16_n61_v128256_bf16_t0.7", "B": B, "nodes": N,
                   "V": V, "logits": "bf16", "temperature": wl.temperature,
                   "input_copies": len(copies), "draw_arithmetic": "f64"},
        "roofline": {"bound": "alu", "kernel": "k_tree_stats", "achieved": achieved,
                     "peak": PEAK_FP64_TOPS, "unit": "Tops/s (fp64)",
                     "frac": achieved / PEAK_FP64_TOPS, "traffic": None,
                     "algorithmic_ops_per_launch": stats_ops,
                     "algorithmic_bytes_per_launch": stats_bytes,
                     "hbm_gbps": stats_bytes / (st_us * 1e-6) / 1e9},
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
        "kernels": kern,
        "mean_accepted": float(acc_np.mean()),
        "cpu_baseline": allc if res_cpu is not None else None,
        "cpu_baseline_1core": one,
        "correctness_gate": gate,
    }
    print(json.dumps(result), flush=True)
    if gate is not None and gate["unflagged"]:
        print("bench: FAILED: tree sampling outputs disagree with the oracle away from any "
              "decision boundary", file=sys.stderr, flush=True)
        sys.exit(1)


def bench_probs(args):
    """One JSON line for the probability-row workload: B=512, k=8, V=128256
    float32 rows with a prescribed overlap alpha in {0.6, 0.8, 0.9}.  Two
    kernels: k_probs_rows (acceptance tests, then one pass over each
    request's rows drawn from -- target and draft row n after a rejection,
    target row k at the bonus -- into per-chunk sums) and k_probs_pick (the
    draw from those sums, reading one 2048-element chunk of those rows
    again).  The row pass is the dominant kernel; its algorithmic bytes are
    the rows drawn from and the gathered acceptance-test values."""
    import numpy as np

    import workloads as W

    print("bench: generating B=512 k=8 V=128256 fp32 probability rows", file=sys.stderr,
          flush=True)
    wl = W.controlled_acceptance()
    B, k, V = wl.B, wl.k, wl.V
    first = args.warmup  # counter base of the first timed step
    legs = None
    if not args.no_cpu_baseline:
        legs = oracle_legs(wl, first, args.steps, args.cpu_seconds, "probability-row")

    import torch

    import verify_accept_sampling_amd as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = torch.from_numpy(wl.target).to(dev)
    d0 = torch.from_numpy(wl.draft).to(dev)
    n_copies = max(1, min(args.copies, 2))  # 4.5 GB per copy, far beyond the caches
    copies = [(t0, d0)] + [(t0.clone(), d0.clone()) for _ in range(n_copies - 1)]
    toks = torch.from_numpy(wl.draft_tokens).to(dev)
    ws = S.Workspace(dev)
    n_u = B * (k + 1) * 2
    acc_all = torch.empty((args.steps, B), dtype=torch.int32, device=dev)
    out_all = torch.empty((args.steps, B, k + 1), dtype=torch.int32, device=dev)
    scratch = (torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B, k + 1), dtype=torch.int32, device=dev))

    def run(i, out):
        t, d = copies[i % len(copies)]
        S.spec_verify_sample(t, d, toks, 1.0, seed=wl.uniform_seed, counter0=i * n_u,
                             kind="probs", workspace=ws, out=out)
        return out

    copy_calibration(args.copy_calibration_mib, dev)

    print(f"bench: warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        run(i, scratch)
    torch.cuda.synchronize()
    ms_step = timed_steps(lambda i: run(i, (acc_all[i - first], out_all[i - first])), first,
                          args.steps, profile=False)
    timed_steps(lambda i: run(i, scratch), first + args.steps, args.steps, profile=True)
    rows_d = np.asarray(S.spec_profile_durations("row_pass")) * 1e3
    pick_d = np.asarray(S.spec_profile_durations("draw")) * 1e3
    acc_np, out_np = acc_all.cpu().numpy(), out_all.cpu().numpy()
    row_bytes = V * 4
    drawn_rows = (acc_np < k).sum(axis=1) + B  # per step: two rows at a rejection, one at the bonus
    gathers = np.minimum(acc_np + 1, k).sum(axis=1) * 2 * 4
    rows_bytes = float(np.mean(drawn_rows * row_bytes + gathers))
    pick_bytes = float(np.mean(drawn_rows * min(V, PROBS_PICK_CHUNK) * 4))
    rows_us, pick_us = float(rows_d.mean()), float(pick_d.mean())
    achieved = rows_bytes / (rows_us * 1e-6) / 1e9
    step_bytes = rows_bytes + pick_bytes
    result = {
        "metric": "verified positions/s (sampling, probability rows, B=512, k=8, V=128256, fp32)",
        "value": B * (k + 1) / (ms_step * 1e-3),
        "unit": "verified positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": "probs_b512_k8_v128256_f32", "B": B, "k": k, "V": V,
                   "alphas": [0.6, 0.8, 0.9], "input_copies": len(copies)},
        "roofline": {"bound": "hbm", "kernel": "k_probs_rows", "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": measured_traffic("probs"),
                     "algorithmic_bytes_per_launch": rows_bytes},
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_frac": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "kernels_avg_us": {"k_probs_rows": rows_us, "k_probs_pick": pick_us},
        "kernel_p10_p90_us": {"k_probs_rows": [float(np.percentile(rows_d, 10)),
                                               float(np.percentile(rows_d, 90))],
                              "k_probs_pick": [float(np.percentile(pick_d, 10)),
                                               float(np.percentile(pick_d, 90))]},
        "mean_accepted": float(acc_np.mean()),
        "workspace_status": S.spec_workspace_status(ws),
    }
    gate = None
    if legs is not None:
        one, allc, res = legs
        result["cpu_baseline"] = allc
        result["cpu_baseline_1core"] = one
        gate = correctness_gate(acc_np, out_np, first, res)
        t, d = copies[first % len(copies)]
        _, _, pr = S.spec_verify_sample(t, d, toks, 1.0, seed=wl.uniform_seed,
                                        counter0=first * n_u, kind="probs", workspace=ws,
                                        probe=True)
        torch.cuda.synchronize()
        gate["probe"], gate["emitted"] = probe_and_emitted_check(wl, acc_np, pr.cpu().numpy())
        result["correctness_gate"] = gate
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    bad = []
    if gate is not None and gate["unflagged"]:
        bad.append("probability-row outputs disagree with the oracle away from any decision "
                   "boundary")
    if gate is not None and gate["probe"]["max_abs_dp"] > 1e-5:
        bad.append(f"probe values differ from the oracle by {gate['probe']['max_abs_dp']:.2e}")
    if gate is not None and gate["emitted"]["z"] is not None and abs(gate["emitted"]["z"]) > 6:
        bad.append(f"mean emitted tokens {gate['emitted']['mean']:.4f} is "
                   f"{gate['emitted']['z']:.1f} standard errors from its expectation")
    if bad:
        print("bench: FAILED: " + "; ".join(bad), file=sys.stderr, flush=True)
        sys.exit(1)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--copies", type=int, default=3, help="input copies rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run a plain elementwise copy (negation) of this many MiB of float32 "
                         "three times before the warmup, as the reference kernel for HBM "
                         "counter scaling")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: turn two rocprofv3 --pmc CSVs (FETCH_SIZE, WRITE_SIZE) "
                         "into the row-statistics traffic file")
    ap.add_argument("--pmc-command", default="", help="command line recorded with --summarize-pmc")
    ap.add_argument("--no-early-exit", action="store_true",
                    help="skip the extra passes of the explicit one-launch schedules (full "
                         "sweep, early exit) on the timed steps' inputs")
    ap.add_argument("--workload",
                    choices=sorted(SAMPLE_WORKLOADS) + ["probs", "serving", "tree_sample"]
                    + sorted(GREEDY_WORKLOADS),
                    default="sample",
                    help="sample (default): the headline sampling workload; sample_v32000: "
                         "B=8 k=4 V=32000; probs: sampling on probability rows (B=512); the "
                         "others print a line for a greedy or serving kernel")
    ap.add_argument("--path", choices=sorted(KERNELS), default="auto",
                    help="auto: the library's default schedule (early exit at the headline "
                         "shape, the full sweep when all rows fit one round); one_launch: the "
                         "one-launch kernel reading every row; two_launch: row pass, then "
                         "draw; early_exit: the one-launch kernel that stops reading rows past "
                         "each request's first rejection.  The roofline line always counts "
                         "the workload's full-sweep bytes; must-read bytes are reported "
                         "beside them")
    args = ap.parse_args()
    if args.summarize_pmc:
        if args.copy_calibration_mib <= 0:
            raise SystemExit("--summarize-pmc needs --copy-calibration-mib of the profiled runs")
        summarize_pmc(*args.summarize_pmc, args.copy_calibration_mib, args.pmc_command,
                      "probs" if args.workload == "probs" else args.path)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the verifier is batch-parallel and this build "
              "runs on a single MI355X (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "probs":
        bench_probs(args)
        return
    if args.workload == "serving":
        bench_serving(args)
        return
    if args.workload == "tree_sample":
        bench_tree_sample(args)
        return
    if args.workload not in SAMPLE_WORKLOADS:
        bench_greedy(args)
        return
    bench_sample(args)


# Sampling workloads with a bench line: name -> (generator, label, traffic file suffix)
SAMPLE_WORKLOADS = {
    "sample": ("sample_chain_llama3", "B=64 k=8 V=128256 bf16 T=0.7",
               "sample_chain_b64_k8_v128256_bf16_t0.7"),
    "sample_v32000": ("sample_chain_v32000", "B=8 k=4 V=32000 bf16 T=1",
                      "sample_chain_b8_k4_v32000_bf16_t1"),
}


def _pct(xs, q):
    import numpy as np

    return float(np.percentile(np.asarray(xs, dtype=np.float64), q)) if len(xs) else None


def bench_sample(args):
    """The sampling chain line (headline or the V=32000 workload)."""
    import numpy as np

    import workloads as W

    gen, label, wname = SAMPLE_WORKLOADS[args.workload]
    headline = args.workload == "sample"
    print(f"bench: generating {label} workload", file=sys.stderr, flush=True)
    wl = getattr(W, gen)()
    B, k, V = wl.B, wl.k, wl.V
    n_u = B * (k + 1) * 2
    first = args.warmup  # counter base of the first timed step

    # CPU legs first: the all-cores leg forks, which must happen before any
    # GPU use in this process.
    legs = None
    if not args.no_cpu_baseline:
        legs = oracle_legs(wl, first, args.steps, args.cpu_seconds, label)

    import torch

    import verify_accept_sampling_amd as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    tgt0, dft0 = dev_bf16(wl.target), dev_bf16(wl.draft)
    # Enough input copies that the rotation's footprint exceeds the 256 MB
    # Infinity Cache (one copy of the headline workload is 279 MB).
    step_in_bytes = (wl.target.nbytes + wl.draft.nbytes)
    n_copies = args.copies if headline else max(args.copies, -(-(600 << 20) // step_in_bytes))
    copies = [(tgt0, dft0)] + [(tgt0.clone(), dft0.clone()) for _ in range(n_copies - 1)]
    toks = torch.from_numpy(wl.draft_tokens).to(dev)
    ws = S.Workspace(dev)
    schedule = SCHEDULE_OF[args.path]
    # Preallocated outputs: one pair per timed step (kept for the gate), one
    # scratch pair for warmup and profiling passes.
    acc_all = torch.empty((args.steps, B), dtype=torch.int32, device=dev)
    out_all = torch.empty((args.steps, B, k + 1), dtype=torch.int32, device=dev)
    scratch = (torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B, k + 1), dtype=torch.int32, device=dev))

    def run(i, out, sched=schedule):
        t, d = copies[i % len(copies)]
        S.spec_verify_sample(t, d, toks, wl.temperature, seed=wl.uniform_seed,
                             counter0=i * n_u, workspace=ws, schedule=sched, out=out)

    copy_calibration(args.copy_calibration_mib, dev)

    print(f"bench: warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        run(i, scratch)
    torch.cuda.synchronize()

    # 1. the timed pass: K steps between two events, outputs kept
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for j in range(args.steps):
        run(first + j, (acc_all[j], out_all[j]))
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    print(f"bench: timed {args.steps} steps, {ms_step * 1e3:.1f} us/step", file=sys.stderr,
          flush=True)

    # 2. step-time spread: an event between consecutive steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for j in range(args.steps):
        run(first + j, scratch)
        evs[j + 1].record()
    torch.cuda.synchronize()
    step_ms = [evs[j].elapsed_time(evs[j + 1]) for j in range(args.steps)]

    # 3. kernel durations: dispatch-stamped events around every launch
    def profiled(sched):
        S.spec_profile_enable(True)
        for j in range(args.steps):
            run(first + j, scratch, sched)
        torch.cuda.synchronize()
        S.spec_profile_enable(False)
        return {kind: S.spec_profile_durations(kind) for kind in ("fused", "row_pass", "draw")}

    durs = profiled(schedule)
    kern = {n: {"launches": len(v), "avg_us": sum(v) / len(v) * 1e3,
                "p10_us": _pct(v, 10) * 1e3, "p50_us": _pct(v, 50) * 1e3,
                "p90_us": _pct(v, 90) * 1e3} for n, v in durs.items() if v}

    acc_np = acc_all.cpu().numpy()
    out_np = out_all.cpu().numpy()
    row_bytes = V * 2
    pass1_bytes = B * (2 * k + 1) * row_bytes
    # rows the final token is drawn from: target and draft row n after a
    # rejection, target row k for the bonus; each read once more, plus the
    # searched chunk of each
    drawn_rows = (acc_np < k).sum(axis=1) + B
    draw_bytes = drawn_rows * row_bytes + drawn_rows * min(V, DRAW_CHUNK) * 2
    # bytes each call must read: per request the target rows 0..n and the
    # draft rows 0..min(n, k-1) (a request's outputs depend on nothing else),
    # plus the draw's re-read
    need_rows = (np.minimum(acc_np + 1, k + 1) + np.minimum(acc_np + 1, k)).sum(axis=1)
    must_bytes = float(np.mean(need_rows * row_bytes + draw_bytes))
    full_bytes = float(np.mean(pass1_bytes + draw_bytes))
    # the schedule that ran: two launches (row pass, draw) when asked for, or
    # when auto picks them for a small row count; else the fused kernel
    if "fused" not in kern:
        dom_name, dom, dom_bytes = "row_pass", kern["row_pass"], float(pass1_bytes)
    else:
        dom_name = "fused"
        dom = kern["fused"]
        dom_bytes = full_bytes
    achieved = dom_bytes / (dom["avg_us"] * 1e-6) / 1e9
    traffic = measured_traffic(args.path) if headline else None
    positions = B * (k + 1)
    result = {
        "metric": METRIC if headline else f"verified positions/sec ({label})",
        "value": positions / (ms_step * 1e-3),
        "unit": "verified positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wname, "B": B, "k": k, "V": V,
                   "logits": "bf16", "temperature": wl.temperature, "input_copies": len(copies),
                   "draw_arithmetic": "f64", "path": args.path},
        "roofline": {"bound": "hbm",
                     "kernel": "k_sample_one" if dom_name == "fused" else "k_row_stats",
                     "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": dom_bytes},
        "kernel_us": {"avg": dom["avg_us"], "p10": dom["p10_us"], "p50": dom["p50_us"],
                      "p90": dom["p90_us"], "launches": dom["launches"]},
        "step_us": {"p10": _pct(step_ms, 10) * 1e3, "p50": _pct(step_ms, 50) * 1e3,
                    "p90": _pct(step_ms, 90) * 1e3},
        "step_hbm_gbps": full_bytes / (ms_step * 1e-3) / 1e9,
        "bytes_basis": "the workload's algorithmic bytes: every logit row once + the draw's "
                       "re-read of the rows drawn from (the early-exit schedule reads fewer: "
                       "must_read_bytes_per_launch, and traffic when measured)",
        "schedule": schedule,
        "schedule_ran": "one launch (k_sample_one)" if dom_name == "fused"
        else "two launches (k_row_stats, k_draw)",
        "must_read_bytes_per_launch": must_bytes,
        "achieved_gbps_over_must_read": must_bytes / (dom["avg_us"] * 1e-6) / 1e9
        if dom_name == "fused" else None,
        "kernels_avg_us": {n: v["avg_us"] for n, v in kern.items()},
        "mean_accepted": float(acc_np.mean()),
        "mean_emitted": float(acc_np.mean() + 1),
    }

    # 4. the explicit one-launch schedules on the same steps (outputs must
    # be identical to the timed ones): the full sweep and early exit
    if schedule != "two_launch" and not args.no_early_exit:
        result["schedules"] = {}
        for other in ("one_launch", "early_exit"):
            acc_e = torch.empty_like(acc_all)
            out_e = torch.empty_like(out_all)
            torch.cuda.synchronize()
            ev0.record()
            for j in range(args.steps):
                run(first + j, (acc_e[j], out_e[j]), other)
            ev1.record()
            torch.cuda.synchronize()
            ms_e = ev0.elapsed_time(ev1) / args.steps
            de = profiled(other)["fused"]
            us_e = sum(de) / len(de) * 1e3
            result["schedules"][other] = {
                "value": positions / (ms_e * 1e-3), "ms_per_step": ms_e,
                "kernel_avg_us": us_e, "kernel_p10_us": _pct(de, 10) * 1e3,
                "kernel_p90_us": _pct(de, 90) * 1e3,
                "achieved_gbps": full_bytes / (us_e * 1e-6) / 1e9,
                "frac": full_bytes / (us_e * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                "outputs_identical": bool(torch.equal(acc_e, acc_all)
                                          and torch.equal(out_e, out_all)),
            }

    status = S.spec_workspace_status(ws)
    result["workspace_status"] = status
    gate = None
    if legs is not None:
        one, allc, res = legs
        result["cpu_baseline"] = allc
        result["cpu_baseline_1core"] = one
        gate = correctness_gate(acc_np, out_np, first, res)
        # one more call with the probe, on the first timed step's inputs
        t, d = copies[first % len(copies)]
        _, _, pr = S.spec_verify_sample(t, d, toks, wl.temperature, seed=wl.uniform_seed,
                                        counter0=first * n_u, workspace=ws, probe=True)
        torch.cuda.synchronize()
        gate["probe"], gate["emitted"] = probe_and_emitted_check(wl, acc_np, pr.cpu().numpy())
        result["correctness_gate"] = gate
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    bad = []
    if status != 0:
        bad.append(f"workspace status {status}")
    if gate is not None and gate["unflagged"]:
        bad.append(f"{gate['unflagged']} requests disagree with the oracle away from any "
                   "decision boundary")
    if gate is not None and gate["probe"]["max_abs_dp"] > 1e-5:
        bad.append(f"probe values differ from the oracle by {gate['probe']['max_abs_dp']:.2e}")
    if gate is not None and gate["emitted"]["z"] is not None and abs(gate["emitted"]["z"]) > 6:
        bad.append(f"mean emitted tokens {gate['emitted']['mean']:.4f} is "
                   f"{gate['emitted']['z']:.1f} standard errors from its expectation")
    for name_, sch in result.get("schedules", {}).items():
        if not sch["outputs_identical"]:
            bad.append(f"the {name_} schedule's outputs differ from the timed schedule's")
    if bad:
        print("bench: FAILED: " + "; ".join(bad), file=sys.stderr, flush=True)
        sys.exit(1)


if __name__ == "__main__":
    main()
