"""Host logic of bench.py: the correctness gate's classification of
disagreements and the scaling of the HBM counter passes (CPU only)."""
import csv
import json

import numpy as np

import bench


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_summarize_pmc_scales_each_counter_by_the_copy(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda key: str(out))
    mib = 4
    # the copy reads and writes 4 MiB; its FETCH_SIZE shows half of it
    fetch = [("void specv::k_probs_rows<4>(...)", 1000.0), ("void specv::k_probs_rows<4>(...)", 1200.0),
             ("at::native::neg_kernel", 2048.0)]
    write = [("void specv::k_probs_rows<4>(...)", 10.0), ("at::native::neg_kernel", 4096.0)]
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), mib, "cmd", "probs")
    t = json.loads(out.read_text())
    assert t["kernel"] == "k_probs_rows" and t["path"] == "probs"
    assert abs(t["fetch_scale"] - 2.0) < 1e-12 and abs(t["write_scale"] - 1.0) < 1e-12
    assert abs(t["hbm_read_bytes_per_launch"] - 1100.0 * 1024 * 2.0) < 1e-6
    assert abs(t["hbm_write_bytes_per_launch"] - 10.0 * 1024) < 1e-6
    assert t["kernel_source_sha"] == bench.kernel_source_sha(bench.PROBS_SOURCES)


def test_correctness_gate_counts_flagged_and_unflagged_mismatches():
    k = 3
    # oracle: (accepted, tokens, accept margins by position, draw margin)
    reqs = [
        (1, [5, 9], {0: 0.5, 1: 0.5}, 0.5),       # GPU agrees
        (1, [5, 9], {0: 0.5, 1: 0.5}, 1e-7),      # GPU draws another token: draw flagged
        (2, [5, 6, 7], {0: 0.5, 1: 2e-6, 2: 0.5}, 0.5),  # GPU stops at 1: that test flagged
        (0, [4], {0: 0.5}, 0.5),                  # GPU draws another token, not flagged
    ]
    acc = np.array([[1, 1, 1, 0]], dtype=np.int32)
    out = np.full((1, 4, k + 1), -1, dtype=np.int32)
    out[0, 0, :2] = [5, 9]
    out[0, 1, :2] = [5, 8]
    out[0, 2, :2] = [5, 3]
    out[0, 3, :1] = [2]
    g = bench.correctness_gate(acc, out, 10, {10: reqs})
    assert g["steps"] == 1 and g["requests"] == 4
    assert g["mismatches"] == 3 and g["unflagged"] == 1
    assert g["draw_decisions"] == 4 and g["accept_decisions"] == 8


def test_probe_and_emitted_check_on_hand_made_rows():
    """Probability rows with p_0(x_0) = 0.2, q_0(x_0) = 0.4 (accept 1/2) and
    p_1(x_1) = 0.3, q_1(x_1) = 0.1 (accept 1): 1 + 1/2 + 1/2 = 2 emitted
    tokens expected; a probe off by 3e-6 reads 3e-6."""
    import types

    target = np.array([[[0.1, 0.2, 0.3, 0.4], [0.4, 0.1, 0.3, 0.2], [0.25, 0.25, 0.25, 0.25]]],
                      dtype=np.float32)
    draft = np.array([[[0.3, 0.4, 0.2, 0.1], [0.5, 0.2, 0.1, 0.2]]], dtype=np.float32)
    wl = types.SimpleNamespace(B=1, k=2, target=target, draft=draft,
                               draft_tokens=np.array([[1, 2]], np.int32), temperature=1.0,
                               kind="probs", dtype="f32")
    probe = np.zeros((1, 3, 4), np.float32)
    probe[0, 0, :2] = [0.2, 0.4]
    probe[0, 1, :2] = [0.3, 0.1 + 3e-6]
    acc = np.array([[1], [0], [2], [1]], np.int32)  # 2, 1, 3, 2 emitted: mean 2
    pr, em = bench.probe_and_emitted_check(wl, acc, probe)
    assert abs(pr["max_abs_dp"] - 3e-6) < 1e-7 and pr["positions"] == 2
    assert abs(em["expected"] - 2.0) < 1e-7
    assert abs(em["mean"] - 2.0) < 1e-12 and em["steps"] == 4 and abs(em["z"]) < 1e-6
