"""Host logic of bench.py (no GPU): the one-GPU refusal, the rule that recorded HBM traffic
is used only while the GEMM source is the profiled one, and the parity report."""
import hashlib
import os
import re
import subprocess
import sys

import types

import numpy as np
import torch

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_recorded_traffic_follows_the_gemm_source():
    src = os.path.join(ROOT, "load_recalibrated_expert_amd", "csrc", "gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for name in ("qwen3_30b_a3b_share", "glm45_106b_a12b_share"):
        path = os.path.join(ROOT, "profiles", f"grouped_gemm_bwd_{name}.md")
        text = open(path).read()
        recorded_sha = re.search(r"gemm_source_sha256:\s*([0-9a-f]{64})", text).group(1)
        recorded = int(re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text).group(1))
        got = bench.recorded_traffic(name)
        assert got == (recorded if recorded_sha == sha else None)
    assert bench.recorded_traffic("no_such_workload") is None


def test_parity_report():
    rng = np.random.default_rng(3)
    E, F, D, T, K = 2, 8, 16, 5, 6
    ref = {"R": rng.random(10) + 0.5, "sel": np.arange(0, 10, 2), "tau": np.array([0.6, 0.6]),
           "dW2": rng.standard_normal((E, F, D)), "dW1": rng.standard_normal((E, D, 2 * F)),
           "dXC": rng.standard_normal((K, D)), "out": rng.standard_normal((T, D))}
    pr = types.SimpleNamespace(cfg=types.SimpleNamespace(swiglu=True),
                               routing=types.SimpleNamespace(seg_off=np.array([0, 6, 10])))
    bufs = {"R": torch.tensor(ref["R"] * (1 + 1e-7)), "sel": torch.tensor(ref["sel"], dtype=torch.int32),
            "g": {"dW2": torch.tensor(ref["dW2"]), "dW1": torch.tensor(ref["dW1"] * 1.001),
                  "dIn": torch.tensor(ref["dXC"] * 1.002)},
            "out": torch.tensor(ref["out"] * 0.997)}
    p = bench.parity(np, bufs, ref, pr)
    assert abs(p["score_max_rel"] - 1e-7) < 1e-12
    assert p["selection_identical"] is True and p["later_steps_on"] == "oracle selection"
    assert abs(p["weight_grad_max_rel_fro"] - 1e-3) < 1e-9
    assert abs(p["input_grad_rel_fro"] - 2e-3) < 1e-9
    assert abs(p["scatter_rel_fro"] - 3e-3) < 1e-9
    bufs["sel"] = torch.tensor(ref["sel"][::-1].copy(), dtype=torch.int32)  # not ascending
    p = bench.parity(np, bufs, ref, pr)
    assert p["selection_identical"] is False and p["selection_within_tie_band"] is False


def test_parity_report_reruns_on_a_tied_gpu_selection():
    """A GPU selection that swaps a pair tied at the threshold is within the band, and the
    GEMM and scatter errors are then taken against the oracle re-run on that selection."""
    import oracle
    from tie_case import swap, tied_problem

    pr, inputs, j1, j2 = tied_problem()
    ref = oracle.backward(**inputs)
    sel = swap(ref["sel"], j1, j2)
    c = oracle.compact(sel, inputs["tok"], inputs["slot"], inputs["alpha"], pr.G, pr.Phi, "bf16", X=pr.X, H=pr.H)
    dW1, dW2, _, dX = oracle.swiglu_expert_backward(ref["cseg_off"], c["Dlt"], c["PhiC"], c["XC"], c["HC"],
                                                    oracle.widen(pr.W1, "bf16"), oracle.widen(pr.W2, "bf16"))
    out = oracle.scatter_tokens(dX, c["ctok"], pr.cfg.T)
    bufs = {"R": torch.tensor(ref["R"]), "sel": torch.tensor(sel, dtype=torch.int32),
            "g": {"dW2": torch.tensor(dW2), "dW1": torch.tensor(dW1), "dIn": torch.tensor(dX)},
            "out": torch.tensor(out)}
    p = bench.parity(np, bufs, ref, pr)
    assert p["selection_identical"] is False and p["selection_within_tie_band"] is True
    assert p["later_steps_on"].startswith("GPU selection")
    assert p["weight_grad_max_rel_fro"] < 1e-12 and p["input_grad_rel_fro"] < 1e-12 and p["scatter_rel_fro"] < 1e-12
