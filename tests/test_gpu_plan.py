"""Quota admission on the GPU (LRMoE paper, section 3.3: Algorithm 1 admits the largest
candidate retention rate whose memory fits, else returns Infeasible): the estimate must
cover what the backward really allocates.

A budget is placed between two candidates' estimates; the planner must admit the lower
one, the next-higher candidate must exceed the budget, and the backward run at the
admitted quotas with fresh buffers (outputs and workspace allocated by the call) must
grow the device's allocated memory by no more than the budget: by the estimate itself,
up to the allocator's rounding. One expert keeps more than 12288 rows, so the workspace
holds split-reduction partials.
"""
import gc

import numpy as np
import pytest
import torch

import load_recalibrated_expert_amd as lr
import oracle
import synth

from gpu_util import DEV, Staged, log

pytestmark = pytest.mark.gpu

RHOS = ["1", "0.8", "0.6", "0.4", "0.2"]


def test_admitted_ratio_fits_its_budget():
    cfg = synth.custom("plan_fit", T=12000, K=4, E=4, D=1024, F=512, counts=(30000, 10000, 5000, 3000), seed=41)
    pr = synth.make_problem(cfg, rho="1")
    counts = np.diff(pr.routing.seg_off)
    est = []
    for r in RHOS:
        P = lr.Problem(E=cfg.E, T=cfg.T, K=cfg.K, D=cfg.D, F=cfg.F, swiglu=True, dtype=lr.BF16,
                       seg_off=pr.routing.seg_off, quota=oracle.ceil_quotas(counts, r).astype(np.int32), device=DEV)
        est.append(lr.backward_bytes(P))
    assert all(est[i] > est[i + 1] for i in range(len(est) - 1)), est
    budget = (est[1] + est[2]) // 2
    i, q, b = lr.plan_quotas(cfg.E, cfg.T, cfg.K, cfg.D, cfg.F, True, lr.BF16, pr.routing.seg_off, RHOS, budget)
    log(f"estimates {est}, budget {budget}: admitted rho={RHOS[i]} ({b} bytes), quotas {q.tolist()}")
    assert i == 2 and b == est[2] <= budget < est[1]
    assert q.tolist() == oracle.ceil_quotas(counts, RHOS[i]).tolist()
    assert int(q.max()) > 12288  # split-reduction partials in the workspace

    pr.quota = q.astype(np.int64)
    s = Staged(pr)  # inputs and the problem's device offsets, allocated before the measurement
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    res = s.backward()
    torch.cuda.synchronize()
    grown = torch.cuda.max_memory_allocated() - base
    log(f"backward at rho={RHOS[i]}: device memory grew by {grown} bytes (estimate {b}, budget {budget})")
    assert grown <= budget
    assert 0.99 * b <= grown <= b + (64 << 10)  # the estimate is the allocation, up to rounding
    assert res["sel"].numel() == int(q.sum()) and bool(torch.isfinite(res["dW1"]).all())
