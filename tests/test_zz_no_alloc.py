"""lrmoe_select_noalloc, the selection for callers that cannot allocate device memory,
against lrmoe_select with a workspace: identical retained indices, keep flags, (token,
slot) map and packed tokens and slots, on two calls in a row (the second with a smaller
problem, so it runs on the array the first call left behind), through the C ABI."""
import numpy as np
import pytest
import torch

import load_recalibrated_expert_amd as lr
import synth
from gpu_util import DEV, Staged, log

pytestmark = pytest.mark.gpu


def _maps(P):
    return {"pmap": torch.full((P.T * P.K,), -7, dtype=torch.int32, device=DEV),
            "ctok": torch.full((max(P.K_tot, 1),), -7, dtype=torch.int32, device=DEV),
            "cslot": torch.full((max(P.K_tot, 1),), -7, dtype=torch.int32, device=DEV)}


def _compare(name, cfg, rho):
    pr = synth.make_problem(cfg, rho=rho)
    s = Staged(pr)
    P = s.P
    R = lr.score(P, s.G, s.Phi, s.alpha, s.tok)
    sel_w, keep_w, m_w = lr.select(P, R, tok=s.tok, slot=s.slot)
    sel = torch.full((max(P.K_tot, 1),), -7, dtype=torch.int32, device=DEV)
    keep = torch.full((max(P.N, 1),), 7, dtype=torch.uint8, device=DEV)
    m = _maps(P)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    lr.select_noalloc(P, R, sel, keep, tok=s.tok, slot=s.slot, maps=m)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    log(f"{name}: N={P.N} K_tot={P.K_tot} E={P.E}")
    assert torch.equal(sel[:P.K_tot], sel_w)
    assert torch.equal(keep[:P.N], keep_w)
    assert torch.equal(m["pmap"], m_w["pmap"])
    assert torch.equal(m["ctok"][:P.K_tot], m_w["ctok"]) and torch.equal(m["cslot"][:P.K_tot], m_w["cslot"])
    # without the map outputs as well
    sel2 = torch.full_like(sel, -7)
    lr.select_noalloc(P, R, sel2)
    torch.cuda.synchronize()
    assert torch.equal(sel2[:P.K_tot], sel_w)


def test_noalloc_select_matches_workspace_select_twice():
    big = synth.custom("noalloc_big", T=30000, K=4, E=16, D=64, F=32,
                       counts=tuple(int(x) for x in np.round(110000 * (np.arange(1, 17) ** -1.2) / np.sum(
                           np.arange(1, 17) ** -1.2))), seed=51)
    small = synth.custom("noalloc_small", T=700, K=4, E=5, D=64, F=32, counts=(900, 0, 610, 333, 7), seed=52)
    _compare("first call", big, "0.6")
    _compare("second call, smaller", small, "0.5")
