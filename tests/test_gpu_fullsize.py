"""GPU parity at the full workload sizes (the configurations the benchmark times), on every
output.

Every check compares the HIP path, run exactly as the benchmark runs it, with the CPU
oracle on the same seeded inputs, on the Qwen3 and GLM shares, the extreme-skew routing and
the quota sweep at all four ratios:
* scores: every pair, |R - R_oracle| <= 1e-6 R_oracle (also the gradient-only criteria);
* selection: every expert, bit-exact (selection on f32 scores on both sides) except for
  pairs inside the 1e-5 tie band of the expert's threshold; steps 3-5 are then checked on
  the GPU's selection, the oracle running on the same choice;
* every output of steps 3-5: packed tokens, slots and PhiW bit for bit; dW1, dW2 per expert,
  dH and the input gradients overall and per packed row, and the scattered token gradients,
  the oracle running expert by expert;
* the zero-masked same-shape baseline equals the packed-Dlt path on every workload.
Tolerances: the spec bar 2e-2 relative (Frobenius) per packed input-gradient row, and
the arithmetic-derived 5e-3 for whole outputs (bf16 storage of PhiW and dH).
"""
import numpy as np
import pytest
import torch

import load_recalibrated_expert_amd as lr
import oracle
import synth

from gpu_util import Staged, as_f64, bits, check_selection, log, reference_selection, rel_fro

pytestmark = pytest.mark.gpu

CASES = [("qwen3_30b_a3b_share", "0.6"), ("glm45_106b_a12b_share", "0.6"), ("extreme_skew", "0.4"),
         ("glm_quota_sweep", "1.0"), ("glm_quota_sweep", "0.8"), ("glm_quota_sweep", "0.5"),
         ("glm_quota_sweep", "0.25")]

BAR, DERIVED = 2e-2, 5e-3


@pytest.fixture(scope="module", params=CASES, ids=[f"{c}-rho{r}" for c, r in CASES])
def full(request):
    name, rho = request.param
    log(f"{name} rho={rho}: generating")
    pr = synth.make_problem(name, rho=rho)
    r = pr.routing
    s = Staged(pr)
    log(f"{name} rho={rho}: GPU path N={s.P.N} K_tot={s.P.K_tot}")
    res = s.backward()
    torch.cuda.synchronize()
    log(f"{name} rho={rho}: oracle scores and selection")
    R_or = oracle.score(pr.G, pr.Phi, r.alpha, r.tok, "bf16")
    sel_or, cseg, tau = oracle.select(R_or.astype(np.float32), r.seg_off, pr.quota)
    yield dict(pr=pr, s=s, res=res, R_or=R_or, sel_or=sel_or, cseg=cseg, name=name, rho=rho)
    del s, res
    torch.cuda.empty_cache()


def test_full_score(full):
    R = full["res"]["R"].cpu().numpy().astype(np.float64)
    ref = full["R_or"]
    assert np.all(np.abs(R - ref) <= 1e-6 * ref + 1e-35)


@pytest.mark.parametrize("criterion", ["grad_sqnorm", "grad_abs"])
def test_full_score_gradient_only_criteria(full, criterion):
    pr, s = full["pr"], full["s"]
    R = lr.score(s.P, s.G, None, None, s.tok, criterion=criterion)
    torch.cuda.synchronize()
    R = R.cpu().numpy().astype(np.float64)
    ref = oracle.score_gradient_only(pr.G, pr.routing.tok, "bf16", criterion)
    assert np.all(np.abs(R - ref) <= 1e-6 * ref + 1e-35)


def test_full_select(full):
    pr = full["pr"]
    sel = full["res"]["sel"].cpu().numpy().astype(np.int64)
    check_selection(sel, full["R_or"], pr.routing.seg_off, pr.quota)
    if full["rho"] == "1.0":  # retention 1.0 keeps every pair
        assert np.array_equal(sel, np.arange(pr.routing.seg_off[-1]))


def _selection(full):
    """The selection steps 3-5 are checked on: the GPU's, after the tie-band check (pairs tied
    at an expert's threshold may be chosen differently; the oracle then runs on the GPU's
    choice)."""
    pr = full["pr"]
    return reference_selection(full["res"]["sel"].cpu().numpy().astype(np.int64), full["R_or"],
                               pr.routing.seg_off, pr.quota)


def test_full_backward_whole_outputs(full):
    """Every output of steps 3-5 against the oracle run on the (checked) selection, expert by
    expert so that host memory stays bounded by the largest expert: the packed rows' tokens
    and slots and the weighted saved rows PhiW bit for bit (the default path packs nothing
    else), dW1 and dW2 per expert, dH and the input gradients overall and per
    packed row, and the scattered token gradients (the oracle's scatter is linear, so the
    per-expert scatters add up to the whole)."""
    pr, res, sel, cseg = full["pr"], full["res"], _selection(full), full["cseg"]
    r = pr.routing
    T, D = pr.cfg.T, pr.cfg.D
    out_ref = np.zeros((T, D))
    sq = {"dIn": [0.0, 0.0], "dH": [0.0, 0.0]}
    for e in range(pr.cfg.E):
        a, b = int(cseg[e]), int(cseg[e + 1])
        if a == b:
            assert not bool(res["dW1"][e].abs().sum()) and not bool(res["dW2"][e].abs().sum()), f"expert {e}"
            continue
        c = oracle.compact(sel[a:b], r.tok, r.slot, r.alpha, pr.G, pr.Phi, "bf16", X=pr.X, H=pr.H)
        assert np.array_equal(bits(res["PhiW"][a:b]), oracle.round_bf16(c["PhiW"])), f"PhiW expert {e}"
        assert np.array_equal(res["ctok"][a:b].cpu().numpy(), c["ctok"]), f"ctok expert {e}"
        assert np.array_equal(res["cslot"][a:b].cpu().numpy(), c["cslot"]), f"cslot expert {e}"
        dW1, dW2, dH, dX = oracle.swiglu_expert_backward(
            np.array([0, b - a]), c["Dlt"], c["PhiC"], c["XC"], c["HC"], oracle.widen(pr.W1[e:e + 1], "bf16"),
            oracle.widen(pr.W2[e:e + 1], "bf16"))
        assert rel_fro(as_f64(res["dW2"][e]), dW2[0]) <= DERIVED, f"dW2 expert {e}"
        assert rel_fro(as_f64(res["dW1"][e]), dW1[0]) <= DERIVED, f"dW1 expert {e}"
        for k, ref in (("dIn", dX), ("dH", dH)):
            got = as_f64(res[k][a:b])
            sq[k][0] += float(np.sum((got - ref) ** 2))
            sq[k][1] += float(np.sum(ref ** 2))
            if k == "dIn":
                num, den = np.linalg.norm(got - ref, axis=1), np.linalg.norm(ref, axis=1)
                assert np.all(num <= BAR * np.maximum(den, 1e-30)), f"dIn rows of expert {e}"
        out_ref += oracle.scatter_tokens(dX, c["ctok"], T)
        log(f"{full['name']} rho={full['rho']}: expert {e} ({b - a} rows) checked")
    for k, (num, den) in sq.items():
        assert np.sqrt(num / den) <= DERIVED, k
    assert rel_fro(as_f64(res["out"]), out_ref) <= DERIVED


def test_full_scatter_beside_is_token_scatter(full):
    """The step as bench.py runs it on bf16 workloads: the scatter on a second stream beside
    the weight gradients (SCATTER_TOKEN_BESIDE) gives the serial token scatter's bits."""
    s, res = full["s"], full["res"]
    side = lr.backward(s.P, G=s.G, Phi=s.Phi, alpha=s.alpha, tok=s.tok, slot=s.slot, W2=s.W2, X=s.X, H=s.H,
                       W1=s.W1, overlap_scatter=True)
    torch.cuda.synchronize()
    assert torch.equal(side["out"], res["out"])
    assert torch.equal(side["dW1"], res["dW1"]) and torch.equal(side["dW2"], res["dW2"])


def test_full_zero_masked_matches(full):
    """Section 3.4: the zero-masked same-shape baseline gives the packed path's results. Both
    store the weighted gradient rows Dlt in bf16, so the baseline is held to the physical
    run that packs Dlt (the default path rounds alpha * phi instead: it is checked against
    the oracle by the sampled tests)."""
    s = full["s"]
    m = s.backward(mode=lr.COMPACT_ZERO_MASKED)
    res = s.backward(packed_dlt=True)
    torch.cuda.synchronize()
    for k in ("dW1", "dW2", "out"):
        a, b = m[k].double(), res[k].double()
        assert float(torch.linalg.norm(a - b) / torch.linalg.norm(b)) <= 1e-5, k
    del m, res
