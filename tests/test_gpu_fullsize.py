"""GPU parity at the full workload sizes (the configurations the benchmark times), on
outputs the oracle can compute one by one.

Every check compares the HIP path, run exactly as the benchmark runs it, with the CPU
oracle on the same seeded inputs:
* scores: every pair, |R - R_oracle| <= 1e-6 R_oracle;
* selection: every expert, bit-exact (selection on f32 scores on both sides) except for
  pairs inside the 1e-5 tie band of the expert's threshold; steps 3-5 are then checked on
  the GPU's selection, the oracle running on the same choice;
* compaction: sampled packed rows and every segment boundary, bit-exact;
* grouped GEMMs: sampled experts (the largest, the smallest non-empty one and two more),
  sampled FC2 input features f: FC2 weight-gradient rows dW2[e][f, :], FC1 weight-gradient
  columns dW1[e][:, f] and dW1[e][:, F+f], dH columns; sampled packed rows of the input
  gradient. Each oracle value comes from the oracle run on the sliced sub-problem (the
  GEMMs are linear in the sliced dimension, so slicing the inputs gives exact samples);
* scatter: sampled tokens;
* the zero-masked same-shape baseline equals the packed path on every workload.
Tolerances: the spec bar 2e-2 relative (Frobenius, per sampled vector), and the
arithmetic-derived 5e-3 for weight-gradient vectors (bf16 storage of PhiW and dH).
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


def test_full_compact_sampled_rows(full):
    pr, res, sel, cseg = full["pr"], full["res"], _selection(full), full["cseg"]
    rng = np.random.default_rng(5)
    K = len(sel)
    rows = np.unique(np.concatenate([rng.integers(0, K, 2048), cseg[:-1][cseg[:-1] < K],
                                     np.maximum(cseg[1:] - 1, 0)]))
    rows_t = torch.from_numpy(rows).to(res["PhiW"].device)
    c = oracle.compact(sel[rows], pr.routing.tok, pr.routing.slot, pr.routing.alpha, pr.G, pr.Phi, "bf16",
                       X=pr.X, H=pr.H)
    assert np.array_equal(bits(res["PhiW"][rows_t]), oracle.round_bf16(c["PhiW"]))
    # the path packs only the weighted saved rows: the GEMMs read G, X and H in place
    assert "Dlt" not in res and "PhiC" not in res and "XC" not in res and "HC" not in res
    assert np.array_equal(res["ctok"][rows_t].cpu().numpy(), c["ctok"])
    assert np.array_equal(res["cslot"][rows_t].cpu().numpy(), c["cslot"])


def _experts(pr, cseg):
    m = np.diff(cseg)
    nz = np.nonzero(m)[0]
    picks = {int(nz[np.argmax(m[nz])]), int(nz[np.argmin(m[nz])])}
    rng = np.random.default_rng(7)
    picks |= set(int(x) for x in rng.choice(nz, size=min(2, len(nz)), replace=False))
    return sorted(picks)


def test_full_grouped_gemm_sampled(full):
    pr, res, sel, cseg = full["pr"], full["res"], _selection(full), full["cseg"]
    F, D = pr.cfg.F, pr.cfg.D
    rng = np.random.default_rng(11)
    W1 = pr.W1
    W2 = pr.W2
    for e in _experts(pr, cseg):
        rows = np.arange(cseg[e], cseg[e + 1])
        f = np.sort(rng.choice(F, size=3, replace=False))
        cols = np.concatenate([f, F + f])
        log(f"{full['name']}: expert {e} ({len(rows)} rows), features {f.tolist()}")
        c = oracle.compact(sel[rows], pr.routing.tok, pr.routing.slot, pr.routing.alpha, pr.G, pr.Phi, "bf16",
                           X=pr.X, H=pr.H)
        sub_off = np.array([0, len(rows)])
        dW1, dW2, dH, _ = oracle.swiglu_expert_backward(
            sub_off, c["Dlt"], c["PhiC"][:, f], c["XC"], c["HC"][:, cols],
            oracle.widen(W1[e][:, cols], "bf16")[None], oracle.widen(W2[e][f, :], "bf16")[None])
        g2 = as_f64(res["dW2"][e][torch.from_numpy(f).to(res["dW2"].device)])
        g1 = as_f64(res["dW1"][e][:, torch.from_numpy(cols).to(res["dW1"].device)])
        gh = as_f64(res["dH"][int(rows[0]):int(rows[-1]) + 1][:, torch.from_numpy(cols).to(res["dH"].device)])
        for i in range(len(f)):
            assert rel_fro(g2[i], dW2[0][i]) <= DERIVED, f"dW2[{e}][{f[i]}]"
        for j in range(len(cols)):
            assert rel_fro(g1[:, j], dW1[0][:, j]) <= DERIVED, f"dW1[{e}][:, {cols[j]}]"
            assert rel_fro(gh[:, j], dH[:, j]) <= DERIVED, f"dH[:, {cols[j]}] expert {e}"


def _row_samples(cseg, K, rng, n=64):
    return np.unique(np.concatenate([rng.integers(0, K, n), cseg[:-1][cseg[:-1] < K]]))


def _oracle_dx_rows(pr, sel, cseg, rows):
    """Oracle input-gradient rows for packed rows `rows` (sub-problem grouped by expert)."""
    e_of = np.searchsorted(cseg, rows, side="right") - 1
    order = np.argsort(e_of, kind="stable")
    rows, e_of = rows[order], e_of[order]
    E = len(cseg) - 1
    counts = np.bincount(e_of, minlength=E)
    sub_off = np.concatenate([[0], np.cumsum(counts)])
    c = oracle.compact(sel[rows], pr.routing.tok, pr.routing.slot, pr.routing.alpha, pr.G, pr.Phi, "bf16",
                       X=pr.X, H=pr.H)
    _, _, _, dX = oracle.swiglu_expert_backward(sub_off, c["Dlt"], c["PhiC"], c["XC"], c["HC"],
                                                oracle.widen(pr.W1, "bf16"), oracle.widen(pr.W2, "bf16"))
    return rows, dX, c["ctok"]


def test_full_input_gradient_rows_sampled(full):
    pr, res, sel, cseg = full["pr"], full["res"], _selection(full), full["cseg"]
    rng = np.random.default_rng(13)
    rows = _row_samples(cseg, len(sel), rng)
    rows, dX, _ = _oracle_dx_rows(pr, sel, cseg, rows)
    got = as_f64(res["dIn"][torch.from_numpy(rows).to(res["dIn"].device)])
    for i in range(len(rows)):
        assert rel_fro(got[i], dX[i]) <= BAR, f"packed row {rows[i]}"
    assert rel_fro(got, dX) <= DERIVED


def test_full_scatter_sampled_tokens(full):
    pr, res, sel, cseg = full["pr"], full["res"], _selection(full), full["cseg"]
    rng = np.random.default_rng(17)
    toks = np.sort(rng.choice(pr.cfg.T, size=24, replace=False))
    ctok_all = pr.routing.tok[sel]
    rows = np.nonzero(np.isin(ctok_all, toks))[0]
    rows, dX, ctok = _oracle_dx_rows(pr, sel, cseg, rows)
    ref = oracle.scatter_tokens(dX, ctok, pr.cfg.T)[toks]
    got = as_f64(res["out"][torch.from_numpy(toks).to(res["out"].device)])
    for i, t in enumerate(toks):
        if np.linalg.norm(ref[i]) == 0:
            assert np.all(got[i] == 0)
        else:
            assert rel_fro(got[i], ref[i]) <= BAR, f"token {t}"


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
