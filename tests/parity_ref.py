"""The oracle's reference for a GPU run, on the GPU's own selection.

Selection keeps, per expert, the q_e largest scores, and ties at an expert's threshold
make several sets equally optimal (LRMoE paper, appendix 7.2, Prop. 7.1). The GPU may
therefore legally pick a different set than the oracle, but only among pairs whose
scores lie within a relative band of the threshold. The later steps (compaction, the
expert backward, the scatter) are then checked against the oracle re-run on the GPU's
selection, so a legal swap is never counted as an arithmetic error and never skipped.

This module only composes the oracle's own step functions; it holds no arithmetic of
the method and imports no GPU code.
"""
from __future__ import annotations

import numpy as np

import oracle

BAND = 1e-5  # relative distance from the threshold inside which selections may differ


def check_selection(sel_gpu, R_or, seg_off, quota, band=BAND):
    """Asserts that ``sel_gpu`` is a valid selection: per expert exactly q_e pair indices,
    inside the expert's segment, strictly ascending, and equal to the oracle's selection
    on the f32-rounded scores except for pairs whose scores lie within ``band`` (relative)
    of the expert's threshold. Returns the oracle's (sel, cseg_off, tau)."""
    sel_gpu = np.asarray(sel_gpu, dtype=np.int64)
    sel_or, cseg, tau = oracle.select(np.asarray(R_or).astype(np.float32), seg_off, quota)
    assert len(sel_gpu) == len(sel_or), "retained pair count differs from the quotas"
    for e in range(len(quota)):
        a = sel_gpu[cseg[e]:cseg[e + 1]]
        b = sel_or[cseg[e]:cseg[e + 1]]
        assert np.all((a >= seg_off[e]) & (a < seg_off[e + 1])), f"expert {e}: index outside its segment"
        assert np.all(np.diff(a) > 0), f"expert {e}: not strictly ascending"
        if np.array_equal(a, b):
            continue
        diff = np.setxor1d(a, b)
        t = tau[e]
        assert np.all(np.abs(R_or[diff] - t) <= band * t), f"expert {e}: selection differs outside the band"
    return sel_or, cseg, tau


def reference_selection(sel_gpu, R_or, seg_off, quota, band=BAND) -> np.ndarray:
    """The selection the later steps are checked on: the GPU's, once it passed the band
    check (an AssertionError otherwise)."""
    check_selection(sel_gpu, R_or, seg_off, quota, band)
    return np.asarray(sel_gpu, dtype=np.int64)


def on_gpu_selection(ref: dict, sel_gpu, *, G, Phi, alpha, tok, slot, seg_off, quota, dtype, T, W2, X=None,
                     H=None, W1=None, band=BAND) -> dict:
    """``ref`` is the oracle's whole-path result (oracle.backward). Returns the reference the
    GPU's steps 3-5 are compared with: ``ref`` itself when the GPU kept the same pairs, else
    a copy whose compaction, backward and scatter outputs the oracle recomputed on
    ``sel_gpu`` (after checking that the two selections differ only inside the band).
    Scores, thresholds and segment offsets are kept: they do not depend on the choice."""
    sel_gpu = reference_selection(sel_gpu, ref["R"], seg_off, quota, band)
    if np.array_equal(sel_gpu, ref["sel"]):
        return ref
    out = dict(ref)
    out["sel"] = sel_gpu
    out["rerun_on_gpu_selection"] = True
    c = oracle.compact(sel_gpu, tok, slot, alpha, G, Phi, dtype, X=X, H=H)
    out.update(c)
    cseg = ref["cseg_off"]
    if H is not None:
        dW1, dW2, dH, dXC = oracle.swiglu_expert_backward(cseg, c["Dlt"], c["PhiC"], c["XC"], c["HC"],
                                                          oracle.widen(W1, dtype), oracle.widen(W2, dtype))
        out.update(dW1=dW1, dW2=dW2, dH=dH, dXC=dXC, out=oracle.scatter_tokens(dXC, c["ctok"], T))
    else:
        dW, dPhi = oracle.linear_expert_backward(cseg, c["Dlt"], c["PhiC"], oracle.widen(W2, dtype))
        out.update(dW2=dW, dPhi=dPhi, out=oracle.scatter_tokens(dPhi, c["ctok"], T))
    return out
