"""A small bf16 SwiGLU problem with an exact score tie placed at one expert's threshold
(test input only: seeded synthetic data, no arithmetic of the method)."""
from __future__ import annotations

import numpy as np

import oracle
import synth


def tied_problem():
    """Pairs j1 < j2 of expert 0 get the same routing weight, the same saved rows and the
    same token row, so their scores are equal; expert 0's quota ends between them, so the
    oracle keeps j1 and drops j2. Returns (problem, inputs for oracle.backward, j1, j2)."""
    cfg = synth.custom("tie_band", T=64, K=3, E=3, D=64, F=32, counts=(60, 50, 40), seed=31)
    pr = synth.make_problem(cfg, rho="0.5")
    r = pr.routing
    seg = r.seg_off
    j1, j2 = int(seg[0]) + 3, int(seg[0]) + 17
    pr.routing.alpha[j2] = r.alpha[j1]
    pr.H[j2] = pr.H[j1]
    pr.Phi[j2] = pr.Phi[j1]
    pr.G[r.tok[j2]] = pr.G[r.tok[j1]]
    R = oracle.score(pr.G, pr.Phi, r.alpha, r.tok, "bf16")
    assert R[j1] == R[j2]
    key = R.astype(np.float32)
    idx = np.arange(seg[0], seg[1])
    order = idx[np.lexsort((idx, -key[idx]))]  # descending score, lower index first
    p1 = int(np.nonzero(order == j1)[0][0])
    assert order[p1 + 1] == j2, "the tied pair is adjacent in the order"
    pr.quota = np.array(pr.quota, dtype=np.int64)
    pr.quota[0] = p1 + 1
    inputs = dict(G=pr.G, Phi=pr.Phi, alpha=r.alpha, tok=r.tok, slot=r.slot, seg_off=seg, quota=pr.quota,
                  dtype="bf16", T=cfg.T, W2=pr.W2, X=pr.X, H=pr.H, W1=pr.W1)
    return pr, inputs, j1, j2


def swap(sel, out_j, in_j):
    """``sel`` with pair out_j replaced by in_j (same expert), kept ascending."""
    s = np.asarray(sel, dtype=np.int64).copy()
    s[s == out_j] = in_j
    return np.sort(s)
