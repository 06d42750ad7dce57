"""Plain fp64 CPU oracle of the LRMoE memory-aware expert backward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module. It shares no
code with the HIP path (no kernels, headers, helpers or constants) and imports
nothing from it.

Every step widens the stored inputs (bf16 bit patterns or float32) to float64
and computes in float64, one obviously-correct step at a time, in the order the
LRMoE paper's Algorithm 1 ("Resource-constrained layer-wise load calibration",
its backward-time calibration block) gives them:

1. ``score``    - the Load Recalibration Metric of every routed pair
                  (section 3.2, Proposition 3.1, Eq. 3; appendix 7.1, Eq. 11-12);
                  ``score_gradient_only`` - the gradient-only criteria it is
                  compared with in the ablation (section 4.7, Table 2).
2. ``select``   - per-expert TopK of the scores under fixed quotas
                  (section 3.3; appendix 7.2, Proposition 7.1 and Eq. 17).
3. ``compact``  - gather of the retained gradient rows and saved activations
                  into contiguous expert-major segments (section 3.1 "compact
                  runtime", section 3.3, section 3.4 / Figure 4).
4. ``swiglu_expert_backward`` / ``linear_expert_backward`` - the four expert
                  backward GEMMs on the retained rows (section 3.4) with the
                  activation backward between FC2 and FC1 (section 3.1).
5. ``scatter_tokens`` / ``scatter_slots`` - the inverse mapping back to token
                  order or to (token, routing-slot) positions in zero-initialised
                  buffers (section 3.1; Algorithm 1's ScatterWithZeros).

Readings taken where the pages are silent (all listed in the design notes):
ties at an expert's quota threshold go to the lower expert-major index; a
compact segment keeps the retained pairs in ascending original order; the
weighted gradient row of a retained pair is ``delta = alpha * g`` (appendix 7.1,
Eq. 5, with alpha applied exactly once); SwiGLU is ``silu(gate) * up`` with the
FC1 output stored as ``[gate | up]``; weights are stored ``[in x out]``.

Pins (what fixes each function independently of itself) live in
``tests/test_oracle_pins.py``; every function here has at least one.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "InfeasibleQuota", "widen", "round_bf16", "score", "score_gradient_only", "select", "compact",
    "swiglu_expert_backward", "linear_expert_backward", "scatter_tokens", "scatter_slots",
    "backward", "ceil_quotas", "backward_bytes", "plan_quotas",
    "swiglu", "expert_forward_fc1", "expert_forward_fc2",
]


class InfeasibleQuota(ValueError):
    """A quota outside 0 <= q_e <= n_e: the admission of Algorithm 1 would have
    returned Infeasible for it (section 3.3)."""


def widen(a, dtype: str) -> np.ndarray:
    """Stored values -> float64. ``dtype`` is "bf16" (uint16 bit patterns) or "f32"."""
    a = np.asarray(a)
    if dtype == "bf16":
        bits = a.astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float64)
    raise ValueError(dtype)


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even) of float64 ``x``, as uint16 bits.

    Written from the definition of round-to-nearest-even: x = m * 2^e with
    0.5 <= |m| < 1; the 8-bit significand is rint(m * 2^8) (numpy's rint rounds
    halves to even). Valid for zero and normal-range values, which is all the
    path produces."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.rint(m * 256.0)
    v = np.ldexp(r, e - 8)                     # exact; r == 256 carries into the exponent
    return (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------- step 1

def score(G, Phi, alpha, tok, dtype: str, chunk: int = 16384) -> np.ndarray:
    """LRM score R_u = alpha_u^2 * ||g_t||^2 * ||phi_u||^2 for every routed pair
    (Proposition 3.1, Eq. 3; Algorithm 1's backward scoring step).

    G: [T, D] upstream gradients *before* the routing weight (appendix 7.1,
    Eq. 4-5); Phi: [N, F] saved input of the protected projection (FC2), one row
    per pair, expert-major; alpha: [N] routing weights; tok: [N] token of each
    pair. Returns float64 [N]."""
    T = G.shape[0]
    gn = np.empty(T, dtype=np.float64)
    for t0 in range(0, T, chunk):
        g = widen(G[t0:t0 + chunk], dtype)
        gn[t0:t0 + chunk] = np.sum(g * g, axis=1)
    N = Phi.shape[0]
    pn = np.empty(N, dtype=np.float64)
    for j0 in range(0, N, chunk):
        p = widen(Phi[j0:j0 + chunk], dtype)
        pn[j0:j0 + chunk] = np.sum(p * p, axis=1)
    a = np.asarray(alpha, dtype=np.float64)
    return a * a * gn[np.asarray(tok, dtype=np.int64)] * pn


def score_gradient_only(G, tok, dtype: str, criterion: str, chunk: int = 16384) -> np.ndarray:
    """Gradient-only selection scores, the alternative criteria of the ablation
    (section 4.7, Table 2: a squared gradient norm and an absolute gradient
    magnitude). A gradient-only rule sees neither the routing weight nor the saved
    activation, so every pair of token t gets the same score, from g_t alone:

      "grad_sqnorm"  sum_i g_{t,i}^2    (the squared norm of the upstream gradient)
      "grad_abs"     sum_i |g_{t,i}|    (its absolute magnitude, read as the L1 sum;
                                         the plain norm would rank like grad_sqnorm)

    G: [T, D] upstream gradients before the routing weight; tok: [N] token of each
    pair. Returns float64 [N]. The random-selection baseline of the same table needs
    no function here: its scores are the random draws themselves, fed to ``select``."""
    if criterion not in ("grad_sqnorm", "grad_abs"):
        raise ValueError(f"unknown criterion {criterion!r}")
    T = G.shape[0]
    gs = np.empty(T, dtype=np.float64)
    for t0 in range(0, T, chunk):
        g = widen(G[t0:t0 + chunk], dtype)
        gs[t0:t0 + chunk] = np.sum(g * g, axis=1) if criterion == "grad_sqnorm" else np.sum(np.abs(g), axis=1)
    return gs[np.asarray(tok, dtype=np.int64)]


# ---------------------------------------------------------------------------- step 2

def select(R, seg_off, quota):
    """Per-expert TopK under fixed quotas (section 3.3; Proposition 7.1).

    Inside each expert segment [seg_off[e], seg_off[e+1]) the q_e pairs with the
    largest scores are kept; among equal scores the lower expert-major index wins.
    The retained indices of a segment are returned in ascending order.

    Returns (sel [K_tot] int64, cseg_off [E+1] int64, tau [E] float64), where
    tau_e is the q_e-th largest score of segment e (NaN when q_e is 0 or n_e, where
    no pair sits at a threshold). Raises InfeasibleQuota unless 0 <= q_e <= n_e."""
    R = np.asarray(R)
    seg_off = np.asarray(seg_off, dtype=np.int64)
    quota = np.asarray(quota, dtype=np.int64)
    E = len(quota)
    sel, tau = [], np.full(E, np.nan)
    cseg_off = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        lo, hi, q = int(seg_off[e]), int(seg_off[e + 1]), int(quota[e])
        if q < 0 or q > hi - lo:
            raise InfeasibleQuota(f"expert {e}: quota {q} outside [0, {hi - lo}]")
        j = np.arange(lo, hi, dtype=np.int64)
        order = np.lexsort((j, -R[lo:hi]))      # score descending, then index ascending
        kept = np.sort(j[order[:q]])
        if 0 < q < hi - lo:
            tau[e] = float(R[lo + order[q - 1]])
        sel.append(kept)
        cseg_off[e + 1] = cseg_off[e] + q
    sel = np.concatenate(sel) if sel else np.zeros(0, dtype=np.int64)
    return sel, cseg_off, tau


# ---------------------------------------------------------------------------- step 3

def compact(sel, tok, slot, alpha, G, Phi, dtype: str, X=None, H=None):
    """Physical compaction of the retained pairs (section 3.1 "compact runtime";
    section 3.4, Figure 4): row c of every output belongs to retained pair
    j = sel[c], so each expert's retained rows form one contiguous segment.

    Dlt[c]  = alpha_j * g_{tok_j}   (the weighted cotangent, Eq. 5; exact in fp64)
    PhiC[c] = Phi[j],  XC[c] = X[tok_j],  HC[c] = H[j]
    ctok[c] = tok_j,   cslot[c] = slot_j
    PhiW[c] = alpha_j * Phi[j]      (exact in fp64)

    PhiW carries the routing weight on the saved activation instead of the gradient: the
    FC2 weight gradient of appendix 7.1 (Eq. 6-8) sums alpha_j phi_j^T g_t over the pairs,
    a product linear in each factor, so PhiW^T g_{ctok} over an expert's rows is the same
    sum as PhiC^T Dlt, and a path that reads g rows by token needs no Dlt at all.
    """
    sel = np.asarray(sel, dtype=np.int64)
    t = np.asarray(tok, dtype=np.int64)[sel]
    a = np.asarray(alpha, dtype=np.float64)[sel]
    out = {
        "Dlt": a[:, None] * widen(np.asarray(G)[t], dtype),
        "PhiC": widen(np.asarray(Phi)[sel], dtype),
        "PhiW": a[:, None] * widen(np.asarray(Phi)[sel], dtype),
        "ctok": t.astype(np.int64),
        "cslot": np.asarray(slot, dtype=np.int64)[sel],
    }
    if X is not None:
        out["XC"] = widen(np.asarray(X)[t], dtype)
    if H is not None:
        out["HC"] = widen(np.asarray(H)[sel], dtype)
    return out


# ---------------------------------------------------------------------------- step 4

def swiglu_expert_backward(row_off, Dlt, PhiC, XC, HC, W1, W2):
    """Backward of SwiGLU experts on their packed rows (section 3.4: the FC2 and FC1
    data- and weight-gradient GEMMs; section 3.1: the activation backward between
    them uses the same retained identities). Weights are stored [in x out]:
    W1[e] is [D, 2F] with columns [0, F) = gate and [F, 2F) = up; W2[e] is [F, D].

    Per expert e over its rows i in [row_off[e], row_off[e+1]):
        dW2_e = PhiC^T Dlt                         [F, D]
        dPhi  = Dlt W2_e^T                         [m, F]
        s = sigmoid(gate), silu = gate*s, silu' = s*(1 + gate*(1 - s))
        dH    = [dPhi * up * silu', dPhi * silu]   [m, 2F]
        dW1_e = XC^T dH                            [D, 2F]
        dXC   = dH W1_e^T                          [m, D]
    All inputs float64; returns (dW1 [E,D,2F], dW2 [E,F,D], dH [rows,2F], dXC [rows,D])."""
    row_off = np.asarray(row_off, dtype=np.int64)
    E = len(row_off) - 1
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    F = W2.shape[1]
    rows, D = Dlt.shape
    dW1 = np.zeros((E, W1.shape[1], W1.shape[2]))
    dW2 = np.zeros((E, F, W2.shape[2]))
    dH = np.zeros((rows, 2 * F))
    dXC = np.zeros((rows, W1.shape[1]))
    for e in range(E):
        r = slice(int(row_off[e]), int(row_off[e + 1]))
        if r.start == r.stop:
            continue
        d, phi, x, h = Dlt[r], PhiC[r], XC[r], HC[r]
        dW2[e] = phi.T @ d
        dphi = d @ W2[e].T
        gate, up = h[:, :F], h[:, F:]
        s = 1.0 / (1.0 + np.exp(-gate))
        silu = gate * s
        dsilu = s * (1.0 + gate * (1.0 - s))
        dh = np.concatenate([dphi * up * dsilu, dphi * silu], axis=1)
        dH[r] = dh
        dW1[e] = x.T @ dh
        dXC[r] = dh @ W1[e].T
    return dW1, dW2, dH, dXC


def linear_expert_backward(row_off, Dlt, PhiC, W):
    """Backward of a single protected projection y = alpha * phi W (W stored [in x out],
    [F, D] per expert): dW_e = PhiC^T Dlt and dPhi = Dlt W_e^T (appendix 7.1, Eq. 6-8,
    with Dlt = alpha * g). Returns (dW [E,F,D], dPhi [rows,F])."""
    row_off = np.asarray(row_off, dtype=np.int64)
    E = len(row_off) - 1
    W = np.asarray(W, dtype=np.float64)
    dW = np.zeros((E, W.shape[1], W.shape[2]))
    dPhi = np.zeros((Dlt.shape[0], W.shape[1]))
    for e in range(E):
        r = slice(int(row_off[e]), int(row_off[e + 1]))
        if r.start == r.stop:
            continue
        dW[e] = PhiC[r].T @ Dlt[r]
        dPhi[r] = Dlt[r] @ W[e].T
    return dW, dPhi


# ---------------------------------------------------------------------------- step 5

def scatter_tokens(rows, ctok, T: int) -> np.ndarray:
    """Inverse mapping to token order: out[t] = sum of the rows whose pair belongs to
    token t; tokens with no retained pair stay zero (section 3.1, section 3.4)."""
    rows = np.asarray(rows, dtype=np.float64)
    out = np.zeros((T, rows.shape[1]))
    for c, t in enumerate(np.asarray(ctok, dtype=np.int64)):
        out[t] += rows[c]
    return out


def scatter_slots(rows, ctok, cslot, T: int, K: int) -> np.ndarray:
    """Inverse mapping to (token, routing-slot) positions of a zero-initialised dense
    buffer [T*K, width] (section 3.1): out[t*K + k] = the row of pair (t, k)."""
    rows = np.asarray(rows, dtype=np.float64)
    out = np.zeros((T * K, rows.shape[1]))
    pos = np.asarray(ctok, dtype=np.int64) * K + np.asarray(cslot, dtype=np.int64)
    for c, p in enumerate(pos):
        out[p] = rows[c]
    return out


# ---------------------------------------------------------------------------- whole path

def backward(*, G, Phi, alpha, tok, slot, seg_off, quota, dtype, T, W2, X=None, H=None,
             W1=None, score_dtype=np.float32):
    """The five steps in order. Selection is taken on the scores rounded to
    ``score_dtype`` (the precision in which the scores are stored and compared);
    pass None to select on the float64 scores. Returns a dict of every output."""
    R = score(G, Phi, alpha, tok, dtype)
    key = R if score_dtype is None else R.astype(score_dtype)
    sel, cseg_off, tau = select(key, seg_off, quota)
    c = compact(sel, tok, slot, alpha, G, Phi, dtype, X=X, H=H)
    out = {"R": R, "sel": sel, "cseg_off": cseg_off, "tau": tau, **c}
    if H is not None:
        dW1, dW2, dH, dXC = swiglu_expert_backward(cseg_off, c["Dlt"], c["PhiC"], c["XC"], c["HC"],
                                                   widen(W1, dtype), widen(W2, dtype))
        out.update(dW1=dW1, dW2=dW2, dH=dH, dXC=dXC, out=scatter_tokens(dXC, c["ctok"], T))
    else:
        dW, dPhi = linear_expert_backward(cseg_off, c["Dlt"], c["PhiC"], widen(W2, dtype))
        out.update(dW2=dW, dPhi=dPhi, out=scatter_tokens(dPhi, c["ctok"], T))
    return out


# ---------------------------------------------------------------------------- quota admission

def ceil_quotas(counts, rho) -> np.ndarray:
    """Retention quotas of one candidate ratio: q_e = min(n_e, ceil(rho * n_e)), rho taken
    as an exact fraction (a string like "0.6", a Fraction, or an int)."""
    from fractions import Fraction
    import math
    r = Fraction(rho)
    return np.array([min(int(n), math.ceil(r * int(n))) for n in counts], dtype=np.int64)


def backward_bytes(*, T, E, D, F, swiglu, dtype, N, K_tot, packed=False, workspace=0) -> int:
    """Device bytes one physical-compaction backward holds besides its inputs (G, Phi, X, H,
    W1, W2, alpha, tok, slot): the memory that the retention quotas decide, the estimate
    Algorithm 1's admission compares with the available HBM. It is ``workspace`` (the
    scratch the backward's implementation asks for at these quotas: the pages fix no
    scratch layout, so the caller supplies it) plus the buffers, listed one by one (e =
    bytes of the storage dtype; w = D for SwiGLU experts, F for an FC2-only expert):
      scores R f32 [N], keep flags u8 [N]; sel, ctok, cslot int32 [K_tot];
      the packed rows of step 3: by default only the weighted saved rows PhiW [K_tot x F] e
      (the gradient, saved-activation and FC1-input rows are then read in place, by token or
      by pair); with ``packed`` the weighted gradient rows Dlt [K_tot x D] e and the saved
      rows PhiC [K_tot x F] e (SwiGLU: XC [K_tot x D], HC [K_tot x 2F] too);
      SwiGLU dH [K_tot x 2F] e; input gradients [K_tot x w] e;
      weight gradients f32: dW2 [E x F x D] (SwiGLU: dW1 [E x D x 2F]); scatter output
      f32 [T x w]."""
    e = 2 if dtype == "bf16" else 4
    w = D if swiglu else F
    b = 4 * N + N
    b += 3 * 4 * K_tot
    if not packed:
        b += K_tot * F * e
    else:
        b += K_tot * D * e + K_tot * F * e
        if swiglu:
            b += K_tot * D * e + K_tot * 2 * F * e
    if swiglu:
        b += K_tot * 2 * F * e
    b += K_tot * w * e
    b += 4 * E * F * D
    if swiglu:
        b += 4 * E * D * 2 * F
    b += 4 * T * w
    return int(b + workspace)


def plan_quotas(counts, rhos, hbm_avail, *, T, D, F, swiglu, dtype, packed=False, workspace=None):
    """Algorithm 1's forward-time admission on one GPU (no replica plan and no
    communication window to check): try the candidate ratios in decreasing order (equal
    ratios in the order given), form their quotas, and admit the first whose
    ``backward_bytes`` fit ``hbm_avail``. ``workspace(quotas)`` gives the implementation's
    scratch bytes at a candidate's quotas (None: no scratch). Returns (index of the
    admitted candidate, quotas, bytes). None fits: Algorithm 1 returns Infeasible - raised
    as InfeasibleQuota."""
    from fractions import Fraction
    counts = [int(n) for n in counts]
    order = sorted(range(len(rhos)), key=lambda i: (-Fraction(rhos[i]), i))
    for i in order:
        q = ceil_quotas(counts, rhos[i])
        b = backward_bytes(T=T, E=len(counts), D=D, F=F, swiglu=swiglu, dtype=dtype, N=sum(counts),
                           K_tot=int(q.sum()), packed=packed, workspace=0 if workspace is None else workspace(q))
        if b <= hbm_avail:
            return i, q, b
    raise InfeasibleQuota("no candidate retention ratio fits the available memory")


# ---------------------------------------------------------------------------- forward and context save

def swiglu(h, F: int) -> np.ndarray:
    """phi = silu(gate) * up for rows h = [gate | up] (float64), silu(x) = x / (1 + e^-x)."""
    h = np.asarray(h, dtype=np.float64)
    gate, up = h[:, :F], h[:, F:]
    return gate / (1.0 + np.exp(-gate)) * up


def expert_forward_fc1(X, tok, seg_off, W1, dtype: str):
    """First half of the expert forward that produces the backward's saved context
    (Algorithm 1's FullForwardAndSaveContext; section 3.1: the forward keeps every routed
    pair). Pair j of expert e (expert-major, j in [seg_off[e], seg_off[e+1])) computes
    h_j = x_{tok[j]} W1[e] ([gate | up], 2F wide) and phi_j = silu(gate_j) * up_j.
    Returns float64 (H [N, 2F], Phi [N, F]); the stored context is their bf16 (or f32)
    rounding."""
    X = widen(X, dtype)
    W1 = widen(W1, dtype)
    seg_off = np.asarray(seg_off, dtype=np.int64)
    tok = np.asarray(tok, dtype=np.int64)
    F = W1.shape[2] // 2
    N = int(seg_off[-1])
    H = np.zeros((N, 2 * F), dtype=np.float64)
    for e in range(len(seg_off) - 1):
        r = slice(seg_off[e], seg_off[e + 1])
        H[r] = X[tok[r]] @ W1[e]
    return H, swiglu(H, F)


def expert_forward_fc2(Phi, alpha, seg_off, W2, dtype: str) -> np.ndarray:
    """Second half: y_j = alpha_j * phi_j W2[e] for the stored phi rows (the FC2 input is
    the saved tensor). Returns float64 [N, D]; the layer output is the token sum of these
    rows (scatter_tokens)."""
    P = widen(Phi, dtype)
    W2 = widen(W2, dtype)
    seg_off = np.asarray(seg_off, dtype=np.int64)
    a = np.asarray(alpha, dtype=np.float64)
    Y = np.zeros((P.shape[0], W2.shape[2]), dtype=np.float64)
    for e in range(len(seg_off) - 1):
        r = slice(seg_off[e], seg_off[e + 1])
        Y[r] = a[r, None] * (P[r] @ W2[e])
    return Y
