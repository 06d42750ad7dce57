"""Pins of the CPU oracle to facts the pages and the mathematics fix (no GPU).

Each check is a function of an oracle-like namespace ``o`` so that the
``test_pins_catch_planted_mistakes`` cases can run the same check against a copy
of the oracle with one plausible mistake planted in it, and see it fail.

Independent references used here (none re-types the oracle's formulas):
* brute force: the pairwise weight-gradient outer products of Eq. 1 / Eq. 8 of
  the LRMoE paper materialised in float64;
* torch autograd (float64, CPU) of the expert *forward*, whose gradient is the
  dense or masked backward the path must reproduce (section 3.4: compact equals
  zero-masked for the same retained pairs; retention 1.0 is the unpruned backward);
* exhaustive subset search (Proposition 7.1);
* the worked examples the pages print (tests/golden/).
"""
import itertools
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _small_swiglu(seed=0, T=6, K=3, E=3, D=5, F=4, counts=(5, 0, 7), dtype="bf16"):
    cfg = synth.custom(T=T, K=K, E=E, D=D, F=F, counts=counts, swiglu=True, dtype=dtype, seed=seed)
    return synth.make_problem(cfg, rho="1.0")


# ----------------------------------------------------------------------------- autograd reference

def autograd_swiglu(p: synth.Problem, keep_mask=None):
    """Gradients of L = sum_t <g_t, sum_{u in t} m_u alpha_u phi_u W2_e> by torch autograd.

    The saved FC1 output H and the saved FC2 input Phi enter with their stored
    values while the gradient flows as if h = x W1 and phi = silu(gate) * up
    (straight-through), which is what a backward over saved state computes."""
    dt = p.cfg.dtype
    r = p.routing
    F = p.cfg.F
    x = torch.tensor(oracle.widen(p.X, dt), requires_grad=True)
    w1 = torch.tensor(oracle.widen(p.W1, dt), requires_grad=True)
    w2 = torch.tensor(oracle.widen(p.W2, dt), requires_grad=True)
    Hs = torch.tensor(oracle.widen(p.H, dt))
    Ps = torch.tensor(oracle.widen(p.Phi, dt))
    g = torch.tensor(oracle.widen(p.G, dt))
    tok = torch.tensor(r.tok.astype(np.int64))
    a = torch.tensor(r.alpha.astype(np.float64))
    if keep_mask is not None:
        a = a * torch.tensor(keep_mask.astype(np.float64))
    e_of = torch.tensor(r.expert.astype(np.int64))
    h_lin = torch.einsum("nd,ndk->nk", x[tok], w1[e_of])
    h = Hs + (h_lin - h_lin.detach())
    phi_c = torch.nn.functional.silu(h[:, :F]) * h[:, F:]
    phi = Ps + (phi_c - phi_c.detach())
    y = a[:, None] * torch.einsum("nf,nfd->nd", phi, w2[e_of])
    out = torch.zeros(p.cfg.T, p.cfg.D, dtype=torch.float64).index_add(0, tok, y)
    (g * out).sum().backward()
    return w1.grad.numpy(), w2.grad.numpy(), x.grad.numpy()


def autograd_linear(p: synth.Problem, keep_mask=None):
    dt = p.cfg.dtype
    r = p.routing
    w = torch.tensor(oracle.widen(p.W2, dt), requires_grad=True)
    phi = torch.tensor(oracle.widen(p.Phi, dt), requires_grad=True)
    g = torch.tensor(oracle.widen(p.G, dt))
    tok = torch.tensor(r.tok.astype(np.int64))
    a = torch.tensor(r.alpha.astype(np.float64))
    if keep_mask is not None:
        a = a * torch.tensor(keep_mask.astype(np.float64))
    e_of = torch.tensor(r.expert.astype(np.int64))
    y = a[:, None] * torch.einsum("nf,nfd->nd", phi, w[e_of])
    out = torch.zeros(p.cfg.T, p.cfg.D, dtype=torch.float64).index_add(0, tok, y)
    (g * out).sum().backward()
    return w.grad.numpy(), phi.grad.numpy()


def _rel(a, b):
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


# ----------------------------------------------------------------------------- checks

def check_score_outer_product(o, dtype="bf16", seed=0):
    """Eq. 3 / Eq. 11-12: R_u is the squared Frobenius norm of (alpha_u g_t) phi_u^T."""
    rng = _rng(seed)
    T, D, N, F = 5, 7, 11, 6
    G = rng.standard_normal((T, D)).astype(np.float32)
    P = rng.standard_normal((N, F)).astype(np.float32)
    if dtype == "bf16":
        G, P = synth.f32_to_bf16_bits(G), synth.f32_to_bf16_bits(P)
    alpha = rng.uniform(0.01, 1.0, N).astype(np.float32)
    tok = rng.integers(0, T, N).astype(np.int32)
    R = o.score(G, P, alpha, tok, dtype)
    g64 = (synth.bf16_bits_to_f32(G) if dtype == "bf16" else G).astype(np.float64)
    p64 = (synth.bf16_bits_to_f32(P) if dtype == "bf16" else P).astype(np.float64)
    for u in range(N):
        Gu = np.outer(float(alpha[u]) * g64[tok[u]], p64[u])   # pair u's weight-gradient contribution
        brute = float(np.sum(Gu * Gu))
        assert abs(R[u] - brute) <= 1e-13 * brute, (u, R[u], brute)


def check_score_dyadic_exact(o):
    """On small dyadic inputs every product and sum is exact, so Eq. 3 holds bit for bit."""
    G = np.array([[1.0, -2.0, 0.5], [3.0, 0.0, -1.0]], dtype=np.float32)
    P = np.array([[0.25, 1.0], [2.0, -2.0], [0.0, 0.0]], dtype=np.float32)
    alpha = np.array([0.5, 0.25, 1.0], dtype=np.float32)
    tok = np.array([0, 1, 1], dtype=np.int32)
    R = o.score(synth.f32_to_bf16_bits(G), synth.f32_to_bf16_bits(P), alpha, tok, "bf16")
    # ||g0||^2 = 5.25, ||g1||^2 = 10, ||p0||^2 = 1.0625, ||p1||^2 = 8, ||p2||^2 = 0
    assert R.tolist() == [0.25 * 5.25 * 1.0625, 0.0625 * 10.0 * 8.0, 0.0]


def check_score_is_omission_change(o, seed=3):
    """Eq. 10/12: R_u equals ||dW_e(all pairs) - dW_e(all but u)||_F^2, the squared change
    of the protected projection's gradient when pair u alone is omitted (autograd)."""
    p = synth.make_problem(synth.custom(T=4, K=2, E=2, D=6, F=5, counts=(5, 3), swiglu=False,
                                        dtype="f32", seed=seed), rho="1.0")
    R = o.score(p.G, p.Phi, p.routing.alpha, p.routing.tok, "f32")
    full, _ = autograd_linear(p)
    for u in range(p.routing.tok.shape[0]):
        m = np.ones(len(R))
        m[u] = 0.0
        part, _ = autograd_linear(p, m)
        diff = float(np.sum((full - part) ** 2))
        assert abs(diff - R[u]) <= 1e-12 * R[u], (u, diff, R[u])


def check_gradient_only_brute_force(o, seed=4):
    """The gradient-only criteria (section 4.7, Table 2) written out element by element with
    exact rational arithmetic on dyadic bf16 inputs: sum of squares and sum of magnitudes
    of the pair's token row, independent of its slot, routing weight and expert."""
    from fractions import Fraction
    rng = _rng(seed)
    T, D, N = 5, 7, 11
    G = (rng.integers(-64, 65, size=(T, D)) / 16.0).astype(np.float32)  # dyadic, exact in bf16
    tok = rng.integers(0, T, size=N).astype(np.int32)
    Gb = synth.f32_to_bf16_bits(G)
    for crit in ("grad_sqnorm", "grad_abs"):
        R = o.score_gradient_only(Gb, tok, "bf16", crit)
        for j in range(N):
            row = [Fraction(float(x)) for x in G[tok[j]]]
            ref = sum(x * x for x in row) if crit == "grad_sqnorm" else sum(abs(x) for x in row)
            assert Fraction(float(R[j])) == ref, (crit, j)


def check_gradient_only_against_lrm(o, seed=5):
    """With alpha = 1 and a saved activation of unit norm (one coordinate equal to 1) the LRM
    score (pinned above by brute-force outer products) reduces to the squared gradient norm;
    the magnitude criterion scales linearly: |c| times for the rows scaled by c = 2^k."""
    rng = _rng(seed)
    T, D, F, N = 6, 9, 4, 13
    G = rng.standard_normal((T, D)).astype(np.float32)
    tok = rng.integers(0, T, size=N).astype(np.int32)
    Phi = np.zeros((N, F), dtype=np.float32)
    Phi[np.arange(N), rng.integers(0, F, size=N)] = 1.0
    Gb = synth.f32_to_bf16_bits(G)
    lrm = o.score(Gb, synth.f32_to_bf16_bits(Phi), np.ones(N, dtype=np.float32), tok, "bf16")
    assert np.array_equal(o.score_gradient_only(Gb, tok, "bf16", "grad_sqnorm"), lrm)
    a1 = o.score_gradient_only(Gb, tok, "bf16", "grad_abs")
    a4 = o.score_gradient_only(synth.f32_to_bf16_bits(-4.0 * G), tok, "bf16", "grad_abs")
    assert np.array_equal(a4, 4.0 * a1)
    with pytest.raises(ValueError):
        o.score_gradient_only(Gb, tok, "bf16", "random")


def check_ceil_quotas_definition(o, seed=6):
    """q_e is the least integer >= rho * n_e, capped at n_e, for exact fractional rho."""
    from fractions import Fraction
    rng = _rng(seed)
    counts = [0, 1, 2, 3, 5, 7, 10, 99, 1000] + [int(x) for x in rng.integers(0, 100000, size=20)]
    for rho in ("0", "1", "0.6", "0.25", "0.75", "0.333", "0.999999", Fraction(2, 3), Fraction(1, 7)):
        q = o.ceil_quotas(counts, rho)
        r = Fraction(rho)
        for n, k in zip(counts, q.tolist()):
            assert 0 <= k <= n
            assert k == n or (k >= r * n and k - 1 < r * n), (rho, n, k)
        if r == 1:
            assert q.tolist() == counts
        if r == 0:
            assert not any(q.tolist())


def _buffer_bytes_of_outputs(o, p, packed):
    """Bytes of the buffers the oracle's own backward returns, from their shapes and the
    dtype each one is stored in on the device."""
    e = 2 if p.cfg.dtype == "bf16" else 4
    r = p.routing
    out = o.backward(G=p.G, Phi=p.Phi, alpha=r.alpha, tok=r.tok, slot=r.slot, seg_off=r.seg_off, quota=p.quota,
                     dtype=p.cfg.dtype, T=p.cfg.T, W2=p.W2, X=p.X, H=p.H, W1=p.W1)
    size = lambda a: int(np.prod(np.asarray(a).shape))  # noqa: E731
    b = 4 * size(out["R"]) + 1 * size(out["R"])          # scores, keep flags
    b += 4 * (size(out["sel"]) + size(out["ctok"]) + size(out["cslot"]))
    if not packed:
        b += e * size(out["PhiW"])
    else:
        b += e * (size(out["Dlt"]) + size(out["PhiC"]))
        if p.cfg.swiglu:
            b += e * (size(out["XC"]) + size(out["HC"]))
    if p.cfg.swiglu:
        b += e * (size(out["dH"]) + size(out["dXC"])) + 4 * (size(out["dW1"]) + size(out["dW2"]))
    else:
        b += e * size(out["dPhi"]) + 4 * size(out["dW2"])
    return b + 4 * size(out["out"])


def check_backward_bytes_from_shapes(o):
    """The admission's memory estimate equals the bytes of the buffers the backward really
    produces (SwiGLU and FC2-only, bf16 and f32, packed or read in place)."""
    for sw, dt, counts in ((True, "bf16", (5, 0, 7)), (False, "f32", (4, 6, 1)), (True, "f32", (3, 3, 3))):
        cfg = synth.custom(T=7, K=3, E=3, D=16, F=8, counts=counts, swiglu=sw, dtype=dt, seed=21)
        p = synth.make_problem(cfg, rho="0.6")
        for packed in (False, True):
            est = o.backward_bytes(T=cfg.T, E=cfg.E, D=cfg.D, F=cfg.F, swiglu=sw, dtype=dt,
                                   N=int(p.routing.seg_off[-1]), K_tot=int(p.quota.sum()), packed=packed)
            assert est == _buffer_bytes_of_outputs(o, p, packed), (sw, dt, packed)


def _scratch_of(q):
    """A quota-dependent scratch size standing in for an implementation's workspace: it
    grows with the largest quota in steps, as split reductions do, and is not monotone in
    the total."""
    q = [int(x) for x in q]
    return 4096 * (1 + max(q) // 37) + 96 * (q[0] % 5)


def check_plan_quotas_brute_force(o, seed=8):
    """Admission picks the largest candidate ratio (ties: the earlier one) whose estimate fits,
    checked against every candidate; with no candidate fitting it reports Infeasible. The
    estimate is the buffers plus the workspace at the candidate's own quotas, run without
    and with a quota-dependent workspace."""
    from fractions import Fraction
    rng = _rng(seed)
    dims = dict(T=300, D=64, F=48, swiglu=True, dtype="bf16")
    counts = [int(x) for x in rng.integers(0, 200, size=6)]
    rhos = ["0.5", "1", "0.75", "0.25", "0.75", "0.9", "0"]
    for ws in (None, _scratch_of):
        est = []
        for r in rhos:
            q = o.ceil_quotas(counts, r)
            b = o.backward_bytes(E=len(counts), N=sum(counts), K_tot=int(q.sum()), **dims)
            est.append(b + (0 if ws is None else ws(q)))
        for budget in sorted(set(est)) + [min(est) - 1, max(est) + 1]:
            ok = [i for i in range(len(rhos)) if est[i] <= budget]
            if not ok:
                with pytest.raises(o.InfeasibleQuota):
                    o.plan_quotas(counts, rhos, budget, workspace=ws, **dims)
                continue
            best = max(ok, key=lambda i: (Fraction(rhos[i]), -i))
            i, q, b = o.plan_quotas(counts, rhos, budget, workspace=ws, **dims)
            assert (i, b) == (best, est[best]) and q.tolist() == o.ceil_quotas(counts, rhos[best]).tolist()


def check_backward_bytes_adds_workspace(o):
    """The workspace enters the estimate once, as given."""
    kw = dict(T=50, E=3, D=32, F=16, swiglu=True, dtype="bf16", N=90, K_tot=40)
    assert o.backward_bytes(workspace=12345, **kw) == o.backward_bytes(**kw) + 12345


def check_swiglu_closed_forms(o):
    """silu(x) = x sigma(x): sigma(0) = 1/2, sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4, and the odd
    part silu(x) - silu(-x) = x for any x; the up half multiplies."""
    ln3 = math.log(3.0)
    h = np.array([[0.0, ln3, -ln3, 2.0, 5.0, -1.5, 3.0, 7.0]])  # F = 4: gate | up
    phi = o.swiglu(h, 4)[0]
    ref = [0.0 * 5.0, 0.75 * ln3 * -1.5, -0.25 * ln3 * 3.0]  # silu(gate_k) * up_k
    for k in range(3):
        assert abs(phi[k] - ref[k]) <= 1e-15 * max(1.0, abs(ref[k])), k
    x = np.linspace(-9.0, 9.0, 37)
    hp = np.stack([x, np.ones_like(x)], axis=1)
    hm = np.stack([-x, np.ones_like(x)], axis=1)
    assert np.allclose(o.swiglu(hp, 1)[:, 0] - o.swiglu(hm, 1)[:, 0], x, rtol=0, atol=1e-14)


def check_forward_exact(o, seed=9):
    """Exact rational brute force of both forward GEMMs on dyadic bf16 inputs: pair j of
    expert e multiplies its token's x by W1[e] (gather through tok, weights stored [in x out])
    and its stored phi by W2[e], scaled by its routing weight."""
    from fractions import Fraction
    rng = _rng(seed)
    T, E, D, F = 4, 2, 3, 2
    tok = np.array([2, 0, 3, 1, 2], dtype=np.int32)
    seg = np.array([0, 2, 5], dtype=np.int64)
    X = (rng.integers(-8, 9, size=(T, D)) / 4.0).astype(np.float32)
    W1 = (rng.integers(-8, 9, size=(E, D, 2 * F)) / 8.0).astype(np.float32)
    W2 = (rng.integers(-8, 9, size=(E, F, D)) / 8.0).astype(np.float32)
    P = (rng.integers(-8, 9, size=(5, F)) / 2.0).astype(np.float32)
    alpha = np.array([0.5, 0.25, 1.0, 0.125, 2.0], dtype=np.float32)
    b = synth.f32_to_bf16_bits
    H, Phi = o.expert_forward_fc1(b(X), tok, seg, b(W1), "bf16")
    Y = o.expert_forward_fc2(b(P), alpha, seg, b(W2), "bf16")
    for j in range(5):
        e = 0 if j < 2 else 1
        for c in range(2 * F):
            ref = sum(Fraction(float(X[tok[j], d])) * Fraction(float(W1[e, d, c])) for d in range(D))
            assert Fraction(float(H[j, c])) == ref, (j, c)
        for d in range(D):
            ref = Fraction(float(alpha[j])) * sum(Fraction(float(P[j, f])) * Fraction(float(W2[e, f, d]))
                                                  for f in range(F))
            assert Fraction(float(Y[j, d])) == ref, (j, d)
    assert np.array_equal(Phi, o.swiglu(H, F))


def check_select_exhaustive(o, seed=1, ties=False):
    """Proposition 7.1: per expert, the retained set maximises the retained score sum
    among all subsets of size q_e (and the dropped set minimises Eq. 13; Eq. 16 links
    the two); with distinct scores the maximiser is unique."""
    rng = _rng(seed)
    for trial in range(25):
        E = int(rng.integers(1, 4))
        counts = rng.integers(0, 10, E)
        seg_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        q = np.array([rng.integers(0, c + 1) for c in counts], dtype=np.int64)
        N = int(seg_off[-1])
        R = (rng.integers(0, 4, N) if ties else rng.permutation(N) + rng.uniform(0, 0.5, N)).astype(np.float64)
        sel, cseg_off, tau = o.select(R, seg_off, q)
        assert cseg_off.tolist() == np.concatenate([[0], np.cumsum(q)]).tolist()
        for e in range(E):
            lo, hi = int(seg_off[e]), int(seg_off[e + 1])
            mine = sel[cseg_off[e]:cseg_off[e + 1]]
            assert np.all(np.diff(mine) > 0) and np.all((mine >= lo) & (mine < hi))
            got = float(R[mine].sum())
            best, argbest = -1.0, []
            for S in itertools.combinations(range(lo, hi), int(q[e])):
                v = float(R[list(S)].sum())
                if v > best + 1e-12:
                    best, argbest = v, [S]
                elif abs(v - best) <= 1e-12:
                    argbest.append(S)
            assert abs(got - best) <= 1e-9, (trial, e)
            dropped = sorted(set(range(lo, hi)) - set(mine.tolist()))
            assert abs(R[dropped].sum() - (R[lo:hi].sum() - got)) <= 1e-9   # Eq. 16
            if not ties:
                assert len(argbest) == 1 and tuple(mine.tolist()) == argbest[0]
            else:
                assert tuple(mine.tolist()) in argbest
                # the reading taken for ties: among equal boundary scores the lower index wins
                if 0 < q[e] < hi - lo:
                    t = tau[e]
                    kept_at = [j for j in mine if R[j] == t]
                    drop_at = [j for j in dropped if R[j] == t]
                    if kept_at and drop_at:
                        assert max(kept_at) < min(drop_at)


def check_select_per_expert(o):
    """Section 3.3: selection ranks pairs inside each expert against that expert's quota,
    not layer-wide; a high-scoring expert cannot take another expert's quota."""
    seg_off = np.array([0, 4, 8])
    R = np.array([9.0, 8.0, 7.0, 6.0, 0.1, 0.4, 0.3, 0.2])
    sel, cseg_off, _ = o.select(R, seg_off, np.array([2, 2]))
    assert sel.tolist() == [0, 1, 5, 6] and cseg_off.tolist() == [0, 2, 4]


def check_fig4_worked_example(o, seed=5):
    """Figure 4: loads [4,2,3] with quotas [3,1,2] pack into segments [3,1,2] at offsets
    [0,3,4,6]; each expert drops its one lowest-scored pair."""
    with open(os.path.join(GOLDEN, "fig4_worked_example.json")) as f:
        ex = json.load(f)
    loads, kept = ex["loads"], ex["retained"]
    seg_off = np.concatenate([[0], np.cumsum(loads)])
    R = _rng(seed).permutation(sum(loads)).astype(np.float64) + 1.0
    sel, cseg_off, _ = o.select(R, seg_off, np.array(kept))
    assert cseg_off.tolist() == ex["packed_offsets"]
    assert np.diff(cseg_off).tolist() == kept
    for e in range(len(loads)):
        seg = list(range(seg_off[e], seg_off[e + 1]))
        dropped = set(seg) - set(sel[cseg_off[e]:cseg_off[e + 1]].tolist())
        assert dropped == {min(seg, key=lambda j: R[j])}


def check_compact_identity(o, seed=2):
    """Section 3.1/3.4: compaction keeps token-expert correspondence. Row c of every packed
    buffer is exactly the source row of retained pair sel[c]; each retained pair appears
    once; the gradient row is alpha times the token's gradient (Eq. 5)."""
    p = _small_swiglu(seed=seed, counts=(6, 0, 9), T=7, K=3)
    r = p.routing
    R = o.score(p.G, p.Phi, r.alpha, r.tok, "bf16")
    q = np.array([4, 0, 5])
    sel, cseg_off, _ = o.select(R.astype(np.float32), r.seg_off, q)
    c = o.compact(sel, r.tok, r.slot, r.alpha, p.G, p.Phi, "bf16", X=p.X, H=p.H)
    assert len(set(sel.tolist())) == len(sel) == q.sum()
    for i, j in enumerate(sel):
        t = r.tok[j]
        assert c["ctok"][i] == t and c["cslot"][i] == r.slot[j]
        np.testing.assert_array_equal(c["PhiC"][i], synth.bf16_bits_to_f32(p.Phi[j]))
        np.testing.assert_array_equal(c["XC"][i], synth.bf16_bits_to_f32(p.X[t]))
        np.testing.assert_array_equal(c["HC"][i], synth.bf16_bits_to_f32(p.H[j]))
        g = synth.bf16_bits_to_f32(p.G[t]).astype(np.float64)
        np.testing.assert_array_equal(c["Dlt"][i], float(r.alpha[j]) * g)


def check_weighted_phi_vs_autograd(o, seed=9):
    """Appendix 7.1 (Eq. 6-8): dW2 sums alpha_j phi_j g_t^T over the retained pairs, so the
    FC2 weight gradient from the alpha-weighted saved rows PhiW and the unweighted token
    gradient rows equals autograd's with dropped pairs masked, and with every routing
    weight 1 PhiW is PhiC itself."""
    p = _small_swiglu(seed=seed, counts=(9, 3, 0, 8), E=4, T=9, K=3, D=6, F=4)
    r = p.routing
    q = synth.quotas(np.diff(r.seg_off), "0.5")
    R = o.score(p.G, p.Phi, r.alpha, r.tok, "bf16")
    sel, cseg_off, _ = o.select(R.astype(np.float32), r.seg_off, q)
    c = o.compact(sel, r.tok, r.slot, r.alpha, p.G, p.Phi, "bf16", X=p.X, H=p.H)
    g_rows = o.widen(p.G, "bf16")[np.asarray(c["ctok"], dtype=np.int64)]
    _, dW2, _, _ = o.swiglu_expert_backward(cseg_off, g_rows, c["PhiW"], c["XC"], c["HC"],
                                            o.widen(p.W1, "bf16"), o.widen(p.W2, "bf16"))
    mask = np.zeros(len(r.tok))
    mask[sel] = 1.0
    _, dW2_ref, _ = autograd_swiglu(p, mask)
    assert _rel(dW2, dW2_ref) < 1e-12
    ones = o.compact(sel, r.tok, r.slot, np.ones_like(r.alpha), p.G, p.Phi, "bf16")
    np.testing.assert_array_equal(ones["PhiW"], ones["PhiC"])


def check_swiglu_dense_vs_autograd(o, seed=4):
    """Retention 1.0 keeps every pair, so the packed backward must equal the unpruned
    dense backward of the expert forward (torch autograd, float64)."""
    p = _small_swiglu(seed=seed, counts=(7, 0, 9, 4), E=4, T=8, K=3, D=6, F=5)
    r = p.routing
    res = o.backward(G=p.G, Phi=p.Phi, alpha=r.alpha, tok=r.tok, slot=r.slot, seg_off=r.seg_off,
                     quota=np.diff(r.seg_off), dtype="bf16", T=p.cfg.T, W2=p.W2, X=p.X, H=p.H, W1=p.W1)
    dW1, dW2, dX = autograd_swiglu(p)
    assert _rel(res["dW1"], dW1) < 1e-12
    assert _rel(res["dW2"], dW2) < 1e-12
    assert _rel(res["out"], dX) < 1e-12


def check_swiglu_masked_vs_autograd(o, seed=6):
    """Section 3.4: the packed backward equals the zero-masked same-shape backward for the
    same retained pairs (here: autograd with dropped pairs' routing weights masked)."""
    p = _small_swiglu(seed=seed, counts=(9, 3, 0, 8), E=4, T=9, K=3, D=6, F=4)
    r = p.routing
    q = synth.quotas(np.diff(r.seg_off), "0.5")
    res = o.backward(G=p.G, Phi=p.Phi, alpha=r.alpha, tok=r.tok, slot=r.slot, seg_off=r.seg_off,
                     quota=q, dtype="bf16", T=p.cfg.T, W2=p.W2, X=p.X, H=p.H, W1=p.W1)
    mask = np.zeros(len(r.tok))
    mask[res["sel"]] = 1.0
    dW1, dW2, dX = autograd_swiglu(p, mask)
    assert _rel(res["dW1"], dW1) < 1e-12
    assert _rel(res["dW2"], dW2) < 1e-12
    assert _rel(res["out"], dX) < 1e-12


def check_linear_masked_vs_autograd(o, seed=7):
    """Single protected projection (appendix 7.1, Eq. 6-8): dW = sum alpha phi g^T over the
    retained pairs and dphi = alpha W g, against autograd with dropped pairs masked."""
    p = synth.make_problem(synth.CONFIGS["tiny"])
    r = p.routing
    res = o.backward(G=p.G, Phi=p.Phi, alpha=r.alpha, tok=r.tok, slot=r.slot, seg_off=r.seg_off,
                     quota=p.quota, dtype="f32", T=p.cfg.T, W2=p.W2)
    mask = np.zeros(len(r.tok))
    mask[res["sel"]] = 1.0
    dW, dphi = autograd_linear(p, mask)
    assert _rel(res["dW2"], dW) < 1e-12
    # autograd's dphi is per pair in pair order; the oracle's rows are packed
    np.testing.assert_allclose(res["dPhi"], dphi[res["sel"]], rtol=1e-12, atol=1e-14)
    assert np.all(dphi[mask == 0] == 0)


def check_aggregate_error_eq19(o, seed=8):
    """Appendix 7.3, Eq. 18-20: ||dW2_all - dW2_kept||^2 = sum_D R + 2 sum_{u<v} <G_u, G_v>
    over the dropped set D, and it is bounded by (sum sqrt R)^2 <= d * sum R."""
    p = _small_swiglu(seed=seed, counts=(8, 6), E=2, T=7, K=2, D=5, F=4)
    r = p.routing
    full = o.backward(G=p.G, Phi=p.Phi, alpha=r.alpha, tok=r.tok, slot=r.slot, seg_off=r.seg_off,
                      quota=np.diff(r.seg_off), dtype="bf16", T=p.cfg.T, W2=p.W2, X=p.X, H=p.H, W1=p.W1)
    q = np.array([3, 2])
    kept = o.backward(G=p.G, Phi=p.Phi, alpha=r.alpha, tok=r.tok, slot=r.slot, seg_off=r.seg_off,
                      quota=q, dtype="bf16", T=p.cfg.T, W2=p.W2, X=p.X, H=p.H, W1=p.W1)
    R = full["R"]
    g64 = synth.bf16_bits_to_f32(p.G).astype(np.float64)
    p64 = synth.bf16_bits_to_f32(p.Phi).astype(np.float64)
    for e in range(2):
        seg = range(r.seg_off[e], r.seg_off[e + 1])
        D_set = sorted(set(seg) - set(kept["sel"].tolist()))
        Gs = [np.outer(p64[u], float(r.alpha[u]) * g64[r.tok[u]]) for u in D_set]  # [in x out]
        lhs = float(np.sum((full["dW2"][e] - kept["dW2"][e]) ** 2))
        cross = sum(float(np.sum(Gs[a] * Gs[b])) for a in range(len(Gs)) for b in range(a + 1, len(Gs)))
        rhs = float(R[D_set].sum()) + 2.0 * cross
        assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs))
        assert lhs <= float(np.sum(np.sqrt(R[D_set]))) ** 2 * (1 + 1e-12)
        assert float(np.sum(np.sqrt(R[D_set]))) ** 2 <= len(D_set) * float(R[D_set].sum()) * (1 + 1e-12)


def check_scatter(o, seed=9):
    """Scatter restores the layout: token mode conserves the row sum and puts each row on
    its token; slot mode writes each row at (token, slot) and leaves every other row 0."""
    rng = _rng(seed)
    T, K, w = 6, 3, 4
    pos = rng.choice(T * K, size=10, replace=False)
    ctok, cslot = pos // K, pos % K
    rows = rng.standard_normal((10, w))
    out = o.scatter_tokens(rows, ctok, T)
    np.testing.assert_allclose(out.sum(axis=0), rows.sum(axis=0), rtol=1e-12)
    for t in range(T):
        np.testing.assert_allclose(out[t], rows[ctok == t].sum(axis=0) if np.any(ctok == t) else 0.0,
                                   rtol=1e-12, atol=0)
    s = o.scatter_slots(rows, ctok, cslot, T, K)
    np.testing.assert_array_equal(s[pos], rows)
    rest = np.setdiff1d(np.arange(T * K), pos)
    assert np.all(s[rest] == 0)


def check_round_bf16(o, seed=10):
    """bf16 round-to-nearest-even, against hand-worked ties and torch's CPU conversion."""
    cases = {1.0: 0x3F80, 1.0 + 2.0 ** -8: 0x3F80, 1.0 + 3 * 2.0 ** -8: 0x3F82,
             -(1.0 + 2.0 ** -8 + 2.0 ** -30): 0xBF81, 0.0: 0x0000, 255.5: 0x4380, 256.0 + 1.0: 0x4380}
    for v, bits in cases.items():
        assert int(o.round_bf16(np.array([v]))[0]) == bits, (v, hex(int(o.round_bf16(np.array([v]))[0])))
    x = _rng(seed).standard_normal(100000).astype(np.float32) * np.float32(3.0)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(o.round_bf16(x.astype(np.float64)), ref)


ALL_CHECKS = {
    "score_outer_product_bf16": lambda o: check_score_outer_product(o, "bf16"),
    "score_outer_product_f32": lambda o: check_score_outer_product(o, "f32"),
    "score_dyadic_exact": check_score_dyadic_exact,
    "score_is_omission_change": check_score_is_omission_change,
    "gradient_only_brute_force": check_gradient_only_brute_force,
    "gradient_only_against_lrm": check_gradient_only_against_lrm,
    "ceil_quotas_definition": check_ceil_quotas_definition,
    "backward_bytes_from_shapes": check_backward_bytes_from_shapes,
    "plan_quotas_brute_force": check_plan_quotas_brute_force,
    "backward_bytes_adds_workspace": check_backward_bytes_adds_workspace,
    "swiglu_closed_forms": check_swiglu_closed_forms,
    "forward_exact": check_forward_exact,
    "select_exhaustive_distinct": lambda o: check_select_exhaustive(o, ties=False),
    "select_exhaustive_ties": lambda o: check_select_exhaustive(o, seed=11, ties=True),
    "select_per_expert": check_select_per_expert,
    "fig4_worked_example": check_fig4_worked_example,
    "compact_identity": check_compact_identity,
    "weighted_phi_vs_autograd": check_weighted_phi_vs_autograd,
    "swiglu_dense_vs_autograd": check_swiglu_dense_vs_autograd,
    "swiglu_masked_vs_autograd": check_swiglu_masked_vs_autograd,
    "linear_masked_vs_autograd": check_linear_masked_vs_autograd,
    "aggregate_error_eq19": check_aggregate_error_eq19,
    "scatter": check_scatter,
    "round_bf16": check_round_bf16,
}


@pytest.mark.parametrize("name", sorted(ALL_CHECKS))
def test_oracle_pin(name):
    ALL_CHECKS[name](oracle)


def test_select_rejects_infeasible_quota():
    with pytest.raises(oracle.InfeasibleQuota):
        oracle.select(np.ones(3), np.array([0, 3]), np.array([4]))
    with pytest.raises(oracle.InfeasibleQuota):
        oracle.select(np.ones(3), np.array([0, 3]), np.array([-1]))


def test_llep_reindex_example_groups_stably():
    """The LLEP page's re-indexing example pins the generator's expert-major grouping."""
    with open(os.path.join(GOLDEN, "llep_reindex_example.json")) as f:
        ex = json.load(f)
    order = synth.group_expert_major(np.array(ex["experts"]))
    assert [ex["tokens"][i] for i in order] == ex["batch_order"]


# ----------------------------------------------------------------------------- planted mistakes

def _mutant(**overrides):
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in oracle.__all__})
    for k, v in overrides.items():
        setattr(ns, k, v)
    # backward() resolves its steps through the module; rebuild it on the namespace
    def backward(**kw):
        return _backward_on(ns, **kw)
    ns.backward = backward
    return ns


def _backward_on(o, *, G, Phi, alpha, tok, slot, seg_off, quota, dtype, T, W2, X=None, H=None,
                 W1=None, score_dtype=np.float32):
    R = o.score(G, Phi, alpha, tok, dtype)
    key = R if score_dtype is None else R.astype(score_dtype)
    sel, cseg_off, tau = o.select(key, seg_off, quota)
    c = o.compact(sel, tok, slot, alpha, G, Phi, dtype, X=X, H=H)
    out = {"R": R, "sel": sel, "cseg_off": cseg_off, "tau": tau, **c}
    if H is not None:
        dW1, dW2, dH, dXC = o.swiglu_expert_backward(cseg_off, c["Dlt"], c["PhiC"], c["XC"], c["HC"],
                                                     o.widen(W1, dtype), o.widen(W2, dtype))
        out.update(dW1=dW1, dW2=dW2, dH=dH, dXC=dXC, out=o.scatter_tokens(dXC, c["ctok"], T))
    else:
        dW, dPhi = o.linear_expert_backward(cseg_off, c["Dlt"], c["PhiC"], o.widen(W2, dtype))
        out.update(dW2=dW, dPhi=dPhi, out=o.scatter_tokens(dPhi, c["ctok"], T))
    return out


def _score_alpha_not_squared(G, Phi, alpha, tok, dtype, chunk=16384):
    return oracle.score(G, Phi, alpha, tok, dtype) / np.asarray(alpha, dtype=np.float64)


def _gradient_only_signed_sum(G, tok, dtype, criterion, chunk=16384):
    if criterion == "grad_abs":
        return oracle.widen(G, dtype).sum(axis=1)[np.asarray(tok, dtype=np.int64)]
    return oracle.score_gradient_only(G, tok, dtype, criterion)


def _gradient_only_by_pair_row(G, tok, dtype, criterion, chunk=16384):
    n = len(tok)
    return oracle.score_gradient_only(G, np.arange(n) % np.asarray(G).shape[0], dtype, criterion)


def _ceil_quotas_floor(counts, rho):
    from fractions import Fraction
    import math
    r = Fraction(rho)
    return np.array([min(int(n), math.floor(r * int(n))) for n in counts], dtype=np.int64)


def _backward_bytes_no_dh(*, T, E, D, F, swiglu, dtype, N, K_tot, packed=False, workspace=0):
    e = 2 if dtype == "bf16" else 4
    return oracle.backward_bytes(T=T, E=E, D=D, F=F, swiglu=swiglu, dtype=dtype, N=N, K_tot=K_tot,
                                 packed=packed, workspace=workspace) - (K_tot * 2 * F * e if swiglu else 0)


def _plan_in_given_order(counts, rhos, hbm_avail, workspace=None, **kw):
    for i, r in enumerate(rhos):
        q = oracle.ceil_quotas(counts, r)
        b = oracle.backward_bytes(E=len(counts), N=sum(int(n) for n in counts), K_tot=int(q.sum()),
                                  workspace=0 if workspace is None else workspace(q), **kw)
        if b <= hbm_avail:
            return i, q, b
    raise oracle.InfeasibleQuota("none")


def _plan_without_workspace(counts, rhos, hbm_avail, workspace=None, **kw):
    return oracle.plan_quotas(counts, rhos, hbm_avail, **kw)


def _backward_bytes_ignores_workspace(*, workspace=0, **kw):
    return oracle.backward_bytes(**kw)


def _swiglu_sigmoid_of_minus(h, F):
    h = np.asarray(h, dtype=np.float64)
    return h[:, :F] / (1.0 + np.exp(h[:, :F])) * h[:, F:]


def _fc1_no_gather(X, tok, seg_off, W1, dtype):
    return oracle.expert_forward_fc1(X, np.arange(len(tok)) % np.asarray(X).shape[0], seg_off, W1, dtype)


def _fc2_alpha_dropped(Phi, alpha, seg_off, W2, dtype):
    return oracle.expert_forward_fc2(Phi, np.ones_like(np.asarray(alpha)), seg_off, W2, dtype)


def _select_smallest(R, seg_off, quota):
    sel, c, tau = oracle.select(-np.asarray(R), seg_off, quota)
    return sel, c, tau


def _select_layer_wide(R, seg_off, quota):
    R = np.asarray(R)
    k = int(np.sum(quota))
    top = np.sort(np.lexsort((np.arange(len(R)), -R))[:k])
    c = np.concatenate([[0], np.cumsum(quota)])
    return top, c, np.full(len(quota), np.nan)


def _select_ties_high_index(R, seg_off, quota):
    R = np.asarray(R)
    n = len(R)
    rev = R[::-1]
    seg_rev = (n - np.asarray(seg_off)[::-1])
    sel, c, tau = oracle.select(rev, seg_rev, np.asarray(quota)[::-1])
    sel = np.sort(n - 1 - sel)
    return sel, np.concatenate([[0], np.cumsum(quota)]), tau[::-1]


def _compact_alpha_twice(sel, tok, slot, alpha, G, Phi, dtype, X=None, H=None):
    out = oracle.compact(sel, tok, slot, alpha, G, Phi, dtype, X=X, H=H)
    out["Dlt"] = out["Dlt"] * np.asarray(alpha, dtype=np.float64)[np.asarray(sel)][:, None]
    return out


def _compact_phiw_unweighted(sel, tok, slot, alpha, G, Phi, dtype, X=None, H=None):
    out = oracle.compact(sel, tok, slot, alpha, G, Phi, dtype, X=X, H=H)
    out["PhiW"] = out["PhiC"]
    return out


def _compact_phiw_alpha_by_packed_row(sel, tok, slot, alpha, G, Phi, dtype, X=None, H=None):
    out = oracle.compact(sel, tok, slot, alpha, G, Phi, dtype, X=X, H=H)
    a = np.asarray(alpha, dtype=np.float64)[: len(sel)]
    out["PhiW"] = a[:, None] * out["PhiC"]
    return out


def _compact_token_off_by_one(sel, tok, slot, alpha, G, Phi, dtype, X=None, H=None):
    t = np.asarray(tok).copy()
    t = np.minimum(t + 1, np.asarray(G).shape[0] - 1)
    return oracle.compact(sel, t, slot, alpha, G, Phi, dtype, X=X, H=H)


def _swiglu_wrong_dsilu(row_off, Dlt, PhiC, XC, HC, W1, W2):
    F = W2.shape[1]
    HC2 = HC.copy()
    # uses silu'(x) = sigmoid(x) (drops the x * s * (1 - s) term) by rescaling the gate
    g = HC[:, :F]
    s = 1.0 / (1.0 + np.exp(-g))
    dW1, dW2, dH, dXC = oracle.swiglu_expert_backward(row_off, Dlt, PhiC, XC, HC2, W1, W2)
    ratio = s / (s * (1.0 + g * (1.0 - s)))
    dH2 = dH.copy()
    dH2[:, :F] *= ratio
    row_off = np.asarray(row_off)
    for e in range(len(row_off) - 1):
        r = slice(row_off[e], row_off[e + 1])
        dW1[e] = XC[r].T @ dH2[r]
        dXC[r] = dH2[r] @ W1[e].T
    return dW1, dW2, dH2, dXC


def _swiglu_gate_up_swapped(row_off, Dlt, PhiC, XC, HC, W1, W2):
    F = W2.shape[1]
    HC2 = np.concatenate([HC[:, F:], HC[:, :F]], axis=1)
    return oracle.swiglu_expert_backward(row_off, Dlt, PhiC, XC, HC2, W1, W2)


def _scatter_drop_last(rows, ctok, T):
    return oracle.scatter_tokens(np.asarray(rows)[:-1], np.asarray(ctok)[:-1], T)


def _round_truncate(x):
    v = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
    return (v >> np.uint32(16)).astype(np.uint16)


PLANTED = [
    ("score_alpha_not_squared", dict(score=_score_alpha_not_squared),
     ["score_outer_product_bf16", "score_dyadic_exact", "score_is_omission_change"]),
    ("gradient_abs_without_abs", dict(score_gradient_only=_gradient_only_signed_sum),
     ["gradient_only_brute_force", "gradient_only_against_lrm"]),
    ("gradient_only_ignores_token", dict(score_gradient_only=_gradient_only_by_pair_row),
     ["gradient_only_brute_force", "gradient_only_against_lrm"]),
    ("quota_rounds_down", dict(ceil_quotas=_ceil_quotas_floor), ["ceil_quotas_definition"]),
    ("bytes_without_dh", dict(backward_bytes=_backward_bytes_no_dh), ["backward_bytes_from_shapes"]),
    ("plan_in_given_order", dict(plan_quotas=_plan_in_given_order), ["plan_quotas_brute_force"]),
    ("plan_without_workspace", dict(plan_quotas=_plan_without_workspace), ["plan_quotas_brute_force"]),
    ("bytes_ignore_workspace", dict(backward_bytes=_backward_bytes_ignores_workspace),
     ["backward_bytes_adds_workspace"]),
    ("silu_with_sigmoid_of_minus_x", dict(swiglu=_swiglu_sigmoid_of_minus), ["swiglu_closed_forms", "forward_exact"]),
    ("fc1_ignores_token_gather", dict(expert_forward_fc1=_fc1_no_gather), ["forward_exact"]),
    ("fc2_drops_routing_weight", dict(expert_forward_fc2=_fc2_alpha_dropped), ["forward_exact"]),
    ("select_keeps_smallest", dict(select=_select_smallest),
     ["select_exhaustive_distinct", "fig4_worked_example", "select_per_expert"]),
    ("select_layer_wide", dict(select=_select_layer_wide), ["select_per_expert"]),
    ("select_ties_to_higher_index", dict(select=_select_ties_high_index), ["select_exhaustive_ties"]),
    ("compact_alpha_applied_twice", dict(compact=_compact_alpha_twice),
     ["compact_identity", "swiglu_dense_vs_autograd", "linear_masked_vs_autograd"]),
    ("compact_phiw_unweighted", dict(compact=_compact_phiw_unweighted), ["weighted_phi_vs_autograd"]),
    ("compact_phiw_alpha_of_packed_row", dict(compact=_compact_phiw_alpha_by_packed_row),
     ["weighted_phi_vs_autograd"]),
    ("compact_wrong_token", dict(compact=_compact_token_off_by_one),
     ["compact_identity", "swiglu_masked_vs_autograd"]),
    ("swiglu_wrong_derivative", dict(swiglu_expert_backward=_swiglu_wrong_dsilu),
     ["swiglu_dense_vs_autograd", "swiglu_masked_vs_autograd"]),
    ("swiglu_gate_up_swapped", dict(swiglu_expert_backward=_swiglu_gate_up_swapped),
     ["swiglu_dense_vs_autograd"]),
    ("scatter_drops_a_row", dict(scatter_tokens=_scatter_drop_last), ["scatter", "swiglu_dense_vs_autograd"]),
    ("round_bf16_truncates", dict(round_bf16=_round_truncate), ["round_bf16"]),
]


@pytest.mark.parametrize("mistake,overrides,checks", PLANTED, ids=[m[0] for m in PLANTED])
def test_pins_catch_planted_mistakes(mistake, overrides, checks):
    """A plausible mistake planted in a copy of the oracle must fail every listed pin."""
    o = _mutant(**overrides)
    for name in checks:
        with pytest.raises((AssertionError, ValueError, IndexError)):
            ALL_CHECKS[name](o)
