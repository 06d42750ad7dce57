"""GPU parity of the forward that saves the backward's context (lrmoe_expert_forward:
Algorithm 1's FullForwardAndSaveContext) against the oracle, and the backward run on the
context that forward saved. Calls go through the C ABI.

Tolerances (derived from the arithmetic): every stored value is one bf16 rounding
(relative error <= 2^-9) of an fp32 sum whose accumulation error is far below that, so
H, Phi and Y agree per element within 2^-8 |ref| + 1e-4 rms(row). Y is compared with the
oracle's FC2 applied to the GPU's own stored Phi (the FC2 input is the saved tensor). The
layer output sums bf16 Y rows in f32: rel. Frobenius <= 5e-3. The backward on the saved
context keeps the backward suite's bound against the exact oracle: rel. Frobenius <= 5e-3.
"""
import dataclasses

import numpy as np
import pytest
import torch

import load_recalibrated_expert_amd as lr
import oracle
import synth

from gpu_util import DEV, Staged, as_f64, bits, log, rel_fro

pytestmark = pytest.mark.gpu

CASES = {
    "ragged": synth.custom("fwd_ragged", T=600, K=4, E=6, D=512, F=384, counts=(700, 0, 513, 300, 257, 1), seed=31),
    "odd_dims": synth.custom("fwd_odd_dims", T=100, K=2, E=4, D=136, F=72, counts=(50, 17, 0, 90), seed=32),
    "many_experts": synth.custom("fwd_many_experts", T=300, K=10, E=40, D=256, F=128,
                                 counts=tuple((0 if e % 3 == 1 else 3 * e + 5) for e in range(40)), seed=33),
    "wide": synth.custom("fwd_wide", T=150, K=3, E=3, D=2304, F=136, counts=(200, 90, 110), seed=34),
    "multi_round": synth.custom("fwd_multi_round", T=16750, K=2, E=3, D=256, F=640, counts=(14000, 12000, 7500),
                                seed=35),
}


def _close_rows(got, ref, rel=2.0 ** -8, floor=1e-4):
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    err = np.abs(got - ref)
    bound = rel * np.abs(ref) + floor * rms
    assert np.all(err <= bound), f"max excess {np.max(err - bound)}"


@pytest.fixture(scope="module", params=sorted(CASES))
def fwd(request):
    log(f"forward case {request.param}: generating")
    pr = synth.make_problem(CASES[request.param], rho="0.6")
    s = Staged(pr)
    r = pr.routing
    out = lr.expert_forward(s.P, s.X, s.tok, s.alpha, s.W1, s.W2)
    torch.cuda.synchronize()
    log(f"forward case {request.param}: N={s.P.N}")
    return request.param, pr, s, out


def test_forward_saved_activations(fwd):
    name, pr, s, out = fwd
    r = pr.routing
    H_or, Phi_or = oracle.expert_forward_fc1(pr.X, r.tok, r.seg_off, pr.W1, "bf16")
    _close_rows(as_f64(out["H"]), H_or)
    _close_rows(as_f64(out["Phi"]), Phi_or)


def test_forward_output_rows_and_layer_output(fwd):
    name, pr, s, out = fwd
    r = pr.routing
    Y_or = oracle.expert_forward_fc2(bits(out["Phi"]), r.alpha, r.seg_off, pr.W2, "bf16")
    _close_rows(as_f64(out["Y"]), Y_or)
    y = lr.scatter(s.P, out["Y"], s.tok, s.slot, n_rows=s.P.N)
    torch.cuda.synchronize()
    ref = oracle.scatter_tokens(Y_or, r.tok, pr.cfg.T)
    assert rel_fro(as_f64(y[:pr.cfg.T]), ref) <= 5e-3


def test_backward_on_the_saved_context(fwd):
    """The backward path run on the H and Phi this forward saved, against the oracle fed the
    same stored values."""
    name, pr0, s, out = fwd
    pr = dataclasses.replace(pr0, H=bits(out["H"]), Phi=bits(out["Phi"]))
    s2 = Staged(pr)
    res = s2.backward()
    torch.cuda.synchronize()
    r = pr.routing
    ref = oracle.backward(G=pr.G, Phi=pr.Phi, alpha=r.alpha, tok=r.tok, slot=r.slot, seg_off=r.seg_off,
                          quota=pr.quota, dtype="bf16", T=pr.cfg.T, W2=pr.W2, X=pr.X, H=pr.H, W1=pr.W1)
    for k in ("dW1", "dW2"):
        got = as_f64(res[k])
        for e in range(pr.cfg.E):
            if np.linalg.norm(ref[k][e]) > 0:
                assert rel_fro(got[e], ref[k][e]) <= 5e-3, (name, k, e)
    assert rel_fro(as_f64(res["out"][:pr.cfg.T]), ref["out"]) <= 5e-3


def test_forward_rejects_unsupported():
    pr = synth.make_problem(synth.custom("fwd_f32", T=20, K=2, E=2, D=64, F=32, counts=(10, 8), dtype="f32",
                                         seed=36), rho="1.0")
    s = Staged(pr)
    with pytest.raises(lr.LrmoeError):
        lr.expert_forward(s.P, s.X, s.tok, s.alpha, s.W1, s.W2)


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_share", "glm45_106b_a12b_share"])
def test_forward_full_size_sampled(name):
    """Full-size workload, the launch bench.py --forward times: 96 sampled pairs (the first
    and last of every expert plus random ones) checked row by row against the oracle."""
    log(f"forward full size {name}: generating")
    pr = synth.make_problem(name)
    s = Staged(pr)
    out = lr.expert_forward(s.P, s.X, s.tok, s.alpha, s.W1, s.W2)
    torch.cuda.synchronize()
    r = pr.routing
    seg = r.seg_off
    rng = np.random.default_rng(5)
    pick = set(rng.integers(0, int(seg[-1]), size=64).tolist())
    for e in range(pr.cfg.E):
        if seg[e + 1] > seg[e]:
            pick.update((int(seg[e]), int(seg[e + 1]) - 1))
    pick = np.array(sorted(pick), dtype=np.int64)
    e_of = np.searchsorted(seg, pick, side="right") - 1
    log(f"forward full size {name}: checking {len(pick)} pairs")
    H = as_f64(out["H"][torch.from_numpy(pick).to(DEV)])
    Phi_bits = bits(out["Phi"][torch.from_numpy(pick).to(DEV)])
    Y = as_f64(out["Y"][torch.from_numpy(pick).to(DEV)])
    X = oracle.widen(pr.X, "bf16")
    F = pr.cfg.F
    H_ref = np.stack([X[r.tok[j]] @ oracle.widen(pr.W1[e], "bf16") for j, e in zip(pick, e_of)])
    _close_rows(H, H_ref)
    _close_rows(oracle.widen(Phi_bits, "bf16"), oracle.swiglu(H_ref, F))
    Y_ref = np.stack([float(r.alpha[j]) * (oracle.widen(Phi_bits[i], "bf16") @ oracle.widen(pr.W2[e], "bf16"))
                      for i, (j, e) in enumerate(zip(pick, e_of))])
    _close_rows(Y, Y_ref)
    del s, out
    torch.cuda.empty_cache()
