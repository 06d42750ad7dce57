"""GPU parity at the largest addresses the path accepts.

The grouped GEMMs read the expert input X and the gradient rows G in place, through the
packed rows' token map, with 32-bit byte offsets; the library accepts that while
T * D * 2 < 2^31 and rejects larger X and G (unsupported). Here T = 2^20 - 1 and D = 1024,
so X and G are 2^31 - 2048 bytes each and the gathered rows of the last tokens sit just
under the limit.
The forward's FC1 launch gathers X the same way. The token-order scatter writes a
[T x D] fp32 output of 4 GiB, past 32-bit byte offsets.

Only a few thousand pairs are routed. Their tokens' rows of G and X are drawn from the
seeded generator; every other row is zero and enters no result. The oracle runs on the
reduced problem (the routed tokens renumbered 0..T'-1), which every step maps one to one:
scores, selection, packed rows, GEMMs and the scattered rows of routed tokens. Tolerances
are those of the small parity cases; rows of unrouted tokens must stay exactly zero.
"""
import numpy as np
import pytest
import torch

import load_recalibrated_expert_amd as lr
import oracle
import synth

from gpu_util import DEV, as_f64, bits, check_selection, log, on_gpu_selection, rel_fro, to_dev

pytestmark = pytest.mark.gpu

T, D, F = (1 << 20) - 1, 1024, 64
BAR, DERIVED = 2e-2, 5e-3


@pytest.fixture(scope="module")
def limit():
    cfg = synth.custom("address_limit", T=T, K=1, E=2, D=D, F=F, counts=(2500, 1500), seed=25)
    rho = "0.75"
    log(f"address limit: T={T} D={D}, X and G {T * D * 2} bytes (limit {1 << 31})")
    r = synth.make_routing(cfg)
    counts = np.diff(r.seg_off)
    quota = synth.quotas(counts, rho)
    N, E = int(r.seg_off[-1]), cfg.E
    toks = np.unique(r.tok)                      # routed tokens, ascending
    tok_r = np.searchsorted(toks, r.tok).astype(np.int32)
    Tr = len(toks)
    G_r = synth.normal_rows(cfg.seed, synth.TID_G, Tr, D, 1.0, "bf16")
    X_r = synth.normal_rows(cfg.seed, synth.TID_X, Tr, D, 1.0, "bf16")
    H = synth.normal_rows(cfg.seed, synth.TID_PAIR, N, 2 * F, 1.0, "bf16")
    Phi = synth.swiglu_forward_phi(H, F)
    W1 = synth.normal_rows(cfg.seed, synth.TID_W1, E * D, 2 * F, 1.0 / np.sqrt(D), "bf16").reshape(E, D, 2 * F)
    W2 = synth.normal_rows(cfg.seed, synth.TID_W2, E * F, D, 1.0 / np.sqrt(F), "bf16").reshape(E, F, D)

    toks_d = torch.from_numpy(toks.astype(np.int64)).to(DEV)
    G = torch.zeros((T, D), dtype=torch.bfloat16, device=DEV)
    X = torch.zeros((T, D), dtype=torch.bfloat16, device=DEV)
    G[toks_d] = to_dev(G_r, "bf16")
    X[toks_d] = to_dev(X_r, "bf16")
    P = lr.Problem(E=E, T=T, K=1, D=D, F=F, swiglu=True, dtype=lr.BF16, seg_off=r.seg_off, quota=quota, device=DEV)
    log(f"address limit: GPU path N={N} K_tot={P.K_tot}, highest routed token {int(toks[-1])}")
    res = lr.backward(P, G=G, Phi=to_dev(Phi, "bf16"), alpha=torch.from_numpy(r.alpha).to(DEV),
                      tok=torch.from_numpy(r.tok).to(DEV), slot=torch.from_numpy(r.slot).to(DEV),
                      W2=to_dev(W2, "bf16"), X=X, H=to_dev(H, "bf16"), W1=to_dev(W1, "bf16"))
    torch.cuda.synchronize()
    log("address limit: oracle on the routed tokens")
    ref = oracle.backward(G=G_r, Phi=Phi, alpha=r.alpha, tok=tok_r, slot=r.slot, seg_off=r.seg_off, quota=quota,
                          dtype="bf16", T=Tr, W2=W2, X=X_r, H=H, W1=W1)
    try:  # steps 3-5 on the GPU's selection (differences only inside the tie band)
        ref = on_gpu_selection(ref, res["sel"].cpu().numpy(), G=G_r, Phi=Phi, alpha=r.alpha, tok=tok_r, slot=r.slot,
                               seg_off=r.seg_off, quota=quota, dtype="bf16", T=Tr, W2=W2, X=X_r, H=H, W1=W1)
    except AssertionError as err:
        log(f"address limit: GPU selection rejected ({err})")
    yield dict(r=r, toks=toks, toks_d=toks_d, quota=quota, res=res, ref=ref, E=E, P=P, X=X, X_r=X_r, tok_r=tok_r,
               W1=W1, W2=W2)
    del res, G, X
    torch.cuda.empty_cache()


def test_limit_inputs_reach_the_limit(limit):
    # the last tokens are routed, so the in-place gather reads within 1 MiB of the limit
    assert (int(limit["toks"][-1]) + 1) * D * 2 > (1 << 31) - (1 << 20)
    assert T * D * 2 < (1 << 31)


def test_limit_score_select_compact(limit):
    res, ref, r = limit["res"], limit["ref"], limit["r"]
    R = as_f64(res["R"])
    assert np.all(np.abs(R - ref["R"]) <= 1e-6 * ref["R"] + 1e-35)
    sel = res["sel"].cpu().numpy().astype(np.int64)
    check_selection(sel, ref["R"], r.seg_off, limit["quota"])
    assert np.array_equal(sel, ref["sel"])
    # ctok holds original token ids; the oracle's are renumbered
    assert np.array_equal(res["ctok"].cpu().numpy(), limit["toks"][ref["ctok"]])
    assert np.array_equal(res["cslot"].cpu().numpy(), ref["cslot"])
    assert np.array_equal(bits(res["PhiW"]), oracle.round_bf16(ref["PhiW"]))


def test_limit_grouped_gemm(limit):
    res, ref = limit["res"], limit["ref"]
    dW1, dW2 = as_f64(res["dW1"]), as_f64(res["dW2"])
    for e in range(limit["E"]):
        assert rel_fro(dW2[e], ref["dW2"][e]) <= DERIVED, f"dW2 expert {e}"
        assert rel_fro(dW1[e], ref["dW1"][e]) <= DERIVED, f"dW1 expert {e}"
    assert rel_fro(as_f64(res["dH"]), ref["dH"]) <= DERIVED
    dIn = as_f64(res["dIn"])
    assert rel_fro(dIn, ref["dXC"]) <= DERIVED
    num = np.linalg.norm(dIn - ref["dXC"], axis=1)
    den = np.linalg.norm(ref["dXC"], axis=1)
    assert np.all(num <= BAR * np.maximum(den, 1e-30))


def test_limit_scatter(limit):
    res, ref, toks_d = limit["res"], limit["ref"], limit["toks_d"]
    out = res["out"]
    assert tuple(out.shape) == (T, D) and out.dtype == torch.float32
    got = as_f64(out[toks_d])
    assert rel_fro(got, ref["out"]) <= DERIVED
    # exactly the routed tokens that kept a pair have nonzero rows; every other row is zero
    nonzero = 0
    for t0 in range(0, T, 1 << 17):
        nonzero += int((out[t0:t0 + (1 << 17)] != 0).any(dim=1).sum())
    assert nonzero == int(np.count_nonzero(np.abs(ref["out"]).sum(axis=1)))


def _close_rows(got, ref, rel=2.0 ** -8, floor=1e-4):
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + floor * rms)


def test_limit_forward(limit):
    """The forward that saves the context, gathering X rows up to the last routed token:
    per element within one bf16 rounding of the oracle (as in the forward parity cases)."""
    r, P = limit["r"], limit["P"]
    out = lr.expert_forward(P, limit["X"], torch.from_numpy(r.tok).to(DEV), torch.from_numpy(r.alpha).to(DEV),
                            to_dev(limit["W1"], "bf16"), to_dev(limit["W2"], "bf16"))
    torch.cuda.synchronize()
    H_or, Phi_or = oracle.expert_forward_fc1(limit["X_r"], limit["tok_r"], r.seg_off, limit["W1"], "bf16")
    _close_rows(as_f64(out["H"]), H_or)
    _close_rows(as_f64(out["Phi"]), Phi_or)
    Y_or = oracle.expert_forward_fc2(bits(out["Phi"]), r.alpha, r.seg_off, limit["W2"], "bf16")
    _close_rows(as_f64(out["Y"]), Y_or)
