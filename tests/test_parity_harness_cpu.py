"""CPU checks of the GPU parity harness's tie-band rule.

Ties at an expert's threshold make several selections optimal (LRMoE paper, appendix 7.2,
Prop. 7.1), so a GPU selection may swap pairs whose scores lie inside the 1e-5 band. The
harness must then re-run the oracle's compaction, expert backward and scatter on the
GPU's choice and compare with that, and must reject a swap outside the band. Here a
synthetic "GPU selection" swaps one pair of an exact tie placed at a threshold.
"""
import numpy as np
import pytest

import oracle
from parity_ref import BAND, on_gpu_selection, reference_selection
from tie_case import swap as _swap, tied_problem


def _rel(a, b):
    d = float(np.linalg.norm(b))
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b))) / (d if d > 0 else 1.0)


@pytest.fixture(scope="module")
def tied():
    """Pairs j1 < j2 of expert 0 score exactly alike, with expert 0's quota ending between
    them: the oracle keeps j1 and drops j2."""
    pr, inputs, j1, j2 = tied_problem()
    ref = oracle.backward(**inputs)
    assert j1 in ref["sel"] and j2 not in ref["sel"]
    return dict(inputs=inputs, ref=ref, j1=j1, j2=j2, R=ref["R"])


def _gpu_like_outputs(inp, sel):
    """What a correct GPU path produces on the selection ``sel`` (the oracle's steps 3-5,
    with the packed gradient rows stored in bf16 as the GPU stores them)."""
    c = oracle.compact(sel, inp["tok"], inp["slot"], inp["alpha"], inp["G"], inp["Phi"], "bf16", X=inp["X"],
                       H=inp["H"])
    cseg = np.concatenate([[0], np.cumsum(inp["quota"])])
    dlt = oracle.widen(oracle.round_bf16(c["Dlt"]), "bf16")
    dW1, dW2, dH, dXC = oracle.swiglu_expert_backward(cseg, dlt, c["PhiC"], c["XC"], c["HC"],
                                                      oracle.widen(inp["W1"], "bf16"), oracle.widen(inp["W2"], "bf16"))
    return dict(sel=sel, ctok=c["ctok"], cslot=c["cslot"], Dlt=oracle.round_bf16(c["Dlt"]), dW1=dW1, dW2=dW2,
                dH=dH, dIn=dXC, out=oracle.scatter_tokens(dXC, c["ctok"], inp["T"]))


def _compare(got, ref, E):
    """The comparisons the GPU parity tests make (index lists and compacted rows bit-exact,
    GEMM and scatter outputs within the derived 5e-3)."""
    assert np.array_equal(got["sel"], ref["sel"])
    assert np.array_equal(got["ctok"], ref["ctok"])
    assert np.array_equal(got["cslot"], ref["cslot"])
    assert np.array_equal(got["Dlt"], oracle.round_bf16(ref["Dlt"]))
    for e in range(E):
        assert _rel(got["dW1"][e], ref["dW1"][e]) <= 5e-3
        assert _rel(got["dW2"][e], ref["dW2"][e]) <= 5e-3
    assert _rel(got["dH"], ref["dH"]) <= 5e-3
    assert _rel(got["dIn"], ref["dXC"]) <= 5e-3
    assert _rel(got["out"], ref["out"]) <= 5e-3


def test_in_band_swap_is_rerun_and_passes(tied):
    inp, ref = tied["inputs"], tied["ref"]
    sel_gpu = _swap(ref["sel"], tied["j1"], tied["j2"])
    got = _gpu_like_outputs(inp, sel_gpu)
    checked = on_gpu_selection(ref, sel_gpu, **inp)
    assert checked is not ref and checked.get("rerun_on_gpu_selection")
    _compare(got, checked, len(inp["quota"]))
    # the oracle's own selection would have failed the index comparisons: the swap is real
    with pytest.raises(AssertionError):
        _compare(got, ref, len(inp["quota"]))


def test_same_selection_keeps_the_oracle_reference(tied):
    inp, ref = tied["inputs"], tied["ref"]
    assert on_gpu_selection(ref, ref["sel"].copy(), **inp) is ref
    _compare(_gpu_like_outputs(inp, ref["sel"]), ref, len(inp["quota"]))


def test_swap_outside_the_band_is_rejected(tied):
    inp, ref, R = tied["inputs"], tied["ref"], tied["R"]
    seg = inp["seg_off"]
    tau = ref["tau"][0]
    dropped = np.setdiff1d(np.arange(seg[0], seg[1]), ref["sel"])
    far = [int(j) for j in dropped if abs(R[j] - tau) > 1e3 * BAND * tau]
    assert far, "a dropped pair well below the threshold"
    sel_bad = _swap(ref["sel"], tied["j1"], far[0])
    with pytest.raises(AssertionError, match="outside the band"):
        on_gpu_selection(ref, sel_bad, **inp)


def test_wrong_count_or_order_is_rejected(tied):
    inp, ref = tied["inputs"], tied["ref"]
    with pytest.raises(AssertionError):
        reference_selection(ref["sel"][:-1], ref["R"], inp["seg_off"], inp["quota"])
    s = ref["sel"].copy()
    s[[0, 1]] = s[[1, 0]]
    with pytest.raises(AssertionError, match="ascending"):
        reference_selection(s, ref["R"], inp["seg_off"], inp["quota"])
