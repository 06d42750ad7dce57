"""C-ABI library checks that need no GPU: it loads, exports every symbol the header
declares, and its host-side validation answers before any launch."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from load_recalibrated_expert_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "lrmoe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\*|lrmoe_status)\s+(lrmoe_\w+)\s*\(", src, re.M)))


def test_header_declares_the_five_steps():
    d = _declared()
    for name in ("lrmoe_score", "lrmoe_select", "lrmoe_compact", "lrmoe_grouped_gemm_bwd", "lrmoe_scatter",
                 "lrmoe_validate", "lrmoe_workspace_size", "lrmoe_status_string", "lrmoe_version"):
        assert name in d


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s+(lrmoe_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(_lib.EXPORTS) <= exported


def _problem(E=3, T=10, K=2, D=64, F=32, swiglu=1, dtype=_lib.BF16, counts=(5, 0, 7), quota=(3, 0, 7)):
    seg = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return _lib.make_problem_struct(E, T, K, D, F, swiglu, dtype, seg, np.array(quota, dtype=np.int32))


def _validate(p):
    k = ctypes.c_int64(-1)
    cseg = np.full(p.E + 1, -7, dtype=np.int64)
    st = _lib.load().lrmoe_validate(ctypes.byref(p), ctypes.byref(k), cseg.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return st, k.value, cseg


def test_validate_accepts_and_returns_packed_offsets():
    p, keep = _problem()
    st, k, cseg = _validate(p)
    assert st == _lib.OK and k == 10 and cseg.tolist() == [0, 3, 3, 10]


def test_validate_worked_example_offsets():
    # loads [4,2,3] retained [3,1,2] (LRMoE Figure 4) -> packed offsets [0,3,4,6]
    p, keep = _problem(counts=(4, 2, 3), quota=(3, 1, 2), T=5)
    st, k, cseg = _validate(p)
    assert st == _lib.OK and k == 6 and cseg.tolist() == [0, 3, 4, 6]


@pytest.mark.parametrize("quota", [(6, 0, 7), (3, -1, 7), (3, 1, 7)])
def test_validate_rejects_infeasible_quota(quota):
    p, keep = _problem(quota=quota)
    assert _validate(p)[0] == _lib.ERR_INFEASIBLE_QUOTA


@pytest.mark.parametrize("kw,expect", [
    (dict(D=60), _lib.ERR_UNSUPPORTED),
    (dict(F=12), _lib.ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.ERR_UNSUPPORTED),
    (dict(T=5), _lib.ERR_INVALID_ARG),          # N = 12 pairs > T*K = 10 positions
    (dict(K=0), _lib.ERR_INVALID_ARG),
])
def test_validate_rejects_bad_shapes(kw, expect):
    p, keep = _problem(**kw)
    assert _validate(p)[0] == expect


def test_validate_rejects_bad_flags():
    p, keep = _problem()
    p.swiglu = 2
    assert _validate(p)[0] == _lib.ERR_INVALID_ARG
    p.swiglu = 1
    p.reserved = 1
    assert _validate(p)[0] == _lib.ERR_INVALID_ARG


def test_validate_rejects_non_monotone_offsets():
    p, keep = _problem()
    keep[0][1] = 9  # seg_off = [0, 9, 5, 12]
    assert _validate(p)[0] == _lib.ERR_INVALID_ARG


def test_workspace_size_and_host_side_rejections():
    lib = _lib.load()
    p, keep = _problem()
    n = ctypes.c_size_t(0)
    assert lib.lrmoe_workspace_size(ctypes.byref(p), _lib.COMPACT_PHYSICAL, ctypes.byref(n)) == _lib.OK
    assert n.value >= 256
    # null device pointers and missing workspaces are refused on the host, before any launch
    assert lib.lrmoe_score(ctypes.byref(p), None, None, None, None, None, None, 0, None) == _lib.ERR_INVALID_ARG
    fake = ctypes.c_void_p(0x1000)
    assert lib.lrmoe_score(ctypes.byref(p), fake, fake, fake, fake, fake, None, 0, None) == _lib.ERR_WORKSPACE
    nomap = [None] * 5  # tok, slot, pmap, ctok, cslot
    assert lib.lrmoe_select(ctypes.byref(p), fake, fake, fake, fake, fake, None, *nomap, None, 0,
                            None) == _lib.ERR_WORKSPACE
    # the (token, slot) map needs the pairs' tokens and slots and the packed rows' outputs
    assert lib.lrmoe_select(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, fake, fake, fake, fake,
                            fake, 1 << 30, None) == _lib.ERR_INVALID_ARG
    assert lib.lrmoe_select(ctypes.byref(p), fake, fake, fake, fake, fake, None, fake, fake, fake, None, fake,
                            fake, 1 << 30, None) == _lib.ERR_INVALID_ARG
    assert lib.lrmoe_select(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, None, None, fake, fake,
                            fake, 1 << 30, None) == _lib.ERR_INVALID_ARG  # ctok without the map
    assert lib.lrmoe_scatter(ctypes.byref(p), 0, 3, 12, _lib.BF16, fake, fake, fake, None, fake, fake, 1 << 20,
                             None) == _lib.ERR_INVALID_ARG  # width not a multiple of 8
    assert lib.lrmoe_scatter(ctypes.byref(p), 3, 3, 16, _lib.BF16, fake, fake, fake, None, fake, fake, 1 << 20,
                             None) == _lib.ERR_INVALID_ARG  # no scatter mode 3 (TOKEN, SLOT, TOKEN_BESIDE)
    # with the selection's map the scatter covers exactly the K_tot packed rows (3 + 0 + 7 = 10 here)
    assert lib.lrmoe_scatter(ctypes.byref(p), 0, 11, 16, _lib.BF16, fake, None, None, fake, fake, None, 0,
                             None) == _lib.ERR_INVALID_ARG
    assert lib.lrmoe_compact(ctypes.byref(p), 5, *([None] * 16), None, 0, None) == _lib.ERR_INVALID_ARG
    sw = [fake] * 15 if p.swiglu else [fake, None, fake, fake, None, None, fake, fake, fake, fake, fake, None,
                                         None, fake, fake]
    assert lib.lrmoe_compact(ctypes.byref(p), _lib.COMPACT_PHYSICAL, *sw, None, None, 0,
                             None) == _lib.ERR_WORKSPACE
    q, keep2 = _problem(quota=(6, 0, 7))
    assert lib.lrmoe_grouped_gemm_bwd(ctypes.byref(q), 0, *([fake] * 14), 0, fake, 1 << 30,
                                      None, None) == _lib.ERR_INFEASIBLE_QUOTA
    assert _lib.status_string(_lib.ERR_INFEASIBLE_QUOTA).startswith("infeasible")
    # packing PhiC needs Phi; packing XC needs X
    args = [fake, None, fake, None, None, None, fake, fake, fake, fake, fake, None, None, fake, fake]
    assert lib.lrmoe_compact(ctypes.byref(p), _lib.COMPACT_PHYSICAL, *args, None, fake, 1 << 30,
                             None) == _lib.ERR_INVALID_ARG
    args = [fake, None, fake, fake, None, None, fake, fake, fake, fake, None, fake, None, fake, fake]
    assert lib.lrmoe_compact(ctypes.byref(p), _lib.COMPACT_PHYSICAL, *args, None, fake, 1 << 30,
                             None) == _lib.ERR_INVALID_ARG
    # zero-masked compaction has no packed rows to map
    args = [None, fake, fake, fake, fake, fake, fake, fake, fake, fake, None, None, None, None, None]
    assert lib.lrmoe_compact(ctypes.byref(p), _lib.COMPACT_ZERO_MASKED, *args, fake, fake, 1 << 30,
                             None) == _lib.ERR_INVALID_ARG


def test_score_criterion_host_checks():
    """lrmoe_score_criterion: unknown criteria, missing pointers and workspaces are refused on the
    host; the gradient-only criteria do not need Phi or alpha (they fail only on the workspace)."""
    lib = _lib.load()
    p, keep = _problem()
    fake = ctypes.c_void_p(0x1000)
    f = lib.lrmoe_score_criterion
    assert f(ctypes.byref(p), 3, fake, fake, fake, fake, fake, fake, 1 << 20, None) == _lib.ERR_INVALID_ARG
    assert f(ctypes.byref(p), -1, fake, fake, fake, fake, fake, fake, 1 << 20, None) == _lib.ERR_INVALID_ARG
    for crit in (1, 2):
        assert f(ctypes.byref(p), crit, fake, None, None, fake, fake, None, 0, None) == _lib.ERR_WORKSPACE
        assert f(ctypes.byref(p), crit, None, None, None, fake, fake, fake, 1 << 20, None) == _lib.ERR_INVALID_ARG
        assert f(ctypes.byref(p), crit, fake, None, None, None, fake, fake, 1 << 20, None) == _lib.ERR_INVALID_ARG
    # criterion 0 is lrmoe_score, which needs Phi and alpha
    assert f(ctypes.byref(p), 0, fake, None, None, fake, fake, fake, 1 << 20, None) == _lib.ERR_INVALID_ARG


def test_expert_forward_host_checks():
    """lrmoe_expert_forward: SwiGLU bf16 only, every pointer required when there are pairs,
    matrices too large for 32-bit offsets refused - all on the host, before any launch."""
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    f = lib.lrmoe_expert_forward
    p, keep = _problem(dtype=_lib.F32)
    assert f(ctypes.byref(p), *([fake] * 9), None) == _lib.ERR_UNSUPPORTED
    p, keep = _problem(swiglu=0)
    assert f(ctypes.byref(p), *([fake] * 9), None) == _lib.ERR_UNSUPPORTED
    p, keep = _problem()
    for i in range(9):
        args = [fake] * 9
        args[i] = None
        assert f(ctypes.byref(p), *args, None) == _lib.ERR_INVALID_ARG, i
    big, keep2 = _problem(T=600000, D=2048, counts=(5, 0, 7))
    assert f(ctypes.byref(big), *([fake] * 9), None) == _lib.ERR_UNSUPPORTED  # X is 2.3 GiB


def _gemm(p, phi_rows=None, x_rows=None, swiglu=True):
    """lrmoe_grouped_gemm_bwd with fake device pointers (only host checks can pass)."""
    fake = ctypes.c_void_p(0x1000)
    w1 = fake if swiglu else None
    return _lib.load().lrmoe_grouped_gemm_bwd(
        ctypes.byref(p), _lib.COMPACT_PHYSICAL, fake, fake, fake, w1, w1, w1, phi_rows, x_rows, fake, w1, fake, w1,
        w1, fake, 0, None, 0, None, None)


def test_row_maps_limited_to_2gib_matrices():
    """Gathered weight-gradient operands are addressed with 32-bit byte offsets: a mapped
    Phi (N x F) or X (T x D) of 2 GiB or more is refused on the host."""
    fake = ctypes.c_void_p(0x1000)
    # N * F * 2 bytes = 2^20 * 1024 * 2 = 2 GiB
    p, keep = _problem(E=1, T=1 << 20, K=1, D=64, F=1024, counts=(1 << 20,), quota=(3,))
    assert _gemm(p, phi_rows=fake) == _lib.ERR_UNSUPPORTED
    # T * D * 2 bytes = 2^24 * 64 * 2 = 2 GiB
    p, keep = _problem(E=1, T=1 << 24, K=1, D=64, F=32, counts=(8,), quota=(3,))
    assert _gemm(p, x_rows=fake) == _lib.ERR_UNSUPPORTED
    # just under: the checks move on (to the missing workspace)
    p, keep = _problem(E=1, T=(1 << 24) - 1, K=1, D=64, F=32, counts=(8,), quota=(3,))
    assert _gemm(p, x_rows=fake) == _lib.ERR_WORKSPACE
    # an X row map without SwiGLU is an argument error
    p, keep = _problem(swiglu=0)
    assert _gemm(p, x_rows=fake, swiglu=False) == _lib.ERR_INVALID_ARG


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "load_recalibrated_expert_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f
                assert "synth" not in re.findall(r"^\s*(?:import|from)\s+(\w+)", text, re.M), f


def test_select_noalloc_refuses_problems_beyond_its_scratch():
    """lrmoe_select_noalloc's fixed 4 MiB scratch holds E x 20 KB of digit histograms: 1100
    experts need more, which is refused on the host before any launch; bad arguments are
    refused as for lrmoe_select."""
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    counts = np.full(1100, 3)
    p, keep = _problem(E=1100, T=4000, K=1, counts=counts, quota=np.ones(1100, dtype=np.int32))
    assert lib.lrmoe_select_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, None, None, None,
                                    None, None) == _lib.ERR_WORKSPACE
    q, keep2 = _problem()
    assert lib.lrmoe_select_noalloc(ctypes.byref(q), None, fake, fake, fake, fake, None, None, None, None, None,
                                    None, None) == _lib.ERR_INVALID_ARG
    assert lib.lrmoe_select_noalloc(ctypes.byref(q), fake, fake, fake, fake, fake, None, None, None, None, fake,
                                    None, None) == _lib.ERR_INVALID_ARG


def _gathered(p, swiglu=True, **kw):
    """lrmoe_grouped_gemm_bwd_gathered with every pointer set (fake device addresses) except
    those overridden; returns the status of the host checks."""
    fake = ctypes.c_void_p(0x1000)
    a = dict(cseg=fake, G=fake, alpha=fake, sel=fake, ctok=fake, PhiW=fake, X=fake if swiglu else None,
             H=fake if swiglu else None, W2=fake, W1=fake if swiglu else None, dW2=fake,
             dW1=fake if swiglu else None, dH=fake if swiglu else None, dIn=fake, acc=0, ws=None, ws_bytes=0)
    a.update(kw)
    return _lib.load().lrmoe_grouped_gemm_bwd_gathered(
        ctypes.byref(p), a["cseg"], a["G"], a["alpha"], a["sel"], a["ctok"], a["PhiW"], a["X"], a["H"], a["W2"],
        a["W1"], a["dW2"], a["dW1"], a["dH"], a["dIn"], a["acc"], a["ws"], a["ws_bytes"], None, None)


def test_gathered_path_host_checks():
    """The path that reads gradient rows by token: lrmoe_compact_weighted and
    lrmoe_grouped_gemm_bwd_gathered refuse missing buffers, SwiGLU-only arguments on a
    linear problem, a G or X of 2 GiB or more (32-bit offsets) and a missing workspace,
    on the host, before any launch."""
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    p, keep = _problem()
    assert lib.lrmoe_compact_weighted(ctypes.byref(p), None, fake, fake, fake, None) == _lib.ERR_INVALID_ARG
    assert lib.lrmoe_compact_weighted(ctypes.byref(p), fake, fake, None, fake, None) == _lib.ERR_INVALID_ARG
    z, keep_z = _problem(quota=(0, 0, 0))  # nothing retained: nothing to check or launch
    assert lib.lrmoe_compact_weighted(ctypes.byref(z), None, None, None, None, None) == _lib.OK
    bad_q, keep_b = _problem(quota=(6, 0, 7))
    assert lib.lrmoe_compact_weighted(ctypes.byref(bad_q), fake, fake, fake, fake, None) == _lib.ERR_INFEASIBLE_QUOTA
    # every buffer the step reads or writes is required
    for k in ("cseg", "G", "alpha", "sel", "ctok", "PhiW", "X", "H", "W2", "W1", "dW2", "dW1", "dH", "dIn"):
        assert _gathered(p, **{k: None}) == _lib.ERR_INVALID_ARG, k
    assert _gathered(p, acc=2) == _lib.ERR_INVALID_ARG
    # the weight-gradient plan needs the workspace the library asks for
    assert _gathered(p) == _lib.ERR_WORKSPACE
    # a linear (FC2-only) problem takes no SwiGLU operands
    lin, keep_l = _problem(swiglu=0)
    assert _gathered(lin, swiglu=False, X=fake) == _lib.ERR_INVALID_ARG
    assert _gathered(lin, swiglu=False, dH=fake) == _lib.ERR_INVALID_ARG
    # G and X of T * D * 2 bytes = 2^24 * 64 * 2 = 2 GiB are read with 32-bit offsets: refused
    big, keep_g = _problem(E=1, T=1 << 24, K=1, D=64, F=32, counts=(8,), quota=(3,))
    assert _gathered(big) == _lib.ERR_UNSUPPORTED
    ok, keep_o = _problem(E=1, T=(1 << 24) - 1, K=1, D=64, F=32, counts=(8,), quota=(3,))
    assert _gathered(ok) == _lib.ERR_WORKSPACE  # the checks move on to the missing workspace
