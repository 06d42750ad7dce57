"""Quota admission on one GPU (host-only C ABI: lrmoe_backward_bytes, lrmoe_plan_quotas)
against the oracle's admission (Algorithm 1's forward-time admission with a single GPU).
The estimate is the backward's buffers plus the library's workspace at each candidate's
quotas; the oracle takes that workspace from lrmoe_workspace_size. Integer results, so
they must agree exactly. No GPU needed."""
import ctypes

import numpy as np
import pytest

import load_recalibrated_expert_amd as lr
import oracle
import synth
from load_recalibrated_expert_amd import _lib

RHOS = ["1", "0.8", "0.6", "0.5", "0.25", "0.1", "0"]


@pytest.fixture(scope="module", params=["qwen3_30b_a3b_share", "extreme_skew", "tiny"])
def workload(request):
    cfg = synth.CONFIGS[request.param]
    return cfg, np.diff(synth.make_routing(cfg).seg_off).astype(np.int64)


def _dims(cfg):
    return dict(T=cfg.T, D=cfg.D, F=cfg.F, swiglu=bool(cfg.swiglu), dtype=cfg.dtype)


def _ws_fn(cfg, seg, mode=_lib.COMPACT_PHYSICAL):
    """The scratch the library asks for at given quotas: lrmoe_workspace_size plus the
    selection's (token, slot) -> packed row map, int32 [T x K]."""
    dt = _lib.BF16 if cfg.dtype == "bf16" else _lib.F32

    def ws(q):
        c, keep = _lib.make_problem_struct(cfg.E, cfg.T, cfg.K, cfg.D, cfg.F, cfg.swiglu, dt, seg,
                                           np.asarray(q, dtype=np.int32))
        n = ctypes.c_size_t(0)
        assert _lib.load().lrmoe_workspace_size(ctypes.byref(c), mode, ctypes.byref(n)) == _lib.OK
        return int(n.value) + 4 * cfg.T * cfg.K
    return ws


@pytest.mark.parametrize("packed", [False, True])
def test_backward_bytes_matches_oracle(workload, packed):
    cfg, counts = workload
    seg = np.concatenate([[0], np.cumsum(counts)])
    for rho in RHOS:
        q = oracle.ceil_quotas(counts, rho).astype(np.int32)
        c, keep = _lib.make_problem_struct(cfg.E, cfg.T, cfg.K, cfg.D, cfg.F, cfg.swiglu,
                                           _lib.BF16 if cfg.dtype == "bf16" else _lib.F32, seg, q)
        n = ctypes.c_size_t(0)
        assert _lib.load().lrmoe_backward_bytes(ctypes.byref(c), int(packed), ctypes.byref(n)) == _lib.OK
        ref = oracle.backward_bytes(E=cfg.E, N=int(seg[-1]), K_tot=int(q.sum()), packed=packed,
                                    workspace=_ws_fn(cfg, seg)(q), **_dims(cfg))
        assert n.value == ref, (cfg.name, rho, packed)


@pytest.mark.parametrize("packed", [False, True])
def test_plan_quotas_matches_oracle(workload, packed):
    cfg, counts = workload
    seg = np.concatenate([[0], np.cumsum(counts)])
    dt = _lib.BF16 if cfg.dtype == "bf16" else _lib.F32
    ws = _ws_fn(cfg, seg)
    est = [oracle.backward_bytes(E=cfg.E, N=int(seg[-1]), K_tot=int(oracle.ceil_quotas(counts, r).sum()),
                                 packed=packed, workspace=ws(oracle.ceil_quotas(counts, r)), **_dims(cfg))
           for r in RHOS]
    for budget in sorted(set(est)) + [max(est) + 1, min(est) - 1]:
        try:
            ref = oracle.plan_quotas(counts, RHOS, budget, packed=packed, workspace=ws, **_dims(cfg))
        except oracle.InfeasibleQuota:
            with pytest.raises(_lib.InfeasibleQuotaError):
                lr.plan_quotas(cfg.E, cfg.T, cfg.K, cfg.D, cfg.F, cfg.swiglu, dt, seg, RHOS, budget, packed=packed)
            continue
        i, q, b = lr.plan_quotas(cfg.E, cfg.T, cfg.K, cfg.D, cfg.F, cfg.swiglu, dt, seg, RHOS, budget, packed=packed)
        assert (i, b) == (ref[0], ref[2])
        assert q.tolist() == ref[1].tolist()


def test_plan_quotas_order_ties_and_rounding():
    """Candidates given out of order and with a duplicate; quotas use the exact ceiling
    (0.6 * 5 = 3, where a floating-point product exceeds 3)."""
    counts = np.array([5, 10, 0, 7], dtype=np.int64)
    seg = np.concatenate([[0], np.cumsum(counts)])
    rhos = ["0.3", "0.6", "0.9", "0.6"]
    dims = dict(T=22, D=64, F=32, swiglu=True, dtype="bf16")
    big = 1 << 40
    i, q, b = lr.plan_quotas(4, 22, 1, 64, 32, 1, _lib.BF16, seg, rhos, big)
    assert i == 2 and q.tolist() == [5, 9, 0, 7]
    cfg = synth.custom(T=22, K=1, E=4, D=64, F=32, counts=tuple(int(n) for n in counts), seed=1)
    q06 = oracle.ceil_quotas(counts, "0.6")
    b06 = oracle.backward_bytes(E=4, N=22, K_tot=int(q06.sum()), workspace=_ws_fn(cfg, seg)(q06), **dims)
    i, q, b = lr.plan_quotas(4, 22, 1, 64, 32, 1, _lib.BF16, seg, rhos, b06)
    assert i == 1 and q.tolist() == [3, 6, 0, 5] and b == b06


def test_plan_quotas_rejects_bad_ratios():
    seg = np.array([0, 3, 5], dtype=np.int64)
    c, keep = _lib.make_problem_struct(2, 5, 1, 64, 32, 1, _lib.BF16, seg, np.zeros(2, dtype=np.int32))
    I32 = ctypes.POINTER(ctypes.c_int32)
    out_i, out_b = ctypes.c_int32(7), ctypes.c_size_t(0)
    q = np.zeros(2, dtype=np.int32)
    for num, den in (([1], [0]), ([3], [2]), ([-1], [2])):
        n, d = np.array(num, dtype=np.int32), np.array(den, dtype=np.int32)
        st = _lib.load().lrmoe_plan_quotas(ctypes.byref(c), n.ctypes.data_as(I32), d.ctypes.data_as(I32), 1, 0,
                                           1 << 40, ctypes.byref(out_i), q.ctypes.data_as(I32), ctypes.byref(out_b))
        assert st == _lib.ERR_INVALID_ARG
    n, d = np.array([1], dtype=np.int32), np.array([2], dtype=np.int32)
    st = _lib.load().lrmoe_plan_quotas(ctypes.byref(c), n.ctypes.data_as(I32), d.ctypes.data_as(I32), 0, 0,
                                       1 << 40, ctypes.byref(out_i), q.ctypes.data_as(I32), ctypes.byref(out_b))
    assert st == _lib.ERR_INVALID_ARG
    st = _lib.load().lrmoe_plan_quotas(ctypes.byref(c), n.ctypes.data_as(I32), d.ctypes.data_as(I32), 1, 0,
                                       0, ctypes.byref(out_i), q.ctypes.data_as(I32), ctypes.byref(out_b))
    assert st == _lib.ERR_INFEASIBLE_QUOTA and out_i.value == -1


def test_workspace_holds_the_split_reduction_partials():
    """At the Qwen3-30B-A3B share's quotas the experts above 12288 retained rows split their
    weight-gradient reduction into chunks of at most 12288 rows, each chunk keeping one
    256 x 256 fp32 partial tile per weight-gradient tile (FC2: F/256 x D/256, FC1:
    D/256 x 2F/256); the workspace, and so the admission estimate, holds all of them."""
    cfg = synth.CONFIGS["qwen3_30b_a3b_share"]
    counts = np.diff(synth.make_routing(cfg).seg_off).astype(np.int64)
    seg = np.concatenate([[0], np.cumsum(counts)])
    tiles = -(-cfg.F // 256) * -(-cfg.D // 256) + -(-cfg.D // 256) * -(-2 * cfg.F // 256)
    for rho in ("0.6", "1"):
        q = oracle.ceil_quotas(counts, rho)
        chunks = [-(-int(m) // 12288) for m in q if m > 12288]
        partials = sum(chunks) * tiles * 256 * 256 * 4
        ws = _ws_fn(cfg, seg)(q)
        pmap = 4 * cfg.T * cfg.K
        assert partials > 0 and partials + pmap <= ws <= partials + pmap + (1 << 20), (rho, partials, ws)
        c, keep = _lib.make_problem_struct(cfg.E, cfg.T, cfg.K, cfg.D, cfg.F, cfg.swiglu, _lib.BF16, seg,
                                           q.astype(np.int32))
        n = ctypes.c_size_t(0)
        assert _lib.load().lrmoe_backward_bytes(ctypes.byref(c), 0, ctypes.byref(n)) == _lib.OK
        bufs = oracle.backward_bytes(E=cfg.E, N=int(seg[-1]), K_tot=int(q.sum()), **_dims(cfg))
        assert n.value == bufs + ws



def _partials_bytes(cfg, q, kc):
    tiles = -(-cfg.F // 256) * -(-cfg.D // 256) + -(-cfg.D // 256) * -(-2 * cfg.F // 256)
    return sum(-(-int(m) // kc) for m in q if m > kc) * tiles * 256 * 256 * 4


@pytest.mark.parametrize("name,rho,kc", [("qwen3_30b_a3b_share", "0.6", 12288),
                                         ("glm45_106b_a12b_share", "0.6", 12288),
                                         ("glm_quota_sweep", "1.0", 12288),
                                         ("extreme_skew", "0.4", 8192)])
def test_chunk_length_follows_the_expert_balance(name, rho, kc):
    """The weight-gradient chunk length is 12288 rows unless one expert's long chunks would
    load the eight XCDs unevenly: with 70% of the retained rows in one expert (the
    extreme-skew routing) 8192-row chunks win despite their extra partial tiles. The
    workspace holds the partials of exactly the chosen length (plus the map and under 1 MiB
    of plan and compaction scratch), so its size tells which length was taken."""
    cfg = synth.CONFIGS[name]
    counts = np.diff(synth.make_routing(cfg).seg_off).astype(np.int64)
    seg = np.concatenate([[0], np.cumsum(counts)])
    q = oracle.ceil_quotas(counts, rho)
    ws = _ws_fn(cfg, seg)(q)
    pmap = 4 * cfg.T * cfg.K
    fits = [c for c in (12288, 8192, 6144) if 0 <= ws - pmap - _partials_bytes(cfg, q, c) <= (1 << 20)]
    assert fits == [kc], (ws, fits)
