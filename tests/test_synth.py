"""Seeded input generator: determinism and the workload shapes (no GPU)."""
import numpy as np

import synth


def test_counts_and_quotas_of_the_large_workloads():
    # 32,768 tokens x top-8 = 262,144 pairs over 16 local experts (LRMoE section 4.1 shapes)
    q = synth.CONFIGS["qwen3_30b_a3b_share"]
    n = synth.expert_counts(q)
    assert n.sum() == 262144 and len(n) == 16 and np.all(np.diff(n) <= 0)
    assert int(synth.quotas(n, "0.6").sum()) == 157292
    x = synth.expert_counts(synth.CONFIGS["extreme_skew"])
    assert x[0] == round(0.7 * 262144) and x.sum() == 262144
    assert int(synth.quotas(x, "0.4").sum()) == 104864
    s = synth.CONFIGS["glm_quota_sweep"]
    ns = synth.expert_counts(s)
    assert [int(synth.quotas(ns, r).sum()) for r in s.rhos] == [262144, 209721, 131077, 65544]


def test_quota_rounding_is_exact_ceil():
    assert synth.quotas([5, 10, 0, 1, 3], "0.6").tolist() == [3, 6, 0, 1, 2]
    assert synth.quotas([7], "1.0").tolist() == [7]


def test_tiny_router_workload():
    p = synth.make_problem("tiny")
    r = p.routing
    assert r.seg_off[-1] == 512 and p.Phi.shape == (512, 32) and p.G.shape == (256, 64)
    assert np.all(np.diff(r.expert) >= 0)
    # each (token, slot) position appears exactly once
    pos = r.tok.astype(np.int64) * 2 + r.slot
    assert len(np.unique(pos)) == 512
    # top-2 of a softmax: slot 0 carries the larger weight of its token
    w = np.zeros((256, 2), dtype=np.float32)
    w[r.tok, r.slot] = r.alpha
    assert np.all(w[:, 0] >= w[:, 1]) and np.all(w.sum(axis=1) <= 1.0 + 1e-6)
    assert np.array_equal(p.quota, np.ceil(0.75 * np.diff(r.seg_off)).astype(np.int32))


def test_generation_is_deterministic_and_chunk_stable():
    cfg = synth.custom(T=50, K=4, E=5, D=24, F=16, counts=(40, 0, 60, 30, 10), seed=77)
    a, b = synth.make_problem(cfg), synth.make_problem(cfg)
    for k in ("G", "X", "H", "Phi", "W1", "W2"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))
    np.testing.assert_array_equal(a.routing.tok, b.routing.tok)
    # N < T*K: every (token, slot) position used at most once
    pos = a.routing.tok.astype(np.int64) * 4 + a.routing.slot
    assert len(np.unique(pos)) == 140


def test_bf16_conversion_round_trip():
    x = np.array([1.0, -2.5, 3.140625, 1e-3], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(b)[:3], x[:3])
