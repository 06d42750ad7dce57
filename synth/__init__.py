"""Seeded synthetic inputs for the memory-aware MoE expert backward (LRMoE).

This module only *draws* inputs. It holds no step of the method: no scoring,
selection, compaction, gradient or scatter arithmetic. The CPU oracle's tests
and the HIP path's tests and benchmark both take their inputs from here, so the
two sides see the same stored values.

What it draws, and from which passage of the pages the shapes come:

* A routed MoE layer on one GPU's share of experts. Every routed token-expert
  pair ``u = (t, e)`` (LRMoE paper, section 2.1) is one row. Pairs are stored
  expert-major: the (token, slot) positions are grouped by expert with a stable
  sort, which is the re-indexing that the Least-Loaded EP page illustrates in its
  "reindexing tokens into per-expert batches" example (tokens a,b,c,d routed to
  experts 2,6,2,1 become the batch order d,a,c,b).
* Routing weights ``alpha``: a softmax over the router logits whose top-K
  probabilities are kept without renormalisation (the LLEP page's MoE output
  formula, where the gate of a selected expert is its softmax score).
* Shapes of the LRMoE evaluation (section 4.1): sequence 8192 x micro-batch 4 =
  32,768 tokens per GPU, 128 experts with top-8 routing, so 16 local experts
  under EP8, hidden 2048 and expert intermediate 768 (Qwen3-30B-A3B shaped),
  and a GLM4.5-106B-A12B-shaped variant with hidden 4096 and intermediate 1408.
* Retention quotas ``q_e = min(n_e, ceil(rho * n_e))``: the LRMoE paper sets the
  quotas once, before the layer call, and the backward does not revise them
  (section 3.1); it does not give the planner's rounding, so this is the plain
  reading.

Random numbers come from numpy's counter-based Philox generator, one stream per
(seed, tensor id, row chunk), so generation is deterministic and can run on
several threads. bf16 tensors are returned as ``uint16`` bit patterns produced
by round-to-nearest-even from float32.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

# Tensor ids that key the random streams.
TID_G = 1        # upstream gradient g_t, [T, D]
TID_PAIR = 2     # per-pair saved state: H = [gate | up] (SwiGLU) or phi (linear)
TID_X = 3        # expert input x_t, [T, D]
TID_W1 = 4       # FC1 weights, [E, D, 2F]
TID_W2 = 5       # FC2 weights, [E, F, D]
TID_ROUTER = 6   # router inputs / logits
TID_SHUFFLE = 7  # placement of expert ids over (token, slot) positions
TID_POS = 8      # choice of (token, slot) positions when N < T*K

_CHUNK_ROWS = 4096


@dataclass(frozen=True)
class Config:
    """One synthetic workload: a single GPU's share of a routed MoE layer."""

    name: str
    T: int            # tokens
    K: int            # routing slots per token (top-K)
    E: int            # local experts
    D: int            # hidden size (width of g_t and x_t)
    F: int            # expert intermediate size (width of phi_u, FC2 input)
    swiglu: bool      # True: SwiGLU experts (FC1 gate/up + FC2); False: one projection
    dtype: str        # storage dtype of activations, gradients and weights: "f32" | "bf16"
    rhos: tuple       # retention ratios, as decimal strings
    seed: int
    skew: tuple       # ("router", s) | ("zipf", s) | ("hot", frac, s)
    n_logits: int = 128
    counts: tuple = field(default=())  # explicit per-expert pair counts (custom problems)
    n_pairs: int = 0  # explicit N when counts are given (N may be < T*K)

    @property
    def N(self) -> int:
        return self.n_pairs if self.counts else self.T * self.K


CONFIGS = {
    # Tiny fp32 down-projection backward: router-determined load, top-2 of 8.
    "tiny": Config("tiny", T=256, K=2, E=8, D=64, F=32, swiglu=False, dtype="f32",
                   rhos=("0.75",), seed=0x5EED0001, skew=("router", 1.0), n_logits=8),
    # Qwen3-30B-A3B-shaped share: D=2048, intermediate 768, 16 local experts, Zipf 1.2.
    "qwen3_30b_a3b_share": Config("qwen3_30b_a3b_share", T=32768, K=8, E=16, D=2048, F=768,
                                  swiglu=True, dtype="bf16", rhos=("0.6",), seed=0x5EED0002,
                                  skew=("zipf", 1.2)),
    # GLM4.5-106B-A12B-shaped share: D=4096, intermediate 1408.
    "glm45_106b_a12b_share": Config("glm45_106b_a12b_share", T=32768, K=8, E=16, D=4096, F=1408,
                                    swiglu=True, dtype="bf16", rhos=("0.6",), seed=0x5EED0003,
                                    skew=("zipf", 1.2)),
    # Extreme imbalance: 70% of pairs on one expert, the rest Zipf 2.0 over the others.
    "extreme_skew": Config("extreme_skew", T=32768, K=8, E=16, D=2048, F=768, swiglu=True,
                           dtype="bf16", rhos=("0.4",), seed=0x5EED0004, skew=("hot", 0.7, 2.0)),
    # Quota sweep at GLM shapes; one dataset for every ratio.
    "glm_quota_sweep": Config("glm_quota_sweep", T=32768, K=8, E=16, D=4096, F=1408, swiglu=True,
                              dtype="bf16", rhos=("1.0", "0.8", "0.5", "0.25"), seed=0x5EED0005,
                              skew=("zipf", 1.2)),
}


def custom(name="custom", *, T, K, E, D, F, counts, swiglu=True, dtype="bf16", seed=1,
           rhos=("0.6",)) -> Config:
    """A small problem with explicit per-expert pair counts (sum may be < T*K)."""
    counts = tuple(int(c) for c in counts)
    if len(counts) != E or sum(counts) > T * K or min(counts) < 0:
        raise ValueError("counts must have E non-negative entries summing to at most T*K")
    return Config(name, T=T, K=K, E=E, D=D, F=F, swiglu=swiglu, dtype=dtype, rhos=tuple(rhos),
                  seed=seed, skew=("explicit",), counts=counts, n_pairs=sum(counts))


# ----------------------------------------------------------------------------- bf16 storage

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b >> np.uint32(16)) & np.uint32(1)
    out = ((b + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------- random streams

def _gen(seed: int, tid: int, chunk: int = 0) -> np.random.Generator:
    key = np.array([seed & 0xFFFFFFFFFFFFFFFF, ((tid & 0xFFFFFFFF) << 32) | (chunk & 0xFFFFFFFF)],
                   dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_rows(seed, tid, rows, cols, std=1.0, out_dtype="f32") -> np.ndarray:
    """[rows, cols] of N(0, std^2), drawn in fixed row chunks (one stream per chunk).

    Returns float32, or uint16 bf16 bits when ``out_dtype == "bf16"``.
    """
    out = np.empty((rows, cols), dtype=np.uint16 if out_dtype == "bf16" else np.float32)
    nchunks = (rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS

    def work(c):
        r0, r1 = c * _CHUNK_ROWS, min(rows, (c + 1) * _CHUNK_ROWS)
        v = _gen(seed, tid, c).standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(v) if out_dtype == "bf16" else v

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


# ----------------------------------------------------------------------------- routing

def apportion(total: int, weights) -> np.ndarray:
    """Largest-remainder apportionment of ``total`` over ``weights`` (ties -> lower index)."""
    w = np.asarray(weights, dtype=np.float64)
    exact = total * w / w.sum()
    base = np.floor(exact).astype(np.int64)
    rem = total - int(base.sum())
    frac = exact - base
    order = np.lexsort((np.arange(len(w)), -frac))  # largest remainder first, lower index on ties
    base[order[:rem]] += 1
    return base


def expert_counts(cfg: Config) -> np.ndarray:
    """Pair counts n_e of the local experts, for the count-driven configs."""
    if cfg.counts:
        return np.asarray(cfg.counts, dtype=np.int64)
    kind = cfg.skew[0]
    N = cfg.N
    if kind == "zipf":
        s = cfg.skew[1]
        return apportion(N, (np.arange(cfg.E) + 1.0) ** (-s))
    if kind == "hot":
        frac, s = cfg.skew[1], cfg.skew[2]
        n0 = int(round(frac * N))
        rest = apportion(N - n0, (np.arange(1, cfg.E) + 0.0) ** (-s))
        return np.concatenate([[n0], rest]).astype(np.int64)
    raise ValueError(f"counts of config {cfg.name} are router-determined")


def quotas(counts, rho: str) -> np.ndarray:
    """q_e = min(n_e, ceil(rho * n_e)), with rho taken as an exact decimal."""
    r = Fraction(rho)
    return np.array([min(int(n), math.ceil(r * int(n))) for n in counts], dtype=np.int32)


@dataclass
class Routing:
    seg_off: np.ndarray   # int64 [E+1]: pair segment of expert e is [seg_off[e], seg_off[e+1])
    tok: np.ndarray       # int32 [N]: token of each pair, expert-major
    slot: np.ndarray      # int32 [N]: routing slot (0..K-1) of each pair
    alpha: np.ndarray     # float32 [N]: routing weight of each pair
    expert: np.ndarray    # int32 [N]: expert of each pair (non-decreasing)


def group_expert_major(expert_of_position: np.ndarray) -> np.ndarray:
    """Stable grouping of (token, slot) positions by expert: returns the position order."""
    return np.argsort(np.asarray(expert_of_position), kind="stable")


def _softmax_topk(logits: np.ndarray, K: int):
    """Softmax over the last axis (fp64), then the K largest probabilities per row, in
    decreasing order (ties -> lower index). Not renormalised."""
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    idx = np.argsort(-p, axis=1, kind="stable")[:, :K]
    return idx, np.take_along_axis(p, idx, axis=1)


def make_routing(cfg: Config) -> Routing:
    T, K, E = cfg.T, cfg.K, cfg.E
    if cfg.skew[0] == "router":
        # u ~ N(0,1)^D, W_r ~ N(0, 1/D), logits = u W_r + log(Zipf weights), softmax, top-K.
        s = cfg.skew[1]
        g = _gen(cfg.seed, TID_ROUTER)
        u = g.standard_normal((T, cfg.D))
        wr = g.standard_normal((cfg.D, E)) / math.sqrt(cfg.D)
        zipf = (np.arange(E) + 1.0) ** (-s)
        logits = u @ wr + np.log(zipf / zipf.sum())
        idx, prob = _softmax_topk(logits, K)
        expert_pos = idx.reshape(-1).astype(np.int32)        # position p = t*K + k
        alpha_pos = prob.reshape(-1).astype(np.float32)
        positions = np.arange(T * K, dtype=np.int64)
    else:
        counts = expert_counts(cfg)
        N = int(counts.sum())
        # alpha: softmax over n_logits router logits per token, top-K kept by slot.
        g = _gen(cfg.seed, TID_ROUTER)
        logits = g.standard_normal((T, cfg.n_logits))
        _, prob = _softmax_topk(logits, K)
        alpha_all = prob.reshape(-1).astype(np.float32)
        if N == T * K:
            positions = np.arange(T * K, dtype=np.int64)
        else:
            positions = np.sort(_gen(cfg.seed, TID_POS).choice(T * K, size=N, replace=False))
        ids = np.repeat(np.arange(E, dtype=np.int32), counts)
        expert_pos = ids[_gen(cfg.seed, TID_SHUFFLE).permutation(N)]
        alpha_pos = alpha_all[positions]
    order = group_expert_major(expert_pos)
    pos = positions[order]
    expert = expert_pos[order].astype(np.int32)
    counts = np.bincount(expert, minlength=E).astype(np.int64)
    seg_off = np.zeros(E + 1, dtype=np.int64)
    np.cumsum(counts, out=seg_off[1:])
    return Routing(seg_off=seg_off, tok=(pos // K).astype(np.int32),
                   slot=(pos % K).astype(np.int32), alpha=alpha_pos[order].astype(np.float32),
                   expert=expert)


# ----------------------------------------------------------------------------- full problem

@dataclass
class Problem:
    cfg: Config
    rho: str
    routing: Routing
    quota: np.ndarray          # int32 [E]
    G: np.ndarray              # [T, D] upstream gradient (bf16 bits or f32)
    Phi: np.ndarray            # [N, F] saved FC2 input, expert-major
    X: np.ndarray | None       # [T, D] expert input (SwiGLU only)
    H: np.ndarray | None       # [N, 2F] saved FC1 output [gate | up] (SwiGLU only)
    W1: np.ndarray | None      # [E, D, 2F] FC1 weights, [in x out]
    W2: np.ndarray             # [E, F, D] FC2 weights, [in x out]

    @property
    def seg_off(self):
        return self.routing.seg_off


def swiglu_forward_phi(H_bits: np.ndarray, F: int) -> np.ndarray:
    """Saved FC2 input of a SwiGLU expert, phi = silu(gate) * up, stored as bf16.

    This is the *forward* activation that produces saved state; it is computed
    in float32 from the stored bf16 gate/up values, row chunk by row chunk."""
    rows = H_bits.shape[0]
    out = np.empty((rows, F), dtype=np.uint16)

    def work(c):
        r0, r1 = c * _CHUNK_ROWS, min(rows, (c + 1) * _CHUNK_ROWS)
        gate = bf16_bits_to_f32(H_bits[r0:r1, :F])
        up = bf16_bits_to_f32(H_bits[r0:r1, F:])
        phi = gate / (np.float32(1.0) + np.exp(-gate)) * up
        out[r0:r1] = f32_to_bf16_bits(phi)

    n = (rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(n)))
    return out


def make_problem(cfg: Config | str, rho: str | None = None, quota=None) -> Problem:
    """Draw every input of one invocation of the expert backward for ``cfg``."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rho = rho if rho is not None else cfg.rhos[0]
    r = make_routing(cfg)
    counts = np.diff(r.seg_off)
    q = np.asarray(quota, dtype=np.int32) if quota is not None else quotas(counts, rho)
    N, T, D, F, E = int(r.seg_off[-1]), cfg.T, cfg.D, cfg.F, cfg.E
    dt = cfg.dtype
    G = normal_rows(cfg.seed, TID_G, T, D, 1.0, dt)
    if cfg.swiglu:
        X = normal_rows(cfg.seed, TID_X, T, D, 1.0, dt)
        H = normal_rows(cfg.seed, TID_PAIR, N, 2 * F, 1.0, dt)
        if dt == "bf16":
            Phi = swiglu_forward_phi(H, F)
        else:
            gate, up = H[:, :F], H[:, F:]
            Phi = (gate / (np.float32(1.0) + np.exp(-gate)) * up).astype(np.float32)
        W1 = normal_rows(cfg.seed, TID_W1, E * D, 2 * F, 1.0 / math.sqrt(D), dt).reshape(E, D, 2 * F)
    else:
        X = H = W1 = None
        Phi = normal_rows(cfg.seed, TID_PAIR, N, F, 1.0, dt)
    W2 = normal_rows(cfg.seed, TID_W2, E * F, D, 1.0 / math.sqrt(F), dt).reshape(E, F, D)
    return Problem(cfg=cfg, rho=rho, routing=r, quota=q, G=G, Phi=Phi, X=X, H=H, W1=W1, W2=W2)
