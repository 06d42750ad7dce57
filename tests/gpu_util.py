"""Helpers for the GPU parity tests: stage generated inputs on the device, read
results back, and compare against the oracle."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import load_recalibrated_expert_amd as lr
import synth
from parity_ref import check_selection, on_gpu_selection, reference_selection  # noqa: F401

DEV = torch.device("cuda:0")


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a, dtype: str):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns; f32 tensor -> float32 array."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Staged:
    """A generated problem copied to the GPU, plus its lr.Problem."""

    def __init__(self, pr: synth.Problem):
        self.pr = pr
        c, r, dt = pr.cfg, pr.routing, pr.cfg.dtype
        self.dt = dt
        self.P = lr.Problem(E=c.E, T=c.T, K=c.K, D=c.D, F=c.F, swiglu=c.swiglu,
                            dtype=lr.BF16 if dt == "bf16" else lr.F32, seg_off=r.seg_off, quota=pr.quota,
                            device=DEV)
        self.G = to_dev(pr.G, dt)
        self.Phi = to_dev(pr.Phi, dt)
        self.W2 = to_dev(pr.W2, dt)
        self.X = to_dev(pr.X, dt) if pr.X is not None else None
        self.H = to_dev(pr.H, dt) if pr.H is not None else None
        self.W1 = to_dev(pr.W1, dt) if pr.W1 is not None else None
        self.alpha = torch.from_numpy(r.alpha).to(DEV)
        self.tok = torch.from_numpy(r.tok).to(DEV)
        self.slot = torch.from_numpy(r.slot).to(DEV)

    def backward(self, mode=lr.COMPACT_PHYSICAL, scatter_mode=lr.SCATTER_TOKEN, bufs=None, packed_dlt=False):
        return lr.backward(self.P, G=self.G, Phi=self.Phi, alpha=self.alpha, tok=self.tok, slot=self.slot,
                           W2=self.W2, X=self.X, H=self.H, W1=self.W1, mode=mode, scatter_mode=scatter_mode,
                           bufs=bufs, packed_dlt=packed_dlt)


def rel_fro(a, b) -> float:
    d = float(np.linalg.norm(b))
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b))) / (d if d > 0 else 1.0)
