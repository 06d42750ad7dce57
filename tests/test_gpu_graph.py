"""One whole backward step (score, select, compact, grouped GEMMs, scatter) captured into a
HIP graph: every replay equals the eager step bit for bit, with eager steps and host
synchronisations between the replays. The path records no memset nodes: every buffer it
clears is cleared by a kernel."""
import pytest
import torch

import load_recalibrated_expert_amd as lr
import synth

pytestmark = pytest.mark.gpu

from gpu_util import Staged, log  # noqa: E402


@pytest.mark.parametrize("name,rho", [("graph_swiglu", "0.6"), ("graph_linear", "0.5")])
def test_backward_step_replays_in_a_graph(name, rho):
    sw = name == "graph_swiglu"
    cfg = synth.custom(name, T=500, K=4, E=5, D=256, F=384 if sw else 264, counts=(600, 0, 513, 300, 257),
                       swiglu=sw, seed=41)
    pr = synth.make_problem(cfg, rho=rho)
    s = Staged(pr)
    bufs = {}

    def step():
        return lr.backward(s.P, G=s.G, Phi=s.Phi, alpha=s.alpha, tok=s.tok, slot=s.slot, W2=s.W2, X=s.X, H=s.H,
                           W1=s.W1, bufs=bufs)

    keys = ("R", "sel", "PhiW", "dW2", "dIn", "out") + (("dW1", "dH") if sw else ())
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for _ in range(3):  # first calls allocate every buffer; capture needs them in place
            res = step()
        torch.cuda.synchronize()
        ref = {k: res[k].clone() for k in keys}
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            gres = step()
    torch.cuda.synchronize()
    for rep in range(3):
        for k in keys:  # clobber the outputs so a replay that skips work cannot pass
            gres[k].zero_() if gres[k].is_floating_point() else gres[k].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(gres[k], ref[k]), (name, rep, k)
        log(f"{name}: replay {rep} equals the eager step")
        with torch.cuda.stream(side):
            step()  # eager work between replays
        torch.cuda.synchronize()
