"""Benchmark of the memory-aware MoE expert backward (LRMoE) on one MI355X.

One step = one pass of the whole path (score -> select -> compact -> grouped GEMM
backward -> scatter) over one layer invocation of the workload, inputs resident in
HBM. Prints ONE JSON line. Default workload: the Qwen3-30B-A3B-shaped single-GPU
expert share (32,768 tokens x top-8 = 262,144 pairs over 16 local experts, D=2048,
intermediate 768, retention 0.6, bf16 with fp32 accumulation), seeded synthetic data.
The line also carries an object timing the GLM4.5-106B-A12B-shaped share the same way
(GPU timing and roofline only), unless --second none.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "retained pairs/s through MoE expert backward; grouped-GEMM % of bf16 MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="qwen3_30b_a3b_share")
    ap.add_argument("--rho", default=None)
    ap.add_argument("--second", default="glm45_106b_a12b_share",
                    help="a second workload timed after the first (GPU timing and roofline only, no oracle), "
                         "reported as an object of its own; 'none' skips it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-masked", action="store_true")
    ap.add_argument("--serial-scatter", action="store_true",
                    help="run the scatter after the whole grouped GEMM call on the same stream, instead of on a "
                         "second stream beside the weight gradients as soon as the input gradients are complete")
    ap.add_argument("--packed", action="store_true",
                    help="compaction also packs the saved Phi and X rows (PhiC, XC) and the GEMMs read the "
                         "packed copies, instead of reading Phi and X in place through sel and ctok")
    ap.add_argument("--path", default="gathered", choices=["gathered", "packed_dlt"],
                    help="physical step 3-4 variant: 'gathered' (default) packs the weighted saved rows "
                         "PhiW = alpha Phi[sel] and the GEMMs read the gradient rows G[ctok] by token; "
                         "'packed_dlt' packs the weighted gradient rows Dlt instead")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="before timing, run 3 device-to-device copies of this many MiB (a plain copy kernel "
                         "of known size, used to scale hardware byte counters)")
    ap.add_argument("--cpu-sample-frac", type=float, default=1.0,
                    help="fraction of the pairs (smallest experts first) the oracle runs on")
    ap.add_argument("--forward", action="store_true",
                    help="also time the forward that saves the backward's context (FC1 + SwiGLU + FC2 over all "
                         "pairs, then the token combine); reported as an extra object, not the headline")
    ap.add_argument("--criterion", default="lrm", choices=["lrm", "grad_sqnorm", "grad_abs", "random"],
                    help="selection criterion: the LRM score (default) or an alternative of the ablation; "
                         "'random' selects on uniform draws made once on the host (no score kernel)")
    return ap.parse_args()


def to_dev(np_mod, torch, a, dtype, dev):
    a = np_mod.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np_mod.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def algorithmic_bytes(cfg, N, K_tot, packed=False, criterion="lrm", path="packed_dlt"):
    """Bytes each step reads once and writes once (storage dtype e; f32 scores/outputs)."""
    e = 2 if cfg.dtype == "bf16" else 4
    T, D, F = cfg.T, cfg.D, cfg.F
    if criterion == "lrm":
        score = (T * D + N * F) * e + N * (4 + 4 + 4)        # G, Phi, alpha, tok -> R
    elif criterion == "random":
        score = 0                                             # the draws are an input
    else:
        score = T * D * e + N * (4 + 4)                       # G, tok -> R
    # compact reads each token's G row once and writes every retained pair's Dlt row once;
    # packed, it also reads each token's X row and each retained pair's Phi row once and
    # writes their copies (the saved [gate | up] rows are always read in place by the GEMM)
    if path == "gathered":  # each retained pair's Phi row read once, its PhiW row written once
        compact = 2 * K_tot * F * e + K_tot * (4 + 4)
    elif not packed:
        compact = T * D * e + K_tot * D * e
    elif cfg.swiglu:
        compact = (2 * T * D + K_tot * F) * e + K_tot * (2 * D + F) * e
    else:
        compact = (T * D + K_tot * F) * e + K_tot * (D + F) * e
    width = D if cfg.swiglu else F
    scatter = K_tot * width * e + T * width * 4
    # selection: the scores, the pairs' tokens and slots read once; sel, keep, the packed rows'
    # tokens and slots and the [T x K] map written once
    select = N * (4 + 8) + N + K_tot * (4 + 8) + cfg.T * cfg.K * 4
    return {"score": score, "compact": compact, "scatter": scatter, "select": select}


def profile_key(cfg, rho):
    """Name of a workload's profiles: the config, plus the retention ratio when it is not the
    config's first one (the quota sweep's other ratios)."""
    return cfg.name if str(rho) == str(cfg.rhos[0]) else f"{cfg.name}_rho{rho}"


def recorded_traffic(workload):
    """HBM bytes per grouped-GEMM call recorded from rocprofv3 byte counters in profiles/,
    valid only while the GEMM source is the one the counters were taken on."""
    path = os.path.join(ROOT, "profiles", f"grouped_gemm_bwd_{workload}.md")
    src = os.path.join(ROOT, "load_recalibrated_expert_amd", "csrc", "gemm.hip")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"gemm_source_sha256:\s*([0-9a-f]{64})", text)
    m_tr = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not (m_sha and m_tr):
        return None
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    return int(m_tr.group(1)) if sha == m_sha.group(1) else None


def gemm_flops(cfg, rows):
    return (12 if cfg.swiglu else 4) * cfg.D * cfg.F * rows


def cpu_baseline(pr, frac):
    """The oracle, as it stands, on the smallest experts holding ~frac of the pairs."""
    import numpy as np
    import oracle
    import synth

    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        threads = 1
    r = pr.routing
    cfg = pr.cfg
    counts = np.diff(r.seg_off)
    order = np.argsort(counts, kind="stable")
    chosen, tot = [], 0
    for e in order:
        if tot >= frac * r.seg_off[-1]:
            break
        chosen.append(int(e))
        tot += int(counts[e])
    chosen.sort()
    idx = np.concatenate([np.arange(r.seg_off[e], r.seg_off[e + 1]) for e in chosen])
    seg = np.concatenate([[0], np.cumsum(counts[chosen])]).astype(np.int64)
    q = pr.quota[chosen]
    W1 = pr.W1[chosen] if pr.W1 is not None else None
    t0 = time.perf_counter()
    out = oracle.backward(G=pr.G, Phi=pr.Phi[idx], alpha=r.alpha[idx], tok=r.tok[idx], slot=r.slot[idx],
                          seg_off=seg, quota=q, dtype=cfg.dtype, T=cfg.T, W2=pr.W2[chosen],
                          X=pr.X, H=pr.H[idx] if pr.H is not None else None, W1=W1)
    dt = time.perf_counter() - t0
    kt = int(q.sum())
    return {"value": kt / dt, "unit": "pairs/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(chosen)} smallest of {cfg.E} experts: {tot} pairs, {kt} retained, full T={cfg.T} token "
                      f"rows; all five steps in fp64 ({dt:.1f} s)",
            "seconds": dt, "retained_pairs": kt, "experts": len(chosen), "_out": out}


def tiny_single_thread():
    """The oracle on the tiny fp32 configuration (388 retained pairs), on one thread: the
    best of five runs of all five steps."""
    import oracle
    import synth
    import threadpoolctl

    pr = synth.make_problem("tiny")
    r = pr.routing
    best = float("inf")
    with threadpoolctl.threadpool_limits(1):
        for _ in range(5):
            t0 = time.perf_counter()
            oracle.backward(G=pr.G, Phi=pr.Phi, alpha=r.alpha, tok=r.tok, slot=r.slot, seg_off=r.seg_off,
                            quota=pr.quota, dtype=pr.cfg.dtype, T=pr.cfg.T, W2=pr.W2)
            best = min(best, time.perf_counter() - t0)
    k = int(pr.quota.sum())
    return {"ms": best * 1e3, "value": k / best, "unit": "pairs/s", "cores": 1, "kind": "oracle",
            "sample": f"tiny config, all {k} retained pairs, best of 5"}


def parity(np, bufs, ref, pr, band=1e-5):
    """Agreement of the last timed step's outputs with the oracle run of the CPU baseline
    when that run covered the whole workload (same inputs), next to the bounds the parity
    tests hold them to. Pairs tied at an expert's threshold may be chosen differently (the
    LRMoE paper's Prop. 7.1): the selection must then differ only inside the band, and the
    later steps are compared with the oracle re-run on the GPU's selection."""
    import oracle

    def f64(t):
        return t.detach().double().cpu().numpy()

    def rel(a, b):
        d = float(np.linalg.norm(b))
        return float(np.linalg.norm(a - b)) / (d if d > 0 else 1.0)

    swiglu = pr.cfg.swiglu
    R = f64(bufs["R"])
    sel = bufs["sel"].cpu().numpy().astype(np.int64)
    identical = bool(np.array_equal(sel, ref["sel"]))
    in_band = identical
    if not identical and len(sel) == len(ref["sel"]) and bool(np.all(np.diff(sel) > 0)):
        diff = np.setxor1d(sel, ref["sel"])
        e_of = np.searchsorted(pr.routing.seg_off, diff, side="right") - 1
        tau = np.asarray(ref["tau"])[e_of]
        in_band = bool(np.all(np.abs(ref["R"][diff] - tau) <= band * tau))
    if not identical and in_band:  # steps 3-5 of the oracle on the GPU's choice
        r = pr.routing
        c = oracle.compact(sel, r.tok, r.slot, r.alpha, pr.G, pr.Phi, pr.cfg.dtype, X=pr.X, H=pr.H)
        ref = dict(ref)
        if swiglu:
            ref["dW1"], ref["dW2"], _, ref["dXC"] = oracle.swiglu_expert_backward(
                ref["cseg_off"], c["Dlt"], c["PhiC"], c["XC"], c["HC"], oracle.widen(pr.W1, pr.cfg.dtype),
                oracle.widen(pr.W2, pr.cfg.dtype))
            ref["out"] = oracle.scatter_tokens(ref["dXC"], c["ctok"], pr.cfg.T)
        else:
            ref["dW2"], ref["dPhi"] = oracle.linear_expert_backward(ref["cseg_off"], c["Dlt"], c["PhiC"],
                                                                    oracle.widen(pr.W2, pr.cfg.dtype))
            ref["out"] = oracle.scatter_tokens(ref["dPhi"], c["ctok"], pr.cfg.T)
    g = bufs["g"]
    dW = [rel(a, b) for a, b in zip(f64(g["dW2"]), ref["dW2"])]
    if swiglu:
        dW += [rel(a, b) for a, b in zip(f64(g["dW1"]), ref["dW1"])]
    return {
        "against": "the cpu_baseline oracle run (whole workload, same inputs)",
        "score_max_rel": float(np.max(np.abs(R - ref["R"]) / np.maximum(ref["R"], 1e-30))),
        "selection_identical": identical,
        "selection_within_tie_band": in_band,
        "later_steps_on": "oracle selection" if identical else "GPU selection (oracle re-run)",
        "weight_grad_max_rel_fro": max(dW),
        "input_grad_rel_fro": rel(f64(g["dIn"]), ref["dXC" if swiglu else "dPhi"]),
        "scatter_rel_fro": rel(f64(bufs["out"]), ref["out"]),
        "bounds": {"score_max_rel": 1e-6, "tie_band": band, "rel_fro": 5e-3},
    }


def main():
    args = parse()
    if args.packed:  # packing the saved rows is a variant of the packed-Dlt path
        args.path = "packed_dlt"
    if args.gpus != 1:
        print(f"bench.py measures one GPU's expert share; --gpus {args.gpus} is not supported "
              f"(it runs on one GPU; the expert-parallel sharding across GPUs is a design, not code here).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import load_recalibrated_expert_amd as lr
    import synth

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    rho = args.rho or cfg.rhos[0]
    def workload(cfg, rho):
        """Times one workload's step on the GPU; returns its measurements and the closures the
        optional extra timings reuse."""
        # bf16 rows: the token scatter runs beside the weight gradients (its kernel fits in the
        # registers they leave free); f32 rows do not fit there, and on the small f32 shapes the
        # second stream's synchronisation would cost more than it hides
        overlap = not args.serial_scatter and cfg.dtype == "bf16"
        t0 = time.time()
        pr = synth.make_problem(cfg, rho=rho)
        gen_s = time.time() - t0
        r = pr.routing
        dt = cfg.dtype
        P = lr.Problem(E=cfg.E, T=cfg.T, K=cfg.K, D=cfg.D, F=cfg.F, swiglu=cfg.swiglu,
                       dtype=lr.BF16 if dt == "bf16" else lr.F32, seg_off=r.seg_off, quota=pr.quota, device=dev)
        T_ = lambda a: to_dev(np, torch, a, dt, dev)  # noqa: E731
        ins = dict(G=T_(pr.G), Phi=T_(pr.Phi), W2=T_(pr.W2), X=T_(pr.X) if pr.X is not None else None,
                   H=T_(pr.H) if pr.H is not None else None, W1=T_(pr.W1) if pr.W1 is not None else None,
                   alpha=torch.from_numpy(r.alpha).to(dev), tok=torch.from_numpy(r.tok).to(dev),
                   slot=torch.from_numpy(r.slot).to(dev))
        print(f"# workload {cfg.name} rho={rho} N={P.N} K_tot={P.K_tot} generated in {gen_s:.1f}s", file=sys.stderr,
              flush=True)

        if args.copy_calib_mib > 0:
            n = args.copy_calib_mib << 20
            src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst

        def run(mode, bufs, timing=None):
            """One step; with `timing`, HIP events bracket each step's call on the stream it runs on
            (the scatter's on the second stream when it overlaps the weight gradients)."""
            G, Phi, alpha, tok, slot = ins["G"], ins["Phi"], ins["alpha"], ins["tok"], ins["slot"]
            main = torch.cuda.current_stream()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)] if timing is not None else None
            rec = (lambda i, s=None: ev[i].record(s if s is not None else main)) if ev else (lambda i, s=None: None)
            if overlap and "side" not in bufs:
                bufs["side"] = torch.cuda.Stream(device=dev)
                bufs["din_ready"] = torch.cuda.Event()
                bufs["side_ws"] = torch.empty_like(P.workspace())
                bufs["out"] = torch.empty(P.T, cfg.D if cfg.swiglu else cfg.F, dtype=torch.float32, device=dev)
            rec(0)
            if args.criterion == "random":  # uniform draws made once on the host: the scores are an input
                if "R" not in bufs:
                    bufs["R"] = torch.from_numpy(np.random.default_rng(cfg.seed).random(P.N).astype(np.float32)).to(dev)
                R = bufs["R"]
            else:
                crit_lrm = args.criterion == "lrm"
                R = lr.score(P, G, Phi if crit_lrm else None, alpha if crit_lrm else None, tok, R=bufs.get("R"),
                             criterion=args.criterion)
                bufs["R"] = R
            rec(1)
            phys = mode == lr.COMPACT_PHYSICAL
            maps = None
            if phys:  # the selection writes the (token, slot) map that compaction and the scatter use
                sel, keep, maps = lr.select(P, R, sel=bufs.get("sel"), keep=bufs.get("keep"), tok=tok, slot=slot,
                                            maps=bufs.get("maps"))
                bufs.setdefault("maps", maps)
            else:
                sel, keep = lr.select(P, R, sel=bufs.get("sel"), keep=bufs.get("keep"))
            bufs.setdefault("sel", sel)
            bufs.setdefault("keep", keep)
            rec(2)
            gathered = phys and args.path == "gathered"
            if gathered:  # weighted saved rows only; the GEMMs read G, X and H in place
                PhiW = lr.compact_weighted(P, sel, Phi, alpha, out=bufs.get("PhiW"))
                bufs.setdefault("PhiW", PhiW)
                c = {"ctok": maps["ctok"], "cslot": maps["cslot"]}
            else:
                c = lr.compact(P, G, Phi, alpha, tok, slot, sel=sel, keep=keep, X=ins["X"] if args.packed else None,
                               mode=mode, out=bufs.get("c"), pack_phi=args.packed, maps=maps)
                bufs.setdefault("c", c)
            rec(3)
            ctok, cslot = (c["ctok"], c["cslot"]) if phys else (tok, slot)
            hc_rows = sel if (phys and cfg.swiglu) else None
            if args.packed:
                PhiC, XC, phi_rows, x_rows = (c["PhiC"] if phys else Phi), c.get("XC"), None, None
            else:  # Phi and X read in place: pair rows through sel, token rows through ctok (tok)
                PhiC, XC = Phi, ins["X"]
                phi_rows = sel if phys else None
                x_rows = ctok if cfg.swiglu else None
            if gathered:
                g = lr.grouped_gemm_bwd_gathered(P, G, alpha, sel, ctok, PhiW, ins["W2"], X=ins["X"], H=ins["H"],
                                                 W1=ins["W1"], out=bufs.get("g"),
                                                 din_ready=bufs["din_ready"] if overlap else None)
            else:
                g = lr.grouped_gemm_bwd(P, c["Dlt"], PhiC, ins["W2"], XC=XC, HC=ins["H"], W1=ins["W1"], mode=mode,
                                        out=bufs.get("g"), hc_rows=hc_rows, phi_rows=phi_rows, x_rows=x_rows,
                                        din_ready=bufs["din_ready"] if overlap else None)
            bufs.setdefault("g", g)
            rec(4)
            bufs["scatter_args"] = (g["dIn"], ctok, cslot, P.rows(mode), maps["pmap"] if maps else None)
            if overlap:  # the scatter runs beside the weight gradients, on the second stream
                side = bufs["side"]
                side.wait_event(bufs["din_ready"])
                rec(6, side)
                lr.scatter(P, g["dIn"], ctok, cslot, n_rows=P.rows(mode), mode=lr.SCATTER_TOKEN_BESIDE,
                           out=bufs["out"], ws=bufs["side_ws"], pmap=maps["pmap"] if maps else None, stream=side)
                rec(7, side)
                main.wait_stream(side)
            else:
                out = lr.scatter(P, g["dIn"], ctok, cslot, n_rows=P.rows(mode), out=bufs.get("out"),
                                 pmap=maps["pmap"] if maps else None)
                bufs.setdefault("out", out)
            rec(5)
            if ev:
                timing.append(ev)

        def measure(mode):
            bufs = {}
            for _ in range(args.warmup):
                run(mode, bufs)
            torch.cuda.synchronize()
            t = time.perf_counter()
            for _ in range(args.steps):
                run(mode, bufs)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t
            # second pass: per-step HIP events (same stream as the launches)
            timing = []
            for _ in range(args.steps):
                run(mode, bufs, timing)
            torch.cuda.synchronize()
            names = ["score", "select", "compact", "grouped_gemm_bwd", "scatter"]
            per = {n: float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in timing])) for i, n in enumerate(names)}
            if overlap:
                per["scatter"] = float(np.mean([ev[6].elapsed_time(ev[7]) for ev in timing]))
            # whole step of the event pass, first to last event (includes the events' own cost)
            per["step_median"] = float(np.median([ev[0].elapsed_time(ev[5]) for ev in timing]))
            if overlap:  # the token scatter alone on the GPU, for its bandwidth (another kernel)
                dIn, ctok, cslot, n_rows, pmap = bufs["scatter_args"]
                bufs.setdefault("out_alone", torch.empty_like(bufs["out"]))
                sev = []
                for i in range(args.warmup + args.steps):
                    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                    e[0].record()
                    lr.scatter(P, dIn, ctok, cslot, n_rows=n_rows, out=bufs["out_alone"], ws=bufs["side_ws"],
                               pmap=pmap)
                    e[1].record()
                    if i >= args.warmup:
                        sev.append(e)
                torch.cuda.synchronize()
                per["scatter_alone"] = float(np.mean([e[0].elapsed_time(e[1]) for e in sev]))
            return wall, per, bufs

        wall, per, phys_bufs = measure(lr.COMPACT_PHYSICAL)
        bytes_ = algorithmic_bytes(cfg, P.N, P.K_tot, packed=args.packed, criterion=args.criterion, path=args.path)
        fl = gemm_flops(cfg, P.K_tot)
        peak = BF16_PEAK_TFLOPS if dt == "bf16" else FP32_PEAK_TFLOPS
        gemm_tf = fl / (per["grouped_gemm_bwd"] * 1e-3) / 1e12
        kernels = {
            "score": ({"ms": per["score"], "GB/s": bytes_["score"] / per["score"] / 1e6,
                       "hbm_frac": bytes_["score"] / per["score"] / 1e6 / HBM_PEAK_GBS} if bytes_["score"] else
                      {"ms": per["score"], "note": "no score kernel: uniform draws made once on the host"}),
            "select": {"ms": per["select"], "GB/s": bytes_["select"] / per["select"] / 1e6,
                       "note": "latency-bound (six launches); bytes for information"},
            "compact": {"ms": per["compact"], "GB/s": bytes_["compact"] / per["compact"] / 1e6,
                        "hbm_frac": bytes_["compact"] / per["compact"] / 1e6 / HBM_PEAK_GBS},
            "grouped_gemm_bwd": {"ms": per["grouped_gemm_bwd"], "TFLOP/s": gemm_tf, "mfma_frac": gemm_tf / peak},
            "scatter": {"ms": per["scatter"], "GB/s": bytes_["scatter"] / per["scatter"] / 1e6,
                        "hbm_frac": bytes_["scatter"] / per["scatter"] / 1e6 / HBM_PEAK_GBS},
        }
        if overlap:
            sa = per["scatter_alone"]
            kernels["scatter"] = {
                "ms": sa, "GB/s": bytes_["scatter"] / sa / 1e6, "hbm_frac": bytes_["scatter"] / sa / 1e6 / HBM_PEAK_GBS,
                "beside_ms": per["scatter"],
                "note": "ms, GB/s: the token scatter alone on the GPU (token_reduce_kernel); in the step it runs "
                        "on a second stream beside the weight gradients (token_reduce_beside_kernel), from the "
                        "input gradients' completion to its end in beside_ms"}
        return dict(pr=pr, P=P, ins=ins, measure=measure, wall=wall, per=per, phys_bufs=phys_bufs,
                    kernels=kernels, gemm_tf=gemm_tf, fl=fl, peak=peak, gen_s=gen_s, overlap=overlap)

    W = workload(cfg, rho)
    pr, P, ins, measure, wall, per, phys_bufs = (W[k] for k in ("pr", "P", "ins", "measure", "wall", "per",
                                                                 "phys_bufs"))
    kernels, gemm_tf, fl, peak = W["kernels"], W["gemm_tf"], W["fl"], W["peak"]
    ms = wall / args.steps * 1e3
    value = P.K_tot * args.steps / wall
    dt = cfg.dtype
    result = {
        "metric": METRIC, "value": value, "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "ms_per_step_median": per["step_median"],
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dt, "data": "synthetic (seeded; pages' shapes, no dataset)",
        "config": {"workload": cfg.name, "T": cfg.T, "top_k": cfg.K, "local_experts": cfg.E, "D": cfg.D,
                   "F": cfg.F, "swiglu": cfg.swiglu, "rho": rho, "pairs": P.N, "retained_pairs": P.K_tot,
                   "mode": "physical compaction", "path": args.path, "criterion": args.criterion,
                   "scatter": "second stream, beside the weight gradients" if W["overlap"] else "after the GEMM call"},
        "roofline": {"bound": "mfma", "achieved": gemm_tf, "peak": peak, "unit": "TFLOP/s",
                     "frac": gemm_tf / peak, "traffic": recorded_traffic(profile_key(cfg, rho)),
                     "kernel": "lrmoe_grouped_gemm_bwd (FC2 dgrad+SwiGLU, FC1 dgrad, FC1+FC2 wgrad launches)",
                     "flops_per_launch": fl},
        "kernels": kernels,
    }
    if not args.no_masked:
        mwall, mper, _ = measure(lr.COMPACT_ZERO_MASKED)
        mfl = gemm_flops(cfg, P.N)
        e_ = 2 if dt == "bf16" else 4
        w_ = cfg.D if cfg.swiglu else cfg.F
        # what each backward holds besides its inputs: the compact run's is the library's own
        # estimate; the masked run keeps N rows of Dlt, dH and dIn and its own workspace
        masked_hold = (5 * P.N + P.N * cfg.D * e_ + (P.N * 2 * cfg.F * e_ if cfg.swiglu else 0) + P.N * w_ * e_
                       + 4 * cfg.E * cfg.F * cfg.D + (4 * cfg.E * cfg.D * 2 * cfg.F if cfg.swiglu else 0)
                       + 4 * cfg.T * w_ + P.workspace_size(lr.COMPACT_ZERO_MASKED))
        result["masked_baseline"] = {
            "ms_per_step": mwall / args.steps * 1e3, "retained_pairs_per_s": P.K_tot * args.steps / mwall,
            "grouped_gemm_ms": mper["grouped_gemm_bwd"], "gemm_rows": P.N, "compact_rows": P.K_tot,
            "gemm_flops": mfl, "speedup_of_compaction": (mwall / args.steps * 1e3) / ms,
            "compact_ms": mper["compact"], "compact_bytes": cfg.T * cfg.D * e_ + P.N * cfg.D * e_,
            "backward_bytes": masked_hold, "backward_bytes_compact": lr.backward_bytes(P),
        }
    if args.forward and cfg.swiglu and dt == "bf16":
        fo, fev = {}, []
        def fwd_step(timing=None):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if timing is not None else None
            if ev:
                ev[0].record()
            f = lr.expert_forward(P, ins["X"], ins["tok"], ins["alpha"], ins["W1"], ins["W2"], out=fo)
            fo.update(f)
            if ev:
                ev[1].record()
            fo["y"] = lr.scatter(P, f["Y"], ins["tok"], ins["slot"], n_rows=P.N, out=fo.get("y"))
            if ev:
                ev[2].record()
                timing.append(ev)
        for _ in range(args.warmup):
            fwd_step()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            fwd_step()
        torch.cuda.synchronize()
        fwall = time.perf_counter() - t
        for _ in range(args.steps):
            fwd_step(fev)
        torch.cuda.synchronize()
        gemm_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in fev]))
        comb_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in fev]))
        ffl = 6.0 * P.N * cfg.D * cfg.F  # FC1 2*N*D*2F + FC2 2*N*F*D
        result["forward"] = {
            "ms_per_step": fwall / args.steps * 1e3, "pairs_per_s": P.N * args.steps / fwall,
            "expert_forward_ms": gemm_ms, "TFLOP/s": ffl / (gemm_ms * 1e-3) / 1e12,
            "mfma_frac": ffl / (gemm_ms * 1e-3) / 1e12 / peak, "flops": ffl, "combine_ms": comb_ms,
            "note": "FC1 with the SwiGLU forward fused, FC2 scaled by the routing weight, over all N pairs; "
                    "then the token combine (scatter)",
        }
    if args.second != "none" and args.second != cfg.name:
        # the pages' second model shape, GPU timing only (no oracle run at this size)
        c2 = synth.CONFIGS[args.second]
        W2_ = workload(c2, c2.rhos[0])
        P2 = W2_["P"]
        result[args.second] = {
            "workload": c2.name, "rho": c2.rhos[0], "pairs": P2.N, "retained_pairs": P2.K_tot,
            "steps": args.steps, "ms_per_step": W2_["wall"] / args.steps * 1e3,
            "value": P2.K_tot * args.steps / W2_["wall"], "unit": "pairs/s",
            "roofline": {"bound": "mfma", "achieved": W2_["gemm_tf"], "peak": W2_["peak"], "unit": "TFLOP/s",
                         "frac": W2_["gemm_tf"] / W2_["peak"],
                         "traffic": recorded_traffic(profile_key(c2, c2.rhos[0])),
                         "flops_per_launch": W2_["fl"]},
            "kernels": W2_["kernels"],
        }
        del W2_, P2
    if not args.no_cpu_baseline and args.criterion == "lrm":  # the oracle's backward scores with LRM
        cb = cpu_baseline(pr, args.cpu_sample_frac)
        ref = cb.pop("_out", None)
        result["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        if cb["experts"] == cfg.E:
            result["parity"] = parity(np, phys_bufs, ref, pr)
        result["cpu_baseline_tiny_one_thread"] = tiny_single_thread()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
