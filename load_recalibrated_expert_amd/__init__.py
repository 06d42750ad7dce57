"""Memory-aware MoE expert backward (LRMoE) on MI355X: Python binding of liblrmoe.

The five steps of the LRMoE paper's backward-time calibration (Algorithm 1,
section 3.3) are calls into ``liblrmoe.so`` (hand-written HIP for gfx950):

    score -> select -> compact_weighted -> grouped_gemm_bwd_gathered -> scatter

(or, packing the weighted gradient rows instead, compact -> grouped_gemm_bwd).

The functions here have the C entry points' names and only marshal arguments:
torch tensors supply device memory and the current HIP stream. ``backward`` chains
the five calls. Nothing falls back to another implementation; if the library is
not built, the first call raises ImportError.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import (BF16, COMPACT_PHYSICAL, COMPACT_ZERO_MASKED, F32, SCATTER_SLOT, SCATTER_TOKEN,
                   SCATTER_TOKEN_BESIDE,
                   InfeasibleQuotaError, LrmoeError)

__all__ = ["Problem", "score", "select", "select_noalloc", "compact", "compact_weighted", "grouped_gemm_bwd",
           "grouped_gemm_bwd_gathered", "expert_forward", "scatter", "backward", "backward_bytes", "plan_quotas",
           "library", "BF16", "F32", "COMPACT_PHYSICAL", "COMPACT_ZERO_MASKED", "SCATTER_TOKEN",
           "SCATTER_SLOT", "SCATTER_TOKEN_BESIDE", "LrmoeError", "InfeasibleQuotaError"]


def library() -> ctypes.CDLL:
    return _lib.load()


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to liblrmoe must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _event(ev, stream=None):
    """Raw handle of a torch.cuda.Event (None -> NULL). torch creates the HIP event on its
    first record, so an event never recorded is recorded once here, on `stream`."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record(stream if stream is not None else torch.cuda.current_stream())
    return ev.cuda_event


class Problem:
    """Shapes, pair segments and quotas of one layer invocation (host + device copies).

    seg_off: int64 [E+1] pair offsets per expert (pairs stored expert-major);
    quota: int32 [E] retention quotas, fixed before the call."""

    def __init__(self, *, E, T, K, D, F, swiglu, dtype, seg_off, quota, device="cuda"):
        lib = library()
        self.E, self.T, self.K, self.D, self.F = int(E), int(T), int(K), int(D), int(F)
        self.swiglu, self.dtype = bool(swiglu), int(dtype)
        self.c, self._keep = _lib.make_problem_struct(self.E, self.T, self.K, self.D, self.F, self.swiglu,
                                                      self.dtype, seg_off, quota)
        k_tot = ctypes.c_int64(0)
        cseg = np.zeros(self.E + 1, dtype=np.int64)
        _lib.check(lib.lrmoe_validate(ctypes.byref(self.c), ctypes.byref(k_tot),
                                      cseg.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))), "lrmoe_validate")
        self.N = int(self._keep[0][-1])
        self.K_tot = int(k_tot.value)
        self.seg_off = self._keep[0]
        self.quota = self._keep[1]
        self.cseg_off = cseg
        self.device = torch.device(device)
        self.seg_off_d = torch.from_numpy(self.seg_off).to(self.device)
        self.quota_d = torch.from_numpy(self.quota).to(self.device)
        self.cseg_off_d = torch.from_numpy(self.cseg_off).to(self.device)
        self._ws = None
        self._ws_size = {}

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == BF16 else torch.float32

    def workspace_size(self, mode=COMPACT_PHYSICAL) -> int:
        """lrmoe_workspace_size, asked once per mode (the quotas are fixed for the problem)."""
        if mode not in self._ws_size:
            n = ctypes.c_size_t(0)
            _lib.check(library().lrmoe_workspace_size(ctypes.byref(self.c), mode, ctypes.byref(n)),
                       "lrmoe_workspace_size")
            self._ws_size[mode] = int(n.value)
        return self._ws_size[mode]

    def workspace(self, mode=COMPACT_PHYSICAL) -> torch.Tensor:
        """The problem's scratch buffer, large enough for every call in ``mode`` (it grows
        once when a zero-masked call needs more than the physical ones)."""
        n = self.workspace_size(mode)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self._ws

    def rows(self, mode=COMPACT_PHYSICAL) -> int:
        return self.K_tot if mode == COMPACT_PHYSICAL else self.N

    def row_off_d(self, mode=COMPACT_PHYSICAL):
        return self.cseg_off_d if mode == COMPACT_PHYSICAL else self.seg_off_d


def backward_bytes(p: Problem, packed=False) -> int:
    """Device bytes one physical-compaction backward holds at p's quotas besides its
    inputs: its buffers and its workspace (host-only; the list is in the header,
    lrmoe_backward_bytes)."""
    n = ctypes.c_size_t(0)
    _lib.check(library().lrmoe_backward_bytes(ctypes.byref(p.c), int(bool(packed)), ctypes.byref(n)),
               "lrmoe_backward_bytes")
    return int(n.value)


def plan_quotas(E, T, K, D, F, swiglu, dtype, seg_off, rhos, hbm_avail, packed=False):
    """Quota admission on one GPU (host-only): the largest candidate ratio in ``rhos``
    (exact decimals such as "0.6", or Fractions) whose backward (buffers and workspace)
    fits ``hbm_avail`` bytes. Returns (index into rhos, quotas [E] int32, bytes); raises InfeasibleQuotaError
    when none fits (Algorithm 1's "return Infeasible")."""
    from fractions import Fraction
    fr = [Fraction(r) for r in rhos]
    num = np.array([f.numerator for f in fr], dtype=np.int32)
    den = np.array([f.denominator for f in fr], dtype=np.int32)
    c, keep = _lib.make_problem_struct(E, T, K, D, F, swiglu, dtype, seg_off, np.zeros(E, dtype=np.int32))
    chosen, nb = ctypes.c_int32(-1), ctypes.c_size_t(0)
    q = np.zeros(E, dtype=np.int32)
    I32 = ctypes.POINTER(ctypes.c_int32)
    _lib.check(library().lrmoe_plan_quotas(ctypes.byref(c), num.ctypes.data_as(I32), den.ctypes.data_as(I32),
                                           len(fr), int(bool(packed)), int(hbm_avail), ctypes.byref(chosen),
                                           q.ctypes.data_as(I32), ctypes.byref(nb)), "lrmoe_plan_quotas")
    return int(chosen.value), q, int(nb.value)


CRITERIA = {"lrm": 0, "grad_sqnorm": 1, "grad_abs": 2}


def score(p: Problem, G, Phi, alpha, tok, R=None, criterion="lrm", stream=None):
    """Step 1. ``criterion``: "lrm" (the LRM score), or the gradient-only criteria of the
    ablation, "grad_sqnorm" / "grad_abs" (Phi and alpha may then be None)."""
    R = R if R is not None else torch.empty(p.N, dtype=torch.float32, device=p.device)
    ws = p.workspace()
    if criterion == "lrm":
        _lib.check(library().lrmoe_score(ctypes.byref(p.c), _ptr(G), _ptr(Phi), _ptr(alpha), _ptr(tok), _ptr(R),
                                         _ptr(ws), ws.numel(), _stream(stream)), "lrmoe_score")
    else:
        if criterion not in CRITERIA:
            raise ValueError(f"unknown criterion {criterion!r}; expected one of {sorted(CRITERIA)}")
        _lib.check(library().lrmoe_score_criterion(ctypes.byref(p.c), CRITERIA[criterion], _ptr(G), _ptr(Phi),
                                                   _ptr(alpha), _ptr(tok), _ptr(R), _ptr(ws), ws.numel(),
                                                   _stream(stream)), "lrmoe_score_criterion")
    return R


def select(p: Problem, R, sel=None, keep=None, want_keep=True, tok=None, slot=None, maps=None, stream=None):
    """Step 2. Returns (sel, keep). With the pairs' ``tok`` and ``slot`` it also writes the
    (token, slot) -> packed row map and the packed rows' tokens and slots, and returns
    (sel, keep, maps) with maps = {"pmap", "ctok", "cslot"} (``maps`` reuses buffers)."""
    sel = sel if sel is not None else torch.empty(max(p.K_tot, 1), dtype=torch.int32, device=p.device)
    if keep is None and want_keep:
        keep = torch.empty(max(p.N, 1), dtype=torch.uint8, device=p.device)
    m = None
    if tok is not None:
        m = dict(maps or {})
        m.setdefault("pmap", torch.empty(max(p.T * p.K, 1), dtype=torch.int32, device=p.device))
        m.setdefault("ctok", torch.empty(max(p.K_tot, 1), dtype=torch.int32, device=p.device))
        m.setdefault("cslot", torch.empty(max(p.K_tot, 1), dtype=torch.int32, device=p.device))
    ws = p.workspace()
    _lib.check(library().lrmoe_select(ctypes.byref(p.c), _ptr(R), _ptr(p.seg_off_d), _ptr(p.quota_d),
                                      _ptr(p.cseg_off_d), _ptr(sel), _ptr(keep), _ptr(tok), _ptr(slot),
                                      _ptr(m["pmap"]) if m else None, _ptr(m["ctok"]) if m else None,
                                      _ptr(m["cslot"]) if m else None, _ptr(ws), ws.numel(), _stream(stream)),
               "lrmoe_select")
    out = (sel[:p.K_tot], (keep[:p.N] if keep is not None else None))
    if m is None:
        return out
    return out + ({"pmap": m["pmap"][:p.T * p.K], "ctok": m["ctok"][:p.K_tot], "cslot": m["cslot"][:p.K_tot]},)


def select_noalloc(p: Problem, R, sel, keep=None, tok=None, slot=None, maps=None, stream=None):
    """lrmoe_select_noalloc: step 2 with the library's fixed per-GPU scratch instead of a
    workspace, for callers that cannot allocate. The caller passes every output (``sel``
    [K_tot], optional ``keep`` [N]; with ``tok``/``slot`` also ``maps`` = {"pmap", "ctok",
    "cslot"}); nothing is allocated here."""
    m = maps if tok is not None else None
    _lib.check(library().lrmoe_select_noalloc(ctypes.byref(p.c), _ptr(R), _ptr(p.seg_off_d), _ptr(p.quota_d),
                                              _ptr(p.cseg_off_d), _ptr(sel), _ptr(keep), _ptr(tok), _ptr(slot),
                                              _ptr(m["pmap"]) if m else None, _ptr(m["ctok"]) if m else None,
                                              _ptr(m["cslot"]) if m else None, _stream(stream)),
               "lrmoe_select_noalloc")
    return sel, keep, m


def compact(p: Problem, G, Phi, alpha, tok, slot, sel=None, keep=None, X=None, H=None,
            mode=COMPACT_PHYSICAL, out=None, pack_phi=True, maps=None, stream=None):
    """Always writes Dlt; ctok/cslot too unless ``maps`` (the map, ctok and cslot that
    select wrote for this sel) is given, in which case they are returned as given and the
    gather runs through that map. The saved rows are packed only on request: PhiC when
    ``pack_phi`` (physical mode), XC when X is given, HC when H is given (physical mode).
    The grouped GEMM can read each of them in place instead, through its row maps (sel for
    Phi and H, ctok or tok for X)."""
    rows = p.rows(mode)
    dt = p.torch_dtype
    o = dict(out or {})
    dev = p.device
    o.setdefault("Dlt", torch.empty(max(rows, 1), p.D, dtype=dt, device=dev))
    if mode == COMPACT_PHYSICAL:
        if pack_phi:
            o.setdefault("PhiC", torch.empty(max(rows, 1), p.F, dtype=dt, device=dev))
        if p.swiglu and H is not None:
            o.setdefault("HC", torch.empty(max(rows, 1), 2 * p.F, dtype=dt, device=dev))
    if p.swiglu and X is not None:
        o.setdefault("XC", torch.empty(max(rows, 1), p.D, dtype=dt, device=dev))
    pmap = None
    if maps is not None:
        o["ctok"], o["cslot"], pmap = maps["ctok"], maps["cslot"], maps["pmap"]
    else:
        o.setdefault("ctok", torch.empty(max(rows, 1), dtype=torch.int32, device=dev))
        o.setdefault("cslot", torch.empty(max(rows, 1), dtype=torch.int32, device=dev))
    ws = p.workspace()
    _lib.check(library().lrmoe_compact(
        ctypes.byref(p.c), mode, _ptr(sel), _ptr(keep), _ptr(G), _ptr(Phi), _ptr(X), _ptr(H), _ptr(alpha),
        _ptr(tok), _ptr(slot), _ptr(o["Dlt"]), _ptr(o.get("PhiC")), _ptr(o.get("XC")), _ptr(o.get("HC")),
        _ptr(o["ctok"]), _ptr(o["cslot"]), _ptr(pmap), _ptr(ws), ws.numel(), _stream(stream)), "lrmoe_compact")
    return {k: v[:rows] for k, v in o.items()}


def grouped_gemm_bwd(p: Problem, Dlt, PhiC, W2, XC=None, HC=None, W1=None, mode=COMPACT_PHYSICAL,
                     out=None, accumulate=False, hc_rows=None, phi_rows=None, x_rows=None, din_ready=None,
                     stream=None):
    """``PhiC``, ``XC`` and ``HC`` are packed rows, or the saved matrices themselves (Phi,
    X, H) with a row map giving, for each packed row, the row to read: ``phi_rows`` and
    ``hc_rows`` index pair rows (e.g. ``sel``), ``x_rows`` token rows (``ctok``, or ``tok``
    in zero-masked mode). ``din_ready`` (a torch.cuda.Event) is recorded on the stream as
    soon as dIn is complete, before the weight-gradient launches."""
    rows = p.rows(mode)
    dt = p.torch_dtype
    dev = p.device
    o = dict(out or {})
    o.setdefault("dW2", torch.empty(p.E, p.F, p.D, dtype=torch.float32, device=dev))
    if p.swiglu:
        o.setdefault("dW1", torch.empty(p.E, p.D, 2 * p.F, dtype=torch.float32, device=dev))
        o.setdefault("dH", torch.empty(max(rows, 1), 2 * p.F, dtype=dt, device=dev))
        o.setdefault("dIn", torch.empty(max(rows, 1), p.D, dtype=dt, device=dev))
    else:
        o.setdefault("dIn", torch.empty(max(rows, 1), p.F, dtype=dt, device=dev))
    ws = p.workspace(mode)
    _lib.check(library().lrmoe_grouped_gemm_bwd(
        ctypes.byref(p.c), mode, _ptr(p.row_off_d(mode)), _ptr(Dlt), _ptr(PhiC), _ptr(XC), _ptr(HC), _ptr(hc_rows),
        _ptr(phi_rows), _ptr(x_rows), _ptr(W2),
        _ptr(W1), _ptr(o["dW2"]), _ptr(o.get("dW1")), _ptr(o.get("dH")), _ptr(o["dIn"]), int(bool(accumulate)),
        _ptr(ws), ws.numel(), _stream(stream), _event(din_ready, stream)), "lrmoe_grouped_gemm_bwd")
    res = dict(o)
    res["dIn"] = o["dIn"][:rows]
    if "dH" in o:
        res["dH"] = o["dH"][:rows]
    return res


def compact_weighted(p: Problem, sel, Phi, alpha, out=None, stream=None):
    """Step 3 for the path that reads gradient rows by token: PhiW[c] = alpha[sel[c]] *
    Phi[sel[c]] over the K_tot packed rows (lrmoe_compact_weighted)."""
    PhiW = out if out is not None else torch.empty(max(p.K_tot, 1), p.F, dtype=p.torch_dtype, device=p.device)
    _lib.check(library().lrmoe_compact_weighted(ctypes.byref(p.c), _ptr(sel), _ptr(Phi), _ptr(alpha), _ptr(PhiW),
                                                _stream(stream)), "lrmoe_compact_weighted")
    return PhiW[:p.K_tot]


def grouped_gemm_bwd_gathered(p: Problem, G, alpha, sel, ctok, PhiW, W2, X=None, H=None, W1=None, out=None,
                              accumulate=False, din_ready=None, stream=None):
    """Step 4 without a packed Dlt (lrmoe_grouped_gemm_bwd_gathered): gradient rows G[ctok]
    and X[ctok] read by token, H[sel] and alpha[sel] by pair, PhiW from compact_weighted.
    Same outputs as grouped_gemm_bwd in physical mode."""
    rows = p.K_tot
    dt = p.torch_dtype
    dev = p.device
    o = dict(out or {})
    o.setdefault("dW2", torch.empty(p.E, p.F, p.D, dtype=torch.float32, device=dev))
    if p.swiglu:
        o.setdefault("dW1", torch.empty(p.E, p.D, 2 * p.F, dtype=torch.float32, device=dev))
        o.setdefault("dH", torch.empty(max(rows, 1), 2 * p.F, dtype=dt, device=dev))
        o.setdefault("dIn", torch.empty(max(rows, 1), p.D, dtype=dt, device=dev))
    else:
        o.setdefault("dIn", torch.empty(max(rows, 1), p.F, dtype=dt, device=dev))
    ws = p.workspace(COMPACT_PHYSICAL)
    _lib.check(library().lrmoe_grouped_gemm_bwd_gathered(
        ctypes.byref(p.c), _ptr(p.cseg_off_d), _ptr(G), _ptr(alpha), _ptr(sel), _ptr(ctok), _ptr(PhiW), _ptr(X),
        _ptr(H), _ptr(W2), _ptr(W1), _ptr(o["dW2"]), _ptr(o.get("dW1")), _ptr(o.get("dH")), _ptr(o["dIn"]),
        int(bool(accumulate)), _ptr(ws), ws.numel(), _stream(stream), _event(din_ready, stream)),
        "lrmoe_grouped_gemm_bwd_gathered")
    res = dict(o)
    res["dIn"] = o["dIn"][:rows]
    if "dH" in o:
        res["dH"] = o["dH"][:rows]
    return res


def expert_forward(p: Problem, X, tok, alpha, W1, W2, out=None, stream=None):
    """The forward that saves the backward's context: H = X[tok] W1 ([gate | up]),
    Phi = silu(gate) * up, Y = alpha * Phi W2 (rows of the N pairs, expert-major).
    The layer output is ``scatter(p, Y, tok, slot, n_rows=p.N)``."""
    dt = torch.bfloat16
    o = out or {}
    H = o.get("H") if o.get("H") is not None else torch.empty(max(p.N, 1), 2 * p.F, dtype=dt, device=p.device)
    Phi = o.get("Phi") if o.get("Phi") is not None else torch.empty(max(p.N, 1), p.F, dtype=dt, device=p.device)
    Y = o.get("Y") if o.get("Y") is not None else torch.empty(max(p.N, 1), p.D, dtype=dt, device=p.device)
    _lib.check(library().lrmoe_expert_forward(ctypes.byref(p.c), _ptr(p.seg_off_d), _ptr(X), _ptr(tok), _ptr(alpha),
                                              _ptr(W1), _ptr(W2), _ptr(H), _ptr(Phi), _ptr(Y), _stream(stream)),
               "lrmoe_expert_forward")
    return {"H": H[:p.N], "Phi": Phi[:p.N], "Y": Y[:p.N]}


def scatter(p: Problem, rows_t, ctok, cslot, n_rows=None, mode=SCATTER_TOKEN, out=None, ws=None, pmap=None,
            stream=None):
    """``pmap``: the (token, slot) map select wrote for these packed rows (then no workspace
    is used). Without it the map is built in ``ws``, which defaults to the problem's
    workspace; a scatter running concurrently with another call of the same problem (on
    another stream) then needs its own."""
    n_rows = rows_t.shape[0] if n_rows is None else n_rows
    width = rows_t.shape[1]
    rdt = BF16 if rows_t.dtype == torch.bfloat16 else F32
    if out is None:
        nout = p.T if mode in (SCATTER_TOKEN, SCATTER_TOKEN_BESIDE) else p.T * p.K
        out = torch.empty(max(nout, 1), width, dtype=torch.float32, device=p.device)
    if pmap is None:
        ws = p.workspace() if ws is None else ws
    _lib.check(library().lrmoe_scatter(ctypes.byref(p.c), mode, n_rows, width, rdt, _ptr(rows_t), _ptr(ctok),
                                       _ptr(cslot), _ptr(pmap), _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(stream)), "lrmoe_scatter")
    return out


def backward(p: Problem, *, G, Phi, alpha, tok, slot, W2, X=None, H=None, W1=None, mode=COMPACT_PHYSICAL,
             scatter_mode=SCATTER_TOKEN, bufs=None, overlap_scatter=False, packed_dlt=False, stream=None):
    """The whole path: score -> select -> compact -> grouped GEMMs -> scatter.

    Physical compaction packs only the weighted saved rows PhiW = alpha Phi[sel] and the
    grouped GEMMs read the gradient rows G[ctok], the FC1 inputs X[ctok] and the saved
    [gate | up] rows H[sel] in place (compact_weighted, grouped_gemm_bwd_gathered). With
    ``packed_dlt`` (and always in zero-masked mode) compaction packs the weighted gradient
    rows Dlt instead and grouped_gemm_bwd reads them.

    ``bufs`` (a dict, optional) carries preallocated outputs between calls; it is
    filled on first use. With ``overlap_scatter`` the scatter runs on a second stream as
    soon as the input gradients are complete, while the weight gradients are computed
    (with a workspace of its own when it builds its map); the calling stream waits for it
    before returning. A token-order scatter then uses SCATTER_TOKEN_BESIDE, whose blocks
    share the compute units the weight-gradient launch occupies (same results, bit for
    bit). Returns a dict of every intermediate and output."""
    b = bufs if bufs is not None else {}
    main = stream if stream is not None else torch.cuda.current_stream()
    b["R"] = score(p, G, Phi, alpha, tok, R=b.get("R"), stream=stream)
    phys = mode == COMPACT_PHYSICAL
    maps = None
    if phys:  # the selection also writes the (token, slot) map that compaction and the scatter use
        sel, keep, maps = select(p, b["R"], sel=b.get("sel_full"), keep=b.get("keep_full"), tok=tok, slot=slot,
                                 maps=b.get("maps"), stream=stream)
        b.setdefault("maps", maps)
    else:
        sel, keep = select(p, b["R"], sel=b.get("sel_full"), keep=b.get("keep_full"), stream=stream)
    b.setdefault("sel_full", sel)
    b.setdefault("keep_full", keep)
    gathered = phys and not packed_dlt
    if gathered:  # the weighted saved rows only; G, X and H are read in place
        PhiW = compact_weighted(p, sel, Phi, alpha, out=b.get("PhiW"), stream=stream)
        b.setdefault("PhiW", PhiW)
        c = {"PhiW": PhiW, "ctok": maps["ctok"], "cslot": maps["cslot"]}
    else:  # the weighted gradient rows; the GEMMs read Phi, X and H in place through sel and ctok
        c = compact(p, G, Phi, alpha, tok, slot, sel=sel, keep=keep, mode=mode, out=b.get("compact"),
                    pack_phi=False, maps=maps, stream=stream)
        b.setdefault("compact", c)
    if mode == COMPACT_PHYSICAL:
        ctok, cslot = c["ctok"], c["cslot"]
        phi_rows = sel
        hc_rows = sel if p.swiglu else None
        x_rows = ctok if p.swiglu else None
    else:
        ctok, cslot = tok, slot
        phi_rows = hc_rows = None
        x_rows = tok if p.swiglu else None
    pmap = maps["pmap"] if maps is not None else None
    if overlap_scatter:
        if "side" not in b:
            b["side"] = torch.cuda.Stream(device=p.device)
            b["din_ready"] = torch.cuda.Event()
            b["side_ws"] = None if pmap is not None else torch.empty_like(p.workspace())
        if "out" not in b:
            nout = p.T if scatter_mode in (SCATTER_TOKEN, SCATTER_TOKEN_BESIDE) else p.T * p.K
            b["out"] = torch.empty(max(nout, 1), p.D if p.swiglu else p.F, dtype=torch.float32, device=p.device)
    if gathered:
        g = grouped_gemm_bwd_gathered(p, G, alpha, sel, ctok, PhiW, W2, X=X, H=H, W1=W1, out=b.get("gemm"),
                                      din_ready=b["din_ready"] if overlap_scatter else None, stream=main)
    else:
        g = grouped_gemm_bwd(p, c["Dlt"], Phi, W2, XC=X, HC=H, W1=W1, mode=mode, out=b.get("gemm"),
                             hc_rows=hc_rows, phi_rows=phi_rows, x_rows=x_rows,
                             din_ready=b["din_ready"] if overlap_scatter else None, stream=main)
    b.setdefault("gemm", g)
    if overlap_scatter:
        side = b["side"]
        side.wait_event(b["din_ready"])
        side_mode = SCATTER_TOKEN_BESIDE if scatter_mode == SCATTER_TOKEN else scatter_mode
        out = scatter(p, g["dIn"], ctok, cslot, n_rows=p.rows(mode), mode=side_mode, out=b["out"],
                      ws=b["side_ws"], pmap=pmap, stream=side)
        main.wait_stream(side)
    else:
        out = scatter(p, g["dIn"], ctok, cslot, n_rows=p.rows(mode), mode=scatter_mode, out=b.get("out"),
                      pmap=pmap, stream=main)
    b.setdefault("out", out)
    return {"R": b["R"], "sel": sel, "keep": keep, **c, **g, "out": out}
