"""The GEMM K loops' wait counts against the gfx950 code the compiler makes of them (CPU only).

The 32-K loop of the weight gradients and the forward waits for a stage's direct-to-LDS
loads with a fixed `s_waitcnt vmcnt(N)`, N = (STAGES - 3) x (direct loads per stage),
computed in the source from the loaders' load counts. That is right only while every
iteration issues exactly that many direct loads and no other vector-memory operation
(whose completion the same counter would track). The 64-K loop of the data gradients
waits with vmcnt(0), right whatever the loads are. This test builds gemm.hip to gfx950
assembly with the library's own flags and checks, in every K loop (a loop holding MFMAs
and direct loads) of every GEMM kernel:
* its only vector-memory instructions are direct-to-LDS loads;
* 32-K loops (weight gradients, forward): every vmcnt wait equals the loop's direct loads
  per iteration (4 stages, so STAGES - 3 = 1 stage left in flight);
* 64-K loops (data gradients): every vmcnt wait is 0.
A loader that issued another number of loads, or any other vector-memory operation, inside
a 32-K loop would make its fixed count wrong and fail here before it reached a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

from load_recalibrated_expert_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                                reason="hipcc is not installed")

VMEM = re.compile(r"^\s+(buffer_|global_|flat_|scratch_)\w+")
WAIT = re.compile(r"s_waitcnt\b[^\n]*?vmcnt\((\d+)\)")
LOOP_HEAD = re.compile(r"^(\.LBB\d+_\d+):.*Loop Header")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    r = subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, "gemm.hip"), "-o",
                        str(out)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    return out.read_text()


def functions(text):
    """(symbol, lines) of every kernel in the assembly."""
    out, name, body = [], None, []
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if name:
                out.append((name, body))
            name, body = m.group(1), []
        elif name:
            body.append(line)
            if line.strip().startswith(".Lfunc_end"):
                out.append((name, body))
                name, body = None, []
    return out


def k_loops(lines):
    """Instructions of the loops that hold MFMAs and direct loads. A loop is its header block
    and every block the compiler marks as inside it (the "in Loop: Header=..." comment of a
    block's label, `.LBB...:` or `; %bb.N:` for a block without a label); a block runs to the
    next block's label."""
    blocks, label, loop_of = {}, None, {}
    for line in lines:
        m = re.match(r"^(\.LBB\d+_\d+|; %bb\.\d+):(.*)$", line)
        if m:
            label = m.group(1)
            blocks[label] = []
            h = re.search(r"Header=(BB\d+_\d+)", m.group(2))
            if "Loop Header" in m.group(2):
                loop_of[label] = label
            elif h:
                loop_of[label] = "." + "L" + h.group(1)
            continue
        if label is not None:
            blocks[label].append(line)
    loops = {}
    for lb, head in loop_of.items():
        loops.setdefault(head, []).extend(blocks[lb])
    return [body for body in loops.values()
            if any("v_mfma" in l for l in body) and any(VMEM.match(l) and " lds" in l for l in body)]


def kind(symbol):
    if "f32_" in symbol:
        return None
    if "dgrad_kernel" in symbol:
        return "k64"
    if "wgrad_kernel" in symbol or "fwd_fc" in symbol:
        return "k32"
    return None


def test_k_loop_waits_match_their_loads(asm):
    checked = {"k32": 0, "k64": 0}
    for sym, lines in functions(asm):
        kd = kind(sym)
        if kd is None:
            continue
        loops = k_loops(lines)
        assert loops, f"{sym}: no K loop found"
        for body in loops:
            vmem = [l.strip() for l in body if VMEM.match(l)]
            other = [l for l in vmem if " lds" not in l]
            assert not other, f"{sym}: vector-memory operations besides the direct loads in its K loop: {other[:3]}"
            waits = {int(w) for l in body for w in WAIT.findall(l)}
            assert waits, f"{sym}: no vmcnt wait in its K loop"
            if kd == "k32":
                assert waits == {len(vmem)}, (f"{sym}: 32-K loop waits {sorted(waits)} with {len(vmem)} direct "
                                              f"loads per iteration")
            else:
                assert waits == {0}, f"{sym}: 64-K loop waits {sorted(waits)}"
            checked[kd] += 1
    # two data-gradient epilogues, six weight-gradient loader mixes, the two forward GEMMs
    assert checked["k64"] >= 2 and checked["k32"] >= 8, checked
