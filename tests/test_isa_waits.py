"""Static checks of the load/wait structure the GEMM kernels rely on, on the AMD
assembly hipcc produces for gfx950 (built here, no GPU needed).

The forward GEMM ends each main-loop step with an explicit `s_waitcnt
vmcnt(N)` and a barrier that does not wait for vector memory (`s_waitcnt
lgkmcnt(4); s_barrier`).  Loads complete in order, so the step's x tile (its
first 8 direct HBM->LDS loads) has landed at the barrier only if exactly N
loads were issued after it: the code tile and the scale loads the source
places there.  A compiler that scheduled any other load into that window would
turn the barrier into a race, so every step of every instantiation is checked.

The decode GEMV waits for each group's direct code loads with explicit counts
that assume no other load is issued after the phase's code loads; checked the
same way.
"""
import os
import re
import subprocess
import shutil

import pytest

from bit_nf4_quantized_15_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    """Device assembly of gemm.hip and gemv.hip, compiled side by side with the library's flags."""
    d = tmp_path_factory.mktemp("isa")
    procs = {}
    for name in ("gemm", "gemv"):
        cmd = [build.HIPCC, *[f for f in build.CFLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
               os.path.join(build.CSRC, f"{name}.hip"), "-o", str(d / f"{name}.s")]
        procs[name] = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE)
    out = {}
    for name, p in procs.items():
        _, err = p.communicate()
        assert p.returncode == 0, err.decode()[-2000:]
        out[name] = (d / f"{name}.s").read_text()
    return out


def _kernels(asm, pattern):
    for m in re.finditer(r"^(_Z\w+):\s*(?:;.*)?$", asm, re.M):
        if pattern in m.group(1):
            end = asm.find(".Lfunc_end", m.start())
            yield m.group(1), [l.strip() for l in asm[m.start():end].split("\n")]


def _ops(lines):
    """vector-memory loads ('D' direct to LDS, 'g' to registers) and vmcnt waits (('c'|'A', n): compiler's
    or the source's inline asm), in program order."""
    ops, in_asm = [], False
    for l in lines:
        if l.startswith(";;#ASMSTART"):
            in_asm = True
        elif l.startswith(";;#ASMEND"):
            in_asm = False
        elif l.startswith("s_waitcnt") and "vmcnt" in l:
            ops.append(("A" if in_asm else "c", int(re.search(r"vmcnt\((\d+)\)", l).group(1))))
        elif l.startswith("buffer_load") and " lds" in l:
            ops.append("D")
        elif l.startswith(("global_load", "buffer_load", "flat_load")):
            ops.append("g")
    return ops


def test_forward_steps_wait_for_exactly_their_x_tile(asm):
    n_kernels = 0
    for name, body in _kernels(asm["gemm"], "nf4_gemm_fwd_kernel"):
        n_kernels += 1
        steps, cur = [], []
        for i, l in enumerate(body):
            cur.append(l)
            if l == "s_barrier":
                if i > 0 and body[i - 1].startswith("s_waitcnt lgkmcnt(4)"):
                    steps.append(cur)
                cur = []
        assert len(steps) >= 6, f"{name}: expected the unrolled main-loop steps, found {len(steps)}"
        for st in steps:
            ops = _ops(st)
            d = [i for i, o in enumerate(ops) if o == "D"]
            assert len(d) >= 8, f"{name}: a step without its x tile"
            # the source's explicit wait (a later compiler wait can only be stricter)
            last_wait = max(i for i, o in enumerate(ops) if isinstance(o, tuple) and o[0] == "A")
            n = ops[last_wait][1]
            after = [o for o in ops[d[7] + 1:last_wait] if o in ("D", "g")]
            assert n == 0 or len(after) == n, \
                f"{name}: wait vmcnt({n}) but {len(after)} loads issued after the x tile"
    assert n_kernels == 16          # scale layout x odd/even blocks x codebook x dtype


def test_gemv_group_waits_follow_the_code_loads(asm):
    n_kernels = 0
    for name, body in _kernels(asm["gemv"], "nf4_gemv_kernel"):
        n_kernels += 1
        since_d = 0
        seen_d = False
        for o in _ops(body):
            if o == "D":
                seen_d, since_d = True, 0
            elif o == "g":
                since_d += 1
            elif o[0] == "A" and seen_d:
                assert since_d == 0, f"{name}: {since_d} register loads between the code loads and a group wait"
    assert n_kernels == 72          # M classes x group counts x scale layout x codebook x dtype


def test_backward_steps_wait_for_their_dy_tile_before_the_barrier(asm):
    """The backward dx GEMM issues the next dy tile by direct loads at the start of a step and
    reads it after the step's closing barrier; loads complete in order, so the tile has landed at
    the barrier if some wait between its last direct load and the barrier allows no more loads in
    flight than were issued after that load.  The step body is written so that the compiler need not
    wait for the tile earlier (its LDS reads are of the other buffers); either way the check holds
    for every step of every instantiation."""
    n_kernels = 0
    for name, body in _kernels(asm["gemm"], "nf4_gemm_bwd_dx_kernel"):
        n_kernels += 1
        if "ILb0E" in name[:60]:        # DYVEC off: dy is staged through registers, no direct loads
            continue
        steps, cur = [], []
        for l in body:
            cur.append(l)
            if l == "s_barrier":
                steps.append(cur)
                cur = []
        checked = 0
        for st in steps:
            ops = _ops(st)
            d = [i for i, o in enumerate(ops) if o == "D"]
            if len(d) < 8:
                continue
            after = ops[d[-1] + 1:]
            waits = [i for i, o in enumerate(after) if isinstance(o, tuple)]
            ok = False
            for wi in waits:
                issued = sum(1 for o in after[:wi] if o in ("D", "g"))
                if after[wi][1] <= issued:
                    ok = True
                    break
            assert ok, f"{name}: no wait covers the dy tile before the barrier"
            checked += 1
        assert checked >= 1, f"{name}: no main-loop step found"
    assert n_kernels == 16
