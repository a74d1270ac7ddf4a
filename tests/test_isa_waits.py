"""Static checks of the load/wait structure the GEMM kernels rely on, on the AMD
assembly hipcc produces for gfx950 (built here, no GPU needed).

The forward GEMM ends each main-loop step with an explicit `s_waitcnt
vmcnt(N)` and a barrier that does not wait for vector memory (`s_waitcnt
lgkmcnt(4); s_barrier`).  Loads complete in order, so the step's x tile (its
first 8 direct HBM->LDS loads) has landed at the barrier only if exactly N
loads were issued after it: the code tile and the scale loads the source
places there.  A compiler that scheduled any other load into that window would
turn the barrier into a race, so every step of every instantiation is checked.

The decode kernels rely on the compiler's own waits; what is checked there is
that no instantiation spills to scratch, that the streaming kernel's waits
never drain its ring of code loads, that the cross-workgroup handshake
of the layer call goes through device-coherent stores and loads, and that no
kernel writes through the scalar data cache.  Every kernel that hands partial
results to another workgroup (the decode layer call, the split sums of the
LoRA products) must have waited for its payload stores before the tag that
publishes them.
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
    """Device assembly of gemm.hip, gemv.hip and lora.hip, compiled side by side with the library's flags."""
    d = tmp_path_factory.mktemp("isa")
    procs = {}
    for name in ("gemm", "gemv", "lora"):
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


def _descriptor(asm, name):
    m = re.search(r"\.amdhsa_kernel " + re.escape(name) + r"\n(.*?)\.end_amdhsa_kernel", asm, re.S)
    assert m, name
    return {k: int(v) for k, v in re.findall(r"\.(amdhsa_\w+) (\d+)", m.group(1))}


def test_gemv_instantiations_keep_everything_in_registers(asm):
    """Every decode-kernel instantiation runs without scratch memory: the phased kernel (batch-row
    classes x scale layout x codebook x dtype x t given or computed in the launch) and the streaming
    kernel (ring depth and tiles per pass x the same four).  The streaming kernel's static LDS is the
    t operand, two slots of partial tiles and their counters (20 KB and at most 64 bytes); its x rows are dynamic
    LDS."""
    counts = {"nf4_gemv_kernel": 0, "nf4_gemv_stream_kernel": 0}
    for kind in counts:
        for name, _ in _kernels(asm["gemv"], kind + "I"):
            counts[kind] += 1
            d = _descriptor(asm["gemv"], name)
            assert d["amdhsa_private_segment_fixed_size"] == 0, f"{name}: uses scratch"
            if kind == "nf4_gemv_stream_kernel":
                assert 20 * 1024 < d["amdhsa_group_segment_fixed_size"] <= 20 * 1024 + 64, f"{name}: static LDS"
                # 8 compute waves and the helper wave: at most 3 waves on a SIMD
                assert d["amdhsa_next_free_vgpr"] <= 168, f"{name}: {d['amdhsa_next_free_vgpr']} VGPRs"
            else:
                assert d["amdhsa_group_segment_fixed_size"] <= 76 * 1024, f"{name}: LDS above 76 KB"
    assert counts == {"nf4_gemv_kernel": 80, "nf4_gemv_stream_kernel": 64}


def test_gemv_main_loop_keeps_the_ring_in_flight(asm):
    """The streaming kernel's block expansions (8 MFMAs each) never drain the ring of code loads: every
    wait before or inside an expansion leaves at least one younger ring entry (4 loads with double
    quantization, 3 without) in flight, and none is a vmcnt(0).  (The compiler's count is exact for the
    first entry of a pass and more cautious for later ones, where the loop-carried state of its wait
    analysis is merged; the bound checked here is the one that keeps loads overlapping the lookups.)"""
    n = 0
    for name, body in _kernels(asm["gemv"], "nf4_gemv_stream_kernelI"):
        m = re.match(r".*nf4_gemv_stream_kernelILi(\d)ELi(\d)ELb(\d)", name)
        D, dq = int(m.group(1)), m.group(3) == "1"
        per = 4 if dq else 3
        blocks, cur = [], []
        for l in body:
            if re.match(r"^\.LBB\S+:|^; %bb", l):
                blocks.append(cur)
                cur = []
            else:
                cur.append(l)
        blocks.append(cur)
        expand = [b for b in blocks if sum(l.startswith("v_mfma") for l in b) == 8]
        assert len(expand) >= D, f"{name}: {len(expand)} expansion blocks"
        for b in expand:
            waits = [int(re.search(r"vmcnt\((\d+)\)", l).group(1)) for l in b
                     if l.startswith("s_waitcnt") and "vmcnt" in l]
            assert waits, f"{name}: an expansion without a wait for its ring entry"
            assert min(waits) >= per, f"{name}: waits {waits} drain the ring"
        n += 1
    assert n == 64


def test_gemv_publication_is_device_scope(asm):
    """The layer call's decode kernels publish partial products of x A to other workgroups, which may run
    on other XCDs with their own L2: the partials and the tag are written with device-coherent (sc1)
    stores and read with device-coherent loads, and the poll loop sleeps between reads.  The kernels
    that take t as an argument have no such traffic (their only waits are on other waves of the same
    workgroup, in LDS)."""
    n_ft = 0
    for kind in ("nf4_gemv_kernelI", "nf4_gemv_stream_kernelI"):
        for name, body in _kernels(asm["gemv"], kind):
            text = "\n".join(body)
            coherent_st = [l for l in body if l.startswith("global_store") and " sc1" in l]
            coherent_ld = [l for l in body if l.startswith("global_load") and " sc1" in l]
            if name.endswith("ELb1EEEvNS0_6GvArgsE"):
                n_ft += 1
                assert coherent_st, f"{name}: no device-coherent stores of the partials and the tag"
                assert any(l.startswith("global_store_dwordx2") for l in coherent_st), f"{name}: no tag store"
                assert any(l.startswith("global_load_dwordx2") for l in coherent_ld), f"{name}: no tag polls"
                assert "s_sleep" in text, f"{name}: the poll loop does not sleep"
            else:
                assert not coherent_st and not coherent_ld, \
                    f"{name}: a kernel with t given should not exchange data with other workgroups"
    assert n_ft == 72


def test_publication_waits_for_the_payload(asm):
    """A tag store (a device-coherent 8-byte store) follows a barrier that every wave reaches only after
    its own device-coherent payload stores have completed: between the last payload store before that
    barrier and the barrier there is an `s_waitcnt vmcnt(0)`.  Without it the tag could reach another
    XCD before the data it announces."""
    counts = {}
    for src in ("gemv", "lora"):
        n = 0
        for name, body in _kernels(asm[src], ""):
            for t in (i for i, l in enumerate(body) if l.startswith("global_store_dwordx2") and " sc1" in l):
                b = max(i for i in range(t) if body[i] == "s_barrier")
                p = max(i for i in range(b) if body[i].startswith(("buffer_store", "global_store")) and " sc1" in body[i])
                assert any(body[i].startswith("s_waitcnt") and "vmcnt(0)" in body[i] for i in range(p, b)), \
                    f"{name}: the tag may overtake the payload"
                n += 1
            # the payload is device-coherent already: no write-back of the whole L2 per workgroup
            assert not any(l.startswith("buffer_wbl2") for l in body), f"{name}: L2 write-back"
        counts[src] = n
    assert counts["gemv"] >= 72 and counts["lora"] >= 64, counts


def test_lora_kernels_keep_everything_in_registers(asm):
    """The LoRA products hold all of a split's loads in registers at once; no instantiation spills."""
    n = 0
    for kind in ("nt_kernelI", "ntb_kernelI", "tn_kernelI", "tn2_kernelI", "tnb_kernelI"):
        for name, _ in _kernels(asm["lora"], kind):
            d = _descriptor(asm["lora"], name)
            assert d["amdhsa_private_segment_fixed_size"] == 0, f"{name}: uses scratch"
            assert d["amdhsa_group_segment_fixed_size"] <= 160 * 1024, name
            n += 1
    assert n == 88 + 88 + 44 + 44 + 44, n


def test_no_scalar_memory_writes(asm):
    """No kernel writes through the scalar data cache (scalar stores, scalar atomics, scalar cache
    write-back or discard): every global write is a vector store."""
    for name in ("gemm", "gemv", "lora"):
        for l in asm[name].split("\n"):
            t = l.strip()
            assert not t.startswith(("s_store", "s_buffer_store", "s_atomic", "s_buffer_atomic", "s_dcache_wb",
                                     "s_dcache_discard")), f"{name}: {t}"


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
            if len(d) < 4:              # a step's dy tile: 4 direct loads per wave (8 waves x 32 rows)
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
