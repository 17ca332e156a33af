"""Checks on the generated gfx950 code (CPU only: hipcc cross-compiles).

The prefill kernels issue their LDS-DMA tile loads (``buffer_load ... lds``)
as inline assembly, whose operands the compiler's hazard checks do not cover.
On this architecture a buffer load must not read a scalar register that a
vector instruction (``v_readfirstlane``, or ``v_readlane`` reloading a
spilled scalar) wrote fewer than 5 wait states earlier; the loads carry those
wait states themselves.  This test compiles the kernels to assembly and scans
every such load: no vector write of one of its scalar operands may sit within
5 wait states before it.  The same statements write the condition code SCC
(their M0 add): no value the compiler put in SCC may be read after one of
them before SCC is written again.  It also checks that no kernel spills
registers to scratch memory inside its main loops, and that no scalar store,
scalar atomic or scalar-cache write-back is generated.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_flashattention_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not found")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in ("prefill_fwd.hip", "decode_splitk.hip", "decode_q4.hip", "merge_partials.hip", "quantize_q4.hip",
                "calibrate.hip", "attn_abi.hip"):
        path = os.path.join(str(d), src + ".s")
        cmd = [hipcc(), "-std=c++17", "-O3", "--offload-arch=gfx950", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-honor-nans",
               "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, src), "-o", path]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out[src] = open(path).read().split("\n")
    return out


def _sregs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _instructions(lines):
    return [l.strip() for l in lines
            if l.strip() and not l.strip().startswith((";", ".")) and not l.strip().endswith(":")]


def test_lds_dma_loads_have_their_wait_states(asm):
    ins = _instructions(asm["prefill_fwd.hip"])
    loads = bad = 0
    for k, line in enumerate(ins):
        if not (line.startswith("buffer_load") and line.endswith(" lds")):
            continue
        loads += 1
        regs = set()
        for tok in line.split(None, 1)[1].split(","):
            regs |= _sregs(tok.strip())
        waits, j = 0, k - 1
        while j >= 0 and waits < 5:
            op = ins[j].split()[0]
            if op.startswith("s_nop"):
                waits += int(ins[j].split()[1], 0) + 1
            else:
                if op.startswith("v_") and len(ins[j].split(None, 1)) > 1:
                    dst = ins[j].split(None, 1)[1].split(",")[0].strip()
                    if _sregs(dst) & regs:
                        bad += 1
                        print(f"hazard: {ins[j]!r} {waits} wait states before {line!r}")
                        break
                waits += 1
            j -= 1
    assert loads > 100, "no LDS-DMA loads found: the scan is not looking at the prefill kernels"
    assert bad == 0


_SCC_READERS = re.compile(r"s_(cbranch_scc[01]|cselect_b(32|64)|addc_u32|subb_u32|cmov_b(32|64)|cmovk_i32)$")
_SCC_WRITERS = re.compile(r"s_(add|sub|addc|subb|and|or|xor|andn2|orn2|nand|nor|xnor|lshl|lshr|ashr|bfe|cmp|min|max|"
                          r"not|abs|absdiff|bcnt|lshl[1-4]_add|quadmask|wqm|bitcmp)[_0-9a-z]*$")


def test_inline_assembly_does_not_cut_through_scc(asm):
    """Every inline-assembly block that writes SCC must be followed, on the
    straight-line path after it, by a write of SCC before any read: a read
    first would see the block's value instead of the one the compiler put
    there."""
    blocks = 0
    for src, lines in asm.items():
        for i, line in enumerate(lines):
            if line.strip() != ";;#ASMSTART":
                continue
            j, body = i + 1, []
            while lines[j].strip() != ";;#ASMEND":
                body.append(lines[j].strip())
                j += 1
            if not any(_SCC_WRITERS.match(b.split()[0]) for b in body if b):
                continue
            blocks += 1
            for line2 in lines[j + 1:]:
                s = line2.split(";")[0].strip()
                if not s or s.startswith("."):
                    continue
                if s.endswith(":"):
                    break  # a label: another path may join here; the path through the block ends
                op = s.split()[0]
                assert not _SCC_READERS.match(op), f"{src}: {s!r} reads SCC written by inline assembly"
                if _SCC_WRITERS.match(op):
                    break
    assert blocks > 100, "no SCC-writing inline assembly found: the scan is not looking at the DMA loads"


def test_no_scalar_memory_writes(asm):
    for src, lines in asm.items():
        for line in _instructions(lines):
            op = line.split()[0]
            assert not re.match(r"s_(store|atomic|buffer_store|buffer_atomic|scratch_store|dcache_wb|dcache_discard)",
                                op), (src, line)


def test_no_spills_in_main_loops(asm):
    """Scratch traffic inside a loop would cost every step; outside the loops
    (a value kept across a kernel's prologue and epilogue) it is harmless.  A
    block belongs to a loop when its label line carries the compiler's
    "Loop Header" / "in Loop" annotation."""
    in_loop, blocks = False, 0
    for src, lines in asm.items():
        for line in lines:
            s = line.strip()
            if s.startswith(".LBB") or s.startswith("; %bb."):
                in_loop = "Loop" in s
                blocks += in_loop
            elif s.endswith(":") and not s.startswith("."):  # a function's entry block
                in_loop = False
            elif in_loop and s.startswith(("scratch_", "buffer_store_dword off", "buffer_load_dword off")):
                raise AssertionError(f"{src}: scratch access inside a loop: {s}")
    assert blocks > 50, "no loop blocks found: the scan is not looking at the kernels' loops"
