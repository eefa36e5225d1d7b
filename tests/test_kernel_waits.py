"""The split-partial kernel's tile loops keep their tile loads in flight.

The tile loads are direct-to-LDS loads written as inline assembly, which the
compiler does not count; each loop waits for them only where it means to (the
wait at the top of every tile).  A wait that the compiler inserts inside a
tile loop, for a value it reloaded from scratch before the loop, is a plain
`s_waitcnt vmcnt(N)` counted as if its own reload were the only load in
flight, so on the hardware it also waits for every tile load in flight, every
iteration.  This test compiles the kernels to gfx950 assembly (no GPU needed)
and checks that no such wait sits in any MFMA loop nested inside a work item
(loop depth 2 or more) of any split-partial instantiation.
"""
from __future__ import annotations

import os
import re
import subprocess
from collections import defaultdict

import pytest

from speculative_decoding_mla_page_amd import build as B

KERNELS = os.path.join(B.PKG, "csrc", "mla_verify_kernels.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "k.s"
    flags = [f for f in B.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-x", "hip", KERNELS, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text().split("\n")


def loop_waits(lines, fn_pattern):
    """{function: [(header, depth, has_mfma, [compiler vmcnt waits])]} per loop."""
    found = {}
    i = 0
    while i < len(lines):
        m = re.match(r"^(_ZN4mlav\w*" + fn_pattern + r"\w*):", lines[i])
        if not m:
            i += 1
            continue
        name = m.group(1)
        loops = defaultdict(lambda: {"depth": 0, "mfma": False, "waits": []})
        cur = None       # header of the current block's innermost loop
        in_asm = False
        i += 1
        while i < len(lines) and not lines[i].startswith(".Lfunc_end"):
            ln = lines[i]
            lab = re.match(r"^(\.LBB\d+_\d+|; %bb\.\d+):", ln)
            if lab:
                nxt = lines[i + 1] if i + 1 < len(lines) else ""
                head = re.search(r"This (?:Inner )?Loop Header: Depth=(\d+)", ln + nxt)
                inl = re.search(r"in Loop: Header=(BB\d+_\d+) Depth=(\d+)", ln)
                if head:
                    cur = lab.group(1).lstrip(".")
                    loops[cur]["depth"] = int(head.group(1))
                elif inl:
                    cur = inl.group(1)
                    loops[cur]["depth"] = int(inl.group(2))
                else:
                    cur = None
            elif "ASMSTART" in ln:
                in_asm = True
            elif "ASMEND" in ln:
                in_asm = False
            elif cur is not None:
                if "v_mfma" in ln:
                    loops[cur]["mfma"] = True
                if not in_asm and "s_waitcnt" in ln and "vmcnt" in ln:
                    loops[cur]["waits"].append(ln.strip())
            i += 1
        found[name] = [(h, v["depth"], v["mfma"], v["waits"]) for h, v in loops.items()]
    return found


def test_no_compiler_vmcnt_wait_in_tile_loops(asm):
    found = loop_waits(asm, "partial_kernel")
    # the <1>, <2> and <4> row-tile instantiations, each with and without the
    # contiguous-prefix fast path
    assert len(found) == 6, sorted(found)
    bad = {}
    for name, loops in found.items():
        tile_loops = [lp for lp in loops if lp[1] >= 2 and lp[2]]
        assert tile_loops, f"{name}: no MFMA loop at depth 2 found"
        for h, depth, _, waits in tile_loops:
            if waits:
                bad[f"{name} loop {h}"] = waits
    assert not bad, bad


def test_no_scratch_in_the_split_partial_kernel(asm):
    """No instantiation spills to scratch: a spill of per-item values costs
    stores from every lane of every workgroup (HBM writes) and reloads whose
    waits the compiler places wherever the value is first used."""
    sizes = {}
    cur = None
    for ln in asm:
        m = re.match(r"^\s*\.amdhsa_kernel (\S+)", ln)
        if m:
            cur = m.group(1)
            continue
        m = re.match(r"^\s*\.amdhsa_private_segment_fixed_size (\d+)", ln)
        if m and cur is not None:
            sizes[cur] = int(m.group(1))
            cur = None
    partial = {k: v for k, v in sizes.items() if "partial_kernel" in k}
    assert len(partial) == 6, sorted(sizes)
    assert all(v == 0 for v in partial.values()), partial
