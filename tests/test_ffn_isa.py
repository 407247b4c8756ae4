"""The expert FFN's stage loop, as compiled for gfx950, holds no wait for
vector memory that the compiler inserted itself, and the kernel keeps no
value in scratch memory.

The stage loop keeps several stages of weight copies in flight and waits for
them only through its own counted waits (blocks without MFMA). A wait that
the compiler adds inside an MFMA block (because some register written by a
load may still be pending there, e.g. a value loaded in cold code and read
only on some paths) would make every stage wait for the copies issued before
it, and the stream would run at a fraction of its rate. This compiles
ffn.hip to assembly with the product flags (no GPU needed) and checks every
basic block of each ffn_kernel instantiation that issues MFMA.

Scratch (private) memory is reached with vector memory instructions too, so
a value kept there (a spill, or a variable the compiler could not keep in
registers) makes the loop wait for the weight copies in flight wherever it
is reloaded: every instantiation must have a private segment of 0 bytes.
"""
import os
import re
import subprocess

import pytest

from aware_expert_routing_amd import build as B


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not installed")
    return _asm(tmp_path_factory.mktemp("isa"))


def _asm(tmp_path, defines=()):
    out = tmp_path / "ffn.s"
    cmd = [B._hipcc(), "-O3", "-std=c++17", f"--offload-arch={B.ARCH}", "--cuda-device-only", "-S",
           *B.DEVICE_FLAGS, *defines, "-x", "hip", os.path.join(B.CSRC, "ffn.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _mfma_blocks_with_waits(asm):
    found = {}
    for m in re.finditer(r"^(_ZN3moe\w*ffn_kernelILi(\d)E\w*):", asm, re.M):
        name, mtx = m.group(1), int(m.group(2))
        end = asm.index(".Lfunc_end", m.end())
        block, mfma, waits = None, 0, []
        bad = []
        for line in asm[m.end():end].splitlines():
            t = line.strip()
            if re.match(r"^\.LBB\d+_\d+:", t):
                if mfma and waits:
                    bad.append((block, waits))
                block, mfma, waits = t.split(":")[0], 0, []
                continue
            if t.startswith("v_mfma"):
                mfma += 1
            elif t.startswith("s_waitcnt") and "vmcnt" in t:
                waits.append(t)
        if mfma and waits:
            bad.append((block, waits))
        found[mtx] = bad
    return found


def test_stage_loop_has_no_compiler_inserted_memory_waits(asm):
    found = _mfma_blocks_with_waits(asm)
    assert sorted(found) == [1, 2, 4], "every ffn_kernel instantiation is compiled"
    for mtx, bad in found.items():
        assert not bad, f"ffn_kernel<{mtx}>: vector-memory waits inside MFMA blocks: {bad}"


def test_ffn_kernels_use_no_scratch(asm):
    sizes = {}
    for m in re.finditer(r"^\s*\.amdhsa_kernel (_ZN3moe\w*ffn_kernelILi(\d)E\w*)\s*$", asm, re.M):
        end = asm.index(".end_amdhsa_kernel", m.end())
        f = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", asm[m.end():end])
        sizes[int(m.group(2))] = int(f.group(1))
    assert sorted(sizes) == [1, 2, 4], sizes
    assert all(v == 0 for v in sizes.values()), f"private segment bytes per lane: {sizes}"
