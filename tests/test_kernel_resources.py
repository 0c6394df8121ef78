"""CPU: the compiler's resource report for every HIP kernel of the build (written by build.py
beside the objects).  No kernel may use scratch memory: a local array indexed at run time was
once kept in scratch and made the decode 12% slower without any other sign.  The decode kernel
on the matrix cores must keep two waves per SIMD (its loads are staggered for exactly that),
and the chunk kernel its two."""

import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ = os.path.join(ROOT, "_build")


def report():
    files = glob.glob(os.path.join(OBJ, "*.hip.resources.txt"))
    if not files:
        import __graft_entry__
        __graft_entry__.build()
        files = glob.glob(os.path.join(OBJ, "*.hip.resources.txt"))
    kernels, cur = {}, None
    for f in files:
        for line in open(f):
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                cur = m.group(1)
                kernels[cur] = {}
                continue
            m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\d+)", line)
            if m and cur:
                kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels


def test_no_kernel_uses_scratch():
    k = report()
    assert len(k) >= 20, "the build wrote no resource report"
    used = {n: v.get("ScratchSize [bytes/lane]") for n, v in k.items()
            if v.get("ScratchSize [bytes/lane]", 0) != 0}
    assert not used, used


@pytest.mark.parametrize("pattern,waves", [(r"decode_mfma_kernelILi128ELi16E", 2),
                                           (r"chunk_kernelILi128ELi32E", 2)])
def test_occupancy_of_the_hot_kernels(pattern, waves):
    k = report()
    hits = [v for n, v in k.items() if re.search(pattern, n)]
    assert hits
    for v in hits:
        assert v["Occupancy [waves/SIMD]"] >= waves, v
        assert v.get("VGPRs Spill", 0) == 0, v  # SGPR spills go to VGPR lanes, not memory
