"""Build libpa.so (host block manager + gfx950 HIP kernels) in-tree with hipcc.

Usage: python -m paged_kv_cache_378_amd.build   (or __graft_entry__.build()).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
PROBE = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-std=c++17", "-O3", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
          f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only; packed-fp32 instructions are switched off.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".cpp", ".hip")))


RESOURCES = os.path.join(OBJ, "kernel_resources.txt")


def _compile(path: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(path) + ".o")
    cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    if path.endswith(".hip"):
        # the compiler's per-kernel resource report (registers, scratch, occupancy, LDS) is kept
        # beside the objects; tests/test_kernel_resources.py reads it
        cmd[1:1] = ["-x", "hip", *DEVICE, "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    remark = "[-Rpass-analysis=kernel-resource-usage]"
    if path.endswith(".hip"):
        with open(os.path.join(OBJ, os.path.basename(path) + ".resources.txt"), "w") as f:
            f.write("\n".join(l for l in res.stderr.splitlines() if remark in l) + "\n")
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and remark not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """libpa.so (the library) and libpa_probe.so (the bandwidth probes bench.py measures the
    achievable read rates with)."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = [os.path.join(CSRC, f) for f in _sources()]
    probes = sorted(os.path.join(PROBE, f) for f in os.listdir(PROBE) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probes))) as ex:
        objs = list(ex.map(_compile, srcs + probes))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
