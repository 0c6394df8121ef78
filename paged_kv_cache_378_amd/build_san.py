"""Build the host half of libpa (block manager, error slot, ABI version) with AddressSanitizer
and UndefinedBehaviorSanitizer into libpa_host_san.so: g++ only, no HIP, no device code.

The library's own tests of the block manager run against it when PA_HOST_LIB names it (the
ASan runtime must then be preloaded into the Python process); tests/test_sanitized_host.py
does both.  Usage: python -m paged_kv_cache_378_amd.build_san
"""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa_host_san.so")
HOST_SOURCES = ("block_manager.cpp", "host_api.cpp")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
CXX = os.environ.get("CXX_HOST", "g++")


def runtime(name: str = "libasan.so") -> str:
    """Path of the compiler's sanitizer runtime (to preload into a process that loads LIB)."""
    return subprocess.run([CXX, f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build(verbose: bool = True) -> str:
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES]
    tmp = LIB + ".tmp"
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", *SAN, f"-I{os.path.join(ROOT, 'include')}",
           f"-I{CSRC}", *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitizer build failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} (ASan + UBSan, host code only)")
    return LIB


def build_driver(src: str, out: str) -> str:
    """A native test driver linked with the same host sources and sanitizers."""
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES]
    cmd = [CXX, "-std=c++17", "-O1", "-g", *SAN, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           src, *srcs, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitizer driver build failed: {' '.join(cmd)}\n{res.stderr}")
    return out


if __name__ == "__main__":
    build()
