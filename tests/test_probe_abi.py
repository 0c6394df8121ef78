"""The probe library (include/pa_probe.h): every declared symbol is exported, and bad arguments
are rejected before any device call, so this runs without a GPU."""

import ctypes as C
import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "paged_kv_cache_378_amd", "libpa_probe.so")


def declared():
    text = open(os.path.join(ROOT, "include", "pa_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_probe_[a-z0-9_]+)\s*\(", text)))


def test_probe_library_exports_every_declared_symbol():
    names = declared()
    assert names == ["pa_probe_mfma", "pa_probe_read_gather", "pa_probe_read_stream"]
    lib = C.CDLL(LIB)
    assert all(hasattr(lib, n) for n in names)
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    assert set(names) <= set(re.findall(r" T (pa_probe_[a-z0-9_]+)$", out, flags=re.M))


def test_probe_calls_reject_bad_arguments():
    lib = C.CDLL(LIB)
    lib.pa_probe_mfma.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                  C.c_void_p, C.c_void_p, C.POINTER(C.c_double), C.c_void_p]
    lib.pa_probe_read_stream.argtypes = [C.c_void_p, C.c_size_t, C.c_int32, C.c_int32, C.c_void_p,
                                         C.POINTER(C.c_size_t), C.c_void_p]
    lib.pa_probe_read_gather.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                         C.c_void_p, C.c_void_p]
    fake = C.c_void_p(0x1000)  # 16-byte aligned, never dereferenced: every call fails validation
    fl = C.c_double()
    for shape, operands, wg, waves, iters in ((24, 0, 256, 4, 10), (32, 2, 256, 4, 10),
                                               (32, 0, 0, 4, 10), (16, 1, 256, 3, 10),
                                               (16, 0, 256, 4, 0)):
        assert lib.pa_probe_mfma(shape, operands, wg, waves, iters, fake, None, C.byref(fl), None) == -1
    assert lib.pa_probe_mfma(32, 1, 256, 4, 10, None, None, C.byref(fl), None) == -1
    got = C.c_size_t()
    assert lib.pa_probe_read_stream(fake, 1 << 30, 256, 0, fake, C.byref(got), None) == -1
    assert lib.pa_probe_read_stream(fake, 1 << 30, 256, 3, fake, C.byref(got), None) == -1
    assert lib.pa_probe_read_stream(fake, 16, 256, 1, fake, C.byref(got), None) == -1  # too small
    assert lib.pa_probe_read_stream(C.c_void_p(0x1004), 1 << 30, 256, 1, fake, C.byref(got), None) == -1
    assert lib.pa_probe_read_gather(fake, fake, 0, 1, 256, fake, None) == -1
    assert lib.pa_probe_read_gather(fake, fake, 16, 3, 256, fake, None) == -1
