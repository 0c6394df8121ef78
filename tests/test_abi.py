"""The C ABI: every symbol include/pa.h declares is exported; argument checks need no GPU."""

import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    # the boundary's calls: block manager (create/destroy, prefill, append, fork, free,
    # tables, stats, reference counts, slot accounting), host table check, device calls
    for must in ("pa_bm_create", "pa_bm_destroy", "pa_bm_add_seq", "pa_bm_append_slots",
                 "pa_bm_fork", "pa_bm_free_seq", "pa_bm_block_tables", "pa_bm_stats",
                 "pa_bm_refcount", "pa_bm_accounting", "pa_validate_tables", "pa_cache_write",
                 "pa_copy_blocks", "pa_decode_workspace_size", "pa_decode", "pa_chunk_attend"):
        assert must in names, must


def test_library_exports_every_declared_symbol(libpa):
    lib = C.CDLL(libpa.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # the binding wraps exactly the declared set
    assert sorted(libpa.EXPORTED) == declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", libpa.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (pa_[a-z0-9_]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_abi_version(libpa):
    assert libpa.pa_abi_version() == 3


def _raw(libpa):
    return libpa._lib


def test_device_calls_reject_bad_arguments_before_launch(libpa):
    # Validation happens on the host before any HIP call, so this runs without a GPU.
    lib = _raw(libpa)
    fake = C.c_void_p(0x1000)  # never dereferenced: every call below fails validation
    st = lib.pa_decode(fake, fake, fake, fake, fake, fake, 4, 4, 4, 96, 16, 10, 10, 100, 0.1,
                       libpa.PA_DTYPE_F32, 0, None, 0, None)
    assert st == libpa.PA_ERR_UNSUPPORTED and b"head_dim" in lib.pa_last_error()
    st = lib.pa_decode(fake, fake, fake, fake, fake, fake, 4, 6, 4, 64, 16, 10, 10, 100, 0.1,
                       libpa.PA_DTYPE_F32, 0, None, 0, None)
    assert st == libpa.PA_ERR_INVALID_ARG
    st = lib.pa_decode(fake, fake, fake, fake, fake, fake, 4, 4, 4, 64, 24, 10, 10, 100, 0.1,
                       libpa.PA_DTYPE_F32, 0, None, 0, None)
    assert st == libpa.PA_ERR_UNSUPPORTED
    st = lib.pa_decode(fake, fake, fake, fake, fake, fake, 4, 4, 4, 64, 16, 10, 10, 500, 0.1,
                       libpa.PA_DTYPE_F32, 0, None, 0, None)
    assert st == libpa.PA_ERR_INVALID_ARG and b"max_ctx_len" in lib.pa_last_error()
    st = lib.pa_decode(fake, fake, fake, fake, fake, fake, 4, 4, 4, 64, 16, 10, 10, 100, 0.1,
                       libpa.PA_DTYPE_F32, 48, None, 0, None)
    assert st == libpa.PA_ERR_INVALID_ARG
    st = lib.pa_decode(fake, fake, fake, fake, fake, fake, 4, 4, 4, 64, 16, 10, 10, 100, 0.1,
                       libpa.PA_DTYPE_F32, 32, None, 0, None)
    assert st == libpa.PA_ERR_WORKSPACE
    st = lib.pa_decode(fake, fake, fake, fake, fake, fake, 4, 4, 4, 64, 16, 10, 10, 100, 0.1,
                       7, 0, None, 0, None)
    assert st == libpa.PA_ERR_UNSUPPORTED
    for bad_scale in (0.0, -0.1, float("inf"), float("nan")):
        st = lib.pa_decode(fake, fake, fake, fake, fake, fake, 4, 4, 4, 64, 16, 10, 10, 100,
                           bad_scale, libpa.PA_DTYPE_F32, 0, None, 0, None)
        assert st == libpa.PA_ERR_INVALID_ARG and b"scale" in lib.pa_last_error()
    st = lib.pa_cache_write(fake, fake, fake, fake, fake, 3, 4, 64, 16, 10, 9, None)
    assert st == libpa.PA_ERR_UNSUPPORTED
    st = lib.pa_cache_write(C.c_void_p(0x1004), fake, fake, fake, fake, 3, 4, 64, 16, 10,
                            libpa.PA_DTYPE_F32, None)
    assert st == libpa.PA_ERR_INVALID_ARG and b"aligned" in lib.pa_last_error()
    st = lib.pa_copy_blocks(fake, fake, fake, -1, 10, 4, 64, 16, libpa.PA_DTYPE_F32, None)
    assert st == libpa.PA_ERR_INVALID_ARG
    # zero-sized work is a no-op that touches nothing
    assert lib.pa_cache_write(None, None, None, None, None, 0, 4, 64, 16, 10,
                              libpa.PA_DTYPE_F32, None) == 0
    assert lib.pa_copy_blocks(None, None, None, 0, 10, 4, 64, 16, libpa.PA_DTYPE_F32, None) == 0


def test_workspace_size(libpa):
    # partial-result slots per (sequence, head): ceil(max_ctx / partition) + 1 (the extra slot is
    # a share group's partition); each slot holds 64 outputs + max + sum in fp32
    one = libpa.pa_decode_workspace_size(4, 4, 64, 100, 128)            # 1 + 1 slots
    four = libpa.pa_decode_workspace_size(4, 4, 64, 100, 32)            # 4 + 1 slots
    assert 0 < one < four
    assert one >= 4 * 4 * 2 * (64 + 2) * 4
    assert four - one >= 4 * 4 * 3 * (64 + 2) * 4
    assert libpa.pa_decode_workspace_size(4, 4, 64, 1000, 0) > 0        # automatic choice
    with pytest.raises(libpa.PaError):
        libpa.pa_decode_workspace_size(4, 4, 64, 100, 40)


def test_noalloc_step_rejects_oversize_batches_before_any_device_call(libpa):
    # The scratch check comes first, so this runs without a GPU (pointers never dereferenced).
    lib = _raw(libpa)
    fake = C.c_void_p(0x1000)
    S, Hq, D, max_ctx = 2048, 64, 128, 8192
    assert libpa.pa_decode_workspace_size(S, Hq, D, max_ctx, 0) > libpa.PA_NOALLOC_SCRATCH_BYTES
    st = lib.pa_decode_step_noalloc(fake, fake, fake, fake, fake, fake, fake, fake, fake, None, S,
                                    Hq, 8, D, 16, 1 << 20, max_ctx // 16, max_ctx, 0.1,
                                    libpa.PA_DTYPE_BF16, 0, None)
    assert st == libpa.PA_ERR_WORKSPACE and b"static scratch" in lib.pa_last_error()
    # the binding's constant is the header's
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    mib = int(re.search(r"#define PA_NOALLOC_SCRATCH_MIB (\d+)", text).group(1))
    assert libpa.PA_NOALLOC_SCRATCH_BYTES == mib << 20
