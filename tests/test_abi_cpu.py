"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/q4.h declares, and rejects bad arguments before making
any HIP call (validation returns before the first HIP call by contract)."""

import ctypes
import os

import pytest

import q4_quantized_speech_amd as q4

pytestmark = pytest.mark.skipif(not os.path.exists(q4.LIB_PATH), reason="libq4mi.so not built")

A = 0x10000  # fake, 16-byte aligned, never dereferenced: validation fails first


def test_exports_every_declared_symbol():
    names = q4.declared_symbols()
    assert "q4_matvec" in names and "q4_lmhead_argmax" in names
    handle = ctypes.CDLL(q4.LIB_PATH)
    missing = [n for n in names if not hasattr(handle, n)]
    assert not missing, missing
    assert set(names) == set(q4._SIGS), "binding signatures out of sync with the header"


def test_basic_queries():
    lib = q4.lib()
    assert lib.q4_abi_version() == 3
    assert lib.q4_row_bytes(3072) == 1728
    assert lib.q4_row_bytes(32) == 18
    assert lib.q4_row_bytes(48) == 0
    assert lib.q4_row_bytes(0) == 0
    for s in range(9):
        assert q4.status_string(s) != "unknown status"
    assert q4.status_string(9) == "unknown status"
    assert lib.q4_lmhead_argmax_workspace_bytes(1, 131072, 3072) > 0
    assert lib.q4_lmhead_argmax_workspace_bytes(0, 131072, 3072) == 0
    assert lib.q4_lmhead_argmax_workspace_bytes(65, 131072, 3072) == 0


def _matmul_no_ws(*args):
    return q4.lib().q4_matmul(*args[:6], None, 0, args[6])


@pytest.mark.parametrize("fn", ["q4_matvec", "q4_matmul", "q4_embed_rows"])
def test_null_shape_align(fn):
    f = _matmul_no_ws if fn == "q4_matmul" else getattr(q4.lib(), fn)
    assert f(None, A, A, 1, 16, 64, None) == q4.Q4_ERR_NULL
    assert f(A, None, A, 1, 16, 64, None) == q4.Q4_ERR_NULL
    assert f(A, A, None, 1, 16, 64, None) == q4.Q4_ERR_NULL
    assert f(A, A, A, 1, 16, 48, None) == q4.Q4_ERR_SHAPE     # K % 32
    assert f(A, A, A, 1, 16, 0, None) == q4.Q4_ERR_SHAPE
    assert f(A, A, A, 0, 16, 64, None) == q4.Q4_ERR_SHAPE     # M = 0
    assert f(A, A, A, 1, 0, 64, None) == q4.Q4_ERR_SHAPE      # N = 0
    assert f(A, A, A, -1, 16, 64, None) == q4.Q4_ERR_SHAPE
    assert f(A + 4, A, A, 1, 16, 64, None) == q4.Q4_ERR_ALIGN
    assert f(A, A + 8, A, 1, 16, 64, None) == q4.Q4_ERR_ALIGN
    assert f(A, A, A + 2, 1, 16, 64, None) == q4.Q4_ERR_ALIGN


def test_matmul_workspace_validation():
    lib = q4.lib()
    f = lib.q4_matmul
    assert f(A, A, A, 4, 16, 64, A + 8, 1024, None) == q4.Q4_ERR_ALIGN   # workspace alignment
    assert f(A, A, A, 4, 16, 1 << 23, None, 0, None) == q4.Q4_ERR_SHAPE  # K above 2^22
    # the split plan: few tiles and a long K ask for a workspace; many tiles do not
    few = lib.q4_matmul_workspace_bytes(100, 200, 4096)
    assert few > 0 and few % (100 * 200 * 4) == 0
    assert lib.q4_matmul_workspace_bytes(1500, 1280, 5120) > 0
    assert lib.q4_matmul_workspace_bytes(3000, 5120, 1280) == 0
    assert lib.q4_matmul_workspace_bytes(100, 200, 4096 + 32) == 0    # K % 64 == 32: no split
    assert lib.q4_matmul_workspace_bytes(0, 200, 4096) == 0
    assert lib.q4_matmul_workspace_bytes(100, 200, 48) == 0


def test_matvec_m_range():
    f = q4.lib().q4_matvec
    assert f(A, A, A, 9, 16, 64, None) == q4.Q4_ERR_SHAPE


def test_lmhead_argmax_validation():
    f = q4.lib().q4_lmhead_argmax
    ws = q4.lib().q4_lmhead_argmax_workspace_bytes(1, 64, 64)
    assert f(None, A, A, None, 1, 64, 64, A, ws, None) == q4.Q4_ERR_NULL
    assert f(A, A, None, None, 1, 64, 64, A, ws, None) == q4.Q4_ERR_NULL
    assert f(A, A, A, None, 0, 64, 64, A, ws, None) == q4.Q4_ERR_SHAPE
    assert f(A, A, A, None, 65, 64, 64, A, ws, None) == q4.Q4_ERR_SHAPE
    assert f(A, A, A, None, 1, 64, 40, A, ws, None) == q4.Q4_ERR_SHAPE
    assert f(A, A, A, None, 1, 64, 64, None, ws, None) == q4.Q4_ERR_WORKSPACE
    assert f(A, A, A, None, 1, 64, 64, A, ws - 1, None) == q4.Q4_ERR_WORKSPACE
    assert f(A, A, A, A + 4, 1, 64, 64, A, ws, None) == q4.Q4_ERR_ALIGN
    assert f(A, A, A, None, 1, 64, 64, A + 8, ws, None) == q4.Q4_ERR_ALIGN


def test_quantize_validation():
    f = q4.lib().q4_quantize
    assert f(None, A, 4, 64, None, None) == q4.Q4_ERR_NULL
    assert f(A, None, 4, 64, None, None) == q4.Q4_ERR_NULL
    assert f(A, A, 0, 64, None, None) == q4.Q4_ERR_SHAPE
    assert f(A, A, 4, 33, None, None) == q4.Q4_ERR_SHAPE
    assert f(A, A + 1, 4, 64, None, None) == q4.Q4_ERR_ALIGN
    assert f(A, A, 4, 64, A + 2, None) == q4.Q4_ERR_ALIGN


def test_python_binding_rejects_bad_tensors():
    import torch
    with pytest.raises(ValueError):
        q4.q4_shape(torch.zeros((4, 17), dtype=torch.uint8))
    with pytest.raises(ValueError):
        q4.q4_shape(torch.zeros((4, 18), dtype=torch.int8))
    with pytest.raises(ValueError):
        q4.matvec(torch.zeros((4, 18), dtype=torch.uint8), torch.zeros(32))  # CPU tensors


def test_header_is_plain_c(tmp_path):
    """include/q4.h compiles as C11 with warnings as errors, and a C program
    linked against the library runs its query and validation paths."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "abi_smoke")
    libdir = os.path.dirname(q4.LIB_PATH)
    cmd = [cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(root, "include"), os.path.join(root, "tests", "c", "abi_smoke.c"),
           "-L", libdir, "-lq4mi", f"-Wl,-rpath,{libdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "abi_smoke ok" in r.stdout, (r.stdout, r.stderr)
