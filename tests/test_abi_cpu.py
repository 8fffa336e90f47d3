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


def test_matmul_residual_validation():
    """Checks that reject a call before anything is enqueued."""
    lib = q4.lib()
    f = lib.q4_matmul_residual
    assert f(None, A, A, A, 4, 16, 64, None, 0, None) == q4.Q4_ERR_NULL
    assert f(A, A, None, A, 4, 16, 64, None, 0, None) == q4.Q4_ERR_NULL   # r
    assert f(A, A, A, None, 4, 16, 64, None, 0, None) == q4.Q4_ERR_NULL   # y
    assert f(A, A, A, A, 4, 16, 48, None, 0, None) == q4.Q4_ERR_SHAPE
    assert f(A, A, A + 4, A, 4, 16, 64, None, 0, None) == q4.Q4_ERR_ALIGN  # r
    assert f(A, A, A, A, 4, 16, 64, A + 8, 1024, None) == q4.Q4_ERR_ALIGN  # workspace
    # in place (r is y) where the add is a second launch: the product needs
    # M*N floats of workspace
    assert f(A, A, A, A, 2, 3072, 3072, None, 0, None) == q4.Q4_ERR_WORKSPACE
    assert f(A, A, A, A, 2, 3072, 3072, A, 2 * 3072 * 4 - 16, None) == q4.Q4_ERR_WORKSPACE
    w = lib.q4_matmul_residual_workspace_bytes
    assert w(2, 3072, 3072) == 2 * 3072 * 4
    # the encoder shapes add r inside the product's kernels: only the K split's workspace
    assert w(1500, 1280, 1280) == lib.q4_matmul_workspace_bytes(1500, 1280, 1280) == 0
    assert w(1500, 1280, 5120) == lib.q4_matmul_workspace_bytes(1500, 1280, 5120) > 0
    assert w(0, 16, 64) == 0


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


# The routing decisions the kernels were measured for.  Without a GPU the
# CU count falls back to 256 (the MI355X's) and the occupancy queries to one
# workgroup per CU, so only the choices that do not depend on occupancy are
# pinned here: the kernel family, and the wide kernel's tile height and split
# (its cost model uses the CU count only).  The GPU tests assert the kernels
# each route reaches.
ROUTES = [
    ((1, 18432, 3072), ("matvec", 1)),      # decode step
    ((2, 9216, 3072), ("matvec", 1)),       # two streams: a pair of rows reads W once
    ((2, 12288, 4096), ("matvec", 1)),      # K past 3072: the pair kernel at any size
    ((2, 18432, 3072), ("stream16", 1)),    # K <= 3072, 20 MiB of weights or more
    ((2, 131072, 3072), ("stream16", 1)),
    ((4, 18432, 3072), ("stream16", 1)),    # four streams: x in two binary16 parts, weights once
    ((3, 3072, 4096), ("stream16", 1)),
    ((4, 3072, 9216), ("small", None)),     # K past 6144, large W: the small-M kernel
    ((4, 300, 6208), ("matvec", 1)),        # 25 chunks, small W: rows through the matvec
    ((2, 64, 12352), ("small", None)),      # K > 12288: beyond the pair kernel
    ((3, 300, 1056), ("matvec", 1)),        # K % 64 == 32 keeps the float32 path
    ((16, 18432, 3072), ("stream16", 1)),   # prompt prefix up to 16 rows: one MFMA tile
    ((5, 3072, 4096), ("stream16", 1)),
    ((8, 3072, 6144), ("stream16", 1)),     # two 256-value chunks per wave
    ((16, 3072, 9216), ("skinny", None)),   # K past 6144: x would outweigh the weights
    ((17, 18432, 3072), ("stream16", 1)),   # two tiles of 16 rows of x, K <= 3072
    ((38, 6144, 3072), ("stream16", 1)),    # the 38-token prefix: three tiles
    ((38, 3072, 4096), ("skinny", None)),   # more than one tile and K past 3072
    ((49, 18432, 3072), ("wide64", 3)),     # past three tiles: the wide kernel
    ((76, 3072, 9216), ("wide96", 16)),     # past 48 rows: the wide kernel's planner
    ((48, 3072, 4096), ("skinny", None)),   # up to 48 rows with K past 3072: skinny
    ((200, 300, 1056), ("simple", 1)),      # K % 64 == 32, binary16 path
    ((300, 256, 1024), ("tile", None)),     # narrow outputs
    ((1500, 3840, 1280), ("wide96", 1)),    # encoder at M = 1500
    ((1500, 1280, 1280), ("wide32", 1)),
    ((1500, 5120, 1280), ("wide128", 1)),
    ((1500, 1280, 5120), ("wide128", 4)),
    ((375, 3072, 5120), ("wide96", 5)),     # adapter at M = 1500 / 4
    ((375, 3840, 1280), ("wide32", 1)),     # encoder at M = 375
    ((375, 5120, 1280), ("wide32", 1)),
    ((375, 1280, 1280), ("wide32", 4)),
    ((375, 1280, 5120), ("wide64", 8)),
    ((3000, 1280, 1280), ("wide64", 1)),    # encoder at M = 3000
    ((3000, 3840, 1280), ("wide96", 1)),
    ((3000, 5120, 1280), ("wide128", 1)),
    ((3000, 1280, 5120), ("wide128", 2)),
    ((750, 3072, 5120), ("wide128", 3)),
]


def test_workspace_sizes_keep_the_plan():
    """Over drawn shapes: the planned workspace gives exactly the plan an
    unlimited one would (the K split it sizes for is the one taken), a
    workspace of zero never splits, and the residual form's size covers
    the plain one's (the same plan, plus room for an in-place product where
    the add is a second launch)."""
    import numpy as np
    lib = q4.lib()
    g = np.random.Generator(np.random.PCG64(123))
    for _ in range(400):
        m = int(g.choice([1, 2, 3, 4, 5, 16, 17, 48, 49, 80, 81, 129, 375, 1500, 3000]))
        n = int(g.integers(1, 20000))
        k = 32 * int(g.integers(1, 400))
        need = int(lib.q4_matmul_workspace_bytes(m, n, k))
        big = q4.matmul_route(m, n, k, 1 << 62)
        assert q4.matmul_route(m, n, k, need) == big, (m, n, k, need)
        assert need == (0 if big[1] == 1 else big[1] * m * n * 4), (m, n, k, need, big)
        assert q4.matmul_route(m, n, k, 0)[1] == 1
        rneed = int(lib.q4_matmul_residual_workspace_bytes(m, n, k))
        assert rneed >= need
        assert q4.matmul_route(m, n, k, rneed) == big, (m, n, k, rneed)
        assert rneed in (need, m * n * 4), (m, n, k, rneed, need)


@pytest.mark.parametrize("shape,want", ROUTES)
def test_matmul_routing(shape, want):
    m, n, k = shape
    need = int(q4.lib().q4_matmul_workspace_bytes(m, n, k))
    kind, splits = q4.matmul_route(m, n, k, need)
    assert kind == want[0], (shape, kind, splits)
    if want[1] is not None:
        assert splits == want[1], (shape, kind, splits)
    # a workspace of size 0 never splits
    assert q4.matmul_route(m, n, k, 0)[1] == 1
