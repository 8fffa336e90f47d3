"""Seeded random shapes through every entry point, each result against the
oracle: rows of x from 1 to 400 (the matvec, small-M, skinny, tile and wide
routes), any N up to 700, K any multiple of 32 up to 4096 (K % 64 == 32 takes
the generic kernels), with and without a K-split workspace; and wider draws
(N up to 12000, K up to 12288, M at every route's edges).  A second call
must give the same bits.  The shapes are drawn, not chosen, so that edges
nobody listed (a tile one row past a multiple, a single output column, a
split that leaves a short last slice) are exercised too."""

import numpy as np
import pytest
import torch

import q4_quantized_speech_amd as q4
from gpu_util import announce, assert_within, dev, host, needs_gpu
from oracle import q4_oracle as O

pytestmark = [pytest.mark.gpu, needs_gpu]

MV = (O.MATVEC_REL, O.MATVEC_ABS)
MF = (O.MFMA_REL, O.MFMA_ABS)


def _draw_m(g):
    band = g.integers(0, 4)
    lo, hi = [(1, 4), (5, 80), (81, 200), (201, 400)][band]
    return int(g.integers(lo, hi + 1))


def _inputs(g, m, n, k):
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = g.standard_normal((m, k)).astype(np.float32)
    return O.quantize_q4_0(w), x


@pytest.mark.parametrize("seed", range(40))
def test_matmul_random_shape(seed):
    g = np.random.Generator(np.random.PCG64(7000 + seed))
    m = _draw_m(g)
    n = int(g.integers(1, 701))
    k = 32 * int(g.integers(1, 129))
    qb, x = _inputs(g, m, n, k)
    ref, b = O.matmul_f64(qb, x, n, k)
    wq, xd = dev(qb), dev(x)
    for ws in (True, None):
        need = int(q4.lib().q4_matmul_workspace_bytes(m, n, k)) if ws else 0
        route = q4.matmul_route(m, n, k, need)
        announce(f"random matmul seed={seed} {m}x{n}x{k} route={route}")
        y1 = host(q4.matmul(wq, xd, workspace=ws))
        y2 = host(q4.matmul(wq, xd, workspace=ws))
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), route
        assert_within(y1, ref, b, *(MV if m <= 4 else MF), f"seed={seed} {m}x{n}x{k} {route}")


@pytest.mark.parametrize("seed", range(48))
def test_matmul_random_wide_shape(seed):
    """Wider draws than above: rows of x at the routes' edges (1-4, 5, 16,
    17, 48, 49, 80, 81, 128, 129 ... 400), N up to 12000 and K up to 12288,
    K % 64 == 0 five times in six (the MFMA kernels), sizes capped so the
    oracle stays fast."""
    g = np.random.Generator(np.random.PCG64(20000 + seed))
    m = int(g.choice([1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 76, 79,
                      80, 81, 96, 97, 127, 128, 129, 200, 257, 300, 375, 383, 385, 400]))
    k = 64 * int(g.integers(1, 193)) if g.random() < 0.85 else 32 * int(g.integers(1, 385))
    nmax = max(1, min(12000, int(2.5e7 // k), int(6e8 // (m * k))))
    n = int(g.integers(1, nmax + 1))
    qb, x = _inputs(g, m, n, k)
    ref, b = O.matmul_f64(qb, x, n, k)
    wq, xd = dev(qb), dev(x)
    for ws in (True, None):
        need = int(q4.lib().q4_matmul_workspace_bytes(m, n, k)) if ws else 0
        route = q4.matmul_route(m, n, k, need)
        announce(f"random wide matmul seed={seed} {m}x{n}x{k} route={route}")
        y1 = host(q4.matmul(wq, xd, workspace=ws))
        y2 = host(q4.matmul(wq, xd, workspace=ws))
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), route
        assert_within(y1, ref, b, *(MV if m <= 4 else MF), f"seed={seed} {m}x{n}x{k} {route}")


@pytest.mark.parametrize("seed", range(20))
def test_matvec_random_shape(seed):
    g = np.random.Generator(np.random.PCG64(8000 + seed))
    m = int(g.integers(1, 9))
    n = int(g.integers(1, 3001))
    k = 32 * int(g.integers(1, 129))
    qb, x = _inputs(g, m, n, k)
    ref, b = O.matmul_f64(qb, x, n, k)
    announce(f"random matvec seed={seed} {m}x{n}x{k} route={q4.matvec_route(n, k)}")
    y = host(q4.matvec(dev(qb), dev(x)))
    assert_within(y, ref, b, *MV, f"seed={seed} {m}x{n}x{k}")


@pytest.mark.parametrize("seed", range(12))
def test_lmhead_argmax_random_shape(seed):
    g = np.random.Generator(np.random.PCG64(9000 + seed))
    m = int(g.integers(1, 4))
    n = int(g.integers(1, 5001))
    k = 32 * int(g.integers(1, 97))
    qb, x = _inputs(g, m, n, k)
    ref, b = O.matmul_f64(qb, x, n, k)
    announce(f"random argmax seed={seed} {m}x{n}x{k} route={q4.matvec_route(n, k, argmax=True)}")
    idx, val = q4.lmhead_argmax(dev(qb), dev(x))
    idx, val = host(idx), host(val)
    for i in range(m):
        assert O.argmax_accepts(ref[i], b[i], int(idx[i])), (seed, i, int(idx[i]))
        j = int(idx[i])
        assert abs(float(val[i]) - ref[i, j]) <= O.tolerance(b[i, j], *MV), (seed, i)


@pytest.mark.parametrize("seed", range(6))
def test_embed_random_shape(seed):
    g = np.random.Generator(np.random.PCG64(9500 + seed))
    n = int(g.integers(1, 2001))
    k = 32 * int(g.integers(1, 129))
    m = int(g.integers(1, 65))
    qb, _ = _inputs(g, 1, n, k)
    ids = g.integers(-3, n + 3, m).astype(np.int32)   # a few out of range: zero rows
    announce(f"random embed seed={seed} {m} ids of {n}x{k}")
    out = host(q4.embed_rows(dev(qb), dev(ids)))
    ref = O.embed_rows(qb, ids, n, k)
    # bit-exact after mapping -0 to +0 (adding +0 does that and nothing else)
    z = np.float32(0.0)
    assert np.array_equal((out + z).view(np.uint32), (ref + z).view(np.uint32))
