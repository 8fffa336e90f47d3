"""Edge cases of every kernel against the oracle, each case checking which
kernel it lands on (q4_matvec_route / q4_matmul_route):

* block scales that are binary16 subnormals (the hand-worked SUBNORMAL and
  ROUNDED_SCALE golden blocks planted, plus random subnormal scales on half
  the blocks): one-hot products return the decoded column exactly (float32
  paths) or its binary16 rounding (matrix-core paths), and full products stay
  within the bounds;
* bit-identical duplicated rows in the LM-head argmax: the lowest index wins
  in every kernel variant (tall tables with four row groups, x in registers,
  the generic kernel for K % 64 == 32).

Q4_0 is the format the pages name for the browser build (section
"Architecture" of "Implémentation en Rust du modèle Voxtral Mini 4B Realtime
de Mistral pour l'exécuter dans le navigateur"); the argmax is the greedy LM
head over the 131072-row table that section "Solutions techniques pour
l'exécution dans le navigateur", item 3, keeps in Q4.
"""

import numpy as np
import pytest

import oracle_checks as oc
import q4_quantized_speech_amd as q4
from gpu_util import announce, assert_within, dev, host, lm_table, needs_gpu
from oracle import q4_oracle as O

pytestmark = [pytest.mark.gpu, needs_gpu]

MV = (O.MATVEC_REL, O.MATVEC_ABS)
MF = (O.MFMA_REL, O.MFMA_ABS)


def subnormal_table(n, k, seed, frac=0.5):
    """Oracle-encoded N(0, 0.02^2) weights whose block scales are replaced,
    on about `frac` of the blocks, by random binary16 subnormal patterns
    (either sign); the golden SUBNORMAL and ROUNDED_SCALE blocks are planted
    at fixed places.  Codes stay as encoded (all 16 levels occur)."""
    g = np.random.Generator(np.random.PCG64(seed))
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    qb = O.quantize_q4_0(w)
    blk = qb.reshape(n, k // 32, 18)
    pick = g.random((n, k // 32)) < frac
    bits = g.integers(1, 1024, (n, k // 32)) | (g.integers(0, 2, (n, k // 32)) << 15)
    blk[..., 0] = np.where(pick, bits & 0xFF, blk[..., 0])
    blk[..., 1] = np.where(pick, bits >> 8, blk[..., 1])
    gold = {gb["name"]: gb for gb in oc.load_golden()}
    for name, (r, b) in {"SUBNORMAL": (0, 0), "ROUNDED_SCALE": (n - 1, k // 32 - 1)}.items():
        blk[r, b] = np.frombuffer(gold[name]["bytes"], np.uint8)
    assert np.any((blk[..., 1] & 0x7C) == 0)
    return qb


# --------------------------------------------------------------------------
# Subnormal scales: matvec variants and the argmax
# --------------------------------------------------------------------------

MV_SHAPES = [(300, 3072), (6144, 3072), (3000, 9216), (2000, 12288), (500, 3104), (70, 96),
             (65600, 1024)]


def test_matvec_variants_are_all_covered():
    routes = {q4.matvec_route(n, k) for n, k in MV_SHAPES}
    routes |= {q4.matvec_route(n, k, argmax=True) for n, k in MV_SHAPES}
    assert routes >= {"pairs_lds", "pairs_lds_g4", "pairs_reg_r1", "pairs_reg_r2", "any"}, routes


@pytest.mark.parametrize("n,k", MV_SHAPES)
def test_subnormal_scales_matvec(n, k):
    qb = subnormal_table(n, k, 7 * n + k)
    wd = O.dequantize_q4_0(qb, n, k)
    wq = dev(qb)
    route = q4.matvec_route(n, k)
    for col in [0, 1, 17, k // 2 + 3, k - 1]:
        x = np.zeros(k, np.float32)
        x[col] = 1.0
        announce(f"subnormal one-hot matvec {route} n={n} k={k} col={col}")
        y = host(q4.matvec(wq, dev(x))) + 0.0       # -0 -> +0 on both sides
        assert np.array_equal(y.view(np.uint32), (wd[:, col] + 0.0).view(np.uint32)), (route, col)
    g = np.random.Generator(np.random.PCG64(n + k))
    x = (g.standard_normal((2, k)) * 1e4).astype(np.float32)
    announce(f"subnormal matvec {route} n={n} k={k}")
    y = host(q4.matvec(wq, dev(x)))
    for i in range(2):
        ref, b = O.lmhead_logits(qb, x[i], n, k)
        assert_within(y[i], ref, b, *MV, f"subnormal matvec {route} {n}x{k} row {i}")


@pytest.mark.parametrize("n,k", MV_SHAPES)
def test_subnormal_scales_argmax(n, k):
    qb = subnormal_table(n, k, 11 * n + k)
    g = np.random.Generator(np.random.PCG64(3 * n + k))
    x = (g.standard_normal((2, k)) * 1e4).astype(np.float32)
    route = q4.matvec_route(n, k, argmax=True)
    announce(f"subnormal argmax {route} n={n} k={k}")
    idx, val = q4.lmhead_argmax(dev(qb), dev(x))
    idx, val = host(idx), host(val)
    for i in range(2):
        y, b = O.lmhead_logits(qb, x[i], n, k)
        assert O.argmax_accepts(y, b, int(idx[i])), (route, i, int(idx[i]), O.argmax_lowest(y))
        assert abs(val[i] - y[idx[i]]) <= O.MATVEC_REL * b[idx[i]] + O.MATVEC_ABS


# --------------------------------------------------------------------------
# Subnormal scales: every matmul kernel
# --------------------------------------------------------------------------

# (M, N, K, workspace?): the kernel each lands on is asserted below
MM_CASES = [
    (2, 64, 3072, False),       # matvec kernel (rows in pairs)
    (4, 64, 12352, True),       # small (weights read once), K split
    (4, 64, 12352, False),      # small, no split
    (4, 300, 2048, False),      # stream16, x in two binary16 parts (the matvec bound)
    (8, 300, 2048, True),       # stream16 (5 to 16 rows, no split; exact weights)
    (20, 300, 2048, True),      # stream16 with two tiles of x (binary16 weights)
    (40, 300, 4096, True),      # skinny (more than one tile of x and K past 3072)
    (1500, 5120, 1280, True),   # wide128
    (1500, 3840, 1280, True),   # wide96
    (375, 3072, 5120, True),    # wide96 with a K split
    (1500, 1280, 1280, True),   # wide32
    (1500, 1280, 5120, True),   # wide128 with a K split
    (375, 1280, 1280, True),    # wide32 with a K split
    (3000, 1280, 1280, True),   # wide64
    (375, 1280, 5120, True),    # wide64 with a K split
    (300, 256, 1024, True),     # tile, K split
    (200, 300, 1056, False),    # simple (K % 64 == 32)
]


def test_matmul_kernels_are_all_covered():
    routes = set()
    for m, n, k, ws in MM_CASES:
        nb = int(q4.lib().q4_matmul_workspace_bytes(m, n, k)) if ws else 0
        r, sp = q4.matmul_route(m, n, k, nb)
        routes.add(r)
        if sp > 1:
            routes.add(r + "+split")
    assert routes >= {"matvec", "small", "small+split", "stream16", "skinny", "wide128", "wide96", "wide64",
                      "wide32", "wide128+split", "wide96+split", "wide64+split", "wide32+split",
                      "tile", "simple"}, routes


def _one_hot_rows(m, k):
    """X [m, k] whose row i is the unit vector at column (i * 37) % k, and
    the columns chosen."""
    cols = (np.arange(m) * 37) % k
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), cols] = 1.0
    return x, cols


@pytest.mark.parametrize("m,n,k,ws", MM_CASES)
def test_subnormal_scales_matmul_one_hot(m, n, k, ws):
    """Y[i, :] = column cols[i] of the decoded weights: exactly on the routes
    whose weights enter unrounded (M <= 4, and the stream16 kernel's q - 8
    with the scale applied in float32 up to 16 rows), its binary16 rounding
    on the other matrix-core routes."""
    qb = subnormal_table(n, k, 5 * m + n + k)
    wd = O.dequantize_q4_0(qb, n, k)
    x, cols = _one_hot_rows(m, k)
    want = wd[:, cols].T + 0.0                      # -0 -> +0
    route = q4.matmul_route(m, n, k, int(q4.lib().q4_matmul_workspace_bytes(m, n, k)) if ws else 0)
    exact = m <= 4 or (route[0] == "stream16" and m <= 16)
    if not exact:
        want = O.round_f16(want) + 0.0
    announce(f"subnormal one-hot matmul {route} {m}x{n}x{k}")
    y = host(q4.matmul(dev(qb), dev(x), workspace=True if ws else None)) + 0.0
    bad = y.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), (route, int(bad.sum()), np.argwhere(bad)[:3].tolist())


@pytest.mark.parametrize("m,n,k,ws", MM_CASES)
def test_subnormal_scales_matmul_bound(m, n, k, ws):
    qb = subnormal_table(n, k, 9 * m + n + k)
    g = np.random.Generator(np.random.PCG64(m + n + k))
    x = (g.standard_normal((m, k)) * 5e3).astype(np.float32)
    ref, b = O.matmul_f64(qb, x, n, k)
    route = q4.matmul_route(m, n, k, int(q4.lib().q4_matmul_workspace_bytes(m, n, k)) if ws else 0)
    announce(f"subnormal matmul {route} {m}x{n}x{k}")
    y = host(q4.matmul(dev(qb), dev(x), workspace=True if ws else None))
    assert_within(y, ref, b, *(MV if m <= 4 else MF), f"subnormal matmul {route} {m}x{n}x{k}")


# --------------------------------------------------------------------------
# Argmax ties: bit-identical rows, lowest index, every variant
# --------------------------------------------------------------------------

def _plant_tie(w, x, rows, scale=0.03):
    """Rows `rows` become identical copies of scale * sign(x): a clear winner
    shared by all of them (every other row is N(0, 0.02^2) noise)."""
    for r in rows:
        w[r] = np.float32(scale) * np.sign(x)


@pytest.mark.parametrize("n,k,rows", [
    (70001, 3072, (1234, 60005)),     # four row groups per workgroup
    (70001, 3072, (4003, 4000)),      # same pass
    (65536, 4096, (65535, 65534)),    # the last pass
    (5000, 3104, (17, 4900)),         # generic kernel (K % 64 == 32)
    (3000, 9216, (2999, 5)),          # x in registers, KS = 9
    (6144, 3072, (100, 6000)),        # x in registers, two rows per lane
])
def test_argmax_tie_lowest_index(n, k, rows):
    g = np.random.Generator(np.random.PCG64(n + k + rows[0]))
    x = g.standard_normal((1, k)).astype(np.float32)
    if n >= 65536:
        qb = lm_table().reshape(-1)[: n * (k // 32) * 18].copy().reshape(n, (k // 32) * 18)
        win = O.quantize_q4_0(np.float32(0.03) * np.sign(x))
        for r in rows:
            qb[r] = win[0]
    else:
        w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
        _plant_tie(w, x[0], rows)
        qb = O.quantize_q4_0(w)
    route = q4.matvec_route(n, k, argmax=True)
    announce(f"argmax tie {route} n={n} k={k} rows={rows}")
    idx, val = q4.lmhead_argmax(dev(qb), dev(x))
    y, b = O.lmhead_logits(qb, x[0], n, k)
    assert y[rows[0]] == y[rows[1]] and O.argmax_lowest(y) == min(rows)
    assert int(host(idx)[0]) == min(rows), (route, int(host(idx)[0]))
    # the tied rows' device logits are bit-identical too
    yy = host(q4.matvec(dev(qb), dev(x[0])))
    assert yy[rows[0]] == yy[rows[1]]
