"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: decoded values bit-exact; q4_matvec within 1e-4*B + 1e-6 per element and
q4_matmul within 2e-3*B + 1e-5, with B = sum_k |w_k x_k| over the exact
weights; argmax indices equal wherever the oracle's top-2 margin exceeds the
two leaders' tolerances (otherwise any row within tolerance of the maximum);
the encoder byte-for-byte.  Shapes follow the decoder (3072), encoder (1280),
adapter (5120 -> 3072) and 131072-row vocabulary of the model the pages run.
"""

import numpy as np
import pytest
import torch

import oracle_checks as oc
import q4_quantized_speech_amd as q4
from gpu_util import (announce, assert_within, dev, host, lm_table, needs_gpu, quantize_panels,
                      weights_q4)
from oracle import q4_oracle as O
from q4_quantized_speech_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]

MV = (O.MATVEC_REL, O.MATVEC_ABS)
MF = (O.MFMA_REL, O.MFMA_ABS)


def _rand_w(n, k, seed, scale=0.02):
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.standard_normal((n, k)) * scale).astype(np.float32)


def _rand_x(m, k, seed):
    return synth.activations(m, k, seed)


# --------------------------------------------------------------------------
# Encoder (device-side quantizer): byte-for-byte
# --------------------------------------------------------------------------

def test_quantize_bit_exact_random():
    g = np.random.Generator(np.random.PCG64(101))
    parts = [
        _rand_w(257, 3072, 1),
        (g.standard_normal((64, 256)) * np.exp2(g.integers(-30, 12, (64, 1)))).astype(np.float32),
        (g.integers(-16, 17, (64, 256)) * 0.25).astype(np.float32),   # exact ties
        np.zeros((2, 256), np.float32),
    ]
    for i, w in enumerate(parts):
        announce(f"quantize part {i} shape {w.shape}")
        got = host(q4.quantize(dev(w)))
        want = O.quantize_q4_0(w)
        assert np.array_equal(got, want), f"part {i}: {int((got != want).sum())} bytes differ"


def test_quantize_golden_blocks():
    for gb in oc.load_golden():
        announce(f"quantize golden {gb['name']}")
        got = host(q4.quantize(dev(gb["x"][None, :]))).tobytes()
        assert got == gb["bytes"], gb["name"]


def test_quantize_flags_nonfinite():
    w = np.zeros((2, 64), np.float32)
    w[1, 40] = np.inf
    announce("quantize inf flag")
    with pytest.raises(ValueError):
        q4.quantize(dev(w))
    w = np.zeros((1, 32), np.float32)
    w[0, 3] = 6.0e5                                   # scale overflows binary16
    with pytest.raises(ValueError):
        q4.quantize(dev(w))


# --------------------------------------------------------------------------
# Embedding rows: exact decode
# --------------------------------------------------------------------------

def test_embed_golden_blocks_bit_exact():
    gold = oc.load_golden()
    table = np.frombuffer(b"".join(gb["bytes"] for gb in gold), np.uint8).reshape(len(gold), 18)
    ids = np.arange(len(gold), dtype=np.int32)
    announce("embed golden")
    got = host(q4.embed_rows(dev(table), dev(ids)))
    for i, gb in enumerate(gold):
        assert np.array_equal(got[i].view(np.uint32), gb["deq"].view(np.uint32)), gb["name"]


@pytest.mark.parametrize("n,k", [(300, 3072), (77, 96), (50, 160), (9, 32)])
def test_embed_bit_exact(n, k):
    qb = O.quantize_q4_0(_rand_w(n, k, 7 + k))
    ids = np.array([0, n - 1, 5 % n, -1, n, 2**31 - 1, 3 % n, 0], np.int32)
    announce(f"embed n={n} k={k}")
    got = host(q4.embed_rows(dev(qb), dev(ids)))
    want = O.embed_rows(qb, ids, n, k)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_embed_full_table_prefix():
    table = lm_table()
    ids = synth.token_ids(synth.PREFIX_TOKENS, synth.seed_for(2, 2))
    announce("embed full table, 38 ids")
    got = host(q4.embed_rows(dev(table), dev(ids)))
    want = O.embed_rows(table, ids, synth.VOCAB, synth.DEC_DIM)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# --------------------------------------------------------------------------
# q4_matvec (float32 FMA path)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(64, 3072), (40, 96), (33, 160), (17, 32), (5, 9216)])
def test_matvec_one_hot_bit_exact(n, k):
    qb = O.quantize_q4_0(_rand_w(n, k, 3 + n))
    w = O.dequantize_q4_0(qb, n, k)
    wq = dev(qb)
    for col in [0, 1, 15, 16, 31, k // 2 + 3, k - 1]:
        x = np.zeros(k, np.float32)
        x[col] = 1.0
        announce(f"matvec one-hot n={n} k={k} col={col}")
        y = host(q4.matvec(wq, dev(x)))
        assert np.array_equal(y, w[:, col]), col


def test_matvec_integer_exact():
    wi, xi = oc.integer_weight_case(31, 96, 3072, 4)
    qb = O.quantize_q4_0(wi)
    ref = xi.astype(np.int64) @ wi.astype(np.int64).T
    announce("matvec integer exact")
    for m in range(4):
        y = host(q4.matvec(dev(qb), dev(xi[m])))
        assert np.array_equal(y.astype(np.float64), ref[m].astype(np.float64))


@pytest.mark.parametrize("n,k,m", [
    (3072, 3072, 1), (1, 64, 1), (17, 64, 1), (100, 96, 1), (129, 160, 2), (257, 320, 1),
    (1000, 1280, 1), (64, 15360, 1), (16, 16384, 1), (300, 4096, 8), (513, 9216, 3), (31, 32, 5)])
def test_matvec_parity(n, k, m):
    qb = O.quantize_q4_0(_rand_w(n, k, n * 7 + k))
    x = _rand_x(m, k, 5 + m)
    announce(f"matvec n={n} k={k} m={m}")
    y = host(q4.matvec(dev(qb), dev(x)))
    ref, b = O.matmul_f64(qb, x, n, k)
    assert_within(y, ref, b, *MV, f"matvec {n}x{k} M={m}")


@pytest.mark.parametrize("name,n,k", synth.DECODER_LAYER)
def test_matvec_decoder_layer_full(name, n, k):
    """One decode step of a decoder layer at its real shapes, all outputs."""
    t = [p[0] for p in synth.DECODER_LAYER].index(name)
    qb = weights_q4(n, k, synth.seed_for(1, t))
    x = synth.activations(1, k, synth.seed_for(1, 10 + t))[0]
    announce(f"matvec decoder {name} {n}x{k}")
    y = host(q4.matvec(dev(qb), dev(x)))
    ref, b = O.matvec_f64(qb, x, n, k)
    assert_within(y, ref, b, *MV, f"decoder {name}")


@pytest.mark.parametrize("k", [1280, 1056, 9216])
@pytest.mark.parametrize("case", ["tiny", "huge", "spread", "outlier_on_zero_weights"])
def test_matvec_x_spread(case, k):
    """The bound holds for x far from 1 and for a few huge x meeting zero
    weights (q = 8): the sums are of (q - 8) x terms, so a large x times a
    zero weight adds nothing, exactly.  K = 1056 takes the generic kernel."""
    n = 96
    w = _rand_w(n, k, 40 + k)
    g = np.random.Generator(np.random.PCG64(41 + k))
    x = g.standard_normal((2, k))
    cols = [3, 77, k // 2 + 5, k - 1]
    if case == "tiny":
        x *= 1e-30
    elif case == "huge":
        x *= 1e8
    elif case == "spread":
        x *= 1e-3
        x[:, 77] = 1e4
    else:
        w[:, cols] = 0.0          # a zero column quantises to code 8 in every row
        x[:, cols] = 1e7
    x = x.astype(np.float32)
    qb = O.quantize_q4_0(w)
    ref, b = O.matmul_f64(qb, x, n, k)
    announce(f"matvec x {case} k={k}")
    y = host(q4.matvec(dev(qb), dev(x)))
    assert_within(y, ref, b, *MV, f"matvec x {case} k={k}")
    idx, val = q4.lmhead_argmax(dev(qb), dev(x))
    idx, val = host(idx), host(val)
    for i in range(2):
        assert O.argmax_accepts(ref[i], b[i], int(idx[i])), (case, i)
        assert abs(val[i] - ref[i, idx[i]]) <= O.MATVEC_REL * b[i, idx[i]] + O.MATVEC_ABS


def test_matvec_single_3072():
    qb = weights_q4(3072, 3072, synth.seed_for(0, 0))
    x = synth.activations(1, 3072, synth.seed_for(0, 1))[0]
    announce("matvec 3072x3072")
    y = host(q4.matvec(dev(qb), dev(x)))
    ref, b = O.matvec_f64(qb, x, 3072, 3072)
    assert_within(y, ref, b, *MV, "matvec 3072")


# --------------------------------------------------------------------------
# q4_matmul (binary16 operands on the matrix cores, float32 accumulation)
# --------------------------------------------------------------------------

def test_matmul_one_hot_f16():
    n, k = 150, 256
    w = _rand_w(n, k, 77)
    qb = O.quantize_q4_0(w)
    # block 2 of row 3 becomes golden block D, whose decoded 0.0624847... and
    # -0.0874786... round to binary16 as the golden file states
    d = {g["name"]: g for g in oc.load_golden()}["D"]
    qb[3, 2 * 18: 3 * 18] = np.frombuffer(d["bytes"], np.uint8)
    wd = O.dequantize_q4_0(qb, n, k)
    for i, v in d["f16"].items():
        assert O.round_f16(wd[3, 64 + i: 65 + i])[0] == v
    x = np.zeros((k, k), np.float32)
    np.fill_diagonal(x, 1.0)
    announce("matmul one-hot")
    y = host(q4.matmul(dev(qb), dev(x)))
    assert np.array_equal(y, O.round_f16(wd.T))


def test_matmul_golden_f16_rounding():
    gold = {g["name"]: g for g in oc.load_golden()}
    d = gold["D"]
    qb = np.frombuffer(d["bytes"], np.uint8).reshape(1, 18)
    x = np.zeros((32, 32), np.float32)
    np.fill_diagonal(x, 1.0)
    announce("matmul golden D")
    y = host(q4.matmul(dev(qb), dev(x)))[:, 0]
    for i, v in d["f16"].items():
        assert y[i] == v, (i, y[i], v)


def test_matmul_integer_exact():
    for (n, k, m) in [(96, 3072, 40), (130, 256, 129), (16, 1280, 16)]:
        wi, xi = oc.integer_weight_case(41 + m, n, k, m)
        qb = O.quantize_q4_0(wi)
        ref = xi.astype(np.int64) @ wi.astype(np.int64).T
        announce(f"matmul integer exact {m}x{n}x{k}")
        y = host(q4.matmul(dev(qb), dev(xi)))
        assert np.array_equal(y.astype(np.float64), ref.astype(np.float64))


@pytest.mark.parametrize("m,n,k", [
    (1, 64, 64), (2, 17, 96), (15, 129, 160), (16, 128, 256), (17, 130, 32), (130, 255, 1280),
    (300, 64, 3072), (3, 3000, 128), (257, 257, 288)])
def test_matmul_parity_small(m, n, k):
    qb = O.quantize_q4_0(_rand_w(n, k, m + n + k))
    x = _rand_x(m, k, 9 + m)
    announce(f"matmul m={m} n={n} k={k}")
    y = host(q4.matmul(dev(qb), dev(x)))
    ref, b = O.matmul_f64(qb, x, n, k)
    assert_within(y, ref, b, *MF, f"matmul {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(100, 200, 4096), (17, 3072, 9216), (129, 130, 1024),
                                   (1, 64, 640)])
def test_matmul_split_k(m, n, k):
    """K split over several workgroups per tile: with the planned workspace, a
    workspace too small for the full plan, and none; all within tolerance, and
    repeatable bit for bit for a given workspace size."""
    qb = O.quantize_q4_0(_rand_w(n, k, 3 * m + n))
    x = _rand_x(m, k, 11 + m)
    ref, b = O.matmul_f64(qb, x, n, k)
    wq, xd = dev(qb), dev(x)
    full = q4.matmul_workspace(m, n, k, "cuda")
    if m * n * k > 1 << 20:
        assert full is not None, "a split is planned for this shape"
    small = None if full is None else full[: 2 * m * n * 4]
    for ws, tag in [(full, "planned"), (small, "two slices"), (None, "none")]:
        announce(f"matmul split-K {m}x{n}x{k} workspace {tag}")
        y1 = host(q4.matmul(wq, xd, workspace=ws))
        assert_within(y1, ref, b, *MF, f"split-K {m}x{n}x{k} {tag}")
        y2 = host(q4.matmul(wq, xd, workspace=ws))
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), tag


@pytest.mark.parametrize("m", [1, 16, 17, 32, 33, 48, 80, 81])
@pytest.mark.parametrize("n,k", [(100, 128), (257, 2048), (130, 640), (70, 192), (33, 64)])
def test_matmul_skinny_edges(m, n, k):
    """Row counts at the 16-row MFMA tile edges of the skinny and stream16
    kernels (up to 48 rows; up to 32 rows a skinny stage is four block pairs,
    so K of 1, 2, 3, 10 pairs ends in a partial stage) and past them (80 and
    81 rows go to the tile kernel at these widths); ragged N; with the
    planned workspace (K split where planned) and without one."""
    qb = O.quantize_q4_0(_rand_w(n, k, 7 * m + n + k))
    x = _rand_x(m, k, 5 + m)
    ref, b = O.matmul_f64(qb, x, n, k)
    wq, xd = dev(qb), dev(x)
    for ws in (True, None):
        announce(f"matmul skinny edge {m}x{n}x{k} workspace={ws is not None}")
        y = host(q4.matmul(wq, xd, workspace=ws))
        assert_within(y, ref, b, *MF, f"skinny {m}x{n}x{k} ws={ws is not None}")


@pytest.mark.parametrize("m,n,k", [(81, 512, 128), (100, 1280, 1280), (129, 1300, 640),
                                   (193, 1280, 5120), (375, 1280, 1280), (93, 3072, 5120),
                                   (257, 768, 320)])
def test_matmul_wide_tiles(m, n, k):
    """The 128 x 256 wave-specialised kernel with 128- or 64-row tiles (the
    planner picks the tile and the K split per shape): ragged M in both tile
    heights, ragged N, with the planned workspace and without one."""
    qb = O.quantize_q4_0(_rand_w(n, k, 11 * m + n + k))
    x = _rand_x(m, k, 13 + m)
    ref, b = O.matmul_f64(qb, x, n, k)
    wq, xd = dev(qb), dev(x)
    for ws in (True, None):
        announce(f"matmul wide {m}x{n}x{k} workspace={ws is not None}")
        y = host(q4.matmul(wq, xd, workspace=ws))
        assert_within(y, ref, b, *MF, f"wide {m}x{n}x{k} ws={ws is not None}")


def split_canary_workspace(m, n, k, sentinel):
    """A workspace of the planned size (splits x M x N partial floats)
    followed by 64 floats, all set to the sentinel.  Returns (ws floats,
    need bytes)."""
    need = int(q4.lib().q4_matmul_workspace_bytes(m, n, k))
    route, splits = q4.matmul_route(m, n, k, need)
    assert need > 0 and splits > 1 and need == splits * m * n * 4, (route, splits, need)
    ws = torch.full((need // 4 + 64,), sentinel, dtype=torch.float32, device="cuda")
    return ws, need


def test_matmul_every_split_count():
    """The fold is compiled once per K-split count (2 to 16): a workspace of
    s partial slices caps the split at s, so every count is reached, on the
    wide kernel (K = 12288 in 192 stages) and the skinny one; each result is
    held to the oracle's binary16 bound and repeats bit for bit."""
    reached = set()
    for (m, n, k) in [(96, 512, 12288), (8, 130, 12288)]:
        qb_h = O.quantize_q4_0(_rand_w(n, k, 31))
        x_h = _rand_x(m, k, 32)
        ref, b = O.matmul_f64(qb_h, x_h, n, k)
        qb, x = dev(qb_h), dev(x_h)
        for s in range(2, 17):
            nbytes = s * m * n * 4
            route, splits = q4.matmul_route(m, n, k, nbytes)
            assert 2 <= splits <= s, (route, splits, s)
            reached.add(splits)
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            announce(f"matmul split count {route} {splits} (cap {s}) {m}x{n}x{k}")
            y1 = host(q4.matmul(qb, x, workspace=ws))
            y2 = host(q4.matmul(qb, x, workspace=ws))
            assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
            assert_within(y1, ref, b, O.MFMA_REL, O.MFMA_ABS, f"{route} splits={splits} {m}x{n}x{k}")
    assert reached == set(range(2, 17)), sorted(reached)


@pytest.mark.parametrize("m,n,k", [(70, 150, 2048), (300, 256, 1024), (375, 1280, 1280),
                                   (1500, 1280, 5120), (40, 3072, 9216)])
def test_matmul_split_k_stays_in_bounds(m, n, k):
    """Partial sums stay inside the workspace, results inside Y, every
    output written, and a second call gives the same bits: the skinny, tile
    and wide kernels with a K split."""
    qb = dev(O.quantize_q4_0(_rand_w(n, k, 8)))
    x = dev(_rand_x(m, k, 9))
    sentinel = -12345.0
    ws, need = split_canary_workspace(m, n, k, sentinel)
    out = torch.full((m * n + 64,), sentinel, dtype=torch.float32, device="cuda")
    announce(f"matmul split-K canary {q4.matmul_route(m, n, k, need)} {m}x{n}x{k}")
    first = None
    for rep in range(2):
        q4.matmul(qb, x, out=out[: m * n].view(m, n), workspace=ws[: need // 4].view(torch.uint8))
        got = host(out)
        assert np.all(host(ws)[need // 4:] == sentinel)
        assert np.all(got[m * n:] == sentinel)
        assert not np.any(got[: m * n] == sentinel)
        if first is None:
            first = got[: m * n].copy()
        else:
            assert np.array_equal(got[: m * n].view(np.uint32), first.view(np.uint32))


@pytest.mark.parametrize("m,n,k,route", [(1500, 1280, 5120, "wide128"), (93, 3072, 5120, None),
                                         (375, 1280, 1280, None), (100, 1030, 4096, None),
                                         (40, 3072, 9216, "skinny")])
def test_matmul_fold_sums_slices_in_order(m, n, k, route):
    """The K split's fold: Y is bit for bit the float32 sum, in split order
    0, 1, ..., of the partial slices the call left in the workspace (the
    wide kernel at every tile height it takes here, ragged N, the skinny
    kernel), on two calls in a row; the result meets the oracle's bound."""
    qb_h = O.quantize_q4_0(_rand_w(n, k, 41 + m))
    x_h = _rand_x(m, k, 43 + n)
    ws = q4.matmul_workspace(m, n, k, "cuda")
    got_route, splits = q4.matmul_route(m, n, k, ws.numel())
    assert splits > 1 and (route is None or got_route == route), (got_route, splits)
    assert ws.numel() == splits * m * n * 4
    qb, x = dev(qb_h), dev(x_h)
    for rep in range(2):
        announce(f"matmul fold order {got_route} splits={splits} {m}x{n}x{k} call {rep}")
        y = host(q4.matmul(qb, x, workspace=ws))
        parts = host(ws).view(np.float32).reshape(splits, m, n)
        acc = parts[0].copy()
        for s in range(1, splits):
            acc += parts[s]
        assert np.array_equal(y.view(np.uint32), acc.view(np.uint32)), \
            f"{int((y.view(np.uint32) != acc.view(np.uint32)).sum())} elements differ"
    ref, b = O.matmul_f64(qb_h, x_h, n, k)
    assert_within(y, ref, b, *MF, f"fold {got_route} {m}x{n}x{k}")


# (M, N, K, route with the residual workspace): every q4_matmul route, the
# wide tiles with and without a K split, ragged N on the wide kernel with
# (its fold) and without a K split (its per-element stores)
RESIDUAL_SHAPES = [
    (1500, 1280, 5120, "wide128"), (1500, 1280, 1280, "wide32"), (3000, 1280, 1280, "wide64"),
    (1500, 3840, 1280, "wide96"), (1500, 5120, 1280, "wide128"), (375, 1280, 1280, "wide32"),
    (1500, 1300, 1280, "wide64"), (1000, 5000, 1280, "wide96"), (93, 3072, 5120, None),
    (300, 1282, 1024, None), (76, 3072, 9216, None), (40, 3072, 9216, "skinny"),
    (16, 3072, 4096, "stream16"), (4, 3072, 9216, "small"), (3, 6144, 3072, "stream16"),
    (2, 3072, 3072, "matvec"), (1, 3072, 4096, "matvec"), (200, 300, 1024, "tile"),
    (130, 200, 96, "simple"), (8, 130, 12288, "skinny"),
]


@pytest.mark.parametrize("m,n,k,route", RESIDUAL_SHAPES)
def test_matmul_residual(m, n, k, route):
    """q4_matmul_residual: Y = R + X deq(W)^T is bit for bit the float32 sum
    of R and q4_matmul's own result (same workspace size) on every route,
    out of place and in place (R is Y), and meets the oracle's bound plus
    the final add's rounding."""
    g = np.random.Generator(np.random.PCG64(m * 7 + n + k))
    qb_h = O.quantize_q4_0((g.standard_normal((n, k)) * 0.02).astype(np.float32))
    x_h = g.standard_normal((m, k)).astype(np.float32)
    r_h = g.standard_normal((m, n)).astype(np.float32)
    wq, x, r = dev(qb_h), dev(x_h), dev(r_h)
    ws = q4.matmul_residual_workspace(m, n, k, "cuda")
    nb = 0 if ws is None else ws.numel()
    got_route = q4.matmul_route(m, n, k, nb)
    assert route is None or got_route[0] == route, got_route
    announce(f"matmul residual {m}x{n}x{k} {got_route}")
    p = host(q4.matmul(wq, x, workspace=ws))
    want = p + r_h                                   # float32, one rounding
    y1 = host(q4.matmul_residual(wq, x, r, workspace=ws))
    y2 = r.clone()
    q4.matmul_residual(wq, x, y2, out=y2, workspace=ws)
    y2 = host(y2)
    for y, tag in ((y1, "out of place"), (y2, "in place")):
        assert np.array_equal(y.view(np.uint32), want.view(np.uint32)), \
            f"{tag}: {int((y.view(np.uint32) != want.view(np.uint32)).sum())} elements differ"
    ref, b = O.matmul_f64(qb_h, x_h, n, k)
    rel, ab = MV if m <= 4 else MF
    tot = ref + r_h.astype(np.float64)
    err = np.abs(y1.astype(np.float64) - tot)
    assert np.all(err <= rel * b + ab + 2.0 ** -23 * np.abs(tot)), float(np.max(err))


def test_matmul_residual_every_split_count():
    """The fold adds R after the slices for every K-split count (2 to 16, a
    workspace of s slices caps the split at s): bit for bit R plus
    q4_matmul's result with the same workspace, in place."""
    reached = set()
    for (m, n, k) in [(96, 512, 12288), (8, 130, 12288)]:
        qb = dev(O.quantize_q4_0(_rand_w(n, k, 61)))
        x = dev(_rand_x(m, k, 62))
        r_h = _rand_x(m, n, 63)
        for s_ in range(2, 17):
            nbytes = s_ * m * n * 4
            route, splits = q4.matmul_route(m, n, k, nbytes)
            assert 2 <= splits <= s_, (route, splits, s_)
            reached.add(splits)
            ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
            announce(f"matmul residual split count {route} {splits} (cap {s_}) {m}x{n}x{k}")
            want = host(q4.matmul(qb, x, workspace=ws)) + r_h
            y = dev(r_h)
            q4.matmul_residual(qb, x, y, out=y, workspace=ws)
            assert np.array_equal(host(y).view(np.uint32), want.view(np.uint32)), (route, splits)
    assert reached == set(range(2, 17)), sorted(reached)


def test_matmul_residual_in_place_needs_workspace():
    """In place on a route that adds R in a second launch, the product needs
    M*N floats of workspace: without them the call is refused and Y is left
    alone; with them it succeeds."""
    m, n, k = 2, 3072, 3072
    assert q4.matmul_route(m, n, k, 0)[0] == "matvec"
    assert int(q4.lib().q4_matmul_residual_workspace_bytes(m, n, k)) == m * n * 4
    qb = dev(O.quantize_q4_0(_rand_w(n, k, 51)))
    x = dev(_rand_x(m, k, 52))
    y = torch.full((m, n), 3.0, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.matmul_residual(qb, x, y, out=y, workspace=None)
    assert e.value.status == q4.Q4_ERR_WORKSPACE
    assert torch.all(y == 3.0)
    q4.matmul_residual(qb, x, y, out=y, workspace=True)
    want = host(q4.matmul(qb, x)) + np.float32(3.0)
    assert np.array_equal(host(y).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("m", [16, 38, 76])
def test_matmul_decoder_prefix_full(m):
    """The decoder projection set at the prefix lengths 16 / 38 / 76."""
    x_all = synth.activations(m, 9216, synth.seed_for(3, 20 + m))
    for t, (name, n, k) in enumerate(synth.DECODER_LAYER):
        qb = weights_q4(n, k, synth.seed_for(1, t))
        x = np.ascontiguousarray(x_all[:, :k])
        announce(f"matmul prefix M={m} {name} {n}x{k}")
        y = host(q4.matmul(dev(qb), dev(x)))
        ref, b = O.matmul_f64(qb, x, n, k)
        assert_within(y, ref, b, *MF, f"prefix M={m} {name}")


@pytest.mark.parametrize("m", [375, 1500, 3000])
def test_matmul_encoder_full(m):
    """Encoder projections (width 1280) and the adapter at floor(M/4) frames."""
    shapes = [(name, n, k, m) for (name, n, k) in synth.ENCODER_LAYER]
    shapes.append((synth.ADAPTER[0], synth.ADAPTER[1], synth.ADAPTER[2], m // 4))
    for t, (name, n, k, mm) in enumerate(shapes):
        qb = weights_q4(n, k, synth.seed_for(4, t))
        x = synth.activations(mm, k, synth.seed_for(4, 10 + t))
        announce(f"matmul encoder M={mm} {name} {n}x{k}")
        y = host(q4.matmul(dev(qb), dev(x)))
        ref, b = O.matmul_f64(qb, x, n, k)
        assert_within(y, ref, b, *MF, f"encoder M={mm} {name}")


def test_adapter_on_strided_view_of_encoder_output():
    """The 4x downsample adapter reads the encoder output in place: rows of 4
    consecutive frames of width 1280 are one row of 5120 in the same memory
    (a view, no copy), and the product matches the oracle on those rows."""
    m = 384
    _, n_up, k_up = synth.ENCODER_LAYER[1]            # any 1280-wide producer: O 1280x1280
    q_o = weights_q4(n_up, k_up, synth.seed_for(4, 1))
    x = synth.activations(m, k_up, synth.seed_for(6, 0))
    announce("adapter on the encoder output viewed as [M/4, 5120]")
    enc = q4.matmul(dev(q_o), dev(x))                  # [384, 1280] on the device
    frames = enc.view(m // 4, 4 * n_up)
    assert frames.data_ptr() == enc.data_ptr()
    name, n, k = synth.ADAPTER
    qa = weights_q4(n, k, synth.seed_for(4, 4))
    y = host(q4.matmul(dev(qa), frames))
    xa = host(enc).reshape(m // 4, 4 * n_up)
    ref, b = O.matmul_f64(qa, xa, n, k)
    assert_within(y, ref, b, *MF, "adapter on the strided view")


# --------------------------------------------------------------------------
# q4_lmhead_argmax
# --------------------------------------------------------------------------

def test_lmhead_ties_and_planted():
    n, k = 5000, 256
    w = _rand_w(n, k, 123)
    x = _rand_x(3, k, 124)
    # row 4321 is a clear winner for x[0]; rows 17 and 900 tie for x[1]
    w[4321] = np.float32(0.02) * np.sign(x[0])
    w[17] = w[900] = np.float32(0.03) * np.sign(x[1])
    qb = O.quantize_q4_0(w)
    announce("lmhead ties/planted M=3")
    idx, val = q4.lmhead_argmax(dev(qb), dev(x))
    idx, val = host(idx), host(val)
    assert idx[0] == 4321
    assert idx[1] == 17                        # lowest of two bit-identical rows
    for i in range(3):
        y, b = O.lmhead_logits(qb, x[i], n, k)
        assert O.argmax_accepts(y, b, int(idx[i])), i
        assert abs(val[i] - y[idx[i]]) <= O.MATVEC_REL * b[idx[i]] + O.MATVEC_ABS


@pytest.mark.parametrize("n,k", [(5000, 3072), (3000, 9216), (700, 96), (40, 256)])
def test_lmhead_all_logits_negative(n, k):
    """Every logit below zero: the workgroups' empty slots (no row yet) must
    never win over a real candidate in the per-workgroup fold."""
    rng = np.random.default_rng(77 + k)
    w = -np.abs(rng.standard_normal((n, k))).astype(np.float32) * np.float32(0.02)
    x = np.abs(rng.standard_normal((2, k))).astype(np.float32) + np.float32(0.1)
    qb = O.quantize_q4_0(w)
    announce(f"lmhead all-negative n={n} k={k}")
    idx, val = q4.lmhead_argmax(dev(qb), dev(x))
    idx, val = host(idx), host(val)
    for i in range(2):
        y, b = O.lmhead_logits(qb, x[i], n, k)
        assert y.max() < 0.0
        assert O.argmax_accepts(y, b, int(idx[i])), (i, int(idx[i]), O.argmax_lowest(y))
        assert abs(val[i] - y[idx[i]]) <= O.MATVEC_REL * b[idx[i]] + O.MATVEC_ABS


def _tall_view(n, k, negative=False):
    """The first n rows of the LM-head table's bytes read as an n x k Q4_0
    matrix (any k % 32 == 0 regroups the same 18-byte blocks).  negative:
    every weight made <= 0 (scale sign set, every code 8..15)."""
    nbytes = n * (k // 32) * 18
    b = lm_table().reshape(-1)[:nbytes].copy()
    if negative:
        blk = b.reshape(-1, 18)
        blk[:, 1] |= 0x80
        blk[:, 2:] |= 0x88
    return b.reshape(n, (k // 32) * 18)


@pytest.mark.parametrize("n,k", [(65549, 1024), (65601, 2048), (70001, 3072), (65536, 4096)])
def test_tall_matvec_and_argmax(n, k):
    """Tables of 65536 rows or more take four row groups per workgroup:
    ragged row counts and every K that keeps x in LDS."""
    qb = _tall_view(n, k)
    x = _rand_x(2, k, 900 + k)
    wq = dev(qb)
    announce(f"tall matvec/argmax n={n} k={k}")
    y = host(q4.matvec(wq, dev(x[0])))
    idx, val = q4.lmhead_argmax(wq, dev(x))
    idx, val = host(idx), host(val)
    ref, b = O.lmhead_logits(qb, x[0], n, k)
    assert_within(y, ref, b, *MV, f"tall matvec n={n} k={k}")
    for i in range(2):
        yi, bi = (ref, b) if i == 0 else O.lmhead_logits(qb, x[i], n, k)
        assert O.argmax_accepts(yi, bi, int(idx[i])), (i, int(idx[i]), O.argmax_lowest(yi))
        assert abs(val[i] - yi[idx[i]]) <= O.MATVEC_REL * bi[idx[i]] + O.MATVEC_ABS


def test_tall_argmax_all_logits_negative():
    n, k = 70001, 3072
    qb = _tall_view(n, k, negative=True)
    x = np.abs(_rand_x(1, k, 4321)) + np.float32(0.1)
    announce("tall argmax all-negative")
    idx, val = q4.lmhead_argmax(dev(qb), dev(x))
    y, b = O.lmhead_logits(qb, x[0], n, k)
    assert y.max() < 0.0
    i = int(host(idx)[0])
    assert O.argmax_accepts(y, b, i), (i, O.argmax_lowest(y))


def test_lmhead_workspace_reuse_and_odd_k():
    """The workspace starts zeroed and every call leaves it zeroed, so calls
    ordered on one stream can share it; K % 64 == 32 takes the generic kernel."""
    for (n, k) in [(700, 96), (5000, 3072)]:
        qb = O.quantize_q4_0(_rand_w(n, k, 5 + k))
        ws = q4.lmhead_workspace(2, "cuda")
        wq = dev(qb)
        for s in range(4):
            x = _rand_x(2, k, 300 + s)
            announce(f"lmhead reuse n={n} k={k} call {s}")
            idx, _ = q4.lmhead_argmax(wq, dev(x), workspace=ws)
            idx = host(idx)
            for i in range(2):
                y, b = O.lmhead_logits(qb, x[i], n, k)
                assert O.argmax_accepts(y, b, int(idx[i]))
            assert not host(ws).any(), "workspace not left zeroed"


def test_lmhead_full_table():
    table = lm_table()
    x = synth.activations(1, synth.DEC_DIM, synth.seed_for(2, 1))
    announce("lmhead full table")
    idx, val = q4.lmhead_argmax(dev(table), dev(x))
    i = int(host(idx)[0])
    y, b = O.lmhead_logits(table, x[0], synth.VOCAB, synth.DEC_DIM)
    assert O.argmax_accepts(y, b, i), (i, O.argmax_lowest(y), O.top2_margin(y))
    assert abs(float(host(val)[0]) - y[i]) <= O.MATVEC_REL * b[i] + O.MATVEC_ABS
    # the full logit vector of the same kernel family agrees everywhere
    yy = host(q4.matvec(dev(table), dev(x[0])))
    assert_within(yy, y, b, *MV, "lmhead logits")


# --------------------------------------------------------------------------
# Determinism and out-of-bounds writes
# --------------------------------------------------------------------------

def test_determinism():
    qb = dev(weights_q4(3072, 3072, synth.seed_for(0, 0)))
    x = dev(synth.activations(76, 3072, 55))
    announce("determinism")
    a = host(q4.matvec(qb, x[0]))
    b = host(q4.matvec(qb, x[0]))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    a = host(q4.matmul(qb, x))
    b = host(q4.matmul(qb, x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    i1, v1 = q4.lmhead_argmax(qb, x[:1])
    i2, v2 = q4.lmhead_argmax(qb, x[:1])
    assert host(i1)[0] == host(i2)[0] and host(v1)[0] == host(v2)[0]


@pytest.mark.parametrize("op,m,n,k", [
    ("matvec", 1, 130, 128), ("matvec", 3, 130, 3072), ("matvec", 2, 131, 9216),
    ("matvec", 1, 5, 4096), ("matmul", 97, 512, 128), ("matmul", 130, 256, 640),
    ("matmul", 16, 130, 320), ("matmul", 40, 257, 192), ("matmul", 2, 70, 1088)])
def test_outputs_written_exactly(op, m, n, k):
    """Every element of Y written and nothing around it: the matvec pair
    kernel stores through a resource covering a pass's rows (the rows past N
    of a ragged last pass dropped by its range check), the wide GEMM drops the
    rows past M the same way, the skinny GEMM ends on a partial stage."""
    qb = dev(O.quantize_q4_0(_rand_w(n, k, 3 + n)))
    x = dev(_rand_x(m, k, 4 + m))
    sentinel = -12345.0
    pad = 64
    buf = torch.full((m * n + 2 * pad,), sentinel, dtype=torch.float32, device="cuda")
    y = buf[pad: pad + m * n].view(m, n)
    announce(f"outputs written exactly: {op} {m}x{n}x{k}")
    if op == "matvec":
        q4.matvec(qb, x, out=y)
    else:
        q4.matmul(qb, x, out=y, workspace=None)
    got = host(buf)
    assert np.all(got[:pad] == sentinel) and np.all(got[pad + m * n:] == sentinel)
    assert not np.any(got[pad: pad + m * n] == sentinel)


def test_no_write_past_outputs():
    n, k, m = 130, 96, 3
    qb = dev(O.quantize_q4_0(_rand_w(n, k, 1)))
    x = dev(_rand_x(m, k, 2))
    sentinel = -12345.0
    announce("canary matvec/matmul/embed")
    buf = torch.full((m * n + 64,), sentinel, dtype=torch.float32, device="cuda")
    q4.matvec(qb, x, out=buf[: m * n].view(m, n))
    assert np.all(host(buf)[m * n:] == sentinel)
    buf.fill_(sentinel)
    q4.matmul(qb, x, out=buf[: m * n].view(m, n))
    assert np.all(host(buf)[m * n:] == sentinel)
    ids = dev(np.array([1, 2, 129], np.int32))
    buf = torch.full((3 * k + 64,), sentinel, dtype=torch.float32, device="cuda")
    q4.embed_rows(qb, ids, out=buf[: 3 * k].view(3, k))
    assert np.all(host(buf)[3 * k:] == sentinel)


@pytest.mark.parametrize("n,k", [(300, 1088), (3000, 3072), (3072, 4096), (700, 9216),
                                 (65600, 1024), (70, 12320), (40, 13312)])
@pytest.mark.parametrize("m", [2, 3, 5, 8])
def test_matvec_rows_as_alone(m, n, k):
    """Rows of x taken in pairs by one workgroup (weights decoded once for
    both) give every row the bits it has in a call with that row alone, on
    every variant (x in LDS, four row groups, x in registers, the generic
    kernel) and with an odd last row; each row also meets the oracle."""
    qb = O.quantize_q4_0(_rand_w(n, k, 41 + m))
    x = _rand_x(m, k, 42 + m)
    wq, xd = dev(qb), dev(x)
    announce(f"matvec rows as alone {q4.matvec_route(n, k)} M={m} {n}x{k}")
    y = host(q4.matvec(wq, xd))
    ref, b = O.matmul_f64(qb, x, n, k)
    assert_within(y, ref, b, *MV, f"rows as alone M={m} {n}x{k}")
    for i in range(m):
        yi = host(q4.matvec(wq, xd[i:i + 1]))[0]
        assert np.array_equal(y[i].view(np.uint32), yi.view(np.uint32)), (m, i)


@pytest.mark.parametrize("n,k", [(65600, 1024), (65549, 3072)])
@pytest.mark.parametrize("m", [2, 3, 5])
def test_lmhead_rows_as_alone(m, n, k):
    """Tall tables take the rows of x in pairs (the table is read once per
    pair): every row gets the index and the bit-identical value of a call
    with that row alone, the odd last row included; each index is accepted
    by the oracle.  At M = 2 row 0 has a planted winner and row 1 a tie
    between two identical rows (lowest index); at M > 2 every weight is
    made non-negative and row 2 of x negative, so all of row 2's logits are
    negative."""
    w = _rand_w(n, k, 61 + m)
    x = _rand_x(m, k, 62 + m)
    if m == 2:
        w[n - 7] = np.float32(0.02) * np.sign(x[0])
        w[123] = w[60000] = np.float32(0.03) * np.sign(x[1])
    else:
        w = np.abs(w)
        x[2] = -np.abs(x[2]) - np.float32(0.5)
    qb = O.quantize_q4_0(w)
    wq, xd = dev(qb), dev(x)
    announce(f"argmax rows as alone {q4.matvec_route(n, k, argmax=True)} M={m} {n}x{k}")
    idx, val = q4.lmhead_argmax(wq, xd)
    idx, val = host(idx), host(val)
    if m == 2:
        assert int(idx[0]) == n - 7 and int(idx[1]) == 123, idx
    for i in range(m):
        ii, vi = q4.lmhead_argmax(wq, xd[i:i + 1])
        assert int(host(ii)[0]) == int(idx[i]), (m, i)
        assert host(vi)[0].view(np.uint32) == val[i].view(np.uint32), (m, i)
        y, b = O.lmhead_logits(qb, x[i], n, k)
        assert O.argmax_accepts(y, b, int(idx[i])), (m, i, int(idx[i]), O.argmax_lowest(y))
        if m > 2 and i == 2:
            assert float(val[i]) < 0.0
