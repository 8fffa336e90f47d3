"""q4_matmul with 1 to 4 rows of x meets the matvec bound (1e-4 * B + 1e-6),
not only the binary16 one, on each of its routes: the matvec kernel (rows of
x in pairs; one or two rows, K % 64 == 32, and K past 6144 with weights whose
repeated reads stay in the caches), the stream16 kernel for three or four
rows with K <= 6144 and the small-M kernel for the rest (both read the
weights once and multiply them on the matrix cores as exact q - 8 operands,
the block scales applied in float32 and x carried as two binary16 parts
after a power-of-two scaling per 256-value chunk).  Row counts just
past it (5 to 16) take binary16 x (the stream16 kernel: weights exact, read
once, one MFMA per block for all the rows) and are held to the binary16
bound.
Shapes follow the decoder of the model the pages run (section "Architecture" of
"Implémentation en Rust du modèle Voxtral Mini 4B Realtime de Mistral pour
l'exécuter dans le navigateur"): several decode streams or a short prefix."""

import numpy as np
import pytest
import torch

import q4_quantized_speech_amd as q4
from gpu_util import announce, assert_within, dev, host, needs_gpu, weights_q4
from test_gpu_parity import split_canary_workspace
from oracle import q4_oracle as O
from q4_quantized_speech_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]

MV = (O.MATVEC_REL, O.MATVEC_ABS)
MF = (O.MFMA_REL, O.MFMA_ABS)


def _bound(m):
    return MV if m <= 4 else MF


def _w(n, k, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return O.quantize_q4_0((g.standard_normal((n, k)) * 0.02).astype(np.float32))


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 15, 16])
@pytest.mark.parametrize("n,k", [(1, 64), (63, 192), (64, 256), (65, 320), (300, 1088),
                                 (130, 2048), (65, 1056), (1, 12352), (63, 12352),
                                 (130, 12352), (64, 12320)])
def test_small_m_matvec_bound(m, n, k):
    """Ragged row tiles (N around 64), chunks cut short (K not a multiple of
    256), several x segments (K > 1024), K % 64 == 32; K = 12352 puts M <= 4
    on the small-M kernel; with and without a K split."""
    qb = _w(n, k, 13 * m + n + k)
    x = synth.activations(m, k, 17 + m + k)
    ref, b = O.matmul_f64(qb, x, n, k)
    wq, xd = dev(qb), dev(x)
    for ws in (True, None):
        announce(f"small-M matmul {m}x{n}x{k} workspace={ws is not None}")
        y = host(q4.matmul(wq, xd, workspace=ws))
        assert_within(y, ref, b, *_bound(m), f"small-M {m}x{n}x{k} ws={ws is not None}")


@pytest.mark.parametrize("k", [1280, 4352, 12352])
@pytest.mark.parametrize("case", ["tiny", "huge", "spread", "zero_row", "mixed_rows",
                                  "outlier_1e9", "outlier_1e11", "outlier_1e30", "outlier_3e38",
                                  "huge_3e35", "tiny_among_normal"])
def test_small_m_x_range(case, k):
    """x far from 1 keeps the bound on the routes with a per-chunk
    power-of-two scaling of x (K = 1280 and 4352: the stream16 kernel with
    one and two chunks per wave; K = 12352: the small-M kernel): all tiny, all huge (past
    binary16's range), one large value among small ones, a row of zeros, rows
    of very different magnitudes; huge values on zero-weight columns (they
    set a chunk's scale but add nothing, so the chunk's other values must
    keep their precision: the kernel's float32 path for wide chunks); chunks
    of +-1e38 against a few nonzero weight columns (scaling them for binary16
    would overflow); tiny values scattered among normal ones."""
    m, n = 4, 96
    g = np.random.Generator(np.random.PCG64(6))
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = g.standard_normal((m, k))
    cols = [3, 77, k // 2 + 5, k - 1]
    if case == "tiny":
        x *= 1e-30
    elif case == "huge":
        x *= 1e6
    elif case == "spread":
        x *= 1e-3
        x[:, 77] = 1e4
    elif case == "zero_row":
        x[2] = 0.0
    elif case == "mixed_rows":
        x *= np.array([1e-20, 1e8, 1e-3, 1e-12])[:, None]
    elif case.startswith("outlier"):
        w[:, cols] = 0.0                       # a zero column quantises to code 8
        x[:, cols] = float(case.split("_")[1])
        x[1, cols] *= -1.0
    elif case == "huge_3e35":
        x *= 3e35
        x[2] *= 1e-10                          # one row far below the others
    else:
        x[:, ::97] *= 1e-9
    qb = O.quantize_q4_0(w)
    x = x.astype(np.float32)
    ref, b = O.matmul_f64(qb, x, n, k)
    announce(f"small-M x range {case} k={k} route={q4.matmul_route(m, n, k, 0)}")
    y = host(q4.matmul(dev(qb), dev(x)))
    assert_within(y, ref, b, *MV, f"x range {case}")
    if case == "zero_row":
        assert np.all(y[2] == 0.0)


@pytest.mark.parametrize("case", ["normal", "huge", "spread", "zero_row", "mixed_rows",
                                  "outlier_1e11", "outlier_3e38", "huge_3e35"])
def test_two_rows_stream16(case):
    """Two rows of x over 20 MiB of weights with K <= 3072 take the stream16
    kernel with x in two binary16 parts; they keep the q4_matvec bound over
    x far from 1 (cases as in the x-range test above, rows 0 and 1)."""
    m, n, k = 2, 12288, 3072
    assert q4.matmul_route(m, n, k, 0) == ("stream16", 1)
    g = np.random.Generator(np.random.PCG64(66))
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = g.standard_normal((m, k))
    cols = [3, 77, k // 2 + 5, k - 1]
    if case == "huge":
        x *= 1e6
    elif case == "spread":
        x *= 1e-3
        x[:, 77] = 1e4
    elif case == "zero_row":
        x[1] = 0.0
    elif case == "mixed_rows":
        x *= np.array([1e-20, 1e8])[:, None]
    elif case.startswith("outlier"):
        w[:, cols] = 0.0
        x[:, cols] = float(case.split("_")[1])
        x[1, cols] *= -1.0
    elif case == "huge_3e35":
        x *= 3e35
        x[1] *= 1e-10
    qb = O.quantize_q4_0(w)
    x = x.astype(np.float32)
    ref, b = O.matmul_f64(qb, x, n, k)
    announce(f"two rows stream16 {case} {m}x{n}x{k}")
    y = host(q4.matmul(dev(qb), dev(x)))
    assert_within(y, ref, b, *MV, f"two rows {case}")
    if case == "zero_row":
        assert np.all(y[1] == 0.0)


@pytest.mark.parametrize("m", [2, 3, 4])
def test_small_m_decoder_layer(m):
    """The four decoder projections at their real shapes, all outputs."""
    x_all = synth.activations(m, 9216, synth.seed_for(3, 40 + m))
    for t, (name, n, k) in enumerate(synth.DECODER_LAYER):
        qb = weights_q4(n, k, synth.seed_for(1, t))
        x = np.ascontiguousarray(x_all[:, :k])
        announce(f"small-M decoder M={m} {name} {n}x{k}")
        y = host(q4.matmul(dev(qb), dev(x)))
        ref, b = O.matmul_f64(qb, x, n, k)
        assert_within(y, ref, b, *MV, f"small-M decoder M={m} {name}")


def test_small_m_deterministic_and_in_bounds():
    """Bit-identical on repeat; partial sums inside the workspace and results
    inside Y (sentinels around both stay untouched)."""
    m, n, k = 3, 200, 12352
    qb = dev(_w(n, k, 21))
    x = dev(synth.activations(m, k, 22))
    sentinel = -12345.0
    ws, need = split_canary_workspace(m, n, k, sentinel)
    out = torch.full((m * n + 64,), sentinel, dtype=torch.float32, device="cuda")
    announce("small-M canary")
    q4.matmul(qb, x, out=out[: m * n].view(m, n), workspace=ws[: need // 4].view(torch.uint8))
    first = host(out)[: m * n].copy()
    assert np.all(host(ws)[need // 4:] == sentinel)
    assert np.all(host(out)[m * n:] == sentinel)
    q4.matmul(qb, x, out=out[: m * n].view(m, n), workspace=ws[: need // 4].view(torch.uint8))
    assert np.array_equal(host(out)[: m * n].view(np.uint32), first.view(np.uint32))


@pytest.mark.parametrize("m", [5, 9, 16])
@pytest.mark.parametrize("n,k", [(1, 64), (17, 256), (33, 4352), (300, 4096), (31, 6080),
                                 (40, 6144)])
def test_stream16_edges(m, n, k):
    """5 to 16 rows of x on the stream16 kernel, at its edges: a workgroup of
    one wave (K = 64: the 256 outputs of a pass taken in turns), one full
    chunk, 17 chunks (two per wave, the last wave's second chunk empty), 16
    waves of one chunk, a last chunk cut short, 24 chunks in 12 waves; N not
    a multiple of the 16 weight rows of a pass.  No workspace is planned, the
    same bits come back on a repeat, and nothing past Y is written."""
    assert q4.matmul_route(m, n, k, 1 << 30) == ("stream16", 1)
    assert int(q4.lib().q4_matmul_workspace_bytes(m, n, k)) == 0
    qb = _w(n, k, 31 * m + n + k)
    x = synth.activations(m, k, 19 + m + k)
    ref, b = O.matmul_f64(qb, x, n, k)
    wq, xd = dev(qb), dev(x)
    sentinel = -12345.0
    out = torch.full((m * n + 64,), sentinel, dtype=torch.float32, device="cuda")
    announce(f"stream16 edge {m}x{n}x{k}")
    q4.matmul(wq, xd, out=out[: m * n].view(m, n))
    first = host(out)
    assert np.all(first[m * n:] == sentinel)
    assert_within(first[: m * n].reshape(m, n), ref, b, *MF, f"stream16 {m}x{n}x{k}")
    q4.matmul(wq, xd, out=out[: m * n].view(m, n))
    assert np.array_equal(host(out).view(np.uint32), first.view(np.uint32))


@pytest.mark.parametrize("m", [17, 32, 33, 38, 48])
@pytest.mark.parametrize("n,k", [(1, 64), (17, 256), (300, 3072), (31, 2880), (70, 1216)])
def test_stream16_tiles_edges(m, n, k):
    """17 to 48 rows of x on the stream16 kernel: two or three tiles of 16
    rows (the last one partly past M), one wave per 256-value chunk up to
    K = 3072, a last chunk cut short, N not a multiple of 16; the binary16
    bound, the same bits on a repeat, nothing written past Y."""
    assert q4.matmul_route(m, n, k, 1 << 30) == ("stream16", 1)
    qb = _w(n, k, 37 * m + n + k)
    x = synth.activations(m, k, 23 + m + k)
    ref, b = O.matmul_f64(qb, x, n, k)
    wq, xd = dev(qb), dev(x)
    sentinel = -12345.0
    out = torch.full((m * n + 64,), sentinel, dtype=torch.float32, device="cuda")
    announce(f"stream16 tiles {m}x{n}x{k}")
    q4.matmul(wq, xd, out=out[: m * n].view(m, n))
    first = host(out)
    assert np.all(first[m * n:] == sentinel)
    assert_within(first[: m * n].reshape(m, n), ref, b, *MF, f"stream16 tiles {m}x{n}x{k}")
    q4.matmul(wq, xd, out=out[: m * n].view(m, n))
    assert np.array_equal(host(out).view(np.uint32), first.view(np.uint32))


@pytest.mark.parametrize("m,n,k", [(1, 6144, 3072), (2, 300, 1088), (4, 300, 6208),
                                   (3, 65, 1056), (2, 9216, 3072), (2, 12288, 4096),
                                   (2, 3072, 9216)])
def test_small_m_stream_route_is_matvec(m, n, k):
    """Where the rows go through the matvec kernel, q4_matmul returns exactly
    q4_matvec's bits (the same kernel, no workspace planned); two rows of x
    take that route unless K <= 3072 with 20 MiB of weights or more."""
    assert int(q4.lib().q4_matmul_workspace_bytes(m, n, k)) == 0
    qb = dev(weights_q4(n, k, synth.seed_for(1, n + k)))
    x = dev(synth.activations(m, k, synth.seed_for(3, m + k)))
    announce(f"small-M stream route {m}x{n}x{k}")
    a = host(q4.matmul(qb, x))
    b = host(q4.matvec(qb, x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
