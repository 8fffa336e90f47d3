"""q4_matmul with 1 to 4 rows of x meets the matvec bound (1e-4 * B + 1e-6),
not only the binary16 one, on both of its routes: the matvec kernel once per
row of x (one row, K % 64 == 32, weights whose repeated reads stay in the
caches) and the small-M kernel (weights read once and multiplied on the matrix
cores with exact q - 8 operands, the block scales applied in float32 and x
carried as two binary16 parts; K > 12288 always takes it).  Row counts just
past it (5 to 16) take the binary16 kernels and are held to the binary16
bound.
Shapes follow the decoder of the model the pages run (section "Architecture" of
"Implémentation en Rust du modèle Voxtral Mini 4B Realtime de Mistral pour
l'exécuter dans le navigateur"): several decode streams or a short prefix."""

import numpy as np
import pytest
import torch

import q4_quantized_speech_amd as q4
from gpu_util import announce, assert_within, dev, host, needs_gpu, weights_q4
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


@pytest.mark.parametrize("k", [1280, 12352])
@pytest.mark.parametrize("case", ["tiny", "huge", "spread", "zero_row", "mixed_rows"])
def test_small_m_x_range(case, k):
    """x far from 1 keeps the bound on both routes (K = 12352: the small-M
    kernel's per-chunk power-of-two scaling): all tiny, all huge (past
    binary16's range), one large value among small ones, a row of zeros, rows
    of very different magnitudes."""
    m, n = 4, 96
    qb = _w(n, k, 5)
    g = np.random.Generator(np.random.PCG64(6))
    x = g.standard_normal((m, k))
    if case == "tiny":
        x *= 1e-30
    elif case == "huge":
        x *= 1e6
    elif case == "spread":
        x *= 1e-3
        x[:, 77] = 1e4
    elif case == "zero_row":
        x[2] = 0.0
    else:
        x *= np.array([1e-20, 1e8, 1e-3, 1e-12])[:, None]
    x = x.astype(np.float32)
    ref, b = O.matmul_f64(qb, x, n, k)
    announce(f"small-M x range {case} k={k}")
    y = host(q4.matmul(dev(qb), dev(x)))
    assert_within(y, ref, b, *MV, f"x range {case}")
    if case == "zero_row":
        assert np.all(y[2] == 0.0)


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
    need = int(q4.lib().q4_matmul_workspace_bytes(m, n, k))
    assert need > 0, "a K split is planned for this shape"
    sentinel = -12345.0
    ws = torch.full((need // 4 + 64,), sentinel, dtype=torch.float32, device="cuda")
    out = torch.full((m * n + 64,), sentinel, dtype=torch.float32, device="cuda")
    announce("small-M canary")
    q4.matmul(qb, x, out=out[: m * n].view(m, n), workspace=ws[: need // 4].view(torch.uint8))
    first = host(out)[: m * n].copy()
    assert np.all(host(ws)[need // 4:] == sentinel)
    assert np.all(host(out)[m * n:] == sentinel)
    q4.matmul(qb, x, out=out[: m * n].view(m, n), workspace=ws[: need // 4].view(torch.uint8))
    assert np.array_equal(host(out)[: m * n].view(np.uint32), first.view(np.uint32))


@pytest.mark.parametrize("m,n,k", [(1, 6144, 3072), (2, 300, 1088), (4, 3072, 4096),
                                   (3, 65, 1056), (2, 18432, 3072)])
def test_small_m_stream_route_is_matvec(m, n, k):
    """Where the rows go through the matvec kernel, q4_matmul returns exactly
    q4_matvec's bits (the same kernel, no workspace planned)."""
    assert int(q4.lib().q4_matmul_workspace_bytes(m, n, k)) == 0
    qb = dev(weights_q4(n, k, synth.seed_for(1, n + k)))
    x = dev(synth.activations(m, k, synth.seed_for(3, m + k)))
    announce(f"small-M stream route {m}x{n}x{k}")
    a = host(q4.matmul(qb, x))
    b = host(q4.matvec(qb, x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
