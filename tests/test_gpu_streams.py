"""Every entry point called on a side stream while the current stream is
busy, with the binding allocating its outputs and scratch (the argmax's zeroed
workspace, the matmul's K-split workspace, the encoder's error flag): those
allocations and fills must be ordered on the stream the kernel runs on.
Results are compared with the oracle."""

import numpy as np
import pytest
import torch

import q4_quantized_speech_amd as q4
from gpu_util import announce, assert_within, dev, needs_gpu
from oracle import q4_oracle as O
from q4_quantized_speech_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]


def _busy(a):
    """Queue a few large products on the current stream."""
    for _ in range(3):
        a = a @ a
        a /= a.abs().max()
    return a


def test_entry_points_on_a_side_stream():
    n, k, m = 2048, 3072, 40
    w = synth.weights(n, k, 4242)
    qb = O.quantize_q4_0(w)
    x = synth.activations(m, k, 4243)
    ids = synth.token_ids(8, 4244, vocab=n)
    wq, xd, idd, wf = dev(qb), dev(x), dev(ids), dev(w)
    busy = torch.randn(4096, 4096, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())      # inputs are ready
    for rep in range(3):
        announce(f"side stream rep {rep}")
        busy = _busy(busy)
        enc = q4.quantize(wf, stream=side)
        yv = q4.matvec(wq, xd[:2], stream=side)
        ym = q4.matmul(wq, xd, stream=side)             # workspace allocated here
        emb = q4.embed_rows(wq, idd, stream=side)
        idx, val = q4.lmhead_argmax(wq, xd[:3], stream=side)
        side.synchronize()
        assert np.array_equal(enc.cpu().numpy(), qb)
        ref, b = O.matmul_f64(qb, x, n, k)
        assert_within(yv.cpu().numpy(), ref[:2], b[:2], O.MATVEC_REL, O.MATVEC_ABS, "matvec side")
        assert_within(ym.cpu().numpy(), ref, b, O.MFMA_REL, O.MFMA_ABS, "matmul side")
        assert np.array_equal(emb.cpu().numpy(), O.embed_rows(qb, ids, n, k))
        for i in range(3):
            assert O.argmax_accepts(ref[i], b[i], int(idx[i].item()))
        del enc, yv, ym, emb, idx, val                  # back to the side stream's pool
    torch.cuda.synchronize()
