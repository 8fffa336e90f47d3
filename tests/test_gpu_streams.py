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
        rr = torch.ones((m, n), device="cuda")
        side.wait_stream(torch.cuda.current_stream())
        yr = q4.matmul_residual(wq, xd, rr, stream=side)
        emb = q4.embed_rows(wq, idd, stream=side)
        idx, val = q4.lmhead_argmax(wq, xd[:3], stream=side)
        side.synchronize()
        assert np.array_equal(enc.cpu().numpy(), qb)
        ref, b = O.matmul_f64(qb, x, n, k)
        assert_within(yv.cpu().numpy(), ref[:2], b[:2], O.MATVEC_REL, O.MATVEC_ABS, "matvec side")
        assert_within(ym.cpu().numpy(), ref, b, O.MFMA_REL, O.MFMA_ABS, "matmul side")
        assert np.array_equal(yr.cpu().numpy().view(np.uint32),
                              (ym.cpu().numpy() + np.float32(1.0)).view(np.uint32))
        assert np.array_equal(emb.cpu().numpy(), O.embed_rows(qb, ids, n, k))
        for i in range(3):
            assert O.argmax_accepts(ref[i], b[i], int(idx[i].item()))
        del enc, yv, ym, yr, rr, emb, idx, val          # back to the side stream's pool
    torch.cuda.synchronize()


def test_host_threads_at_once():
    """Four host threads, each with its own stream, call the entry points at
    the same time (the binding's ctypes calls release the interpreter lock,
    so the library's first calls and their cached device and occupancy
    figures race for real); every result is checked against the oracle."""
    import threading

    cases = [(1, 3072, 3072), (2, 1536, 4096), (40, 2048, 3072), (300, 1280, 1280)]
    inputs = []
    for t, (m, n, k) in enumerate(cases):
        qb = O.quantize_q4_0(synth.weights(n, k, 4300 + t))
        x = synth.activations(m, k, 4310 + t)
        ref, b = O.matmul_f64(qb, x, n, k)
        inputs.append((m, n, k, qb, x, ref, b, dev(qb), dev(x)))
    torch.cuda.synchronize()
    results, errors = {}, []

    def work(t):
        try:
            m, n, k, _, _, _, _, wq, xd = inputs[t]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = []
                for _ in range(5):
                    outs.append((q4.matvec(wq, xd[:min(m, 8)], stream=s),
                                 q4.matmul(wq, xd, stream=s),
                                 q4.lmhead_argmax(wq, xd[:1], stream=s)))
            s.synchronize()
            results[t] = [(a.cpu().numpy(), c.cpu().numpy(), int(i[0].item()))
                          for a, c, (i, _) in outs]
        except Exception as e:  # reported below, on the main thread
            errors.append((t, repr(e)))

    announce("four host threads at once")
    threads = [threading.Thread(target=work, args=(t,)) for t in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=90)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    for t, (m, n, k, qb, x, ref, b, _, _) in enumerate(inputs):
        mv = min(m, 8)
        for yv, ym, idx in results[t]:
            assert_within(yv, ref[:mv], b[:mv], O.MATVEC_REL, O.MATVEC_ABS, f"thread {t} matvec")
            assert_within(ym, ref, b, *((O.MATVEC_REL, O.MATVEC_ABS) if m <= 4
                                        else (O.MFMA_REL, O.MFMA_ABS)), f"thread {t} matmul")
            assert O.argmax_accepts(ref[0], b[0], idx), (t, idx)
