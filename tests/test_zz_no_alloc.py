"""q4_lmhead_argmax_noalloc (the argmax with the library's own per-device
scratch, for callers that cannot allocate) against q4_lmhead_argmax with a
caller workspace: same index, bit-identical value, and the oracle's
acceptance, on two calls in a row, the second with a smaller input (fewer
rows of x and a smaller table), so the scratch left by the first call must
be clean for the second.  Runs alone in a fresh process and after the other
GPU tests."""

import numpy as np
import pytest
import torch

import q4_quantized_speech_amd as q4
from gpu_util import announce, dev, host, needs_gpu
from oracle import q4_oracle as O
from q4_quantized_speech_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]


def _case(n, k, m, seed):
    qb = O.quantize_q4_0(synth.weights(n, k, seed))
    x = synth.activations(m, k, seed + 1)
    return qb, x


def test_noalloc_argmax_matches_workspace_entry_point():
    cases = [(20000, 3072, 5, 7100), (3000, 1024, 2, 7200), (70001, 1024, 64, 7300),
             (257, 96, 1, 7400)]
    for n, k, m, seed in cases:
        qb, x = _case(n, k, m, seed)
        wq, xd = dev(qb), dev(x)
        announce(f"noalloc argmax n={n} k={k} m={m}")
        oi = torch.full((m,), -7, dtype=torch.int32, device="cuda")
        ov = torch.full((m,), -7.0, dtype=torch.float32, device="cuda")
        q4.lmhead_argmax_noalloc(wq, xd, oi, ov)
        ri, rv = q4.lmhead_argmax(wq, xd)
        gi, gv, ri, rv = host(oi), host(ov), host(ri), host(rv)
        assert np.array_equal(gi, ri), (n, k, m)
        assert np.array_equal(gv.view(np.uint32), rv.view(np.uint32)), (n, k, m)
        for i in range(m):
            y, b = O.lmhead_logits(qb, x[i], n, k)
            assert O.argmax_accepts(y, b, int(gi[i])), (n, k, m, i)
    # value output optional
    oi = torch.empty(1, dtype=torch.int32, device="cuda")
    q4.lmhead_argmax_noalloc(wq, xd[:1], oi)
    assert int(host(oi)[0]) == int(ri[0])


def test_noalloc_argmax_rejects_more_rows_than_its_scratch():
    qb, x = _case(64, 64, 65, 7500)
    oi = torch.empty(65, dtype=torch.int32, device="cuda")
    with pytest.raises(q4.Q4Error, match="out of range"):
        q4.lmhead_argmax_noalloc(dev(qb), dev(x), oi)
