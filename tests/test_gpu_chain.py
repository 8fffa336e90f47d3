"""q4_decode_chain -- a greedy decode step's Q4_0 work as one call (section
"Architecture" of "Implémentation en Rust du modèle Voxtral Mini 4B Realtime
de Mistral pour l'exécuter dans le navigateur": the decoder's projections
once per token; section "Solutions techniques pour l'exécution dans le
navigateur", item 3: the Q4 table gives the logits and the next token's
embedding) -- against the oracle, bit for bit.

Each step's x is a slice of the previous step's y on the device, so the
dependency is real.  The inputs are chosen so that every product and every
partial sum is an integer below 2^24, exact in float32 whatever the order of
the additions: block scales of 1.0, weights in {-1, 0, 1} (codes 7, 8, 9)
with a few nonzero weights per row, and integer x.  The device's y, the
argmax index (lowest on ties), its value and the chosen token's decoded row
must then equal the oracle's float64 chain exactly, and the input of every
step is the same on both sides without any device value entering the
oracle.  (The matvec's accuracy on real-valued data is what the q4_matvec
and q4_lmhead_argmax parity tests check; here the composition is checked.)"""

import ctypes

import numpy as np
import pytest
import torch

import q4_quantized_speech_amd as q4
from gpu_util import announce, dev, host, needs_gpu
from oracle import q4_oracle as O
from q4_quantized_speech_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]

ONE = (0x00, 0x3C)   # binary16 1.0, little-endian


def ternary_q4(n, k, nnz, seed):
    """Q4_0 bytes of an n x k matrix with scale 1.0 in every block and `nnz`
    weights of +-1 per row at random columns (code 9 or 7), code 8 elsewhere."""
    g = np.random.Generator(np.random.PCG64(seed))
    nb = k // 32
    b = np.empty((n, nb, 18), np.uint8)
    b[..., 0], b[..., 1] = ONE
    b[..., 2:] = 0x88
    cols = np.argsort(g.random((n, k)), axis=1)[:, :nnz]
    sign = g.integers(0, 2, (n, nnz)) * 2 - 1
    rows = np.repeat(np.arange(n), nnz)
    c = cols.reshape(-1)
    blk, e = c // 32, c % 32
    byte = 2 + (e % 16)
    shift = np.where(e < 16, 0, 4)
    code = (8 + sign.reshape(-1)).astype(np.uint8)
    cur = b[rows, blk, byte]
    b[rows, blk, byte] = (cur & ~(0x0F << shift).astype(np.uint8)) | (code << shift).astype(np.uint8)
    return b.reshape(n, nb * 18)


def oracle_chain(steps, x0):
    """steps: [(qb, n, k, slice of the previous y that is x)]; float64."""
    ys = []
    x = np.asarray(x0, np.float64)
    for i, (qb, n, k, sl) in enumerate(steps):
        if i > 0:
            x = ys[-1][sl[0]:sl[1]]
        ys.append(O.dequantize_q4_0(qb, n, k).astype(np.float64) @ x)
    return ys


def run_chain(steps, x0, table=None, head_slice=None, workspace=None):
    dw = [dev(qb) for (qb, _, _, _) in steps]
    ys = [torch.full((n,), np.nan, dtype=torch.float32, device="cuda") for (_, n, _, _) in steps]
    xd = dev(x0)
    call = [(dw[i], xd if i == 0 else ys[i - 1][sl[0]:sl[1]], ys[i])
            for i, (_, _, _, sl) in enumerate(steps)]
    kw = {}
    if table is not None:
        src = ys[-1] if steps else xd
        kw = dict(table_q4=dev(table), head_x=src[head_slice[0]:head_slice[1]],
                  out_val=torch.empty(1, device="cuda"), workspace=workspace,
                  out_embed=torch.full((head_slice[1] - head_slice[0],), np.nan,
                                       dtype=torch.float32, device="cuda"))
    idx, val, emb = q4.decode_chain(call, **kw)
    torch.cuda.synchronize()
    return [host(y) for y in ys], idx, val, emb


def check_chain(steps, x0, table=None, vocab=0, dim=0, head_slice=None):
    ref = oracle_chain(steps, x0)
    assert all(np.all(np.abs(y) < 2 ** 24) for y in ref), "inputs leave the exact range"
    ys, idx, val, emb = run_chain(steps, x0, table, head_slice)
    for i, (y_ref, y) in enumerate(zip(ref, ys)):
        assert np.array_equal(y.astype(np.float64), y_ref), (i, int((y != y_ref).sum()))
    if table is None:
        return
    hx = (ref[-1] if steps else np.asarray(x0, np.float64))[head_slice[0]:head_slice[1]]
    y, _ = O.lmhead_logits(table, hx.astype(np.float32), vocab, dim)
    assert np.all(np.abs(y) < 2 ** 24)
    best = O.argmax_lowest(y)
    assert int(host(idx)[0]) == best
    assert float(host(val)[0]) == y[best]
    want = O.embed_rows(table, np.array([best], np.int32), vocab, dim)[0]
    got = host(emb)
    assert np.array_equal((got + 0.0).view(np.uint32), (want + 0.0).view(np.uint32))
    return best, y


def test_decode_chain_decoder_layer_and_lm_head():
    """The real shapes: QKV 6144x3072 -> O 3072x4096 (x = the first 4096
    outputs of QKV, where attention would be) -> gate+up 18432x3072 -> down
    3072x9216 (x = the first 9216 outputs of gate+up, where the gated
    activation would be) -> the LM-head argmax over a 131072 x 3072 table and
    the chosen token's embedding row."""
    slices = {"qkv": None, "o": (0, 4096), "gate_up": (0, 3072), "down": (0, 9216)}
    steps = [(ternary_q4(n, k, 4, 100 + t), n, k, slices[name])
             for t, (name, n, k) in enumerate(synth.DECODER_LAYER)]
    g = np.random.Generator(np.random.PCG64(7))
    x0 = g.integers(-4, 5, 3072).astype(np.float32)
    V, D = synth.VOCAB, synth.DEC_DIM
    table = ternary_q4(V, D, 6, 200)
    announce("decode chain: decoder layer + LM head + embed")
    best, y = check_chain(steps, x0, table, V, D, (0, D))
    assert np.sum(y == y[best]) >= 1


def test_decode_chain_tie_goes_to_the_lowest_index():
    """Two identical table rows share the maximum: the lower index wins."""
    steps = [(ternary_q4(256, 512, 3, 1), 256, 512, None)]
    x0 = np.random.Generator(np.random.PCG64(2)).integers(-3, 4, 512).astype(np.float32)
    hx = oracle_chain(steps, x0)[-1][:256]
    table = ternary_q4(5000, 256, 3, 3)
    top = np.argsort(-np.abs(hx))[:8]                 # the 8 largest |x|: a clear winner
    row = np.zeros(256, np.float32)
    row[top] = np.sign(hx[top])
    wq = ternary_q4(1, 256, 0, 4)
    blk = wq.reshape(8, 18)
    for c in top:
        code = 8 + int(row[c])
        bi, e = int(c) // 32, int(c) % 32
        shift = 0 if e < 16 else 4
        old = int(blk[bi, 2 + e % 16])
        blk[bi, 2 + e % 16] = (old & (0xF0 >> shift)) | (code << shift)
    assert np.array_equal(O.dequantize_q4_0(wq, 1, 256)[0], row)
    table[4321] = table[77] = wq[0]
    announce("decode chain tie")
    best, _ = check_chain(steps, x0, table, 5000, 256, (0, 256))
    assert best == 77


@pytest.mark.parametrize("case", ["ragged", "generic_k", "head_only", "steps_only", "tall_head"])
def test_decode_chain_small(case):
    if case == "ragged":
        # slices start on 16-byte boundaries (the ABI's alignment)
        shapes = [(100, 128, None), (300, 64, (12, 76)), (257, 256, (0, 256)), (96, 192, (40, 232))]
        vocab, dim, hs = 5000, 64, (8, 72)
    elif case == "generic_k":
        shapes = [(160, 96, None), (70, 160, (0, 160)), (33, 32, (20, 52))]
        vocab, dim, hs = 700, 32, (0, 32)
    elif case == "head_only":
        shapes = []
        vocab, dim, hs = 3000, 1024, (0, 1024)
    elif case == "steps_only":
        shapes = [(512, 1024, None), (1024, 512, (0, 512)), (64, 1024, (0, 1024))]
        vocab = dim = 0
        hs = None
    else:
        shapes = [(2048, 1024, None), (1024, 2048, (0, 2048))]
        vocab, dim, hs = 70001, 1024, (0, 1024)
    steps = [(ternary_q4(n, k, 4, 10 * i + len(case)), n, k, sl)
             for i, (n, k, sl) in enumerate(shapes)]
    k0 = shapes[0][1] if shapes else dim
    x0 = np.random.Generator(np.random.PCG64(31)).integers(-4, 5, k0).astype(np.float32)
    announce(f"decode chain {case}")
    if vocab == 0:
        check_chain(steps, x0)
    else:
        check_chain(steps, x0, ternary_q4(vocab, dim, 5, 99), vocab, dim, hs)


def test_decode_chain_workspace_left_zero_and_repeatable():
    wq = dev(ternary_q4(256, 512, 4, 5))
    tq = dev(ternary_q4(4000, 256, 4, 6))
    ws = q4.lmhead_workspace(1, "cuda")
    x0 = dev(np.random.Generator(np.random.PCG64(8)).integers(-4, 5, 512).astype(np.float32))
    y = torch.empty(256, device="cuda")
    emb = torch.empty(256, device="cuda")
    outs = []
    for r in range(3):
        announce(f"decode chain repeat {r}")
        idx, val, _ = q4.decode_chain([(wq, x0, y)], table_q4=tq, head_x=y,
                                      out_val=torch.empty(1, device="cuda"), out_embed=emb,
                                      workspace=ws)
        outs.append((int(host(idx)[0]), host(val).copy(), host(emb).copy()))
        assert not host(ws).any()
    assert all(o[0] == outs[0][0] for o in outs)
    assert all(np.array_equal(o[2].view(np.uint32), outs[0][2].view(np.uint32)) for o in outs)


def test_decode_chain_rejects_before_enqueueing():
    qb = dev(ternary_q4(64, 64, 2, 1))
    x = torch.zeros(64, device="cuda")
    y = torch.full((64,), 7.0, device="cuda")
    bad = torch.zeros(96, device="cuda")[:48]                   # K of 48
    with pytest.raises(ValueError):
        q4.decode_chain([(qb, x, y), (qb, bad, y)])
    # the C entry point directly: a table without a workspace
    arr = (q4._Step * 1)(q4._Step(qb.data_ptr(), x.data_ptr(), y.data_ptr(), 64, 64))
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    st = q4.lib().q4_decode_chain(ctypes.cast(arr, ctypes.c_void_p), 1,
                                  ctypes.c_void_p(qb.data_ptr()), 64, 64,
                                  ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                                  None, None, None, 0, None)
    assert st == q4.Q4_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 7.0), "a rejected chain enqueued work"
