"""The entry points captured in a HIP graph, as the benchmark times them:
every replay gives the bits of the same calls made eagerly.

Outputs, workspaces and the argmax keys are allocated before the capture
(nothing is allocated inside it).  Before each replay the outputs are filled
with NaN by ordinary kernels on the stream (not memset nodes) and other work
runs on the stream; every replay is checked, not only the first, so a
kernel that leaves state behind for the next call (the argmax's workspace,
which its last workgroup clears; the no-allocation argmax's static scratch)
would show on the second; q4_matmul_residual is captured with its add in
the wide kernel's stores, in the fold, and in a second launch.  The shapes
reach every q4_matmul route that a
graph of the model's calls would: the matvec kernel, stream16 (one tile and
two binary16 parts of x), the small-M kernel, the skinny kernel and the wide
kernel, the last two with a K split and its fold."""

import numpy as np
import pytest
import torch

import q4_quantized_speech_amd as q4
from gpu_util import announce, needs_gpu
from oracle import q4_oracle as O
from q4_quantized_speech_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]

# (M, N, K, route) of the q4_matmul calls in the graph
MATMULS = [
    (2, 1000, 3072, "matvec"),
    (4, 700, 2048, "stream16"),
    (8, 700, 3072, "stream16"),
    (4, 300, 12352, "small"),
    (40, 600, 4096, "skinny"),
    (1500, 1280, 5120, "wide128"),
]


def _w(n, k, seed):
    return torch.from_numpy(O.quantize_q4_0(synth.weights(n, k, seed))).cuda()


def _x(m, k, seed):
    return torch.from_numpy(synth.activations(m, k, seed)).cuda()


def test_graph_replays_match_eager():
    s = torch.cuda.Stream()
    calls = []   # (name, function of the stream, output tensors)
    keep = []
    with torch.cuda.stream(s):
        for i, (m, n, k, route) in enumerate(MATMULS):
            ws_bytes = int(q4.lib().q4_matmul_workspace_bytes(m, n, k))
            assert q4.matmul_route(m, n, k, ws_bytes)[0] == route, (m, n, k)
            w, x = _w(n, k, 500 + i), _x(m, k, 600 + i)
            y = torch.empty((m, n), device="cuda")
            ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
            keep += [w, x, ws]
            calls.append((f"matmul {m}x{n}x{k} {route}",
                          lambda st, w=w, x=x, y=y, ws=ws: q4.matmul(w, x, out=y, workspace=ws,
                                                                     stream=st), [y]))
        # the residual epilogue: fused in the wide kernel's stores (no K
        # split), in the fold (K split), and as a second launch (matvec route)
        for i, (m, n, k) in enumerate([(1500, 1280, 1280), (375, 1280, 5120), (2, 1000, 3072)]):
            w, x = _w(n, k, 740 + i), _x(m, k, 750 + i)
            rr = _x(m, n, 760 + i)
            y = torch.empty((m, n), device="cuda")
            ws = q4.matmul_residual_workspace(m, n, k, "cuda")
            keep += [w, x, rr, ws]
            calls.append((f"matmul_residual {m}x{n}x{k}",
                          lambda st, w=w, x=x, rr=rr, y=y, ws=ws: q4.matmul_residual(
                              w, x, rr, out=y, workspace=ws, stream=st), [y]))
        wv, xv = _w(3000, 3072, 700), _x(1, 3072, 701)[0]
        yv = torch.empty(3000, device="cuda")
        keep += [wv, xv]
        calls.append(("matvec 3000x3072", lambda st: q4.matvec(wv, xv, out=yv, stream=st), [yv]))

        table = _w(70001, 1024, 710)
        xh = _x(2, 1024, 711)
        lws = q4.lmhead_workspace(2, "cuda")
        li = torch.empty(2, dtype=torch.int32, device="cuda")
        lv = torch.empty(2, device="cuda")
        ni = torch.empty(2, dtype=torch.int32, device="cuda")
        nv = torch.empty(2, device="cuda")
        keep += [table, xh, lws]
        calls.append(("lmhead_argmax 2 rows", lambda st: q4.lmhead_argmax(
            table, xh, workspace=lws, out_idx=li, out_val=lv, stream=st), [li, lv]))
        calls.append(("lmhead_argmax_noalloc 2 rows", lambda st: q4.lmhead_argmax_noalloc(
            table, xh, ni, nv, stream=st), [ni, nv]))

        ids = torch.tensor([0, 70000, 12345, -1, 70001, 38], dtype=torch.int32, device="cuda")
        emb = torch.empty((ids.numel(), 1024), device="cuda")
        keep.append(ids)
        calls.append(("embed_rows", lambda st: q4.embed_rows(table, ids, out=emb, stream=st),
                      [emb]))

        # a two-step chain whose second x is a slice of the first y, then the
        # argmax over the table and the chosen row's embedding
        w1, w2 = _w(2048, 1024, 720), _w(1024, 1536, 721)
        x1 = _x(1, 1024, 722)[0]
        y1 = torch.empty(2048, device="cuda")
        y2 = torch.empty(1024, device="cuda")
        cws = q4.lmhead_workspace(1, "cuda")
        ci = torch.empty(1, dtype=torch.int32, device="cuda")
        cv = torch.empty(1, device="cuda")
        ce = torch.empty((1, 1024), device="cuda")
        keep += [w1, w2, x1, cws]
        steps = [(w1, x1, y1), (w2, y1[256:1792], y2)]
        calls.append(("decode_chain", lambda st: q4.decode_chain(
            steps, table, y2, out_idx=ci, out_val=cv, out_embed=ce, workspace=cws, stream=st),
            [y1, y2, ci, cv, ce]))

        def run_all():
            for _name, fn, _outs in calls:
                fn(s)

        announce("graph: eager calls")
        run_all()
    torch.cuda.synchronize()
    eager = [[o.clone() for o in outs] for _n, _f, outs in calls]

    def poison():
        with torch.cuda.stream(s):
            for _n, _f, outs in calls:
                for o in outs:
                    o.fill_(-7 if o.dtype == torch.int32 else float("nan"))

    poison()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    announce("graph: capture")
    with torch.cuda.graph(graph, stream=s):
        run_all()
    torch.cuda.synchronize()

    other_w, other_x = _w(512, 1024, 730), _x(8, 1024, 731)
    for rep in range(3):
        poison()
        with torch.cuda.stream(s):   # unrelated eager work on the stream between replays
            q4.matmul(other_w, other_x, stream=s)
        torch.cuda.synchronize()
        announce(f"graph: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for (name, _f, outs), ref in zip(calls, eager):
            for o, r in zip(outs, ref):
                a, b = o.cpu().numpy(), r.cpu().numpy()
                same = np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b)
                assert same, (rep, name)
    del graph, keep
