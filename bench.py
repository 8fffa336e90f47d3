#!/usr/bin/env python3
"""Benchmark of the Q4_0 hot path on one MI355X.

One step = one decode step of a decoder layer at M = 1: the four Q4_0
projections QKV 6144x3072, O 3072x4096, gate+up 18432x3072, down 3072x9216
(65,470,464 weight bytes), launched back to back on one stream.  ``value`` is
weight bytes streamed per second over the timed steps (inputs resident in HBM,
weights rotated over enough copies that the 256 MB Infinity Cache cannot serve
them).

The same run also measures, each in its own timed loop: the second half of the
metric (q4_matmul TFLOP/s over the encoder layer at M = 1500 plus the adapter at
M = 375), the LM-head argmax and embedding gather over the 131072 x 3072 table,
one greedy decode step as a chain (q4_decode_chain: the four projections,
each reading the previous one's output, the LM-head argmax and the embedding
row of the chosen token), small batches (M = 2 .. 15), the
single 3072 x 3072 matvec, and the prefix GEMMs (M = 16 / 38 / 76).  Kernel
durations come from HIP events recorded on the launch stream around each
launch.  The CPU baseline is the oracle (float64 dequantise + BLAS dgemv) on a
bounded sample of the same workload, timed on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
Prints one JSON line.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q4_0 matvec weight GB/s (% HBM peak) at M=1; matmul TFLOP/s (% MFMA) at M=1500"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
F16_PEAK_TFLOPS = 2500.0     # MI355X dense f16 MFMA, TFLOP/s
CACHE_DEFEAT_BYTES = 1 << 30  # rotate weight copies over >= 1 GiB


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    return p.parse_args()


def weight_bytes(n: int, k: int) -> int:
    return n * (k // 32) * 18


def copies_for(nbytes: int) -> int:
    return max(2, -(-CACHE_DEFEAT_BYTES // nbytes))


def stored_traffic(kernel_key: str):
    """HBM bytes per launch measured with rocprofv3 --pmc, if the summary in
    profiles/ was taken on the current sources of that kernel; else None."""
    from q4_quantized_speech_amd.profile_driver import source_hash
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.lstrip().startswith("#"):
                k, _, v = line.partition(":")
                vals[k.strip()] = v.strip()
    if vals.get(f"{kernel_key}.source_hash") != source_hash(kernel_key):
        return None
    v = vals.get(f"{kernel_key}.hbm_bytes_per_launch")
    return float(v) if v else None


def profile_figures(workload: str, work: float, peak_per_us: float):
    """The committed rocprofv3 kernel trace of `workload` (profiles/, taken in
    this benchmark's timing mode): its kernel time per call and the fraction
    of peak it gives, beside the live HIP-event figure; empty if the trace
    is missing or was taken on other sources."""
    from q4_quantized_speech_amd.profile_driver import profile_call_us
    name = f"kernel_trace_{workload}.txt"
    us = profile_call_us(os.path.join(ROOT, "profiles", name), workload)
    if us is None:
        return {"profile": None}
    return {"profile": {"file": f"profiles/{name}", "kernel_us_per_call": round(us, 3),
                        "frac": round(work / us / peak_per_us, 4)}}


class GraphTimer:
    """Capture `fn(i)` for i in range(n) into one HIP graph on `stream`, then
    time `reps` replays with HIP events recorded on that stream."""

    def __init__(self, torch, stream, fn, n):
        self.torch, self.stream, self.n = torch, stream, n
        with torch.cuda.stream(stream):
            for i in range(min(n, 3)):        # initialise lazily cached state
                fn(i)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=stream):
            for i in range(n):
                fn(i)
        torch.cuda.synchronize()

    def time_us(self, reps, warmup=10):
        """Mean microseconds per captured call over `reps` replays, after
        `warmup` untimed replays (the first replays over freshly written weight
        copies run several percent slow)."""
        ev = self.torch.cuda.Event
        with self.torch.cuda.stream(self.stream):
            for _ in range(warmup):
                self.graph.replay()
            a, b = ev(enable_timing=True), ev(enable_timing=True)
            a.record(self.stream)
            for _ in range(reps):
                self.graph.replay()
            b.record(self.stream)
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * self.n)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    steps, warmup = max(1, args.steps), max(0, args.warmup)

    import numpy as np
    import torch

    import q4_quantized_speech_amd as q4
    from q4_quantized_speech_amd import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    q4.lib()
    stream = torch.cuda.Stream()

    def encode(n, k, seed):
        w = torch.from_numpy(synth.weights(n, k, seed)).cuda()
        out = q4.quantize(w)
        del w
        return out

    # ---------------- decode step: one decoder layer at M = 1 ----------------
    log("preparing decoder layer weights")
    layer = []
    layer_bytes = 0
    for t, (name, n, k) in enumerate(synth.DECODER_LAYER):
        layer.append((name, n, k, encode(n, k, synth.seed_for(1, t)),
                      torch.from_numpy(synth.activations(1, k, synth.seed_for(1, 10 + t))[0]).cuda(),
                      torch.empty(n, dtype=torch.float32, device="cuda")))
        layer_bytes += weight_bytes(n, k)
    r_layer = copies_for(layer_bytes)
    copies = [[w.clone() for (_, _, _, w, _, _) in layer] for _ in range(r_layer)]
    torch.cuda.synchronize()

    def layer_step(i):
        ws = copies[i % r_layer]
        for j, (name, n, k, _, x, y) in enumerate(layer):
            q4.matvec(ws[j], x, out=y, stream=stream)

    # warmup: a graph of `warmup` decode steps replayed once, untimed; timed:
    # one replay of a graph holding exactly `steps` decode steps (4 launches
    # each, weights rotated over r_layer copies)
    log(f"decode step: {layer_bytes} B over {r_layer} copies; warmup {warmup}, steps {steps}")
    if warmup > 0:
        gw = GraphTimer(torch, stream, layer_step, warmup)
        gw.time_us(1, warmup=0)
        del gw
    gt = GraphTimer(torch, stream, layer_step, steps)
    us_step = gt.time_us(1, warmup=0)
    ms_per_step = us_step * 1e-3
    value_gbs = layer_bytes / (us_step * 1e-6) / 1e9
    log(f"decode step {us_step:.2f} us -> {value_gbs:.1f} GB/s ({steps} steps)")
    del gt

    def timed(fn, n, min_launches=200):
        """Mean microseconds per launch: a graph of at least `min_launches`
        launches (the rotation of n weight copies repeated), so the boundary
        between graph replays adds little per launch; at least ~400 untimed
        launches first (replays over freshly cloned weight copies, the LM
        head's 1.1 GB above all, run slow for a while)."""
        n_graph = n * max(1, -(-min_launches // n))
        g = GraphTimer(torch, stream, fn, n_graph)
        us = g.time_us(max(3, 800 // n_graph), warmup=max(2, 400 // n_graph))
        del g
        return us

    # per-launch durations of each projection: graphs of its rotated launches
    per_proj = {}
    for j, (name, n, k, _, x, y) in enumerate(layer):
        us = timed(lambda i, j=j, x=x, y=y: q4.matvec(copies[i % r_layer][j], x, out=y, stream=stream),
                   r_layer)
        per_proj[name] = {"us": round(us, 3), "gbs": round(weight_bytes(n, k) / (us * 1e-6) / 1e9, 1),
                          "frac_hbm": round(weight_bytes(n, k) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    dominant = max(per_proj, key=lambda nm: per_proj[nm]["us"])
    dn, dk = [(n, k) for (nm, n, k, *_rest) in layer if nm == dominant][0]
    dom_bytes = weight_bytes(dn, dk)
    achieved = dom_bytes / (per_proj[dominant]["us"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": stored_traffic(f"matvec_{dominant}"),
                "kernel": f"q4_matvec {dominant} {dn}x{dk}",
                "bytes_per_launch": dom_bytes,
                "launch_us_mean": per_proj[dominant]["us"]}
    roofline.update(profile_figures(f"matvec_{dominant}", dom_bytes, HBM_PEAK_GBS * 1e3))
    rows = {"decode_layer_projections": per_proj}

    # Measured read ceiling: a plain coalesced read kernel (libq4probe.so, not
    # part of the library) over buffers of the dominant kernel's size rotated
    # the same way, and over 1 GiB; best of a few grid sizes.
    probe_path = os.path.join(ROOT, "q4_quantized_speech_amd", "libq4probe.so")
    probe = ctypes.CDLL(probe_path) if os.path.exists(probe_path) else None
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    if probe is not None:
        probe.q4probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
        probe.q4probe_read.restype = ctypes.c_int

    def read_ceiling(nbytes):
        r = copies_for(nbytes)
        bufs = [torch.full((nbytes,), i & 255, dtype=torch.uint8, device="cuda") for i in range(r)]
        torch.cuda.synchronize()
        if probe.q4probe_read(bufs[0].data_ptr(), nbytes, 256, sink.data_ptr(), stream.cuda_stream):
            raise RuntimeError("read probe launch failed")
        best = None
        for grid in (512, 1024, 2048, 4096):
            us = timed(lambda i, grid=grid: probe.q4probe_read(bufs[i % r].data_ptr(), nbytes, grid,
                                                              sink.data_ptr(), stream.cuda_stream),
                       r, min_launches=200 if nbytes < (64 << 20) else 16)
            if best is None or us < best[0]:
                best = (us, grid)
        del bufs
        torch.cuda.empty_cache()
        return {"us": round(best[0], 3), "gbs": round(nbytes / (best[0] * 1e-6) / 1e9, 1),
                "grid": best[1]}

    if probe is not None:
        log("read ceiling")
        ceil_dom = read_ceiling(dom_bytes)
        ceil_big = read_ceiling(1 << 30)
        rows["read_ceiling"] = {f"bytes_{dom_bytes}": ceil_dom, "bytes_1073741824": ceil_big}
        roofline["ceiling_measured_gbs"] = ceil_dom["gbs"]
        roofline["frac_of_ceiling"] = round(achieved / ceil_dom["gbs"], 4)
    else:
        log("libq4probe.so not built: no measured read ceiling")

    # ---------------- single 3072 x 3072 matvec ----------------
    n = k = 3072
    w1 = encode(n, k, synth.seed_for(0, 0))
    r1 = copies_for(weight_bytes(n, k))
    w1c = [w1] + [w1.clone() for _ in range(r1 - 1)]
    x1 = torch.from_numpy(synth.activations(1, k, synth.seed_for(0, 1))[0]).cuda()
    y1 = torch.empty(n, device="cuda")
    us = timed(lambda i: q4.matvec(w1c[i % r1], x1, out=y1, stream=stream), r1)
    rows["matvec_3072x3072"] = {"us": round(us, 3), "gbs": round(weight_bytes(n, k) / (us * 1e-6) / 1e9, 1)}
    del w1c, w1

    # ---------------- LM head argmax + embedding rows ----------------
    log("preparing 131072 x 3072 table")
    V, D = synth.VOCAB, synth.DEC_DIM
    table = encode(V, D, synth.seed_for(2, 0))
    rt = copies_for(weight_bytes(V, D))
    tables = [table] + [table.clone() for _ in range(rt - 1)]
    xl = torch.from_numpy(synth.activations(1, D, synth.seed_for(2, 1))).cuda()
    ws = q4.lmhead_workspace(1, "cuda")
    oi = torch.empty(1, dtype=torch.int32, device="cuda")
    ov = torch.empty(1, dtype=torch.float32, device="cuda")
    us = timed(lambda i: q4.lmhead_argmax(tables[i % rt], xl, workspace=ws, out_idx=oi, out_val=ov,
                                          stream=stream), rt)
    lm_gbs = weight_bytes(V, D) / (us * 1e-6) / 1e9
    rows["lmhead_argmax_131072x3072"] = {"us": round(us, 3), "gbs": round(lm_gbs, 1),
                                         "frac_hbm": round(lm_gbs / HBM_PEAK_GBS, 4)}
    # two decode streams at once: one call with two rows of x (the table is
    # read once for both)
    xl2 = torch.from_numpy(synth.activations(2, D, synth.seed_for(2, 3))).cuda()
    ws2 = q4.lmhead_workspace(2, "cuda")
    oi2 = torch.empty(2, dtype=torch.int32, device="cuda")
    ov2 = torch.empty(2, dtype=torch.float32, device="cuda")
    us = timed(lambda i: q4.lmhead_argmax(tables[i % rt], xl2, workspace=ws2, out_idx=oi2,
                                          out_val=ov2, stream=stream), rt)
    rows["lmhead_argmax_M2_131072x3072"] = {
        "us": round(us, 3), "table_gbs": round(weight_bytes(V, D) / (us * 1e-6) / 1e9, 1)}
    ids = torch.from_numpy(synth.token_ids(synth.PREFIX_TOKENS, synth.seed_for(2, 2))).cuda()
    emb = torch.empty((synth.PREFIX_TOKENS, D), device="cuda")
    us = timed(lambda i: q4.embed_rows(tables[i % rt], ids, out=emb, stream=stream), rt)
    rows["embed_rows_38x3072"] = {"us": round(us, 3)}

    # ---------------- one greedy decode step as a chain (q4_decode_chain) ----------------
    # the four projections, each reading a slice of the previous one's output
    # (QKV -> O reads the first 4096 outputs, where attention would be;
    # gate+up -> down the first 9216, where the gated activation would be),
    # then the LM-head argmax over the down projection's output and the
    # chosen token's embedding row, in one call; weights rotated over the
    # layer and table copies
    emb1 = torch.empty(D, device="cuda")
    x0 = layer[0][4]
    ys = [y for (_, _, _, _, _, y) in layer]
    chain_x = [x0, ys[0][:4096], ys[1], ys[2][:9216]]

    def chain_step(i):
        steps = [(copies[i % r_layer][j], chain_x[j], ys[j]) for j in range(len(layer))]
        q4.decode_chain(steps, table_q4=tables[i % rt], head_x=ys[3], out_idx=oi, out_val=ov,
                        out_embed=emb1, workspace=ws, stream=stream)

    us = timed(chain_step, max(r_layer, rt))
    chain_bytes = layer_bytes + weight_bytes(V, D) + weight_bytes(1, D)
    rows["decode_chain_layer_lmhead_embed"] = {
        "us": round(us, 3), "gbs": round(chain_bytes / (us * 1e-6) / 1e9, 1),
        "frac_hbm": round(chain_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "bytes": chain_bytes, "launches": 5,
        "entry_point": "q4_decode_chain (4 dependent matvec steps + argmax with the chosen "
                       "token's embedding row in the same launch)"}
    del tables, table

    # ---------------- small batches: M = 2 .. 15 over the decoder layer ----------------
    # q4_matvec takes the rows of x in pairs (M <= 8; each pair reads W once,
    # pairs after the first mostly from the caches); q4_matmul picks per
    # projection between that and kernels that read W once
    for m in (2, 4, 8, 15):
        xs = [torch.from_numpy(synth.activations(m, k, synth.seed_for(5, 10 + t))).cuda()
              for t, (_, n, k) in enumerate(synth.DECODER_LAYER)]
        ys = [torch.empty((m, n), device="cuda") for (_, n, _) in synth.DECODER_LAYER]
        wss = [q4.matmul_workspace(m, n, k, "cuda") for (_, n, k) in synth.DECODER_LAYER]
        row = {}
        paths = [("matmul", lambda w, x, y, j: q4.matmul(w, x, out=y, workspace=wss[j], stream=stream))]
        if m <= 8:
            paths.insert(0, ("matvec", lambda w, x, y, j: q4.matvec(w, x, out=y, stream=stream)))
        for pname, call in paths:
            tot = 0.0
            for j in range(len(synth.DECODER_LAYER)):
                tot += timed(lambda i, j=j: call(copies[i % r_layer][j], xs[j], ys[j], j), r_layer)
            row[f"{pname}_layer_us"] = round(tot, 3)
            row[f"{pname}_layer_weight_gbs"] = round(layer_bytes / (tot * 1e-6) / 1e9, 1)
        rows[f"small_batch_M{m}"] = row
        del xs, ys, wss
    del copies
    torch.cuda.empty_cache()
    torch.cuda.empty_cache()

    # ---------------- matmul: encoder layer at M = 1500 + adapter at 375 ----------------
    def gemm_set(shapes, m_of, seed_cfg):
        out = {}
        tot_flop, tot_us = 0.0, 0.0
        for t, (name, n, k) in enumerate(shapes):
            m = m_of(name)
            w = encode(n, k, synth.seed_for(seed_cfg, t))
            r = copies_for(weight_bytes(n, k))
            wc = [w] + [w.clone() for _ in range(r - 1)]
            x = torch.from_numpy(synth.activations(m, k, synth.seed_for(seed_cfg, 10 + t))).cuda()
            y = torch.empty((m, n), device="cuda")
            ws = q4.matmul_workspace(m, n, k, "cuda")
            us = timed(lambda i: q4.matmul(wc[i % r], x, out=y, workspace=ws, stream=stream), r)
            flop = 2.0 * m * n * k
            out[f"{name}_M{m}_{n}x{k}"] = {
                "us": round(us, 3), "tflops": round(flop / (us * 1e-6) / 1e12, 2),
                "weight_gbs": round(weight_bytes(n, k) / (us * 1e-6) / 1e9, 1)}
            tot_flop += flop
            tot_us += us
            del wc, w, x, y, ws
        return out, tot_flop, tot_us

    enc_shapes = list(synth.ENCODER_LAYER) + [synth.ADAPTER]
    m_enc = 1500
    enc_rows, enc_flop, enc_us = gemm_set(
        enc_shapes, lambda nm: m_enc // 4 if nm == "adapter" else m_enc, 4)
    enc_tflops = enc_flop / (enc_us * 1e-6) / 1e12
    dom_gemm = max(enc_rows, key=lambda nm: enc_rows[nm]["us"])
    _m, _nk = dom_gemm.split("_M")[1].split("_", 1)
    m_dom, (n_dom, k_dom) = int(_m), map(int, _nk.split("x"))
    matmul = {
        "metric": "q4_matmul TFLOP/s, encoder layer (QKV 3840x1280, O 1280x1280, up 5120x1280, "
                  "down 1280x5120) at M=1500 + adapter 3072x5120 at M=375",
        "value": round(enc_tflops, 2), "unit": "TFLOP/s",
        "roofline": {"bound": "mfma", "achieved": enc_rows[dom_gemm]["tflops"],
                     "peak": F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(enc_rows[dom_gemm]["tflops"] / F16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic(f"matmul_{dom_gemm}"), "kernel": f"q4_matmul {dom_gemm}",
                     "launch_us_mean": enc_rows[dom_gemm]["us"],
                     **profile_figures(f"matmul_{dom_gemm}", 2.0 * m_dom * n_dom * k_dom,
                                       F16_PEAK_TFLOPS * 1e6)},
        "frac_of_peak_whole_layer": round(enc_tflops / F16_PEAK_TFLOPS, 4),
        "per_projection": enc_rows}
    # the 1280-wide encoder projections with the residual add fused into the
    # product (q4_matmul_residual) against q4_matmul followed by a separate add
    res_rows = {}
    for t, (name, n, k) in enumerate(synth.ENCODER_LAYER):
        if n != 1280:
            continue
        w = encode(n, k, synth.seed_for(4, t))
        r = copies_for(weight_bytes(n, k))
        wc = [w] + [w.clone() for _ in range(r - 1)]
        x = torch.from_numpy(synth.activations(m_enc, k, synth.seed_for(4, 10 + t))).cuda()
        resid = torch.from_numpy(synth.activations(m_enc, n, synth.seed_for(4, 20 + t))).cuda()
        y = torch.empty((m_enc, n), device="cuda")
        ws = q4.matmul_residual_workspace(m_enc, n, k, "cuda")
        fused = timed(lambda i: q4.matmul_residual(wc[i % r], x, resid, out=y, workspace=ws,
                                                   stream=stream), r)

        def unfused(i):
            q4.matmul(wc[i % r], x, out=y, workspace=ws, stream=stream)
            with torch.cuda.stream(stream):
                torch.add(y, resid, out=y)
        res_rows[f"{name}_M{m_enc}_{n}x{k}"] = {"fused_us": round(fused, 3),
                                                 "matmul_then_add_us": round(timed(unfused, r), 3)}
        del wc, w, x, resid, y, ws
    rows[f"encoder_residual_M{m_enc}"] = res_rows
    for m in (375, 3000):
        r, f, u = gemm_set(enc_shapes, lambda nm, m=m: m // 4 if nm == "adapter" else m, 4)
        rows[f"encoder_M{m}"] = dict(r, layer_tflops=round(f / (u * 1e-6) / 1e12, 2))
    for m in (16, 38, 76):
        r, f, u = gemm_set(list(synth.DECODER_LAYER), lambda nm, m=m: m, 3)
        rows[f"prefix_M{m}"] = dict(
            r, layer_weight_gbs=round(layer_bytes / (u * 1e-6) / 1e9, 1),
            layer_tflops=round(f / (u * 1e-6) / 1e12, 2))

    # ---------------- CPU baseline: the oracle on the host cores ----------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline()
        matmul["cpu_baseline"] = cpu_baseline_matmul(m_enc)

    line = {
        "metric": METRIC,
        "value": round(value_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decoder-layer decode step at M=1: Q4_0 projections QKV 6144x3072, "
                               "O 3072x4096, gate+up 18432x3072, down 3072x9216",
                   "weight_bytes_per_step": layer_bytes, "weight_copies_rotated": r_layer,
                   "frac_hbm_peak": round(value_gbs / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "matmul": matmul,
        "rows": rows,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_matmul(m_enc):
    """The oracle (float64 dequantise + BLAS dgemm, with its error bound) over
    the encoder layer + adapter at the GPU workload's shapes."""
    import numpy as np

    from oracle import q4_oracle as O
    from q4_quantized_speech_amd import synth

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    log("cpu baseline (matmul): encoding the encoder layer with the oracle (untimed)")
    mats = []
    for t, (name, n, k) in enumerate(list(synth.ENCODER_LAYER) + [synth.ADAPTER]):
        m = m_enc // 4 if name == "adapter" else m_enc
        qb = O.quantize_q4_0(synth.weights(n, k, synth.seed_for(4, t)))
        x = synth.activations(m, k, synth.seed_for(4, 10 + t))
        mats.append((qb, x, n, k, m))
    flop = sum(2.0 * m * n * k for (_, _, n, k, m) in mats)
    times = []
    t_start = time.perf_counter()
    # about 10 s of timed oracle work (at least 3 layers, at most 40 or 25 s)
    while len(times) < 3 or (time.perf_counter() - t_start < 10.0 and len(times) < 40):
        t0 = time.perf_counter()
        for qb, x, n, k, m in mats:
            O.matmul_f64(qb, x, n, k)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > 25.0:
            break
    med = statistics.median(times)
    log(f"cpu baseline (matmul): {med * 1e3:.1f} ms per encoder layer + adapter")
    return {"value": round(flop / med / 1e12, 4), "unit": "TFLOP/s", "cores": int(blas_threads),
            "host_cores_available": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{len(times)} full encoder layers + adapter at M={m_enc} "
                      f"({flop / 1e9:.1f} GFLOP), median {med * 1e3:.1f} ms; float64 dequantise "
                      f"(numpy, 1 thread) + dgemm and the |X||W| bound dgemm (BLAS, "
                      f"{blas_threads} threads)"}


def cpu_baseline():
    """The oracle (float64 dequantise + BLAS dgemv) over the decode-step layer."""
    import numpy as np

    from oracle import q4_oracle as O
    from q4_quantized_speech_amd import synth

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    log("cpu baseline: encoding the layer with the oracle (untimed)")
    mats = []
    for t, (name, n, k) in enumerate(synth.DECODER_LAYER):
        qb = O.quantize_q4_0(synth.weights(n, k, synth.seed_for(1, t)))
        x = synth.activations(1, k, synth.seed_for(1, 10 + t))[0]
        mats.append((qb, x, n, k))
    total = sum(weight_bytes(n, k) for (_, _, n, k) in mats)
    times = []
    budget = 25.0
    t_start = time.perf_counter()
    # about 10 s of timed oracle work (at least 3 steps, at most 40 or 25 s)
    while len(times) < 3 or (time.perf_counter() - t_start < 10.0 and len(times) < 40):
        t0 = time.perf_counter()
        for qb, x, n, k in mats:
            O.matvec_f64(qb, x, n, k)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget:
            break
    med = statistics.median(times)
    log(f"cpu baseline: {med * 1e3:.1f} ms per layer step")
    return {"value": round(total / med / 1e9, 3), "unit": "GB/s", "cores": int(blas_threads),
            "host_cores_available": cores, "kind": "oracle",
            "sample": f"{len(times)} full decode-layer steps (4 projections, {total} weight bytes), "
                      f"median {med * 1e3:.1f} ms; float64 dequantise (numpy, 1 thread) + dgemv "
                      f"(BLAS, {blas_threads} threads)"}


if __name__ == "__main__":
    main()
