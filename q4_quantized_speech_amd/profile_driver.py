"""Profiling driver: runs one benchmark workload eagerly, for rocprofv3.

    python -m q4_quantized_speech_amd.profile_driver run WORKLOAD [--iters N] [--graph]
    python -m q4_quantized_speech_amd.profile_driver traffic WORKLOAD \
        --fetch FETCH.csv --write WRITE.csv [--out FILE]
    python -m q4_quantized_speech_amd.profile_driver trace KERNEL_TRACE.csv [--out FILE] \
        [--last N --workload WORKLOAD] [--cmd TEXT ...]
    python -m q4_quantized_speech_amd.profile_driver counters COUNTERS.csv [--out FILE] [--cmd TEXT ...]

``run`` builds the inputs of one workload with the same seeds and shapes as
bench.py, rotates enough weight copies (>= 1 GiB) that the Infinity Cache
cannot serve them, and calls the library N times, eagerly or (``--graph``)
as replays of one HIP graph of the rotated calls, which is how bench.py
times them (it then prints the mean per call from HIP events); it then runs a plain
element-wise kernel over 256 MiB (``torch.neg``: 256 MiB read, 256 MiB
written) whose counter readings calibrate the HBM counters.

``traffic`` turns two ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE``
counter files of such a run into HBM bytes per call: the counters (KiB per
dispatch) of the library's kernels, summed over the dispatches one call makes,
each scaled by (true bytes / counter reading) of the calibration kernel.  The
result goes into a key-value file that bench.py reads, each workload tagged
with a hash of its kernels' sources so that stale figures are ignored.

``trace`` summarises a ``rocprofv3 --kernel-trace`` CSV per kernel and grid
size (the library launches one kernel template for several shapes; the grid
tells them apart); with ``--last N`` it also gives each library kernel's mean
over its last N dispatches (the timed window of a ``run --graph``), tagged
with the workload's source hash, which bench.py reads back.

``counters`` gives, per library kernel and grid, the mean of each counter of
a ``rocprofv3 --pmc`` run and the MFMA busy fraction.

``--cmd`` lines (repeatable) go at the top of a summary as '# ' comments: the
commands that produced it.

Workload names are the keys bench.py reports:
    matvec_{qkv,o,gate_up,down}      decoder projections at M = 1
    decode_step                      the four of them back to back
    matvec_3072x3072                 the single matvec
    lmhead_argmax_131072x3072        LM-head argmax at M = 1
    embed_rows_38x3072               embedding gather of 38 ids
    matmul_<proj>_M<m>_<n>x<k>       encoder, adapter or prefix GEMMs
    encoder_layer_M<m>               the encoder projections at M and the adapter at M / 4
    prefix_layer_M<m>                the decoder projections at a prefix of M tokens
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CACHE_DEFEAT_BYTES = 1 << 30
XCDS = 8                       # accelerator complex dies of the MI355X (GRBM counter instances)
CAL_BYTES = 256 << 20          # calibration kernel: reads and writes this many bytes
CAL_KERNEL = "neg_kernel"      # substring of torch's element-wise negation kernel
MARKER_KERNEL = "bitwise_not"  # launched right before the timed replays of ``run --graph``
LIB_KERNEL = "q4::"            # namespace of the library's kernels
SETUP_KERNELS = ("quantize_kernel",)  # library kernels that only prepare inputs


def weight_bytes(n: int, k: int) -> int:
    return n * (k // 32) * 18


# Sources that define each workload family's kernels: a stored counter
# figure stays valid while their code (comments and blank space aside) is
# unchanged.
KERNEL_SOURCES = {
    "matvec": ("q4_matvec.hip", "q4_device.h"),
    "lmhead": ("q4_matvec.hip", "q4_device.h"),
    "matmul": ("q4_matmul.hip", "q4_smallm.hip", "q4_device.h"),
    "encoder": ("q4_matmul.hip", "q4_smallm.hip", "q4_device.h"),
    "prefix": ("q4_matmul.hip", "q4_smallm.hip", "q4_device.h"),
    "decode": ("q4_matvec.hip", "q4_device.h"),
    "embed": ("q4_embed_quant.hip", "q4_device.h"),
}


def _code_only(text: str) -> str:
    """C++ source without comments and with runs of blank space collapsed
    (string literals in these sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(workload: str) -> str:
    """Hash of the code of the HIP sources of the workload's kernels."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[workload.split("_")[0]]:
        with open(os.path.join(ROOT, "q4_quantized_speech_amd", "csrc", name), encoding="utf-8") as fh:
            h.update(name.encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def profile_call_us(path: str, workload: str):
    """Kernel time per call of a workload from a trace summary in profiles/
    (the sum of its library kernels' timed-window means), if the summary was
    taken on the current sources of those kernels; else None."""
    if not os.path.exists(path):
        return None
    total, found, hash_ok, per_call = 0.0, False, False, None
    with open(path) as fh:
        for line in fh:
            if line.startswith("source_hash:"):
                hash_ok = line.split(":", 1)[1].strip() == source_hash(workload)
            elif line.startswith("window_mean_us["):
                total += float(line.split("]:", 1)[1].split()[0])
                found = True
            elif line.startswith("call_kernel_us:"):
                per_call = float(line.split(":", 1)[1].split()[0])
    if not hash_ok:
        return None
    if per_call is not None:
        return per_call
    return total if found else None


def dispatches_per_call(workload: str) -> int:
    """Distinct library kernels one call of the workload launches."""
    if workload.startswith("matmul_"):
        return 0  # one or two (the K-split fold), decided by the shape
    return 1


# ----------------------------------------------------------------------------- run

def _run(workload: str, iters: int, graph: bool = False) -> None:
    import torch

    import q4_quantized_speech_amd as q4
    from q4_quantized_speech_amd import synth

    dev = "cuda"
    torch.cuda.set_device(0)
    q4.lib()
    s = torch.cuda.Stream()

    def encode(n, k, seed):
        w = torch.from_numpy(synth.weights(n, k, seed)).to(dev)
        out = q4.quantize(w)
        del w
        return out

    def copies(nbytes):
        return max(2, -(-CACHE_DEFEAT_BYTES // nbytes))

    def rotate(w):
        return [w] + [w.clone() for _ in range(copies(w.numel()) - 1)]

    def act(m, k, seed):
        return torch.from_numpy(synth.activations(m, k, seed)).to(dev)

    call = None
    m = re.fullmatch(r"matvec_(qkv|o|gate_up|down)", workload)
    if m:
        t = [p[0] for p in synth.DECODER_LAYER].index(m.group(1))
        _, n, k = synth.DECODER_LAYER[t]
        ws = rotate(encode(n, k, synth.seed_for(1, t)))
        x = act(1, k, synth.seed_for(1, 10 + t))[0]
        y = torch.empty(n, device=dev)
        call = lambda i: q4.matvec(ws[i % len(ws)], x, out=y, stream=s)  # noqa: E731
    elif workload == "decode_step":
        # the four projections of a decoder layer at M = 1, back to back,
        # weights rotated as one set (the bench's decode step)
        layer = [(n, k, encode(n, k, synth.seed_for(1, t)),
                  act(1, k, synth.seed_for(1, 10 + t))[0], torch.empty(n, device=dev))
                 for t, (_, n, k) in enumerate(synth.DECODER_LAYER)]
        nb = sum(weight_bytes(n, k) for (n, k, *_r) in layer)
        ws = [[w for (_, _, w, _, _) in layer]]
        ws += [[w.clone() for w in ws[0]] for _ in range(copies(nb) - 1)]

        def call(i):
            for j, (_, _, _, x, y) in enumerate(layer):
                q4.matvec(ws[i % len(ws)][j], x, out=y, stream=s)
    elif re.fullmatch(r"encoder_layer_M\d+", workload) or re.fullmatch(r"prefix_layer_M\d+", workload):
        # every projection of the encoder layer (+ the adapter at M / 4), or
        # of the decoder layer at a prefix length, back to back
        mm = int(workload.rsplit("M", 1)[1])
        if workload.startswith("encoder"):
            shapes = [(nm, n, k, mm // 4 if nm == "adapter" else mm, 4, t)
                      for t, (nm, n, k) in enumerate(list(synth.ENCODER_LAYER) + [synth.ADAPTER])]
        else:
            shapes = [(nm, n, k, mm, 3, t) for t, (nm, n, k) in enumerate(synth.DECODER_LAYER)]
        mats = []
        for (nm, n, k, m_, cfg, t) in shapes:
            w0 = encode(n, k, synth.seed_for(cfg, t))
            mats.append((w0, act(m_, k, synth.seed_for(cfg, 10 + t)),
                         torch.empty((m_, n), device=dev), q4.matmul_workspace(m_, n, k, dev)))
        nb = sum(w0.numel() for (w0, *_r) in mats)
        ws = [[w0 for (w0, *_r) in mats]]
        ws += [[w0.clone() for w0 in ws[0]] for _ in range(copies(nb) - 1)]

        def call(i):
            for j, (_, x, y, wsp) in enumerate(mats):
                q4.matmul(ws[i % len(ws)][j], x, out=y, workspace=wsp, stream=s)
    elif workload == "matvec_3072x3072":
        ws = rotate(encode(3072, 3072, synth.seed_for(0, 0)))
        x = act(1, 3072, synth.seed_for(0, 1))[0]
        y = torch.empty(3072, device=dev)
        call = lambda i: q4.matvec(ws[i % len(ws)], x, out=y, stream=s)  # noqa: E731
    elif workload in ("lmhead_argmax_131072x3072", "embed_rows_38x3072"):
        ws = rotate(encode(synth.VOCAB, synth.DEC_DIM, synth.seed_for(2, 0)))
        if workload.startswith("lmhead"):
            x = act(1, synth.DEC_DIM, synth.seed_for(2, 1))
            wsp = q4.lmhead_workspace(1, dev)
            oi = torch.empty(1, dtype=torch.int32, device=dev)
            ov = torch.empty(1, device=dev)
            call = lambda i: q4.lmhead_argmax(ws[i % len(ws)], x, workspace=wsp,  # noqa: E731
                                              out_idx=oi, out_val=ov, stream=s)
        else:
            ids = torch.from_numpy(synth.token_ids(synth.PREFIX_TOKENS, synth.seed_for(2, 2))).to(dev)
            out = torch.empty((synth.PREFIX_TOKENS, synth.DEC_DIM), device=dev)
            call = lambda i: q4.embed_rows(ws[i % len(ws)], ids, out=out, stream=s)  # noqa: E731
    else:
        m = re.fullmatch(r"matmul_([a-z_]+)_M(\d+)_(\d+)x(\d+)", workload)
        if not m:
            raise SystemExit(f"unknown workload {workload!r}")
        name, mm, n, k = m.group(1), int(m.group(2)), int(m.group(3)), int(m.group(4))
        enc = list(synth.ENCODER_LAYER) + [synth.ADAPTER]
        found = [(4, t) for t, p in enumerate(enc) if p == (name, n, k)]
        found += [(3, t) for t, p in enumerate(synth.DECODER_LAYER) if p == (name, n, k)]
        if not found:
            raise SystemExit(f"no projection {name} {n}x{k}")
        cfg, t = found[0]
        ws = rotate(encode(n, k, synth.seed_for(cfg, t)))
        x = act(mm, k, synth.seed_for(cfg, 10 + t))
        y = torch.empty((mm, n), device=dev)
        wsp = q4.matmul_workspace(mm, n, k, dev)
        call = lambda i: q4.matmul(ws[i % len(ws)], x, out=y, workspace=wsp,  # noqa: E731
                                   stream=s)

    torch.cuda.synchronize()
    r = len(ws)
    if graph:
        # the bench's timing mode (bench.py, timed()): one HIP graph of the r
        # rotated calls repeated to at least 200 calls on the launch stream,
        # max(2, 400 // n) untimed replays, then max(3, iters // n) timed
        # ones; mean per call from HIP events on that stream
        n = r * max(1, -(-200 // r))
        with torch.cuda.stream(s):
            for i in range(min(r, 3)):
                call(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                call(i)
        torch.cuda.synchronize()
        reps = max(3, iters // n)
        warm = max(2, 400 // n)
        print(f"[profile] {workload}: graph of {n} calls, {warm} untimed + {reps} timed replays",
              flush=True)
        marker = torch.zeros(1, dtype=torch.int32, device=dev)
        with torch.cuda.stream(s):
            for _ in range(warm):
                g.replay()
            # a kernel no other step launches: the trace's timed window
            # begins at its dispatch
            torch.bitwise_not(marker, out=marker)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            for _ in range(reps):
                g.replay()
            b.record(s)
        b.synchronize()
        print(f"[profile] HIP events: {a.elapsed_time(b) * 1e3 / (reps * n):.3f} us per call "
              f"over the {reps * n} timed calls (the last {reps * n} calls of the run)", flush=True)
        del g
    else:
        print(f"[profile] {workload}: {iters} calls", flush=True)
        with torch.cuda.stream(s):
            for i in range(iters):
                call(i)
    torch.cuda.synchronize()
    del ws
    torch.cuda.empty_cache()
    a = torch.empty(CAL_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    print(f"[profile] calibration: torch.neg over {CAL_BYTES} B, {iters} calls", flush=True)
    for _ in range(iters):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print("[profile] done", flush=True)


# ----------------------------------------------------------------------------- traffic

def _counter_means(path: str, counter: str):
    """{kernel name: mean counter value per dispatch} and dispatch counts."""
    vals = defaultdict(list)
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def _per_call(path: str, counter: str, workload: str):
    means, counts = _counter_means(path, counter)
    cal = [k for k in means if CAL_KERNEL in k]
    if len(cal) != 1:
        raise SystemExit(f"{path}: calibration kernel not found (or ambiguous): {cal}")
    factor = CAL_BYTES / (means[cal[0]] * 1024.0)
    lib = {k: v for k, v in means.items()
           if LIB_KERNEL in k and not any(s in k for s in SETUP_KERNELS)}
    if dispatches_per_call(workload) and len(lib) != dispatches_per_call(workload):
        raise SystemExit(f"{path}: expected {dispatches_per_call(workload)} library kernels, "
                         f"found {sorted(lib)}")
    kib = sum(lib.values())
    return kib, factor, {k: (v, counts[k]) for k, v in lib.items()}, means[cal[0]]


def _read_kv(path: str):
    vals, order = {}, []
    if os.path.exists(path):
        with open(path) as fh:
            for line in fh:
                if ":" in line and not line.lstrip().startswith("#"):
                    k, _, v = line.partition(":")
                    vals[k.strip()] = v.strip()
                    order.append(k.strip())
    return vals, order


def _traffic(workload: str, fetch: str, write: str, out: str) -> None:
    f_kib, f_fac, f_k, f_cal = _per_call(fetch, "FETCH_SIZE", workload)
    w_kib, w_fac, w_k, w_cal = _per_call(write, "WRITE_SIZE", workload)
    read_b = f_kib * 1024.0 * f_fac
    write_b = w_kib * 1024.0 * w_fac
    vals, order = _read_kv(out)
    vals.pop("source_hash", None)  # a single hash for all workloads (older files)
    order = [k for k in order if k != "source_hash"]
    new = {
        f"{workload}.source_hash": source_hash(workload),
        f"{workload}.fetch_kib_per_call_raw": f"{f_kib:.1f}",
        f"{workload}.write_kib_per_call_raw": f"{w_kib:.1f}",
        f"{workload}.fetch_scale": f"{f_fac:.4f}",
        f"{workload}.write_scale": f"{w_fac:.4f}",
        f"{workload}.hbm_read_bytes_per_launch": f"{read_b:.0f}",
        f"{workload}.hbm_write_bytes_per_launch": f"{write_b:.0f}",
        f"{workload}.hbm_bytes_per_launch": f"{read_b + write_b:.0f}",
    }
    for k, v in new.items():
        if k not in vals:
            order.append(k)
        vals[k] = v
    with open(out, "w") as fh:
        fh.write("# HBM traffic per call from rocprofv3 counters (KiB per dispatch), scaled by\n"
                 f"# the reading of a plain copy kernel (torch.neg over {CAL_BYTES} B: reads and\n"
                 "# writes that many bytes).  Commands, per workload W, from /tmp:\n"
                 "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -o run -- \\\n"
                 "#     python3 <repo>/q4_quantized_speech_amd/profile_driver.py run W --iters 20\n"
                 "#   (same with --pmc WRITE_SIZE into <Wr>)\n"
                 "#   python -m q4_quantized_speech_amd.profile_driver traffic W \\\n"
                 "#     --fetch <F>/run_counter_collection.csv --write <Wr>/run_counter_collection.csv\n"
                 "# W.source_hash ties W's figures to the code of its kernels' sources (comments aside).\n")
        for k in order:
            fh.write(f"{k}: {vals[k]}\n")
    print(f"{workload}: read {read_b / 1e6:.3f} MB (raw {f_kib:.0f} KiB x {f_fac:.3f}), "
          f"write {write_b / 1e6:.3f} MB (raw {w_kib:.0f} KiB x {w_fac:.3f}); "
          f"calibration raw fetch {f_cal:.0f} KiB, write {w_cal:.0f} KiB")
    for k, (v, c) in f_k.items():
        print(f"  FETCH_SIZE {v:.1f} KiB x{c}  {k[:100]}")
    for k, (v, c) in w_k.items():
        print(f"  WRITE_SIZE {v:.1f} KiB x{c}  {k[:100]}")


# ----------------------------------------------------------------------------- counters

def _header(cmds) -> list:
    """'# ' lines naming the commands that produced a summary."""
    return [f"# {c}" for c in (cmds or [])]


def _counters(path: str, out: str | None, cmds=None) -> None:
    """Per library kernel (and grid): mean of each counter per dispatch, and
    the MFMA busy fraction where both counters were collected: busy cycles
    summed over the 1024 SIMDs / (1024 x the kernel's GPU-active cycles).
    rocprofv3 reports GRBM_GUI_ACTIVE summed over the chip's 8 XCDs (each
    counts the same active cycles), so the active cycles are that sum / 8 --
    the maximum over XCDs that rocprofv3's own MfmaUtil takes."""
    vals = defaultdict(lambda: defaultdict(list))
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            if LIB_KERNEL not in r["Kernel_Name"] or any(k in r["Kernel_Name"] for k in SETUP_KERNELS):
                continue
            grid = r.get("Grid_Size") or r.get("Grid_Size_X", "")
            vals[(_short(r["Kernel_Name"]), grid)][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for v in vals.values() for c in v})
    lines = _header(cmds) + [f"{'kernel':44s} {'grid':>8s} {'n':>5s} " + " ".join(f"{c[:24]:>24s}" for c in names)
             + ("  mfma_busy_%" if {"SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"} <= set(names) else "")]
    for (k, g), v in sorted(vals.items()):
        n = max(len(x) for x in v.values())
        means = {c: sum(x) / len(x) for c, x in v.items()}
        line = f"{k[:44]:44s} {g:>8s} {n:5d} " + " ".join(f"{means.get(c, float('nan')):24.1f}"
                                                          for c in names)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in means and "GRBM_GUI_ACTIVE" in means:
            active = means["GRBM_GUI_ACTIVE"] / XCDS
            line += f"  {100.0 * means['SQ_VALU_MFMA_BUSY_CYCLES'] / (active * 1024):11.1f}"
        lines.append(line)
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)


# ----------------------------------------------------------------------------- trace

def _short(name: str) -> str:
    name = name.replace("q4::(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name).replace("void ", "")


def _trace(path: str, out: str | None, last: int = 0, workload: str | None = None,
           cmds=None) -> None:
    rows = defaultdict(list)
    timeline = []
    markers = []                # start times of the marker kernel
    order = defaultdict(list)   # (kernel, grid) -> [(start, ns)] for the timed window
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            ns = t1 - t0
            grid = r.get("Grid_Size") or r.get("Grid_Size_X", "")
            wg = r.get("Workgroup_Size") or r.get("Workgroup_Size_X", "")
            rows[(_short(r["Kernel_Name"]), grid, wg)].append(ns)
            if MARKER_KERNEL in r["Kernel_Name"]:
                markers.append(t0)
            order[(_short(r["Kernel_Name"]), grid)].append((t0, ns))
            if LIB_KERNEL in r["Kernel_Name"] and not any(k in r["Kernel_Name"] for k in SETUP_KERNELS):
                timeline.append((t0, t1, _short(r["Kernel_Name"])))
    lines = _header(cmds)
    stats = path.replace("_kernel_trace.csv", "_kernel_stats.csv")
    if stats != path and os.path.exists(stats):  # rocprofv3 --stats of the same run
        lines.append("## rocprofv3 --stats (per kernel name)")
        lines.append(f"{'kernel':58s} {'calls':>7s} {'avg_us':>9s} {'min_us':>8s} {'max_us':>8s} {'pct':>6s}")
        with open(stats, newline="") as fh:
            for r in csv.DictReader(fh):
                lines.append(f"{_short(r['Name'])[:58]:58s} {int(r['Calls']):7d} "
                             f"{float(r['AverageNs']) / 1e3:9.3f} {float(r['MinNs']) / 1e3:8.3f} "
                             f"{float(r['MaxNs']) / 1e3:8.3f} {float(r['Percentage']):6.2f}")
        lines.append("## per kernel and grid (from the same trace)")
    lines.append(f"{'kernel':58s} {'grid(thr)':>10s} {'wg':>4s} {'calls':>7s} {'avg_us':>9s} "
                 f"{'median_us':>9s} {'min_us':>8s}")
    for (k, g, w), v in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(v)
        lines.append(f"{k[:58]:58s} {g:>10s} {w:>4s} {len(v):7d} {sum(v) / len(v) / 1e3:9.3f} "
                     f"{v[len(v) // 2] / 1e3:9.3f} {v[0] / 1e3:8.3f}")
    if last > 0:
        lib_names = {t[2] for t in timeline}
        if markers:
            # the timed window: every library dispatch after the last marker
            t0 = max(markers)
            lines.append(f"## timed window: library dispatches after the marker kernel "
                         f"({last} calls)")
            if workload:
                lines.append(f"source_hash: {source_hash(workload)}")
            total = 0
            for (k, g), v in sorted(order.items(), key=lambda kv: -sum(x[1] for x in kv[1])):
                if k not in lib_names:
                    continue
                v = [ns for st, ns in v if st > t0]
                if not v:
                    continue
                total += sum(v)
                lines.append(f"window_mean_us[{k} grid={g}]: {sum(v) / len(v) / 1e3:.3f}  "
                             f"(n={len(v)}, {len(v) / last:g} per call)")
            lines.append(f"call_kernel_us: {total / last / 1e3:.3f}  (sum of the window's "
                         f"library kernel time / {last} calls)")
        else:
            # no marker (older runs): the last `last` dispatches of each
            # (kernel, grid); kernels sharing a grid are then counted once
            lines.append(f"## timed window: mean over the last dispatches of each library kernel "
                         f"({last} calls)")
            if workload:
                lines.append(f"source_hash: {source_hash(workload)}")
            for (k, g), v in sorted(order.items(), key=lambda kv: -sum(x[1] for x in kv[1])):
                if k not in lib_names:
                    continue
                v = [ns for _, ns in sorted(v)][-last:]
                lines.append(f"window_mean_us[{k} grid={g}]: {sum(v) / len(v) / 1e3:.3f}  "
                             f"(n={len(v)})")
    if len(timeline) > 1:
        # idle time between one library kernel's end and the next one's start
        timeline.sort()
        gaps = defaultdict(list)
        for (a0, a1, an), (b0, b1, bn) in zip(timeline, timeline[1:]):
            gaps[(an, bn)].append(b0 - a1)
        lines.append("## gaps between consecutive library kernels (next start - previous end)")
        lines.append(f"{'previous kernel -> next kernel':90s} {'count':>6s} {'median_us':>9s} "
                     f"{'min_us':>8s}")
        for (an, bn), v in sorted(gaps.items(), key=lambda kv: -len(kv[1])):
            v = sorted(v)
            lines.append(f"{(an[:44] + ' -> ' + bn[:42]):90s} {len(v):6d} {v[len(v) // 2] / 1e3:9.3f} "
                         f"{v[0] / 1e3:8.3f}")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("workload")
    r.add_argument("--iters", type=int, default=20)
    r.add_argument("--graph", action="store_true",
                   help="replay a HIP graph of rotated calls (the bench's timing mode)")
    t = sub.add_parser("traffic")
    t.add_argument("workload")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--out", default=os.path.join(ROOT, "profiles", "hbm_traffic_counters.txt"))
    s = sub.add_parser("trace")
    s.add_argument("csv")
    s.add_argument("--out")
    s.add_argument("--last", type=int, default=0,
                   help="also report each library kernel's mean over its last N dispatches")
    s.add_argument("--workload", help="tag the summary with this workload's source hash")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--out")
    for q in (s, c):
        q.add_argument("--cmd", action="append", dest="cmds",
                       help="a command that produced the CSV, written as a '# ' header line")
    a = p.parse_args(argv)
    if a.cmd == "run":
        _run(a.workload, a.iters, a.graph)
    elif a.cmd == "traffic":
        _traffic(a.workload, a.fetch, a.write, a.out)
    elif a.cmd == "counters":
        _counters(a.csv, a.out, a.cmds)
    else:
        _trace(a.csv, a.out, a.last, a.workload, a.cmds)


if __name__ == "__main__":
    main()
