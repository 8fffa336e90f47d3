"""Profiling driver: runs one benchmark workload eagerly, for rocprofv3.

    python -m q4_quantized_speech_amd.profile_driver run WORKLOAD [--iters N]
    python -m q4_quantized_speech_amd.profile_driver traffic WORKLOAD \
        --fetch FETCH.csv --write WRITE.csv [--out FILE]
    python -m q4_quantized_speech_amd.profile_driver trace KERNEL_TRACE.csv [--out FILE]

``run`` builds the inputs of one workload with the same seeds and shapes as
bench.py, rotates enough weight copies (>= 1 GiB) that the Infinity Cache
cannot serve them, and calls the library N times; it then runs a plain
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
tells them apart).

Workload names are the keys bench.py reports:
    matvec_{qkv,o,gate_up,down}      decoder projections at M = 1
    matvec_3072x3072                 the single matvec
    lmhead_argmax_131072x3072        LM-head argmax at M = 1
    embed_rows_38x3072               embedding gather of 38 ids
    matmul_<proj>_M<m>_<n>x<k>       encoder, adapter or prefix GEMMs
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
CAL_BYTES = 256 << 20          # calibration kernel: reads and writes this many bytes
CAL_KERNEL = "neg_kernel"      # substring of torch's element-wise negation kernel
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


def dispatches_per_call(workload: str) -> int:
    """Distinct library kernels one call of the workload launches."""
    if workload.startswith("matmul_"):
        return 0  # one or two (the K-split fold), decided by the shape
    return 1


# ----------------------------------------------------------------------------- run

def _run(workload: str, iters: int) -> None:
    import torch

    import q4_quantized_speech_amd as q4
    from q4_quantized_speech_amd import synth

    dev = "cuda"
    torch.cuda.set_device(0)
    q4.lib()

    def encode(n, k, seed):
        w = torch.from_numpy(synth.weights(n, k, seed)).to(dev)
        out = q4.quantize(w)
        del w
        return out

    def rotate(w):
        r = max(2, -(-CACHE_DEFEAT_BYTES // w.numel()))
        return [w] + [w.clone() for _ in range(r - 1)]

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
        call = lambda i: q4.matvec(ws[i % len(ws)], x, out=y)  # noqa: E731
    elif workload == "matvec_3072x3072":
        ws = rotate(encode(3072, 3072, synth.seed_for(0, 0)))
        x = act(1, 3072, synth.seed_for(0, 1))[0]
        y = torch.empty(3072, device=dev)
        call = lambda i: q4.matvec(ws[i % len(ws)], x, out=y)  # noqa: E731
    elif workload in ("lmhead_argmax_131072x3072", "embed_rows_38x3072"):
        ws = rotate(encode(synth.VOCAB, synth.DEC_DIM, synth.seed_for(2, 0)))
        if workload.startswith("lmhead"):
            x = act(1, synth.DEC_DIM, synth.seed_for(2, 1))
            wsp = q4.lmhead_workspace(1, dev)
            call = lambda i: q4.lmhead_argmax(ws[i % len(ws)], x, workspace=wsp)  # noqa: E731
        else:
            ids = torch.from_numpy(synth.token_ids(synth.PREFIX_TOKENS, synth.seed_for(2, 2))).to(dev)
            out = torch.empty((synth.PREFIX_TOKENS, synth.DEC_DIM), device=dev)
            call = lambda i: q4.embed_rows(ws[i % len(ws)], ids, out=out)  # noqa: E731
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
        call = lambda i: q4.matmul(ws[i % len(ws)], x, out=y, workspace=wsp)  # noqa: E731

    torch.cuda.synchronize()
    print(f"[profile] {workload}: {iters} calls", flush=True)
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


# ----------------------------------------------------------------------------- trace

def _short(name: str) -> str:
    name = name.replace("q4::(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name).replace("void ", "")


def _trace(path: str, out: str | None) -> None:
    rows = defaultdict(list)
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            grid = r.get("Grid_Size") or r.get("Grid_Size_X", "")
            wg = r.get("Workgroup_Size") or r.get("Workgroup_Size_X", "")
            rows[(_short(r["Kernel_Name"]), grid, wg)].append(ns)
    lines = []
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
    t = sub.add_parser("traffic")
    t.add_argument("workload")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--out", default=os.path.join(ROOT, "profiles", "hbm_traffic_counters.txt"))
    s = sub.add_parser("trace")
    s.add_argument("csv")
    s.add_argument("--out")
    a = p.parse_args(argv)
    if a.cmd == "run":
        _run(a.workload, a.iters)
    elif a.cmd == "traffic":
        _traffic(a.workload, a.fetch, a.write, a.out)
    else:
        _trace(a.csv, a.out)


if __name__ == "__main__":
    main()
