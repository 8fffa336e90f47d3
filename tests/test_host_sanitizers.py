"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the C ABI's argument validation over every combination of extreme
sizes, and the GGUF reader -- which parses the untrusted bytes of the model's
pieces (section "Préparation du modèle et sharding" of "Implémentation en Rust
du modèle Voxtral Mini 4B Realtime de Mistral pour l'exécuter dans le
navigateur") -- over valid files, byte-split pieces, every malformed case of
the reader's own tests, and a seeded mutation fuzz of a valid file.

Built with clang throughout (one sanitizer runtime): the ABI source for the
host only, the reader and tests/c/san_driver.cpp as plain C++, the kernel
launchers replaced by the driver's stubs.  Any sanitizer report aborts the
driver with a non-zero status."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import gguf_writer as W
from test_gguf_cpu import _model, malformed_cases

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "q4_quantized_speech_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(HIPCC)),
                                reason="ROCm clang/hipcc not available")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    steps = [
        [HIPCC, "--offload-host-only", "-O1", "-g", "-std=c++17", *inc, *host_san, "-c",
         os.path.join(CSRC, "q4_abi.hip"), "-o", str(d / "abi.o")],
        [CLANG, "-O1", "-g", "-std=c++17", *inc, *SAN, "-c", os.path.join(CSRC, "q4_gguf.cpp"),
         "-o", str(d / "gguf.o")],
        [CLANG, "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *inc,
         *SAN, "-c", os.path.join(ROOT, "tests", "c", "san_driver.cpp"), "-o", str(d / "drv.o")],
        [CLANG, *SAN, str(d / "abi.o"), str(d / "gguf.o"), str(d / "drv.o"), "-L/opt/rocm/lib",
         "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(d / "san_driver")],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return str(d / "san_driver"), d


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=600)
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.returncode, r.stderr[-4000:])
    return r.stdout


def test_abi_validation_under_sanitizers(driver):
    exe, _ = driver
    assert _run(exe, "abi").strip() == "abi ok"


def _mutants(blob, seed, count):
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(count):
        b = bytearray(blob)
        kind = int(g.integers(0, 4))
        if kind == 0:                                   # flip a few bytes
            for p in g.integers(0, len(b), int(g.integers(1, 6))):
                b[p] = int(g.integers(0, 256))
        elif kind == 1:                                 # truncate
            b = b[: int(g.integers(0, len(b)))]
        elif kind == 2:                                 # large value in a count or length field
            p = int(g.integers(0, max(1, len(b) - 8)))
            b[p:p + 8] = int(g.integers(0, 2**63)).to_bytes(8, "little")
        else:                                           # insert or delete a run
            p = int(g.integers(0, len(b)))
            if g.random() < 0.5:
                b[p:p] = bytes(int(g.integers(1, 40)))
            else:
                del b[p:p + int(g.integers(1, 40))]
        out.append(bytes(b))
    return out


def test_gguf_reader_under_sanitizers(driver):
    exe, d = driver
    cases = []

    def add(blob, pieces=None):
        i = len(cases)
        if pieces is None:
            p = str(d / f"c{i}.gguf")
            with open(p, "wb") as f:
                f.write(blob)
            cases.append([p])
        else:
            cases.append(W.write_shards(blob, str(d / f"c{i}.gguf"), pieces))

    valid = []
    for alignment, version in [(32, 3), (64, 3), (256, 2), (1, 3)]:
        blob = _model(alignment, version)[0]
        valid.append(len(cases))
        add(blob)
    blob = _model()[0]
    for cuts in ([1], [5, 40], [100, 101, 1500], [24, 24, 700]):
        valid.append(len(cases))
        add(blob, cuts)
    bad = []
    for _, b in malformed_cases():
        bad.append(len(cases))
        add(b)
    for m in _mutants(blob, 2024, 400):
        add(m)
    with open(d / "list.txt", "w") as f:
        for c in cases:
            f.write(";".join(c) + "\n")
    status = [int(s) for s in _run(exe, "gguf", str(d / "list.txt")).split()]
    assert len(status) == len(cases)
    assert all(status[i] == 0 for i in valid)
    assert all(status[i] == 6 for i in bad)          # Q4_ERR_FORMAT
    assert set(status) <= {0, 6}, sorted(set(status))
