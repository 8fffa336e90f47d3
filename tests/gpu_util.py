"""Helpers for the GPU parity tests: device transfer, cached oracle inputs."""

from __future__ import annotations

import functools
import sys

import numpy as np
import pytest
import torch

from oracle import q4_oracle as O
from q4_quantized_speech_amd import synth


def have_gpu() -> bool:
    return torch.cuda.is_available()


needs_gpu = pytest.mark.skipif(not have_gpu(), reason="no HIP device visible")


def announce(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def quantize_panels(w: np.ndarray, panel: int = 4096) -> np.ndarray:
    """Oracle encoding of a tall matrix, a row panel at a time (memory bound)."""
    out = np.empty((w.shape[0], O.row_bytes(w.shape[1])), dtype=np.uint8)
    for s in range(0, w.shape[0], panel):
        out[s:s + panel] = O.quantize_q4_0(w[s:s + panel])
    return out


@functools.lru_cache(maxsize=None)
def weights_q4(n: int, k: int, seed: int) -> np.ndarray:
    """Oracle-encoded synthetic weights N(0, 0.02^2), cached per session."""
    return quantize_panels(synth.weights(n, k, seed))


@functools.lru_cache(maxsize=4)
def lm_table() -> np.ndarray:
    """The 131072 x 3072 Q4_0 table (encoded by the oracle)."""
    return weights_q4(synth.VOCAB, synth.DEC_DIM, synth.seed_for(2, 0))


def assert_within(y: np.ndarray, ref: np.ndarray, bound: np.ndarray, rel: float, abs_: float,
                  what: str) -> None:
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - ref)
    tol = rel * bound + abs_
    bad = err > tol
    if np.any(bad):
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
            f"got {y[i]!r} want {ref[i]!r} err {err[i]:.3e} tol {tol[i]:.3e}")
