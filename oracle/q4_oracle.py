"""CPU oracle for the GGUF Q4_0 hot path (test infrastructure only).

This module is the plain, slow, obviously-correct statement of what the GPU
library computes.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the library itself never does, and this file
imports nothing from the library.

Sources.  The pages are the five copies of the news item "Implémentation en
Rust du modèle Voxtral Mini 4B Realtime de Mistral pour l'exécuter dans le
navigateur" (fr/es/id/hi.news.hada.io) and the blog post "Voxtral Mini 4B:
Implementación Rust y WebGPU para transcripción local" (usedby.ai).  Their
section *Architecture* says the browser path runs the model from a GGUF Q4_0
file with custom shaders, over an encoder of width 1280 and a decoder of width
3072 with GQA 32Q/8KV; section *Solutions techniques pour l'exécution dans le
navigateur* (item 3) says the 1.5 GiB embedding table is kept as Q4 on the GPU
with a row lookup.  The pages do not spell out Q4_0 itself, so this oracle
follows the GGUF/ggml Q4_0 convention:

* a block holds 32 consecutive weights of one row: an IEEE binary16 scale
  ``d`` (little-endian, bytes 0-1) and 16 bytes ``qs``; weight ``j`` of the
  block is the low nibble of ``qs[j]`` and weight ``j+16`` the high nibble;
  its value is ``(q - 8) * d``;
* the encoder picks the element ``m`` of largest magnitude (first one on a
  tie, sign kept), sets ``d = m / -8`` and ``q = clamp(round(x / d) + 8, 0, 15)``.

Readings where that convention leaves a step open (each is listed with its
reason in the design notes): ties on ``|x|`` go to the first index; ``d`` is
computed in float32 and stored with round-to-nearest-even to binary16; the
codes are decided against the *stored* binary16 ``d``, dividing in float64;
"round" is half-up (``floor(t + 1/2)``, the direction of ggml's own encoder);
a block whose stored ``d`` is zero gets ``q = 8`` everywhere; a scale that
overflows binary16, or a non-finite input, is an error.

Arithmetic: dequantised weights are exact in float32 (a 5-bit integer times an
11-bit significand); products and sums are carried in float64 with a BLAS
routine as the only library step.  Every function below states the definition
it writes out.  No function here is "parity unpinned": each is checked in
``tests/test_oracle_pins.py`` against hand-worked blocks, exact rational
arithmetic on tiny inputs, and invariants that the mathematics fixes.
"""

from __future__ import annotations

import numpy as np

QK = 32                      # weights per Q4_0 block
BLOCK_BYTES = 2 + QK // 2    # binary16 scale + 16 bytes of nibbles = 18

# Acceptance bounds (per output element), with B = sum_k |w_k x_k| in float64
# over the exact dequantised weights w.
MATVEC_REL, MATVEC_ABS = 1e-4, 1e-6      # float32 FMA path
MFMA_REL, MFMA_ABS = 2e-3, 1e-5          # binary16-operand matrix-core path


def _check_k(k: int) -> None:
    if k <= 0 or k % QK:
        raise ValueError(f"K must be a positive multiple of {QK}, got {k}")


def row_bytes(k: int) -> int:
    """Bytes of one Q4_0 row of K weights (K/32 blocks of 18 bytes)."""
    _check_k(k)
    return (k // QK) * BLOCK_BYTES


# --------------------------------------------------------------------------
# Encoding (runs only here: the GPU kernels never see float weights except in
# the device-side encoder, which is checked byte-for-byte against this one).
# --------------------------------------------------------------------------

def quantize_q4_0(w) -> np.ndarray:
    """Encode a float32 matrix [N, K] as Q4_0 rows, returned as uint8 [N, K/32*18].

    Steps, per block of 32 consecutive values x[0..31] of a row (GGUF Q4_0, the
    format named in section *Architecture* of the pages):
      1. i* = first index of the largest |x_i|; m = x[i*] with its sign.
      2. d = m / -8 in float32; d16 = binary16(d), round to nearest even.
      3. if d16 == 0 every code is 8; otherwise t_i = x_i / d16 in float64 and
         q_i = clamp(floor(t_i + 1/2) + 8, 0, 15), with the half-up rounding
         taken on the exact fractional part of t_i.
      4. bytes: d16 little-endian, then qs[j] = q_j | (q_{j+16} << 4), j < 16.
    """
    x = np.asarray(w, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("expected a 2-D [N, K] array")
    n, k = x.shape
    _check_k(k)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite weight")
    blocks = x.reshape(n, k // QK, QK)

    # step 1: first index of the largest magnitude (np.argmax keeps the first)
    i_star = np.argmax(np.abs(blocks), axis=-1)
    m = np.take_along_axis(blocks, i_star[..., None], axis=-1)[..., 0]

    # step 2: scale, float32 division then binary16 storage
    d32 = (m / np.float32(-8.0)).astype(np.float32)
    d16 = d32.astype(np.float16)
    if np.any(np.isinf(d16)):
        raise ValueError("block scale overflows binary16 (|max| > 524,032)")

    # step 3: codes decided against the stored scale, in float64
    zero = d16 == 0
    safe_d = np.where(zero, np.float16(1.0), d16).astype(np.float64)
    t = blocks.astype(np.float64) / safe_d[..., None]
    fl = np.floor(t)
    r = fl + ((t - fl) >= 0.5)          # half-up; t - floor(t) is exact
    q = np.clip(r + 8.0, 0.0, 15.0)
    q = np.where(zero[..., None], 8.0, q).astype(np.uint8)

    # step 4: pack
    out = np.empty((n, k // QK, BLOCK_BYTES), dtype=np.uint8)
    bits = d16.view(np.uint16)
    out[..., 0] = (bits & 0xFF).astype(np.uint8)
    out[..., 1] = (bits >> 8).astype(np.uint8)
    out[..., 2:] = q[..., :16] | (q[..., 16:] << 4)
    return out.reshape(n, (k // QK) * BLOCK_BYTES)


# --------------------------------------------------------------------------
# Decoding
# --------------------------------------------------------------------------

def _blocks(qbytes, n: int, k: int) -> np.ndarray:
    _check_k(k)
    b = np.asarray(qbytes, dtype=np.uint8)
    if b.size != n * row_bytes(k):
        raise ValueError(f"expected {n * row_bytes(k)} bytes, got {b.size}")
    return b.reshape(n, k // QK, BLOCK_BYTES)


def block_scales(qbytes, n: int, k: int) -> np.ndarray:
    """The stored binary16 scales d16 as float32, shape [N, K/32]."""
    blk = _blocks(qbytes, n, k)
    bits = blk[..., 0].astype(np.uint16) | (blk[..., 1].astype(np.uint16) << 8)
    return bits.view(np.float16).astype(np.float32)


def block_codes(qbytes, n: int, k: int) -> np.ndarray:
    """The 4-bit codes q in element order, uint8 [N, K/32, 32]."""
    blk = _blocks(qbytes, n, k)
    qs = blk[..., 2:]
    return np.concatenate([qs & 0x0F, qs >> 4], axis=-1)


def dequantize_q4_0(qbytes, n: int, k: int) -> np.ndarray:
    """w[n, k] = (q - 8) * d16 as float32 [N, K].

    The float32 product is exact: q - 8 needs 4 bits and d16 11 significant
    bits, so no rounding happens and this is the value every kernel must see.
    """
    d = block_scales(qbytes, n, k)
    q = block_codes(qbytes, n, k).astype(np.float32) - np.float32(8.0)
    return (q * d[..., None]).reshape(n, k).astype(np.float32)


# --------------------------------------------------------------------------
# Products (float64 accumulation) and the error bound
# --------------------------------------------------------------------------

def matvec_f64(qbytes, x, n: int, k: int):
    """y[n] = sum_k w[n,k] x[k] and B[n] = sum_k |w[n,k] x[k]|, both float64.

    Definition of the decode-step projection (M = 1) over the dequantised
    weights; dgemv on the float64 panel is the only library step.
    """
    xv = np.asarray(x, dtype=np.float32).astype(np.float64)
    if xv.shape != (k,):
        raise ValueError("x must have shape [K]")
    w = dequantize_q4_0(qbytes, n, k).astype(np.float64)
    return w @ xv, np.abs(w) @ np.abs(xv)


def matmul_f64(qbytes, x, n: int, k: int):
    """Y[m,n] = sum_k X[m,k] w[n,k] and B[m,n] = sum_k |X[m,k] w[n,k]| (float64).

    X is float32 [M, K] row-major; the result is X times the transpose of the
    dequantised weight matrix, as in every projection of section
    *Architecture* (rows of X are tokens or audio frames).
    """
    xm = np.asarray(x, dtype=np.float32).astype(np.float64)
    if xm.ndim != 2 or xm.shape[1] != k:
        raise ValueError("X must have shape [M, K]")
    w = dequantize_q4_0(qbytes, n, k).astype(np.float64)
    return xm @ w.T, np.abs(xm) @ np.abs(w).T


def tolerance(bound, rel: float, abs_: float):
    """Per-element acceptance bound rel * B + abs."""
    return rel * np.asarray(bound, dtype=np.float64) + abs_


def round_f16(w) -> np.ndarray:
    """binary16 round-to-nearest-even of float32 values, returned as float32.

    The matrix-core path feeds weights and activations to the hardware as
    binary16; this is the value a one-hot probe of that path returns.
    """
    return np.asarray(w, dtype=np.float32).astype(np.float16).astype(np.float32)


# --------------------------------------------------------------------------
# Embedding rows and the LM-head argmax
# --------------------------------------------------------------------------

def embed_rows(table, ids, n: int, k: int) -> np.ndarray:
    """out[i, :] = dequantised row ids[i] of the Q4 table (float32 [M, K]).

    Section *Solutions techniques pour l'exécution dans le navigateur*, item 3:
    the token-embedding table stays in Q4 and rows are looked up by id.  An id
    outside [0, N) yields a row of zeros (the library's documented behaviour
    for ids it cannot check on the host).
    """
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    blk = _blocks(table, n, k)
    out = np.zeros((ids.size, k), dtype=np.float32)
    for i, r in enumerate(ids):
        if 0 <= r < n:
            out[i] = dequantize_q4_0(blk[r].reshape(-1), 1, k)[0]
    return out


def lmhead_logits(table, x, n: int, k: int, panel: int = 8192):
    """Logits y = T x and bounds B = |T| |x| over the table, in float64.

    Processed in row panels only to bound memory; the arithmetic per row is
    exactly matvec_f64.
    """
    xv = np.asarray(x, dtype=np.float32).astype(np.float64)
    blk = _blocks(table, n, k)
    y = np.empty(n, dtype=np.float64)
    b = np.empty(n, dtype=np.float64)
    for s in range(0, n, panel):
        e = min(n, s + panel)
        w = dequantize_q4_0(blk[s:e].reshape(-1), e - s, k).astype(np.float64)
        y[s:e] = w @ xv
        b[s:e] = np.abs(w) @ np.abs(xv)
    return y, b


def argmax_lowest(y) -> int:
    """Lowest index attaining the maximum of y (np.argmax keeps the first)."""
    return int(np.argmax(np.asarray(y)))


def argmax_accepts(y, bound, idx: int, rel: float = MATVEC_REL,
                   abs_: float = MATVEC_ABS) -> bool:
    """Whether a device argmax ``idx`` is consistent with exact logits ``y``.

    The leaders are the oracle's argmax (lowest index of the maximum) and the
    runner-up (lowest index of the largest logit among the other rows).  If
    the margin between them exceeds the sum of those two rows' tolerances, the
    index must be the oracle's, whatever the tolerances of the other rows.
    Otherwise the race is too close to call and any row whose exact logit lies
    within tol_best + tol_idx of the maximum is accepted.
    """
    y = np.asarray(y, dtype=np.float64)
    tol = tolerance(bound, rel, abs_)
    best = argmax_lowest(y)
    if not 0 <= idx < y.size:
        return False
    if idx == best:
        return True
    if y.size > 1:
        rest = y.copy()
        rest[best] = -np.inf
        second = argmax_lowest(rest)
        if y[best] - y[second] > tol[best] + tol[second]:
            return False
    return bool(y[idx] >= y[best] - (tol[best] + tol[idx]))


def top2_margin(y) -> float:
    """y_(1) - y_(2), the gap between the two largest logits."""
    s = np.sort(np.asarray(y, dtype=np.float64))
    return float(s[-1] - s[-2]) if s.size > 1 else float("inf")
