"""The small-M kernel's two-part binary16 activations, emulated on the CPU.

For up to four rows of x with large weights, q4_matmul multiplies exact
centred codes on the matrix cores and carries x as two binary16 parts after
scaling each 256-value chunk of a row so that its largest magnitude lies in
[2^14, 2^15).  A value far below its chunk's largest then falls into the
binary16 subnormals and loses its relative precision.  The kernel therefore
keeps a chunk whose nonzero magnitudes span more than 2^20 (or whose largest
is 2^124 or more) off the matrix cores and sums it in float32.  This test
emulates that arithmetic with numpy's binary16 (round to nearest even,
subnormals kept) and checks it against the oracle's bound 1e-4 * B + 1e-6:
with the rule every case passes; without it an outlier on zero-weight
columns breaks the bound, which is the failure the rule exists for.
"""

import numpy as np
import pytest

from oracle import q4_oracle as O

CHUNK = 256


def _scale_exp(cmax: float) -> int:
    """Power of two putting cmax in [2^14, 2^15), clamped to +-110 (the
    kernel's clamp keeps the scale and its inverse normal floats)."""
    if cmax == 0.0:
        return 110
    e = int(np.floor(np.log2(cmax)))
    return int(np.clip(14 - e, -110, 110))


def emulate_row(w: np.ndarray, x: np.ndarray, wide_rule: bool) -> np.ndarray:
    """y = w @ x with x represented as the kernel represents it: per chunk,
    either exactly (float32 path, emulated in float64: its rounding is that
    of the matvec, far inside the bound) or as hi + lo binary16 parts of the
    scaled chunk.  Products and sums in float64: only the representation of
    x is emulated."""
    xr = np.empty(x.size, dtype=np.float64)
    for c in range(0, x.size, CHUNK):
        v = x[c:c + CHUNK].astype(np.float32)
        a = np.abs(v)
        cmax = float(a.max())
        nz = a[a > 0]
        cmin = float(nz.min()) if nz.size else np.inf
        wide = not (cmax < 2.0 ** 124) or cmin < cmax * 2.0 ** -20
        if wide and wide_rule:
            xr[c:c + CHUNK] = v.astype(np.float64)
            continue
        se = _scale_exp(cmax)
        xs = (v.astype(np.float64) * 2.0 ** se).astype(np.float32)
        hi = xs.astype(np.float16)
        lo = (xs - hi.astype(np.float32)).astype(np.float16)
        xr[c:c + CHUNK] = (hi.astype(np.float64) + lo.astype(np.float64)) * 2.0 ** -se
    return w.astype(np.float64) @ xr


def _case(kind: str, k: int, seed: int):
    g = np.random.Generator(np.random.PCG64(seed))
    n = 32
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = g.standard_normal(k)
    cols = [3, 77, k // 2 + 5, k - 1]
    if kind.startswith("outlier"):
        w[:, cols] = 0.0                       # zero columns: code 8 in every row
        x[cols] = float(kind.split("_")[1])
    elif kind == "huge_3e35":
        x *= 3e35                              # the top of the float32 block sums
    elif kind == "tiny_among_normal":
        x[::97] *= 1e-9
    elif kind == "normal":
        pass
    qb = O.quantize_q4_0(w)
    wd = O.dequantize_q4_0(qb, n, k)
    return qb, wd, x.astype(np.float32), n


@pytest.mark.parametrize("kind", ["normal", "tiny_among_normal", "outlier_1e6", "outlier_1e9",
                                  "outlier_1e11", "outlier_1e20", "outlier_3e38",
                                  "huge_3e35"])
def test_two_part_x_with_wide_chunks_meets_matvec_bound(kind):
    k = 12352
    qb, wd, x, n = _case(kind, k, 17)
    ref, b = O.matvec_f64(qb, x, n, k)
    y = emulate_row(wd, x, wide_rule=True)
    tol = O.tolerance(b, O.MATVEC_REL, O.MATVEC_ABS)
    assert np.all(np.abs(y - ref) <= tol), float(np.max(np.abs(y - ref) / tol))


@pytest.mark.parametrize("kind", ["outlier_1e11", "outlier_1e20", "outlier_3e38"])
def test_without_the_rule_outliers_break_the_bound(kind):
    """The failure the rule prevents: a huge x on zero-weight columns sets the
    chunk's scale, the other values become binary16 subnormals."""
    k = 12352
    qb, wd, x, n = _case(kind, k, 17)
    ref, b = O.matvec_f64(qb, x, n, k)
    y = emulate_row(wd, x, wide_rule=False)
    tol = O.tolerance(b, O.MATVEC_REL, O.MATVEC_ABS)
    assert np.any(~(np.abs(y - ref) <= tol))       # NaN (an overflowed part) counts


def test_normal_activations_rarely_take_the_float32_path():
    """N(0, 1) activations: under 1 % of 256-value chunks are wide."""
    g = np.random.Generator(np.random.PCG64(3))
    x = g.standard_normal((4000, CHUNK)).astype(np.float32)
    a = np.abs(x)
    cmax = a.max(axis=1)
    cmin = np.where(a > 0, a, np.inf).min(axis=1)
    wide = cmin < cmax * 2.0 ** -20
    assert wide.mean() < 0.01
