"""Checks that pin the CPU oracle to facts outside itself.

Each ``check_*`` function takes the oracle module (or a deliberately broken
copy of it, see test_oracle_mutants.py) and raises AssertionError on a
mismatch.  The expected values never come from the oracle under test: they
come from the hand-worked blocks in golden/q4_0_blocks.txt, from an
independent bit-level binary16 decoder with exact rational arithmetic
(fractions.Fraction), from integer arithmetic, or from invariants the
mathematics of the Q4_0 rule fixes.
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q4_0_blocks.txt")


# --------------------------------------------------------------------------
# Independent exact decoder (bit level, Fraction arithmetic)
# --------------------------------------------------------------------------

def half_bits_to_fraction(bits: int) -> Fraction:
    """Exact value of an IEEE binary16 bit pattern (finite only)."""
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    if e == 0x1F:
        raise ValueError("inf/nan")
    if e == 0:
        return s * Fraction(f, 1 << 24)
    return s * Fraction(1024 + f, 1 << 10) * (Fraction(2) ** (e - 15))


def exact_block(block18) -> list:
    """The 32 exact decoded values of one 18-byte block, element order."""
    b = [int(v) for v in block18]
    d = half_bits_to_fraction(b[0] | (b[1] << 8))
    lo = [(b[2 + j] & 0x0F) - 8 for j in range(16)]
    hi = [(b[2 + j] >> 4) - 8 for j in range(16)]
    return [q * d for q in lo + hi]


def exact_matrix(qbytes, n, k) -> list:
    rb = k // 32 * 18
    raw = np.asarray(qbytes, dtype=np.uint8).reshape(n, rb)
    rows = []
    for r in range(n):
        row = []
        for b in range(k // 32):
            row += exact_block(raw[r, 18 * b:18 * b + 18])
        rows.append(row)
    return rows


def rne_f16(v: Fraction) -> Fraction:
    """Round a rational to binary16, nearest with ties to even, by bisection
    over the bit patterns (positive finite patterns 0x0000..0x7BFF increase
    with their value).  Overflow is outside what the callers pass."""
    a = abs(v)
    lo, hi = 0, 0x7BFF
    if a >= half_bits_to_fraction(hi):
        r = half_bits_to_fraction(hi)
    else:
        while hi - lo > 1:                  # invariant: val(lo) <= a < val(hi)
            mid = (lo + hi) // 2
            if half_bits_to_fraction(mid) <= a:
                lo = mid
            else:
                hi = mid
        dl = a - half_bits_to_fraction(lo)
        dh = half_bits_to_fraction(hi) - a
        pick = lo if (dl < dh or (dl == dh and lo % 2 == 0)) else hi
        r = half_bits_to_fraction(pick)
    return -r if v < 0 else r


# --------------------------------------------------------------------------
# Golden blocks
# --------------------------------------------------------------------------

def _pairs(text, default):
    vals = [default] * 32
    text = text.strip()
    if text.startswith("all"):
        parts = text.split()[1:]
        assert len(parts) == 32
        return parts
    for tok in text.split():
        i, v = tok.split("=")
        vals[int(i)] = v
    return vals


def load_golden():
    blocks, cur = [], None
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.rstrip("\n")
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = {"name": line.strip("[]")}
                blocks.append(cur)
                continue
            key, _, val = line.partition(":")
            cur[key.strip()] = val.strip()
    out = []
    for b in blocks:
        x = np.array([np.float32(v) for v in _pairs(b.get("x", ""), "0")], dtype=np.float32)
        rest = b.get("deq_rest", "0.0")
        deq = np.array([np.float32(v) for v in _pairs(b["deq"], rest)], dtype=np.float32)
        f16 = {}
        if "f16" in b:
            for tok in b["f16"].split():
                i, v = tok.split("=")
                f16[int(i)] = np.float32(v)
        out.append(dict(name=b["name"], x=x, bytes=bytes.fromhex(b["bytes"]), deq=deq, f16=f16))
    return out


def check_golden_blocks(o):
    for g in load_golden():
        got = o.quantize_q4_0(g["x"][None, :]).tobytes()
        assert got == g["bytes"], f"block {g['name']}: {got.hex(' ')} != {g['bytes'].hex(' ')}"
        deq = o.dequantize_q4_0(np.frombuffer(g["bytes"], np.uint8), 1, 32)[0]
        # bit patterns, signed zeros included
        assert np.array_equal(deq.view(np.uint32), g["deq"].view(np.uint32)), g["name"]
        for i, v in g["f16"].items():
            assert o.round_f16(deq[i:i + 1])[0] == v, (g["name"], i)


# --------------------------------------------------------------------------
# Quantizer against its characterisation
# --------------------------------------------------------------------------

def _random_blocks(seed, nblocks):
    g = np.random.Generator(np.random.PCG64(seed))
    parts = [
        g.standard_normal((nblocks, 32), dtype=np.float32) * np.float32(0.02),
        g.standard_normal((nblocks, 32), dtype=np.float32),
        # integer grids create exact ties on |x| and exact half-way codes
        g.integers(-16, 17, (nblocks, 32)).astype(np.float32) * np.float32(0.25),
        # wide dynamic range
        (g.standard_normal((nblocks, 32)) * np.exp2(g.integers(-30, 10, (nblocks, 1)))).astype(np.float32),
    ]
    return np.concatenate(parts, axis=0)


def check_quantizer_exact(o, nblocks=400, seed=11):
    """d16 = RNE16(m / -8) and q = the nearest of the 16 levels (ties to the
    larger code), both decided in exact rational arithmetic."""
    x = _random_blocks(seed, nblocks // 4)
    qb = o.quantize_q4_0(x)
    for r in range(x.shape[0]):
        blk = [Fraction(float(v)) for v in x[r]]
        mags = [abs(v) for v in blk]
        i_star = mags.index(max(mags))
        m = blk[i_star]
        # m / -8 is exact in float32 unless it underflows; the inputs here stay
        # far from the float32 subnormal range.
        d16 = rne_f16(m / -8) if m != 0 else Fraction(0)
        got = exact_block(qb[r])
        b0, b1 = int(qb[r][0]), int(qb[r][1])
        got_d = half_bits_to_fraction(b0 | (b1 << 8))
        assert got_d == d16, (r, got_d, d16)
        for i in range(32):
            if d16 == 0:
                assert got[i] == 0
                continue
            levels = [(abs(blk[i] - (q - 8) * d16), -q, q) for q in range(16)]
            qbest = min(levels)[2]
            assert got[i] == (qbest - 8) * d16, (r, i)


def check_quantizer_invariants(o, nblocks=25000, seed=7):
    x = _random_blocks(seed, nblocks)              # 4 * nblocks blocks
    qb = o.quantize_q4_0(x)
    d = o.block_scales(qb, x.shape[0], 32)[:, 0].astype(np.float64)
    q = o.block_codes(qb, x.shape[0], 32)[:, 0, :].astype(np.int64)
    deq = o.dequantize_q4_0(qb, x.shape[0], 32).astype(np.float64)
    xd = x.astype(np.float64)
    nz = d != 0
    # a normal binary16 scale is within 2^-11 (relative) of m/-8; a subnormal
    # one can be much coarser, and then the two invariants marked (*) below
    # do not hold (e.g. m/-8 = 1.5 * 2^-24 stores as 2^-23 and m gets code 2)
    normal = np.abs(d) >= 2.0 ** -14
    assert np.any(nz & ~normal) and np.any(normal)   # both kinds are exercised
    # decoded values lie on the 16-level grid of their block
    assert np.array_equal(deq[nz], (q[nz] - 8) * d[nz, None])
    # (*) the element of largest magnitude (first on ties) encodes to code 0
    i_star = np.argmax(np.abs(x), axis=1)
    assert np.all(q[np.arange(x.shape[0]), i_star][normal] == 0)
    # |x - deq| <= |d|/2 wherever the code is not clamped, i.e. -8.5 <= t <= 7.5
    # with t = x/d16 (t = 7.5 clamps 16 -> 15 but still lands |d|/2 away)
    t = xd[nz] / d[nz, None]
    inside = (t >= -8.5) & (t <= 7.5)
    err = np.abs(xd[nz] - deq[nz])
    half = np.abs(d[nz, None] / 2).repeat(32, 1)
    assert np.all(err[inside] <= half[inside])
    # clamped from above -> code 15; from below (only possible with a
    # subnormal scale) -> code 0
    assert np.all(q[nz][t > 7.5] == 15)
    assert np.all(q[nz][t < -8.5] == 0)
    assert not np.any((t < -8.5) & normal[nz, None])
    # monotone in x whatever the sign of d
    order = np.argsort(xd, axis=1, kind="stable")
    sd = np.take_along_axis(deq, order, axis=1)
    assert np.all(np.diff(sd, axis=1) >= 0)
    # (*) idempotent on blocks with a normal scale
    again = o.quantize_q4_0(o.dequantize_q4_0(qb, x.shape[0], 32))
    assert np.array_equal(again[normal], qb[normal])
    # zero-scale blocks carry code 8 everywhere
    assert np.all(q[~nz] == 8)


def check_quantizer_errors(o):
    import pytest
    with pytest.raises(ValueError):
        o.quantize_q4_0(np.full((1, 32), 6.0e5, np.float32))      # d overflows binary16
    with pytest.raises(ValueError):
        o.quantize_q4_0(np.array([[np.nan] + [0.0] * 31], np.float32))
    with pytest.raises(ValueError):
        o.quantize_q4_0(np.zeros((1, 48), np.float32))            # K % 32 != 0
    # largest finite scale: |m| = 524000 -> d = -65500 -> binary16 65504
    qb = o.quantize_q4_0(np.array([[524000.0] + [0.0] * 31], np.float32))
    assert half_bits_to_fraction(int(qb[0, 0]) | int(qb[0, 1]) << 8) == -65504


# --------------------------------------------------------------------------
# Decoder against the exact bit-level decoder
# --------------------------------------------------------------------------

def check_dequantizer_exact(o, seed=3, nrows=64, k=128):
    g = np.random.Generator(np.random.PCG64(seed))
    raw = g.integers(0, 256, (nrows, k // 32, 18), dtype=np.uint8)
    # keep scales finite: clear the exponent's top bit when it would be 0x1F
    hi = raw[..., 1]
    raw[..., 1] = np.where((hi & 0x7C) == 0x7C, hi & 0xBF, hi)
    qb = raw.reshape(nrows, -1)
    got = o.dequantize_q4_0(qb, nrows, k)
    ref = exact_matrix(qb, nrows, k)
    for r in range(nrows):
        for c in range(k):
            assert Fraction(float(got[r, c])) == ref[r][c], (r, c)


# --------------------------------------------------------------------------
# Products
# --------------------------------------------------------------------------

def _tiny_case(g, n, k, m):
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    return w, g.standard_normal((m, k)).astype(np.float32)


def check_products_exact(o, seed=5):
    g = np.random.Generator(np.random.PCG64(seed))
    for n, k, m in [(1, 32, 1), (3, 64, 2), (4, 96, 3), (2, 32, 3), (4, 64, 1)]:
        w, x = _tiny_case(g, n, k, m)
        qb = o.quantize_q4_0(w)
        ew = exact_matrix(qb, n, k)
        ex = [[Fraction(float(v)) for v in row] for row in x]
        y, b = o.matmul_f64(qb, x, n, k)
        assert y.shape == (m, n)
        for i in range(m):
            for j in range(n):
                yy = sum(ex[i][kk] * ew[j][kk] for kk in range(k))
                bb = sum(abs(ex[i][kk] * ew[j][kk]) for kk in range(k))
                assert abs(Fraction(float(y[i, j])) - yy) <= Fraction(1, 10**12) * bb
                assert abs(Fraction(float(b[i, j])) - bb) <= Fraction(1, 10**12) * bb
        yv, bv = o.matvec_f64(qb, x[0], n, k)
        for j in range(n):
            yy = sum(ex[0][kk] * ew[j][kk] for kk in range(k))
            assert abs(Fraction(float(yv[j])) - yy) <= Fraction(1, 10**12) * abs(Fraction(float(bv[j])))


def integer_weight_case(seed, n, k, m, xmax=4):
    """Blocks whose stored scale is exactly 1 (codes hold the integers -8..7)
    and small-integer activations: every product and partial sum is exact in
    binary16/float32, so device results must equal integer arithmetic."""
    g = np.random.Generator(np.random.PCG64(seed))
    wi = g.integers(-8, 8, (n, k)).astype(np.float32)
    wi[:, ::32] = -8.0             # each block's first element is the max: d = 1
    xi = g.integers(-xmax, xmax + 1, (m, k)).astype(np.float32)
    return wi, xi


def check_integer_special_case(o, seed=9):
    n, k, m = 24, 256, 5
    wi, xi = integer_weight_case(seed, n, k, m)
    qb = o.quantize_q4_0(wi)
    ref = xi.astype(np.int64) @ wi.astype(np.int64).T
    y, _ = o.matmul_f64(qb, xi, n, k)
    assert np.array_equal(y, ref.astype(np.float64))
    yv, _ = o.matvec_f64(qb, xi[2], n, k)
    assert np.array_equal(yv, ref[2].astype(np.float64))


def check_product_properties(o, seed=13):
    g = np.random.Generator(np.random.PCG64(seed))
    n, k, m = 40, 192, 6
    w, x = _tiny_case(g, n, k, m)
    qb = o.quantize_q4_0(w)
    y, b = o.matmul_f64(qb, x, n, k)
    # linearity in x
    x2 = g.standard_normal((m, k)).astype(np.float32)
    y2, _ = o.matmul_f64(qb, x2, n, k)
    ys, _ = o.matmul_f64(qb, (x.astype(np.float64) + x2).astype(np.float32), n, k)
    # x + x2 rounded to float32 perturbs each term by <= 2^-24 relative
    _, bs = o.matmul_f64(qb, np.abs(x) + np.abs(x2), n, k)
    assert np.all(np.abs(ys - (y + y2)) <= 1e-6 * bs + 1e-12)
    # permuting rows of X permutes rows of Y
    p = g.permutation(m)
    yp, _ = o.matmul_f64(qb, x[p], n, k)
    assert np.array_equal(yp, y[p])
    # the matvec is the M = 1 row
    for i in range(m):
        yv, bv = o.matvec_f64(qb, x[i], n, k)
        assert np.allclose(yv, y[i], rtol=0, atol=1e-12 * float(b.max()))
        assert np.allclose(bv, b[i], rtol=0, atol=1e-12 * float(b.max()))


# --------------------------------------------------------------------------
# Embedding rows and argmax
# --------------------------------------------------------------------------

def check_embed(o, seed=17):
    g = np.random.Generator(np.random.PCG64(seed))
    n, k = 10, 96
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    qb = o.quantize_q4_0(w)
    ids = np.array([3, 0, 9, 3, -1, 10, 7], dtype=np.int32)
    out = o.embed_rows(qb, ids, n, k)
    ew = exact_matrix(qb, n, k)
    for i, r in enumerate(ids):
        for c in range(k):
            want = ew[r][c] if 0 <= r < n else Fraction(0)
            assert Fraction(float(out[i, c])) == want


def check_argmax(o, seed=19):
    g = np.random.Generator(np.random.PCG64(seed))
    n, k = 12, 64
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[7] = w[2]                 # duplicated rows: identical logits
    x = g.standard_normal(k).astype(np.float32)
    # make rows 2 and 7 the winners
    w[2] = w[7] = np.float32(0.02) * np.sign(x)
    qb = o.quantize_q4_0(w)
    y, b = o.lmhead_logits(qb, x, n, k, panel=5)
    ew = exact_matrix(qb, n, k)
    ex = [Fraction(float(v)) for v in x]
    exact = [sum(ew[r][c] * ex[c] for c in range(k)) for r in range(n)]
    best = max(range(n), key=lambda r: (exact[r], -r))
    assert best == 2
    assert o.argmax_lowest(y) == best
    assert o.argmax_accepts(y, b, 2)
    assert o.argmax_accepts(y, b, 7)          # exact tie: either is acceptable
    assert not o.argmax_accepts(y, b, 0)
    assert o.top2_margin(y) == 0.0
    yv, _ = o.matvec_f64(qb, x, n, k)
    assert np.array_equal(yv, y)
    # a clear margin demands the exact index
    yy = np.array([0.0, 1.0, 0.5])
    bb = np.array([1.0, 1.0, 1.0])
    assert o.argmax_accepts(yy, bb, 1) and not o.argmax_accepts(yy, bb, 2)
    # a margin inside the tolerance admits the runner-up
    yy = np.array([0.0, 1.0, 1.0 - 1e-5])
    bb = np.array([1.0, 1.0, 1.0])
    assert o.argmax_accepts(yy, bb, 2) and not o.argmax_accepts(yy, bb, 0)
    check_argmax_clear_margin(o)


def check_argmax_clear_margin(o):
    """The clear-margin clause with unequal bounds: once the top-2 margin
    exceeds the two leaders' tolerances only the oracle's index is accepted,
    even where a third row's own tolerance is wide enough to reach the
    maximum; with a close race that row is accepted.  The absolute term of
    the bound (1e-6) decides races between rows whose sums of |w x| are 0."""
    rel, abs_ = o.MATVEC_REL, o.MATVEC_ABS
    # leaders 1.0 and 0.9 with zero bounds: margin 0.1 >> 2e-6; row 2 lies
    # 0.15 below the maximum but its bound 2000 gives it a tolerance of 0.2
    yy = np.array([1.0, 0.9, 0.85])
    bb = np.array([0.0, 0.0, 2000.0])
    assert o.argmax_accepts(yy, bb, 0)
    assert not o.argmax_accepts(yy, bb, 1)
    assert not o.argmax_accepts(yy, bb, 2)
    # the same third row in a close race (runner-up 1e-6 below) is accepted
    yy = np.array([1.0, 1.0 - 1e-6, 0.85])
    assert o.argmax_accepts(yy, bb, 1) and o.argmax_accepts(yy, bb, 2)
    # the runner-up is the largest other logit, not the next index, and its
    # own bound counts: a margin of 0.05 against tolerances 0 + 0.1 is close
    yy = np.array([0.2, 1.0, 0.3, 0.95])
    bb = np.array([0.0, 0.0, 0.0, 1000.0])
    assert o.argmax_accepts(yy, bb, 3)
    assert not o.argmax_accepts(yy, bb, 2)       # 0.7 below, tolerance 1e-6
    bb = np.array([1000.0, 0.0, 0.0, 0.0])       # the wide bound on a non-leader
    assert not o.argmax_accepts(yy, bb, 3)
    assert not o.argmax_accepts(yy, bb, 0)
    # rows whose sums of |w x| are 0 (all-zero weights): only the absolute
    # term separates them, so a gap of 1e-7 < 2e-6 is a close race
    yy = np.array([1e-7, 0.0])
    bb = np.array([0.0, 0.0])
    assert o.argmax_accepts(yy, bb, 0) and o.argmax_accepts(yy, bb, 1)
    # and a gap of 3e-6 > 2e-6 is not
    yy = np.array([3e-6, 0.0])
    assert not o.argmax_accepts(yy, bb, 1)
    # the relative term: logits 1 and 1 - 1.5e-4 with bounds 1 each give
    # tolerances 1.01e-4, a close race; with bounds 0.5 (5.1e-5) a clear one
    yy = np.array([1.0, 1.0 - 1.5e-4])
    assert o.argmax_accepts(yy, np.array([1.0, 1.0]), 1)
    assert not o.argmax_accepts(yy, np.array([0.5, 0.5]), 1)
    # a single row: only index 0
    assert o.argmax_accepts(np.array([5.0]), np.array([1.0]), 0)
    assert not o.argmax_accepts(np.array([5.0]), np.array([1.0]), 1)
    assert abs(rel - 1e-4) == 0 and abs(abs_ - 1e-6) == 0


ALL_CHECKS = [
    check_golden_blocks,
    check_quantizer_exact,
    check_quantizer_invariants,
    check_quantizer_errors,
    check_dequantizer_exact,
    check_products_exact,
    check_integer_special_case,
    check_product_properties,
    check_embed,
    check_argmax,
]
