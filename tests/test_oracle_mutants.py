"""Plant plausible mistakes in a copy of the oracle (on the CPU) and require
that the pins in oracle_checks.py catch every one of them."""

import os
import types

import pytest

import oracle_checks as oc

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "q4_oracle.py")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("nibble order swapped",
     "np.concatenate([qs & 0x0F, qs >> 4], axis=-1)",
     "np.concatenate([qs >> 4, qs & 0x0F], axis=-1)"),
    ("pack order swapped",
     "q[..., :16] | (q[..., 16:] << 4)",
     "q[..., 16:] | (q[..., :16] << 4)"),
    ("last index wins a |x| tie",
     "i_star = np.argmax(np.abs(blocks), axis=-1)",
     "i_star = 31 - np.argmax(np.abs(blocks)[..., ::-1], axis=-1)"),
    ("magnitude instead of signed max",
     "m = np.take_along_axis(blocks, i_star[..., None], axis=-1)[..., 0]",
     "m = np.abs(np.take_along_axis(blocks, i_star[..., None], axis=-1)[..., 0])"),
    ("scale sign flipped",
     "d32 = (m / np.float32(-8.0)).astype(np.float32)",
     "d32 = (m / np.float32(8.0)).astype(np.float32)"),
    ("round half to even",
     "r = fl + ((t - fl) >= 0.5)",
     "r = np.round(t)"),
    ("round half away from zero",
     "r = fl + ((t - fl) >= 0.5)",
     "r = np.sign(t) * np.floor(np.abs(t) + 0.5)"),
    ("codes from the unrounded float32 scale",
     "safe_d = np.where(zero, np.float16(1.0), d16).astype(np.float64)",
     "safe_d = np.where(zero, np.float32(1.0), d32).astype(np.float64)"),
    ("upper clamp dropped to 14",
     "q = np.clip(r + 8.0, 0.0, 15.0)",
     "q = np.clip(r + 8.0, 0.0, 14.0)"),
    ("offset 7 instead of 8 in the decoder",
     "q = block_codes(qbytes, n, k).astype(np.float32) - np.float32(8.0)",
     "q = block_codes(qbytes, n, k).astype(np.float32) - np.float32(7.0)"),
    ("scale bytes read big-endian",
     "bits = blk[..., 0].astype(np.uint16) | (blk[..., 1].astype(np.uint16) << 8)",
     "bits = blk[..., 1].astype(np.uint16) | (blk[..., 0].astype(np.uint16) << 8)"),
    ("matmul bound without |x|",
     "return xm @ w.T, np.abs(xm) @ np.abs(w).T",
     "return xm @ w.T, xm @ np.abs(w).T"),
    ("matmul operand transposed",
     "return xm @ w.T, np.abs(xm) @ np.abs(w).T",
     "return (w @ xm.T).T[:, ::-1], np.abs(xm) @ np.abs(w).T"),
    ("matvec in float32",
     "return w @ xv, np.abs(w) @ np.abs(xv)",
     "return (w.astype(np.float32) @ xv.astype(np.float32)).astype(np.float64), np.abs(w) @ np.abs(xv)"),
    ("embed wraps negative ids",
     "if 0 <= r < n:",
     "if -n <= r < n:"),
    ("argmax keeps the last of equal maxima",
     "return int(np.argmax(np.asarray(y)))",
     "return int(np.asarray(y).size - 1 - np.argmax(np.asarray(y)[::-1]))"),
    ("zero scale keeps computed codes",
     "q = np.where(zero[..., None], 8.0, q).astype(np.uint8)",
     "q = np.where(zero[..., None], 0.0, q).astype(np.uint8)"),
    ("lmhead panel offset",
     "y[s:e] = w @ xv",
     "y[s:e] = np.roll(w @ xv, 1)"),
    ("clear margin admits a third row",
     "if y[best] - y[second] > tol[best] + tol[second]:",
     "if False:"),
    ("tolerance without abs",
     "return rel * np.asarray(bound, dtype=np.float64) + abs_",
     "return rel * np.asarray(bound, dtype=np.float64)"),
    ("runner-up is the next index",
     "second = argmax_lowest(rest)",
     "second = (best + 1) % y.size"),
    ("runner-up's bound replaced by the leader's",
     "if y[best] - y[second] > tol[best] + tol[second]:",
     "if y[best] - y[second] > 2 * tol[best]:"),
]


def _load_mutant(old, new):
    with open(SRC) as fh:
        text = fh.read()
    assert text.count(old) == 1, f"mutation site not found once: {old!r}"
    mod = types.ModuleType("q4_oracle_mutant")
    exec(compile(text.replace(old, new), "q4_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    caught = []
    for check in oc.ALL_CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError) as e:  # a failing pin
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"mutant '{name}' passed every pin"
