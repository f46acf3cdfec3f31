"""Pins for the AllReduce oracle: checks that do not come from the oracle.

Each ``check_*`` takes an implementation ``impl(inputs, dtype) -> y`` (the
reduced buffer, storage convention of oracle/allreduce.py) and raises
AssertionError when it disagrees with a fact fixed independently of it:

* closed forms (integer sums are exact in every element type used here);
* exact rational sums (fractions.Fraction) wherever every binary32 prefix sum
  is representable, followed by a from-definition rounding;
* a scalar brute force that emulates binary32 adds with Python floats and the
  C library's float cast (correct by the double-rounding theorem, since
  53 >= 2*24 + 2) and rounds with a from-definition Fraction routine;
* hand-derived special cases from tests/golden/hand_cases.txt;
* invariants (replication, R = 1 identity, one-hot, x + (-x), R*x).

The same checks run against deliberately wrong implementations in
test_oracle_mutants.py, to show that each plausible mistake is caught.

Reading of the pages used throughout: AllReduce with the sum operator, binary32
accumulation in rank order 0..R-1 starting from rank 0's value, one final
round-to-nearest-even to the element type, output replicated to all ranks.
"""

from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# (significand bits incl. hidden bit, min normal exponent, max exponent)
FORMATS = {"fp32": (24, -126, 127), "fp16": (11, -14, 15), "bf16": (8, -126, 127)}
FIELDS = {"fp32": (8, 23), "fp16": (5, 10), "bf16": (8, 7)}  # exponent bits, fraction bits
STORAGE = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}


# ----------------------------------------------------------------------------
# From-definition decoding / rounding (independent of NumPy's conversions)
# ----------------------------------------------------------------------------

def bits_of(x, dtype):
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if dtype == "fp16":
        return np.ascontiguousarray(x, dtype=np.float16).view(np.uint16)
    return np.ascontiguousarray(x, dtype=np.uint16)


def from_bits(b, dtype):
    b = np.asarray(b)
    if dtype == "fp32":
        return b.astype(np.uint32).view(np.float32)
    if dtype == "fp16":
        return b.astype(np.uint16).view(np.float16)
    return b.astype(np.uint16)


def decode(bits: int, dtype: str):
    """Value of one stored pattern: ('num', sign, Fraction) / ('inf', sign) / ('nan',)."""
    ebits, fbits = FIELDS[dtype]
    sign = (bits >> (ebits + fbits)) & 1
    e = (bits >> fbits) & ((1 << ebits) - 1)
    f = bits & ((1 << fbits) - 1)
    bias = (1 << (ebits - 1)) - 1
    if e == (1 << ebits) - 1:
        return ("nan",) if f else ("inf", sign)
    if e == 0:
        mag = Fraction(f, 1 << fbits) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(f, 1 << fbits)) * Fraction(2) ** (e - bias)
    return ("num", sign, mag)


def round_def(v: Fraction, dtype: str):
    """Round a nonzero-or-zero rational to the nearest value of `dtype`, ties
    to even significand; returns ('num', sign, Fraction) or ('inf', sign).
    The sign of an exact zero is the caller's business."""
    p, emin, emax = FORMATS[dtype]
    sign = 1 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return ("num", sign, Fraction(0))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    q = a / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (emax + 1):
        return ("inf", sign)
    return ("num", sign, r)


def same_value(got_bits: int, want, dtype: str) -> bool:
    g = decode(int(got_bits), dtype)
    if want[0] == "nan":
        return g[0] == "nan"
    if want[0] == "inf":
        return g[0] == "inf" and g[1] == want[1]
    if g[0] != "num":
        return False
    if want[2] == 0:
        return g[2] == 0 and g[1] == want[1]
    return g[1] == want[1] and g[2] == want[2]


def f32_round(x: float) -> float:
    """Round a binary64 value to binary32 (RNE) through the C float cast."""
    if math.isnan(x) or math.isinf(x):
        return x
    # At or beyond the midpoint between the largest binary32 value
    # (2^128 - 2^104, odd significand) and 2^128, nearest-even goes to 2^128:
    # infinity.  (The C cast would do the same; struct refuses to pack it.)
    if abs(x) >= 2.0 ** 128 - 2.0 ** 103:
        return math.copysign(math.inf, x)
    return struct.unpack("<f", struct.pack("<f", x))[0]


def scalar_value(bits: int, dtype: str) -> float:
    d = decode(int(bits), dtype)
    if d[0] == "nan":
        return math.nan
    if d[0] == "inf":
        return -math.inf if d[1] else math.inf
    v = float(d[2])  # exact: every fp32/fp16/bf16 value is a binary64 value
    return -v if d[1] else v


def brute_force_element(col_bits, dtype: str):
    """Reduce one element's R stored patterns by emulation; returns the
    expected ('num'|'inf'|'nan', ...) tuple."""
    a = scalar_value(col_bits[0], dtype)
    for b in col_bits[1:]:
        a = f32_round(a + scalar_value(b, dtype))
    if math.isnan(a):
        return ("nan",)
    if math.isinf(a):
        return ("inf", 1 if a < 0 else 0)
    if a == 0.0:
        return ("num", 1 if math.copysign(1.0, a) < 0 else 0, Fraction(0))
    return round_def(Fraction(a), dtype)


def f32_exact(q: Fraction) -> bool:
    if q == 0:
        return True
    d = float(q)  # correctly rounded
    if math.isinf(d):
        return False
    return Fraction(float(np.float32(d))) == q


# ----------------------------------------------------------------------------
# Input helpers (small, local, deterministic)
# ----------------------------------------------------------------------------

def rng(seed):
    return np.random.default_rng(np.random.SeedSequence([7_000_001, seed]))


def rand_inputs(R, n, dtype, seed, scale=1.0):
    g = rng(seed)
    out = []
    for _ in range(R):
        x = (g.standard_normal(n) * scale).astype(np.float32)
        if dtype == "fp32":
            out.append(x)
        elif dtype == "fp16":
            out.append(x.astype(np.float16))
        else:
            import torch
            out.append(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy())
    return out


def special_patterns(dtype):
    """Stored patterns that exercise zeros, subnormals, extremes, Inf and NaN."""
    if dtype == "fp32":
        pats = [0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x007FFFFF, 0x00800000, 0x3F800000,
                0xBF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000, 0x7FC00000, 0x4B800000,
                0x33800000, 0x3F800001]
    elif dtype == "fp16":
        pats = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x3C00, 0xBC00, 0x7BFF, 0xFBFF,
                0x7C00, 0xFC00, 0x7E00, 0x3C01, 0x1400, 0x6800]
    else:
        pats = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F,
                0x7F80, 0xFF80, 0x7FC0, 0x3F81, 0x4780, 0x3B80]
    return pats


# ----------------------------------------------------------------------------
# Checks
# ----------------------------------------------------------------------------

def check_integer_closed_form(impl):
    """Integers in [-8, 8]: every prefix sum is a small integer, exact in
    binary32, and the total (|s| <= 128) is exact in fp16 and bf16 too, so
    the result must be the exact integer sum in every dtype."""
    for dtype in ("fp32", "fp16", "bf16"):
        for R in (1, 2, 3, 4, 5, 8, 13, 16):
            g = rng(100 + R)
            ints = [g.integers(-8, 9, size=257) for _ in range(R)]
            xs = []
            for v in ints:
                f = v.astype(np.float32)
                if dtype == "fp32":
                    xs.append(f)
                elif dtype == "fp16":
                    xs.append(f.astype(np.float16))
                else:
                    xs.append((f.view(np.uint32) >> 16).astype(np.uint16))  # exact: low halves are zero
            y = impl(xs, dtype)
            want = np.sum(np.stack(ints), axis=0)
            got = [scalar_value(b, dtype) for b in bits_of(y, dtype)]
            for i, (gv, wv) in enumerate(zip(got, want)):
                assert gv == float(wv), f"{dtype} R={R} elem {i}: {gv} != exact {wv}"
                if wv == 0:
                    # all-integer columns that cancel: +0 (no -0 unless every input is -0)
                    assert math.copysign(1.0, gv) > 0 or all(math.copysign(1.0, float(v[i])) < 0 for v in ints), \
                        f"{dtype} R={R} elem {i}: sign of zero"


def check_integer_workload(impl, xs):
    """The 16 KiB R=4 fp32 integer workload: bit-exact integer sums."""
    y = impl(xs, "fp32")
    want = np.sum(np.stack([x.astype(np.float64) for x in xs]), axis=0)
    assert np.array_equal(np.asarray(y, dtype=np.float64), want), "integer workload sum not exact"


def check_fraction_exact(impl, dtype="bf16", R=8, n=1500, seed=3):
    """Where every rank-order prefix sum is exactly representable in binary32,
    the binary32 accumulator equals the exact rational sum; the output must
    then be that sum rounded once (from definition) to the element type."""
    xs = rand_inputs(R, n, dtype, seed)
    if dtype == "fp32":
        # keep 16 significant bits so that most prefix sums stay exact
        xs = [(x.view(np.uint32) & np.uint32(0xFFFFFF00)).view(np.float32) for x in xs]
    y = bits_of(impl(xs, dtype), dtype)
    cols = np.stack([bits_of(x, dtype) for x in xs])
    checked = 0
    for i in range(n):
        vals = [decode(int(b), dtype) for b in cols[:, i]]
        fr = [(-v[2] if v[1] else v[2]) for v in vals]
        s = Fraction(0)
        exact = True
        for k, q in enumerate(fr):
            s = q if k == 0 else s + q
            if not f32_exact(s):
                exact = False
                break
        if not exact:
            continue
        checked += 1
        if s == 0:
            continue  # sign of zero pinned elsewhere
        want = round_def(s, dtype)
        assert same_value(y[i], want, dtype), f"elem {i}: got {y[i]:#x}, exact sum {s} rounds to {want}"
    assert checked > n // 2, f"too few exactly-representable columns ({checked})"


def check_brute_force(impl, dtypes=("fp32", "fp16", "bf16"), ranks=tuple(range(1, 17)),
                      sizes=(1, 7, 67), seed=11):
    """Scalar emulation over R = 1..16 and ragged lengths, with special
    patterns mixed into the normal values."""
    for dtype in dtypes:
        specials = special_patterns(dtype)
        for R in ranks:
            for n in sizes:
                xs = rand_inputs(R, n, dtype, seed * 1000 + R * 10 + n, scale=4.0)
                g = rng(seed + R + n)
                bitsx = [bits_of(x, dtype).copy() for x in xs]
                for b in bitsx:  # sprinkle specials
                    m = g.random(n) < 0.1
                    b[m] = g.choice(specials, size=int(m.sum()))
                xs = [from_bits(b, dtype) for b in bitsx]
                y = bits_of(impl(xs, dtype), dtype)
                cols = np.stack(bitsx)
                for i in range(n):
                    want = brute_force_element([int(v) for v in cols[:, i]], dtype)
                    assert same_value(y[i], want, dtype), \
                        f"{dtype} R={R} n={n} elem {i}: inputs {[hex(int(v)) for v in cols[:, i]]} got {int(y[i]):#x} want {want}"


def load_hand_cases():
    cases = []
    with open(os.path.join(GOLDEN, "hand_cases.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            dtype, ins, want = line.split()
            cases.append((dtype, [int(t, 16) for t in ins.split(",")], want))
    return cases


def check_hand_cases(impl):
    """Hand-derived cases: double rounding, order dependence, signed zero,
    Inf/NaN propagation, binary16 overflow, subnormals (tests/golden)."""
    for dtype, ins, want in load_hand_cases():
        xs = [from_bits(np.array([v]), dtype) for v in ins]
        y = int(bits_of(impl(xs, dtype), dtype)[0])
        if want == "nan":
            assert decode(y, dtype)[0] == "nan", f"{dtype} {ins}: want NaN, got {y:#x}"
        else:
            assert y == int(want, 16), f"{dtype} {[hex(v) for v in ins]}: got {y:#x}, want {want}"


def check_invariants(impl):
    """Identity at R=1; one-hot rank; x + (-x) = +0; R*x exact for R a power
    of two and short significands."""
    for dtype in ("fp32", "fp16", "bf16"):
        xs = rand_inputs(1, 300, dtype, 21)
        assert np.array_equal(bits_of(impl(xs, dtype), dtype), bits_of(xs[0], dtype)), f"{dtype} R=1 identity"
        for R in (2, 5, 16):
            hot = rand_inputs(1, 300, dtype, 22 + R)[0]
            hb = bits_of(hot, dtype).copy()
            ebits, fbits = FIELDS[dtype]
            hb[(hb & ((1 << (ebits + fbits)) - 1)) == 0] |= 1  # no zeros in the hot rank
            zero = from_bits(np.zeros(300, dtype=hb.dtype), dtype)
            for k in (0, R - 1, R // 2):
                xs = [zero.copy() for _ in range(R)]
                xs[k] = from_bits(hb, dtype)
                y = bits_of(impl(xs, dtype), dtype)
                assert np.array_equal(y, hb), f"{dtype} one-hot rank {k} of {R}"
        x = rand_inputs(1, 300, dtype, 40)[0]
        xb = bits_of(x, dtype)
        sign = 1 << (sum(FIELDS[dtype]))
        neg = from_bits(xb ^ sign, dtype)
        y = bits_of(impl([x, neg], dtype), dtype)
        assert np.all(y == 0), f"{dtype} x + (-x) must be +0"
        for R in (2, 4, 8, 16):
            g = rng(50 + R)
            base = g.integers(1, 1 << 7, size=300) * np.power(2.0, g.integers(-20, 10, size=300))
            base = base * np.where(g.random(300) < 0.5, -1, 1)
            f = base.astype(np.float32)
            if dtype == "fp32":
                xv = f
            elif dtype == "fp16":
                xv = f.astype(np.float16)  # 7-bit integers times 2^k: exact when in range
            else:
                xv = (f.view(np.uint32) >> 16).astype(np.uint16)  # 7 significant bits: exact
            y = bits_of(impl([xv] * R, dtype), dtype)
            for i in range(300):
                v = scalar_value(bits_of(xv, dtype)[i], dtype)
                want = round_def(Fraction(v) * R, dtype)
                assert same_value(y[i], want, dtype), f"{dtype} {R}*x elem {i}"


def check_replication(impl_outputs, xs, dtype):
    outs = impl_outputs(xs, dtype)
    assert len(outs) == len(xs)
    b0 = bits_of(outs[0], dtype)
    for o in outs[1:]:
        assert np.array_equal(bits_of(o, dtype), b0), "outputs differ between ranks"


ALL_CHECKS = (check_integer_closed_form, check_fraction_exact, check_brute_force,
              check_hand_cases, check_invariants)
