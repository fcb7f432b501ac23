"""Pins for the oracle's reduce and check phases (not GPU).

Reduce: the owner receives the sum of every rank's gradient, delivered in the
16-bit communication type (ZeRO 优化器, "ZeRO Stage 1" gradient states after
reduce; ZeRO-2 source walkthrough, section 三).  The pages leave the
accumulation open; the reading is fp32 additions in rank order starting from
+0, then one rounding to the 16-bit type.  The expected value here follows
IEEE 754 from its definition, on exact rationals (fractions.Fraction of the
values decoded by numpy / torch): every partial sum is the exact rational sum
rounded to the nearest fp32 value (24-bit significand, ties to even,
subnormal quantum 2^-149, overflow to infinity), infinities and NaN follow the
IEEE rules, and the final fp32 value is rounded by brute force to the nearest
16-bit value, ties to even.  Hand-derived columns show where fp32
accumulation and an exact sum part ways.

Check: overflow = any non-finite element; sumsq = the correctly rounded sum
(math.fsum) of the exact squares of the unscaled values, each the fp32 product
of the value and inv_scale (numpy float32 arithmetic).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

FP16, BF16 = oracle.FP16, oracle.BF16


def _values(bits: np.ndarray, dtype: int) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == FP16:
        return bits.view(np.float16).astype(np.float64)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


class _Rounder:
    """Nearest finite 16-bit value of an exact rational, ties to even."""

    def __init__(self, dtype):
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        vals = _values(bits, dtype)
        keep = np.isfinite(vals) & (vals >= 0) & ~((vals == 0) & np.signbit(vals))
        order = np.argsort(vals[keep])
        self.vals = [Fraction(float(v)) for v in vals[keep][order]]
        self.bits = [int(b) for b in bits[keep][order]]
        top, below = self.vals[-1], self.vals[-2]
        self.overflow_at = top + (top - below) / 2
        self.inf = 0x7C00 if dtype == FP16 else 0x7F80

    def __call__(self, q: Fraction, negative_zero: bool) -> int:
        sign = 0x8000 if (q < 0 or (q == 0 and negative_zero)) else 0
        a = abs(q)
        if a >= self.overflow_at:
            return sign | self.inf
        lo, hi = 0, len(self.vals) - 1
        while hi - lo > 1:               # bracket a between vals[lo] and vals[hi]
            mid = (lo + hi) // 2
            if self.vals[mid] <= a:
                lo = mid
            else:
                hi = mid
        dl, dh = a - self.vals[lo], self.vals[hi] - a
        if dl < dh or (dl == dh and self.bits[lo] % 2 == 0):
            return sign | self.bits[lo]
        return sign | self.bits[hi]


F32_MAX = Fraction(2 ** 24 - 1) * Fraction(2) ** 104
F32_OVERFLOW = F32_MAX + Fraction(2) ** 103          # halfway to 2^128


def _round_f32(q: Fraction):
    """Nearest fp32 value of an exact rational, ties to even; "+inf"/"-inf"
    past the overflow threshold."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    if a >= F32_OVERFLOW:
        return "+inf" if q > 0 else "-inf"
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:                    # now 2^e <= a < 2^(e+1)
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    r = k * quantum
    return r if q > 0 else -r


def _expected_sum(col_bits, dtype, rounder):
    """-> (expected pattern or "nan", whether every partial sum was exact)."""
    vals = _values(np.array(col_bits), dtype)
    acc, exact = Fraction(0), True                   # +0
    for v in vals:
        if acc == "nan" or np.isnan(v):
            acc = "nan"
        elif np.isinf(v) or isinstance(acc, str):
            signs = {acc} if isinstance(acc, str) else set()
            if np.isinf(v):
                signs.add("+inf" if v > 0 else "-inf")
            acc = "nan" if len(signs) == 2 else signs.pop()
        else:
            q = acc + Fraction(float(v))
            acc = _round_f32(q)
            exact = exact and acc == q
    if acc == "nan":
        return "nan", exact
    if acc in ("+inf", "-inf"):
        inf = 0x7C00 if dtype == FP16 else 0x7F80
        return (inf if acc == "+inf" else 0x8000 | inf), exact
    # an fp32 sum that starts from +0 is never -0 (x + -x is +0 to nearest)
    return rounder(acc, False), exact


def _is_nan16(b, dtype):
    expo, frac = (0x7C00, 0x3FF) if dtype == FP16 else (0x7F80, 0x7F)
    return (b & expo) == expo and (b & frac) != 0


SPECIAL_FP16 = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x3C00, 0xBC00, 0x7BFF, 0xFBFF,
                0x7B53,  # 60000 (eight of them overflow the sum)
                0x3C01, 0x1400, 0x7C00, 0xFC00, 0x7E00]
SPECIAL_BF16 = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F,
                0x7F00, 0x3F81, 0x3B80, 0x7F80, 0xFF80, 0x7FC0]


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_reduce_brute_force_specials(dtype):
    rng = np.random.default_rng(21 + dtype)
    rounder = _Rounder(dtype)
    special = SPECIAL_FP16 if dtype == FP16 else SPECIAL_BF16
    checked = inexact = 0
    for n_ranks in (1, 2, 3, 8, 16):
        for trial in range(60):
            phi = 10
            srcs = []
            for r in range(n_ranks):
                pick = rng.random(phi) < 0.5
                s = np.where(pick, rng.choice(special, phi),
                             rng.integers(0, 65536, phi)).astype(np.uint16)
                if dtype == BF16 and trial % 2 == 0:
                    # moderate exponent spread (fields 110..140) and +-0 / inf / NaN
                    e = rng.integers(110, 141, phi).astype(np.uint16)
                    s = (s & 0x807F) | (e << 7)
                    s = np.where(rng.random(phi) < 0.1, rng.choice(
                        [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0], phi), s).astype(np.uint16)
                srcs.append(s)
            got = oracle.reduce(srcs, dtype)
            for i in range(phi):
                want, exact = _expected_sum([int(s[i]) for s in srcs], dtype, rounder)
                if want == "nan":
                    assert _is_nan16(int(got[i]), dtype)
                else:
                    assert int(got[i]) == want, (n_ranks, [hex(int(s[i])) for s in srcs])
                checked += 1
                inexact += not exact
    assert checked == 5 * 60 * 10
    assert 0 < inexact < checked // 2          # both kinds of column are exercised


def test_reduce_sum_overflow_and_cancellation():
    sixty_k = np.full(4, 0x7B53, dtype=np.uint16)                  # 60000.0
    # 8 x 60000 overflows binary16 -> +inf; 60000 + (-60000) cancels to +0
    assert (oracle.reduce([sixty_k] * 8, FP16) == 0x7C00).all()
    assert (oracle.reduce([sixty_k, sixty_k | 0x8000], FP16) == 0x0000).all()
    # the sum starts from +0, so -0 columns give +0 (also with one rank)
    negz = np.full(2, 0x8000, dtype=np.uint16)
    assert (oracle.reduce([negz, negz], FP16) == 0x0000).all()
    assert (oracle.reduce([negz], BF16) == 0x0000).all()
    # +inf + -inf is NaN; two bf16 maxima overflow fp32 itself -> +inf
    pinf, ninf = np.full(1, 0x7C00, np.uint16), np.full(1, 0xFC00, np.uint16)
    assert _is_nan16(int(oracle.reduce([pinf, ninf], FP16)[0]), FP16)
    bmax = np.full(1, 0x7F7F, np.uint16)
    assert int(oracle.reduce([bmax, bmax], BF16)[0]) == 0x7F80


def test_reduce_fp32_accumulation_worked_examples():
    """Columns worked by hand where fp32 accumulation and the exact sum round
    to different 16-bit values.
    binary16 [2048, 1, 2^-14]: 2048 + 1 = 2049 exactly; 2049 + 2^-14 rounds
    back to 2049 in fp32 (a quarter of its 2^-12 quantum); 2049 is halfway
    between the binary16 neighbours 2048 and 2050 and goes to the even 2048.
    The exact sum 2049.00006... would round up to 2050.
    bfloat16 [1, 2^-8, 2^-32]: 1 + 2^-8 is exact; adding 2^-32 (below half of
    the 2^-23 quantum) leaves 1 + 2^-8, halfway between 1 and 1 + 2^-7, which
    goes to the even 1.0.  The exact sum is above the midpoint: 1 + 2^-7."""
    col = lambda *b: [np.array([x], np.uint16) for x in b]
    assert int(oracle.reduce(col(0x6800, 0x3C00, 0x0400), FP16)[0]) == 0x6800
    assert int(oracle.reduce(col(0x3F80, 0x3B80, 0x2F80), BF16)[0]) == 0x3F80
    # the same addends with the tiny one first: 2^-14 + 1 is exact in fp32,
    # + 2048 gives 2049.00006 -> rounds to 2049 in fp32 -> 2048 again
    assert int(oracle.reduce(col(0x0400, 0x3C00, 0x6800), FP16)[0]) == 0x6800
    # an exact column agrees with the exact sum: 2048 + 1 + 1 = 2050
    assert int(oracle.reduce(col(0x6800, 0x3C00, 0x3C00), FP16)[0]) == 0x6801


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_check_flag_and_norm(dtype):
    rng = np.random.default_rng(5)
    for trial in range(50):
        n = int(rng.integers(0, 2000))
        bits = rng.integers(0, 65536, n).astype(np.uint16)
        vals = _values(bits, dtype)
        finite = np.isfinite(vals)
        if trial % 2 == 0:                        # half the cases all finite
            bits = np.where(finite, bits, np.uint16(0))
            vals = _values(bits, dtype)
        inv = 2.0 ** -int(rng.integers(0, 20))
        if trial % 5 == 4:
            inv = float(np.float32(1.0 / (1024 * 3)))   # a divisor that is not a power of two
        flag, sumsq = oracle.check(bits, dtype, inv)
        assert flag == int((~np.isfinite(vals)).any())
        if not flag:
            g = vals.astype(np.float32) * np.float32(inv)     # fp32 products
            want = math.fsum(float(x) ** 2 for x in g)
            assert sumsq == pytest.approx(want, rel=1e-13, abs=0)


def test_check_accumulates_over_owner_ranges():
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 0x7000, 1000).astype(np.uint16)
    whole = oracle.check(bits, FP16, 1.0)
    acc = (0, 0.0)
    for lo, hi in ((0, 250), (250, 600), (600, 1000)):
        acc = oracle.check(bits[lo:hi], FP16, 1.0, *acc)
    assert acc[0] == whole[0]
    assert acc[1] == pytest.approx(whole[1], rel=1e-14)
    bits[777] = 0x7E00
    acc = (0, 0.0)
    for lo, hi in ((0, 500), (500, 1000)):
        acc = oracle.check(bits[lo:hi], FP16, 1.0, *acc)
    assert acc[0] == 1


def test_clip_coef_matches_torch_clip_grad_norm():
    rng = np.random.default_rng(4)
    for max_norm in (0.0, -1.0, 0.5, 1.0, 1e6):
        g = rng.standard_normal(3000) * 0.05
        sumsq = math.fsum(x * x for x in g)
        coef = oracle.clip_coef(max_norm, sumsq)
        if max_norm <= 0:
            assert coef == 1.0
            continue
        p = torch.nn.Parameter(torch.zeros(3000, dtype=torch.float64))
        p.grad = torch.from_numpy(g.copy())
        total = float(torch.nn.utils.clip_grad_norm_([p], max_norm))
        assert total == pytest.approx(math.sqrt(sumsq), rel=1e-12)
        # clip_grad_norm_ scales by min(1, max_norm / (norm + 1e-6))
        ratio = float(p.grad[0] / g[0]) if g[0] != 0 else 1.0
        assert coef == pytest.approx(ratio, rel=2 ** -23)
