"""Pins for the oracle's reduce and check phases (not GPU).

Reduce: the owner receives the sum of every rank's gradient, delivered in the
16-bit communication type (ZeRO 优化器, "ZeRO Stage 1" gradient states after
reduce; ZeRO-2 source walkthrough, section 三).  The expected value here is the
exact rational sum (fractions.Fraction of the values decoded by numpy / torch),
rounded by brute force to the nearest 16-bit value with ties to even, with
IEEE rules for infinities and NaN.  For binary16 inputs the oracle's fp64 sum
is exact, so the two must agree everywhere.  For bfloat16 the fp64 sum is exact
unless the addends' exponents spread over more than ~45 bits; there the
oracle's definition (fp64 additions in rank order, one final rounding) is
checked instead, with the same brute-force rounding of that double.

Check: overflow = any non-finite element; sumsq = the correctly rounded sum
(math.fsum) of the exact squares of the unscaled values.
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


def _expected_sum(col_bits, dtype, rounder):
    """-> (expected pattern or "nan", whether the fp64 sum was exact)."""
    vals = _values(np.array(col_bits), dtype)
    if np.isnan(vals).any() or (np.isposinf(vals).any() and np.isneginf(vals).any()):
        return "nan", True
    if np.isposinf(vals).any():
        return (0x7C00 if dtype == FP16 else 0x7F80), True
    if np.isneginf(vals).any():
        return (0xFC00 if dtype == FP16 else 0xFF80), True
    q = sum((Fraction(float(v)) for v in vals), Fraction(0))
    d = float(vals[0])
    for v in vals[1:]:
        d = d + float(v)            # IEEE double additions in rank order
    exact = Fraction(d) == q
    if not exact:
        return rounder(Fraction(d), math.copysign(1, d) < 0), False
    all_neg_zero = all(v == 0 and math.copysign(1, v) < 0 for v in vals)
    return rounder(q, all_neg_zero), True


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
    if dtype == FP16:
        assert inexact == 0         # binary16 sums are always exact in fp64
    else:
        assert checked - inexact > checked // 2


def test_reduce_sum_overflow_and_cancellation():
    sixty_k = np.full(4, 0x7B53, dtype=np.uint16)                  # 60000.0
    # 8 x 60000 overflows binary16 -> +inf; 60000 + (-60000) cancels to +0
    assert (oracle.reduce([sixty_k] * 8, FP16) == 0x7C00).all()
    assert (oracle.reduce([sixty_k, sixty_k | 0x8000], FP16) == 0x0000).all()
    # -0 + -0 stays -0; +inf + -inf is NaN
    negz = np.full(2, 0x8000, dtype=np.uint16)
    assert (oracle.reduce([negz, negz], FP16) == 0x8000).all()
    pinf, ninf = np.full(1, 0x7C00, np.uint16), np.full(1, 0xFC00, np.uint16)
    assert _is_nan16(int(oracle.reduce([pinf, ninf], FP16)[0]), FP16)


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
        flag, sumsq = oracle.check(bits, dtype, inv)
        assert flag == int((~np.isfinite(vals)).any())
        if not flag:
            want = math.fsum(float(Fraction(float(v)) * Fraction(inv)) ** 2 for v in vals)
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
