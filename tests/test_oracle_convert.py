"""Pins for the oracle's 16-bit converters (not GPU).

The converters are written from the binary16 / bfloat16 definitions; here they
are checked against independent implementations: numpy's float16 casts, torch's
bfloat16 casts, and a brute-force nearest-value search over every finite
16-bit value.  NaN results compare as "both NaN" (payloads are free).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle

FP16, BF16 = oracle.FP16, oracle.BF16
THREADS = min(8, os.cpu_count() or 1)


def _same16(got: np.ndarray, want: np.ndarray, dtype: int) -> np.ndarray:
    """Elementwise: equal patterns, or both NaN."""
    expo = 0x7C00 if dtype == FP16 else 0x7F80
    frac = 0x03FF if dtype == FP16 else 0x007F
    nan_g = ((got & expo) == expo) & ((got & frac) != 0)
    nan_w = ((want & expo) == expo) & ((want & frac) != 0)
    return (got == want) | (nan_g & nan_w)


def test_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode16(bits, FP16)
    want = bits.view(np.float16).astype(np.float64)
    ok = (got == want) | (np.isnan(got) & np.isnan(want))
    assert ok.all()
    got = oracle.decode16(bits, BF16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ok = (got == want) | (np.isnan(got) & np.isnan(want))
    assert ok.all()


def _f32_chunk(lo: int, n: int) -> np.ndarray:
    return (np.arange(n, dtype=np.uint64) + np.uint64(lo)).astype(np.uint32).view(np.float32)


def _library_cast(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == FP16:
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_encode_from_f32_structured(dtype):
    """Every sign/exponent/upper-fraction prefix of fp32 with the low bits set
    to the patterns that decide rounding (0, 1, tie-1, tie, tie+1, all ones,
    and random), plus 2^22 random patterns, round like the library cast."""
    low_bits = 13 if dtype == FP16 else 16
    tie = 1 << (low_bits - 1)
    rng = np.random.default_rng(3)
    lows = np.array([0, 1, tie - 1, tie, tie + 1, (1 << low_bits) - 1,
                     *rng.integers(0, 1 << low_bits, 10)], dtype=np.uint64)
    n_high = 1 << (32 - low_bits)
    step = 1 << 16                       # prefixes per chunk: small, reused buffers
    for h0 in range(0, n_high, step):
        highs = np.arange(h0, h0 + step, dtype=np.uint32) << np.uint32(low_bits)
        x = (highs[:, None] | lows.astype(np.uint32)[None, :]).ravel().view(np.float32)
        assert _same16(oracle.encode16(x, dtype), _library_cast(x, dtype), dtype).all(), h0
    for k in range(4):
        x = rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
        assert _same16(oracle.encode16(x, dtype), _library_cast(x, dtype), dtype).all()


@pytest.mark.slow
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_encode_from_f32_exhaustive(dtype):
    """Every one of the 2^32 fp32 patterns rounds like the library cast
    (about two minutes on 8 cores; run with --run-slow)."""
    chunk = 1 << 24

    def work(c):
        x = _f32_chunk(c * chunk, chunk)
        got = oracle.encode16(x, dtype)
        return int((~_same16(got, _library_cast(x, dtype), dtype)).sum())

    with ThreadPoolExecutor(THREADS) as ex:
        bad = sum(ex.map(work, range((1 << 32) // chunk)))
    assert bad == 0


def _all_finite_values(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if dtype == FP16:
        vals = bits.view(np.float16).astype(np.float64)
    else:
        vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    keep = np.isfinite(vals) & ~((vals == 0) & (np.signbit(vals)))
    return vals[keep], bits[keep]


def _nearest_even(x: np.ndarray, dtype: int) -> np.ndarray:
    """Brute force: the nearest finite 16-bit value, ties to the even pattern;
    beyond the largest finite value by half an ulp or more -> inf."""
    vals, bits = _all_finite_values(dtype)
    order = np.argsort(vals)
    vals, bits = vals[order], bits[order]
    big = vals[-1]
    # half an ulp above the largest finite value
    ulp_top = vals[-1] - vals[-2]
    inf_bits = 0x7C00 if dtype == FP16 else 0x7F80
    out = np.empty(x.size, dtype=np.uint16)
    for k, v in enumerate(x):
        a = abs(v)
        if a >= big + ulp_top / 2:
            r = inf_bits
        else:
            j = np.searchsorted(vals, a)
            cands = [i for i in (j - 1, j) if 0 <= i < vals.size]
            best = min(cands, key=lambda i: (abs(vals[i] - a), int(bits[i]) & 1))
            r = int(bits[best])
        if np.signbit(v):
            r |= 0x8000
        out[k] = r
    return out


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_encode_from_f64_brute_force(dtype):
    """Doubles that are not fp32 values (so a cast through fp32 would round
    twice) round to the nearest 16-bit value, ties to even."""
    rng = np.random.default_rng(7)
    vals, _ = _all_finite_values(dtype)
    vals = np.sort(vals)
    # midpoints between neighbours (exact ties), and points just off them
    mids = (vals[:-1] + vals[1:]) / 2
    pick = rng.choice(mids.size, 3000, replace=False)
    m = mids[pick]
    off = np.abs(m) * 2.0 ** -40 + 1e-300
    x = np.concatenate([m, m + off, m - off,
                        rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 5, 3000)])
    x = np.concatenate([x, -x])
    got = oracle.encode16(x.astype(np.float64), dtype)
    want = _nearest_even(x, dtype)
    assert np.array_equal(got, want)
    if dtype == FP16:
        # numpy's double->half cast rounds once, directly from the double
        with np.errstate(over="ignore"):
            assert np.array_equal(got, x.astype(np.float16).view(np.uint16))


def test_encode_specials():
    x = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 3 * 2.0 ** -25], dtype=np.float64)
    got = oracle.encode16(x, FP16)
    assert got[0] == 0x7C00 and got[1] == 0xFC00
    assert (got[2] & 0x7C00) == 0x7C00 and (got[2] & 0x3FF) != 0
    assert got[3] == 0 and got[4] == 0x8000
    assert got[5] == 0x7BFF and got[6] == 0x7BFF and got[7] == 0x7C00
    # half the smallest subnormal ties to zero; just above rounds up; 1.5 ulp ties to 2
    assert got[8] == 0 and got[9] == 1 and got[10] == 2
