"""The reduce's fp32 rank-order accumulation on the GPU, on inputs whose sums
round: uniformly random finite 16-bit patterns with a wide exponent spread.

The workload generators put every rank's value on one binary grid, so their
sums are exact in fp32 whatever the order.  Here most columns are not: each
element has a random sign, a random fraction and an exponent field drawn
uniformly over a wide range (binary16: subnormals up to 2^10, so that 16
values cannot overflow; bfloat16: 41 binades around a random exponent per
column).  Checked for 8 ranks (the LDS-staged whole blocks) and 16 ranks
(register path), binary16 and bfloat16, counts that reach the vector body,
several blocks and a ragged tail, at an aligned and a misaligned start, through
zero_reduce_owned, zero_reduce_check_owned and zero_reduce_check_buckets:

* the reduced values equal the oracle's (fp32 additions in rank order from
  +0, one rounding to 16 bits) bit for bit;
* most columns of the sample are inexact in fp32 (the rank-order sum differs
  from the exact one), and summing the ranks in reverse order changes the
  16-bit result of some columns, so a reduce with another order would fail;
* the overflow flag is exact and the squared norm is within the bound any
  summation order of non-negative terms meets, 2 (n - 1) 2^-53 relative.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import zero_partitioned_mixed_shard_amd as Z
from _common import assert_bits16_equal, to_np16

pytestmark = pytest.mark.gpu


def sum_bound(n):
    """Relative bound on two fp64 sums of the same n non-negative terms in
    different orders: each is within (n - 1) 2^-53 of the exact sum."""
    return 2 * max(n - 1, 1) * 2.0 ** -53

FP16, BF16 = 1, 2
COUNT = (1 << 20) + 3          # 256 whole blocks of 4096 elements and a ragged tail


def random_patterns(n_ranks, count, dtype, seed):
    """n_ranks arrays of finite 16-bit patterns with a wide exponent spread."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, (n_ranks, count)).astype(np.uint16) << 15
    if dtype == FP16:
        expo = rng.integers(0, 0x1A, (n_ranks, count))          # subnormals .. 2^10
        frac = rng.integers(0, 1 << 10, (n_ranks, count))
        bits = sign | (expo << 10).astype(np.uint16) | frac.astype(np.uint16)
    else:
        base = rng.integers(0x40, 0xC0, count)                    # per column
        expo = np.clip(base[None, :] + rng.integers(-20, 21, (n_ranks, count)), 1, 0xF0)
        frac = rng.integers(0, 1 << 7, (n_ranks, count))
        bits = sign | (expo << 7).astype(np.uint16) | frac.astype(np.uint16)
    return [np.ascontiguousarray(b) for b in bits]


def device_copy(a, dtype, offset):
    base = torch.zeros(a.size + offset + 8, dtype=torch.int16, device="cuda")
    base[offset:offset + a.size] = torch.from_numpy(a.view(np.int16)).cuda()
    return base.view(torch.float16 if dtype == FP16 else torch.bfloat16)[offset:offset + a.size]


def inexact_fraction(host, dtype, sample=20000):
    """Fraction of the first `sample` columns whose rank-order fp32 sum
    differs from the exact sum (math.fsum of the exact values)."""
    vals = [oracle.decode16(h[:sample], dtype).astype(np.float64) for h in host]
    acc = np.zeros(sample, np.float32)
    for v in vals:
        acc = (acc + v.astype(np.float32)).astype(np.float32)
    cols = np.stack(vals, axis=1)
    exact = np.array([math.fsum(c) for c in cols])
    return float(np.mean(acc.astype(np.float64) != exact))


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("n_ranks", [8, 16])
@pytest.mark.parametrize("offset", [0, 3])
def test_reduce_rounds_in_rank_order(dtype, n_ranks, offset):
    seed = 100 * dtype + n_ranks + offset
    host = random_patterns(n_ranks, COUNT, dtype, seed)
    want = oracle.reduce(host, dtype)
    # the inputs exercise rounding, and the order is observable in the result
    assert inexact_fraction(host, dtype) > 0.5
    reverse = oracle.reduce(host[::-1], dtype)
    assert np.count_nonzero(reverse != want) > 0
    inv = 2.0 ** -10
    flag_o, sumsq_o = oracle.check(want, dtype, inv)
    srcs = [device_copy(h, dtype, offset) for h in host]

    dst = device_copy(np.zeros(COUNT, np.uint16), dtype, offset)
    Z.zero_reduce_owned(dst, srcs)
    torch.cuda.synchronize()
    assert_bits16_equal(to_np16(dst), want, dtype, "zero_reduce_owned")

    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(Z.zero_check_workspace_bytes(COUNT) // 8 + 1, dtype=torch.float64,
                     device="cuda")
    dst = device_copy(np.zeros(COUNT, np.uint16), dtype, offset)
    Z.zero_reduce_check_owned(dst, srcs, inv, res, ws)
    r = Z.read_result(res)
    assert_bits16_equal(to_np16(dst), want, dtype, "zero_reduce_check_owned")
    assert r.overflow == flag_o
    assert r.sumsq == pytest.approx(sumsq_o, rel=sum_bound(COUNT))

    # the same columns as three reduce windows, each with rank buffers of its own
    cuts = [0, 4096 * 70 + 5, 4096 * 200, COUNT]
    windows = [(a, b - a) for a, b in zip(cuts, cuts[1:])]
    per_window = [[device_copy(h[a:b], dtype, (offset + a) % 8) for h in host]
                  for a, b in zip(cuts, cuts[1:])]
    dst = device_copy(np.zeros(COUNT, np.uint16), dtype, offset)
    ws = torch.empty(Z.zero_range_workspace_bytes(windows) // 8 + 1, dtype=torch.float64,
                     device="cuda")
    Z.zero_reduce_check_buckets(dst, windows, per_window, inv, res, ws)
    r = Z.read_result(res)
    assert_bits16_equal(to_np16(dst), want, dtype, "zero_reduce_check_buckets")
    assert r.overflow == flag_o
    assert r.sumsq == pytest.approx(sumsq_o, rel=sum_bound(COUNT))
