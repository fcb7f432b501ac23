"""zero_reduce_check_buckets on window lists beyond the ones a step's
bucketing produces: windows out of dst order, empty windows, gaps between
windows (left untouched), rank slices on and off the 16-byte grid of dst,
one window reduced in place into one of its own rank slices, the call
accumulating onto an earlier zero_reduce_check_owned result, the unscale
factor taken from a device step control, and an inf in one rank's slice.
3 ranks, 8 (whole blocks staged in LDS) and 16, binary16 and bfloat16.

Against the oracle (ZeRO-2 source walkthrough section 4.2: each bucket's part
of the owner's partition is the sum over the N ranks): the reduced values bit
for bit, the overflow flag exactly, the squared norm within the bound any
summation order of non-negative terms meets, 2 (n - 1) 2^-53 relative.
"""
import numpy as np
import pytest
import torch

import oracle
import zero_partitioned_mixed_shard_amd as Z
from _common import assert_bits16_equal, to_np16
from test_gpu_reduce_rounding import BF16, FP16, device_copy, random_patterns, sum_bound

pytestmark = pytest.mark.gpu

TOTAL = 80_000
# (offset, count) in dst, not in dst order, with gaps, empty windows and a
# one-element window; the fifth is reduced in place (rank 2's slice is dst's)
WINDOWS = [(40_000, 3 * 4096 + 5), (3, 2 * 4096), (70_001, 0), (20_000, 1),
           (20_010, 9_999), (60_000, 4096 + 8), (0, 0)]
IN_PLACE_WINDOW, IN_PLACE_RANK = 5, 2


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("n_ranks,dst_off,use_ctl,inf_at", [
    (3, 0, False, None), (8, 5, False, None), (8, 0, True, (0, 6, 1234)),
    (16, 3, False, (4, 15, 9_000))])
def test_bucket_window_lists(dtype, n_ranks, dst_off, use_ctl, inf_at):
    rng = np.random.default_rng(1000 * dtype + 10 * n_ranks + dst_off)
    inv = 2.0 ** -7
    host = [random_patterns(n_ranks, c, dtype, int(rng.integers(1 << 30))) for _, c in WINDOWS]
    if inf_at is not None:
        w, r, i = inf_at
        host[w][r][i] = 0x7C00 if dtype == FP16 else 0x7F80
    sentinel = rng.integers(0, 65536, TOTAL).astype(np.uint16)
    want = sentinel.copy()
    for (a, c), h in zip(WINDOWS, host):
        if c:
            want[a:a + c] = oracle.reduce(h, dtype)
    if IN_PLACE_WINDOW is not None:
        a, c = WINDOWS[IN_PLACE_WINDOW]
        sentinel[a:a + c] = host[IN_PLACE_WINDOW][IN_PLACE_RANK]
    dst = device_copy(sentinel, dtype, dst_off)
    srcs = []
    for w, ((a, c), h) in enumerate(zip(WINDOWS, host)):
        # even windows share dst's alignment (vector body), odd ones do not
        shift = (dst_off + a + (0 if w % 2 == 0 else 3)) % 8
        ranks = [device_copy(x, dtype, shift) for x in h]
        if w == IN_PLACE_WINDOW:
            ranks[IN_PLACE_RANK] = dst[a:a + c]
        srcs.append(ranks)

    # an earlier reduce+check over another buffer that this call accumulates onto
    pre = random_patterns(n_ranks, 5_000, dtype, 7)
    pre_dst = device_copy(np.zeros(5_000, np.uint16), dtype, 1)
    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(Z.zero_check_workspace_bytes(5_000),
                         Z.zero_range_workspace_bytes(WINDOWS)) // 8 + 1,
                     dtype=torch.float64, device="cuda")
    Z.zero_reduce_check_owned(pre_dst, [device_copy(x, dtype, 1) for x in pre], inv, res, ws)

    ctl_dev = None
    if use_ctl:
        ctl = Z.zero_step_control_init(2.0 ** 9, divisor=4.0)
        ctl_dev = Z.control_to_device(ctl)
        inv = float(np.float32(ctl.inv_scale))
    Z.zero_reduce_check_buckets(dst, WINDOWS, srcs, 99.0 if use_ctl else inv, res, ws,
                                accumulate=True, ctl_dev=ctl_dev)
    r = Z.read_result(res)
    assert_bits16_equal(to_np16(dst), want, dtype, "zero_reduce_check_buckets")

    flag, sumsq = oracle.check(oracle.reduce(pre, dtype), dtype, 2.0 ** -7)
    for (a, c) in WINDOWS:
        if c:
            flag, sumsq = oracle.check(want[a:a + c], dtype, inv, flag, sumsq)
    assert r.overflow == flag
    assert bool(flag) == (inf_at is not None)
    assert r.inv_scale == np.float32(inv)
    if not flag:
        n = 5_000 + sum(c for _, c in WINDOWS)
        assert r.sumsq == pytest.approx(sumsq, rel=sum_bound(n))
