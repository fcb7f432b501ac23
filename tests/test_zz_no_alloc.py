"""The allocation-free fused reduce+check, zero_reduce_check_owned_noalloc,
called through the C ABI against zero_reduce_check_owned with a workspace of
the caller's: two calls in a row on one device, the second with a smaller
input (other rank count, other 16-bit type, misaligned start), then an
accumulating call.  Both calls run the same kernels with the same fold order,
so the reduced values and the whole 16-byte result must be bit-identical;
the reduced values also equal the oracle's.  A count beyond the scratch
array's limit is refused before anything is launched."""
import ctypes

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


def _patterns(n_ranks, count, dtype, seed):
    """Finite 16-bit patterns, exponents spread wide enough that sums round
    but no sum of 16 leaves the format (plus a few exact zeros)."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, (n_ranks, count)).astype(np.uint16) << 15
    if dtype == FP16:
        expo = rng.integers(0, 0x1A, (n_ranks, count)).astype(np.uint16) << 10
        frac = rng.integers(0, 1 << 10, (n_ranks, count)).astype(np.uint16)
    else:
        expo = rng.integers(0x60, 0x90, (n_ranks, count)).astype(np.uint16) << 7
        frac = rng.integers(0, 1 << 7, (n_ranks, count)).astype(np.uint16)
    bits = sign | expo | frac
    bits[:, ::997] = 0
    return [np.ascontiguousarray(b) for b in bits]


def _device(a, dtype, offset):
    base = torch.zeros(a.size + offset + 8, dtype=torch.int16, device="cuda")
    base[offset:offset + a.size] = torch.from_numpy(a.view(np.int16)).cuda()
    return base.view(torch.float16 if dtype == FP16 else torch.bfloat16)[offset:offset + a.size]


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _noalloc(dst, srcs, count, dtype, inv, res, accumulate=0):
    ptrs = (ctypes.c_void_p * len(srcs))(*[s.data_ptr() for s in srcs])
    return Z.lib().zero_reduce_check_owned_noalloc(dst.data_ptr(), ptrs, len(srcs), count, dtype,
                                                   inv, res.data_ptr(), accumulate, _stream())


def _with_workspace(dst, srcs, count, dtype, inv, res, ws, accumulate=0):
    ptrs = (ctypes.c_void_p * len(srcs))(*[s.data_ptr() for s in srcs])
    return Z.lib().zero_reduce_check_owned(dst.data_ptr(), ptrs, len(srcs), count, dtype, inv,
                                           res.data_ptr(), ws.data_ptr(),
                                           ws.numel() * ws.element_size(), accumulate, _stream())


def _result_bytes(res):
    torch.cuda.synchronize()
    return res.cpu().numpy().tobytes()


@pytest.mark.parametrize("order", ["noalloc first", "workspace first"])
def test_noalloc_matches_workspace_call(order):
    cases = [(8, 5_000_011, BF16, 0, 2.0 ** -3),        # LDS-staged blocks, tail
             (3, 100_003, FP16, 3, 2.0 ** -16)]          # second call: smaller, misaligned
    for k, (n_ranks, count, dtype, offset, inv) in enumerate(cases):
        host = _patterns(n_ranks, count, dtype, seed=17 + k)
        srcs = [_device(h, dtype, offset) for h in host]
        want = oracle.reduce(host, dtype)
        flag_o, sumsq_o = oracle.check(want, dtype, inv)
        dst_a = _device(np.zeros(count, np.uint16), dtype, offset)
        dst_b = _device(np.zeros(count, np.uint16), dtype, offset)
        res_a = torch.zeros(4, dtype=torch.int32, device="cuda")
        res_b = torch.full((4,), -1, dtype=torch.int32, device="cuda")
        ws = torch.empty(Z.zero_check_workspace_bytes(count) // 8 + 1, dtype=torch.float64,
                         device="cuda")
        calls = [lambda: _noalloc(dst_a, srcs, count, dtype, inv, res_a),
                 lambda: _with_workspace(dst_b, srcs, count, dtype, inv, res_b, ws)]
        if order == "workspace first":
            calls.reverse()
        for call in calls:
            assert call() == Z.ZERO_OK
        where = f"call {k + 1} ({n_ranks} ranks, {count} elements)"
        assert_bits16_equal(to_np16(dst_a), to_np16(dst_b), dtype, where)
        assert_bits16_equal(to_np16(dst_a), want, dtype, where + " vs oracle")
        assert _result_bytes(res_a) == _result_bytes(res_b), where
        r = Z.read_result(res_a)
        assert r.overflow == flag_o
        assert r.sumsq == pytest.approx(sumsq_o, rel=sum_bound(count))
    # an accumulating call adds to the last result in both forms alike
    assert _noalloc(dst_a, srcs, count, dtype, inv, res_a, accumulate=1) == Z.ZERO_OK
    assert _with_workspace(dst_b, srcs, count, dtype, inv, res_b, ws, accumulate=1) == Z.ZERO_OK
    assert _result_bytes(res_a) == _result_bytes(res_b)
    assert Z.read_result(res_a).sumsq == pytest.approx(2 * sumsq_o, rel=2 * sum_bound(count))


def test_noalloc_limits():
    fake = ctypes.c_void_p(0x10000)                   # never dereferenced: refused first
    srcs = (ctypes.c_void_p * 2)(fake, fake)
    L = Z.lib()
    assert L.zero_reduce_check_owned_noalloc(fake, srcs, 2, (1 << 32) + 1, BF16, 1.0, fake, 0,
                                             None) == Z.ZERO_ERANGE
    assert L.zero_reduce_check_owned_noalloc(fake, srcs, 2, -1, BF16, 1.0, fake, 0,
                                             None) == Z.ZERO_EINVAL
    assert L.zero_reduce_check_owned_noalloc(fake, srcs, 0, 10, BF16, 1.0, fake, 0,
                                             None) == Z.ZERO_EINVAL
    # the binding's wrapper on an empty input touches nothing and succeeds
    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    empty = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    Z.zero_reduce_check_owned_noalloc(empty, [empty, empty], 1.0, res)
    r = Z.read_result(res)
    assert r.overflow == 0 and r.sumsq == 0.0
