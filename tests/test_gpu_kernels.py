"""GPU parity of each C-ABI call against the oracle, element by element.

Sizes span several 128-bit tiles and ragged tails (0, 1, 7, 8, 9, 4095,
100003 elements), start offsets that are not 16-byte aligned (the vector path
then peels a scalar head), pointers with different alignments (scalar path),
1..16 ranks, binary16 and bfloat16, special values (+-0, subnormals, the
largest finite value, sums that overflow, inf, NaN), in-place reduction, the
skip path and accumulation over several owner ranges.

Tolerances: reduced gradients, overflow flags and skip decisions bit-exact;
fp32 master / m / v bit-equal or within 2e-6 relative; 16-bit copy within 1 ulp;
sumsq within 1e-12 relative here (fp64 sums of the exact squares of the fp32
unscaled values; only the summation order differs).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import zero_partitioned_mixed_shard_amd as Z
from _common import (assert_bits16_equal, assert_f32_close, assert_p16_close, from_np16,
                     to_np16, to_np32)

pytestmark = pytest.mark.gpu

FP16, BF16 = 1, 2
# 4096 and 8200: AdamW blocks of 2048 elements all whole (no register-path
# tail at offset 0), then one lane tile past them
COUNTS = [0, 1, 7, 8, 9, 4095, 4096, 8200, 100003]
# the reduce takes two block-wide rows of 256 lane tiles per block (4096
# elements): a last block with one full row and an empty second row, and one
# whose second row holds a single lane tile; 8192 and 12296: every block whole
# (at 8 ranks all staged in LDS, at offset 0), then one lane tile past them
REDUCE_COUNTS = COUNTS + [10240, 6152, 8192, 12296]
SPECIAL = {FP16: [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x7BFF, 0xFBFF, 0x7B53, 0x7C00, 0xFC00,
                  0x7E00],
           BF16: [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x7F7F, 0xFF7F, 0x7F00, 0x7F80, 0xFF80,
                  0x7FC0]}


def _rand16(n, dtype, rng, specials=0.0, sigma=1e-3, scale=2.0 ** 10):
    spec = synth.normal_spec(sigma, dtype)
    if dtype == FP16:
        spec = synth.scaled(spec, scale)
    a = np.empty(n, np.uint16)
    synth.fill_host(a, int(rng.integers(0, 2 ** 40)), int(rng.integers(0, 2 ** 63)), spec)
    if specials:
        pick = rng.random(n) < specials
        a[pick] = rng.choice(SPECIAL[dtype], int(pick.sum()))
    return a


def _dev16(a, dtype, offset=0):
    """Device copy of `a` starting `offset` elements into a fresh allocation."""
    base = torch.zeros(a.size + offset + 8, dtype=torch.int16, device="cuda")
    base[offset:offset + a.size] = torch.from_numpy(a.view(np.int16)).cuda()
    tdt = torch.float16 if dtype == FP16 else torch.bfloat16
    return base.view(tdt)[offset:offset + a.size]


def _dev32(a, offset=0):
    base = torch.zeros(a.size + offset + 8, dtype=torch.float32, device="cuda")
    base[offset:offset + a.size] = torch.from_numpy(a).cuda()
    return base[offset:offset + a.size]


# ----------------------------------------------------------- generator ----
@pytest.mark.parametrize("first", [0, 12345, 2 ** 33 + 7])
def test_device_generator_matches_host(first):
    for spec in (synth.scaled(synth.normal_spec(1e-3, FP16), 2.0 ** 16),
                 synth.normal_spec(1e-4, BF16), synth.normal_spec(0.02, FP16),
                 synth.normal_spec(0.02, BF16)):
        key = synth.stream_key(3, synth.KIND_GRAD, 2, 5)
        host = np.empty(100003, np.uint16)
        synth.fill_host(host, first, key, spec)
        dev = torch.empty(100003, dtype=torch.int16, device="cuda")
        synth.fill_device(dev.data_ptr(), dev.numel(), first, key, spec)
        torch.cuda.synchronize()
        assert np.array_equal(to_np16(dev), host)


# --------------------------------------------------------------- init ------
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_init_master(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    master = torch.empty(bits.size, dtype=torch.float32, device="cuda")
    Z.zero_init_master(master, from_np16(bits, dtype))
    want = oracle.init_master(bits, dtype)
    got = to_np32(master)
    ok = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    assert ok.all()


# ------------------------------------------------------------- reduce ------
@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("n_ranks", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("count", REDUCE_COUNTS)
@pytest.mark.parametrize("offset", [0, 3])
def test_reduce_parity(dtype, n_ranks, count, offset):
    rng = np.random.default_rng(1000 * dtype + 100 * n_ranks + count % 97 + offset)
    host = [_rand16(count, dtype, rng, specials=0.02) for _ in range(n_ranks)]
    srcs = [_dev16(h, dtype, offset) for h in host]
    dst = _dev16(np.zeros(count, np.uint16), dtype, offset)
    Z.zero_reduce_owned(dst, srcs)
    torch.cuda.synchronize()
    if count:
        assert_bits16_equal(to_np16(dst), oracle.reduce(host, dtype), dtype, "reduce")


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_reduce_mixed_alignment_and_in_place(dtype):
    rng = np.random.default_rng(77)
    count = 50001
    host = [_rand16(count, dtype, rng, specials=0.01) for _ in range(8)]
    want = oracle.reduce(host, dtype)
    # sources at different alignments: the scalar path
    srcs = [_dev16(h, dtype, k % 5) for k, h in enumerate(host)]
    dst = _dev16(np.zeros(count, np.uint16), dtype, 1)
    Z.zero_reduce_owned(dst, srcs)
    torch.cuda.synchronize()
    assert_bits16_equal(to_np16(dst), want, dtype, "reduce, mixed alignment")
    # in place into the owner's own rank buffer
    srcs = [_dev16(h, dtype, 2) for h in host]
    Z.zero_reduce_owned(srcs[5], srcs)
    torch.cuda.synchronize()
    assert_bits16_equal(to_np16(srcs[5]), want, dtype, "reduce, in place")


def test_reduce_overflow_specials():
    # 8 x 60000 overflows binary16; 60000 - 60000 cancels; inf - inf is NaN
    a = np.array([0x7B53, 0x7B53, 0x7C00, 0x8000], np.uint16)
    b = np.array([0x7B53, 0xFB53, 0xFC00, 0x8000], np.uint16)
    host = [a] * 7 + [b]
    dst = _dev16(np.zeros(4, np.uint16), FP16)
    Z.zero_reduce_owned(dst, [_dev16(h, FP16) for h in host])
    torch.cuda.synchronize()
    assert_bits16_equal(to_np16(dst), oracle.reduce(host, FP16), FP16)


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_reduce_fp32_accumulation_columns(dtype):
    # columns where fp32 accumulation from +0 and an exact sum round differently
    # (binary16 [2048, 1, 2^-14] -> 2048; bfloat16 [1, 2^-8, 2^-32] -> 1), the
    # same addends in another order, and -0 columns (the sum starts from +0)
    cols = {FP16: [(0x6800, 0x3C00, 0x0400), (0x0400, 0x3C00, 0x6800), (0x8000, 0x8000, 0x8000)],
            BF16: [(0x3F80, 0x3B80, 0x2F80), (0x2F80, 0x3F80, 0x3B80), (0x8000, 0x8000, 0x8000)]}
    want_hand = {FP16: [0x6800, 0x6800, 0x0000], BF16: [0x3F80, 0x3F80, 0x0000]}
    reps = 4099                                  # vector path plus a ragged tail
    host = [np.tile(np.array([c[r] for c in cols[dtype]], np.uint16), reps) for r in range(3)]
    want = oracle.reduce(host, dtype)
    assert want[:3].tolist() == want_hand[dtype]
    dst = _dev16(np.zeros(host[0].size, np.uint16), dtype)
    Z.zero_reduce_owned(dst, [_dev16(h, dtype) for h in host])
    torch.cuda.synchronize()
    assert_bits16_equal(to_np16(dst), want, dtype, "fp32 accumulation columns")


# -------------------------------------------------------------- check ------
def _res_tensor():
    return torch.zeros(4, dtype=torch.int32, device="cuda")


def _ws(count):
    return torch.empty((Z.zero_check_workspace_bytes(count) + 7) // 8, dtype=torch.float64,
                       device="cuda")


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("count", COUNTS + [3_000_017, 10_000_019])
@pytest.mark.parametrize("offset", [0, 5])
@pytest.mark.parametrize("specials", [0.0, 1e-4])
def test_check_parity(dtype, count, offset, specials):
    rng = np.random.default_rng(count + offset + dtype)
    host = _rand16(count, dtype, rng)
    if specials and count:
        host[int(rng.integers(0, count))] = SPECIAL[dtype][-1 - int(rng.integers(0, 3))]
    inv = 2.0 ** -10
    res = _res_tensor()
    Z.zero_unscale_check_norm(_dev16(host, dtype, offset), inv, res, _ws(count))
    r = Z.read_result(res)
    flag, sumsq = oracle.check(host, dtype, inv)
    assert r.overflow == flag
    assert r.inv_scale == inv
    if not flag:
        assert r.sumsq == pytest.approx(sumsq, rel=1e-12, abs=0)


# the large size only at the workload rank counts
FUSED_CASES = ([(n, c) for n in (1, 3, 8, 16) for c in REDUCE_COUNTS]
               + [(n, 10_000_019) for n in (8, 16)])


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("n_ranks,count", FUSED_CASES)
@pytest.mark.parametrize("offset", [0, 3])
def test_reduce_check_fused_parity(dtype, n_ranks, count, offset):
    """zero_reduce_check_owned = reduce then check; 10,000,019 elements give
    2,442 block partials, folded by the one-block final pass."""
    rng = np.random.default_rng(7 * dtype + 31 * n_ranks + count % 101 + offset)
    host = [_rand16(count, dtype, rng, specials=0.0 if count > 1000 else 0.01)
            for _ in range(n_ranks)]
    srcs = [_dev16(h, dtype, offset) for h in host]
    dst = _dev16(np.zeros(count, np.uint16), dtype, offset)
    inv = 2.0 ** -10
    res = _res_tensor()
    Z.zero_reduce_check_owned(dst, srcs, inv, res, _ws(count))
    r = Z.read_result(res)
    want = oracle.reduce(host, dtype) if count else np.zeros(0, np.uint16)
    if count:
        assert_bits16_equal(to_np16(dst), want, dtype, "fused reduce")
    flag, sumsq = oracle.check(want, dtype, inv)
    assert r.overflow == flag and r.inv_scale == inv
    if not flag:
        assert r.sumsq == pytest.approx(sumsq, rel=1e-12, abs=0)


@pytest.mark.parametrize("entry", ["fused", "check"])
def test_norm_through_fold_levels(entry):
    """Past 16,384 block partials the partials go through a fold pass before
    the final one: the fused reduce+check over 70,000,019 elements (17,090
    partials) and the check over 40,000,003 (19,532 partials), against the
    oracle's norm."""
    dtype = BF16
    rng = np.random.default_rng(23 if entry == "fused" else 29)
    count = 70_000_019 if entry == "fused" else 40_000_003
    n_ranks = 8 if entry == "fused" else 1
    host = [_rand16(count, dtype, rng) for _ in range(n_ranks)]
    want = oracle.reduce(host, dtype) if entry == "fused" else host[0]
    res = _res_tensor()
    inv = 2.0 ** -3
    if entry == "fused":
        dst = _dev16(np.zeros(count, np.uint16), dtype, 3)
        Z.zero_reduce_check_owned(dst, [_dev16(h, dtype, 3) for h in host], inv, res, _ws(count))
        assert_bits16_equal(to_np16(dst), want, dtype, "fused reduce, fold levels")
    else:
        Z.zero_unscale_check_norm(_dev16(host[0], dtype, 3), inv, res, _ws(count))
    r = Z.read_result(res)
    flag, sumsq = oracle.check(want, dtype, inv)
    assert r.overflow == flag == 0
    assert r.sumsq == pytest.approx(sumsq, rel=1e-12, abs=0)


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_reduce_check_fused_unaligned_and_windows(dtype):
    rng = np.random.default_rng(17)
    count = 3_000_001
    host = [_rand16(count, dtype, rng) for _ in range(8)]
    want = oracle.reduce(host, dtype)
    # sources at different alignments: every lane walks its 8 elements one by one
    srcs = [_dev16(h, dtype, k % 3) for k, h in enumerate(host)]
    dst = _dev16(np.zeros(count, np.uint16), dtype, 1)
    res = _res_tensor()
    Z.zero_reduce_check_owned(dst, srcs, 1.0, res, _ws(count))
    r = Z.read_result(res)
    assert_bits16_equal(to_np16(dst), want, dtype, "fused, mixed alignment")
    flag, sumsq = oracle.check(want, dtype, 1.0)
    assert r.overflow == flag == 0 and r.sumsq == pytest.approx(sumsq, rel=1e-12)
    # three windows accumulated into one result, a NaN in the middle one
    srcs = [_dev16(h, dtype) for h in host]
    srcs[4][1_500_000] = float("nan")
    dst = _dev16(np.zeros(count, np.uint16), dtype)
    cuts = [0, 1_000_000, 2_000_003, count]
    ws = _ws(count)
    for k in range(3):
        a, b = cuts[k], cuts[k + 1]
        Z.zero_reduce_check_owned(dst[a:b], [x[a:b] for x in srcs], 1.0, res, ws,
                                  accumulate=k > 0)
    assert Z.read_result(res).overflow == 1


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_check_accumulates_over_owners(dtype):
    rng = np.random.default_rng(8)
    host = _rand16(1_000_003, dtype, rng)
    dev = _dev16(host, dtype)
    bounds = [0, 100, 333_333, 900_001, 1_000_003]
    ws = _ws(host.size)
    res = _res_tensor()
    for k in range(len(bounds) - 1):
        Z.zero_unscale_check_norm(dev[bounds[k]:bounds[k + 1]], 1.0, res, ws, accumulate=k > 0)
    r = Z.read_result(res)
    flag, sumsq = 0, 0.0
    for k in range(len(bounds) - 1):
        flag, sumsq = oracle.check(host[bounds[k]:bounds[k + 1]], dtype, 1.0, flag, sumsq)
    assert r.overflow == flag == 0
    assert r.sumsq == pytest.approx(sumsq, rel=1e-12)
    # a NaN in the last range sets the global flag
    dev[1_000_000] = float("nan")
    for k in range(len(bounds) - 1):
        Z.zero_unscale_check_norm(dev[bounds[k]:bounds[k + 1]], 1.0, res, ws, accumulate=k > 0)
    assert Z.read_result(res).overflow == 1


def test_check_repeatable_bits():
    rng = np.random.default_rng(3)
    host = _rand16(5_000_000, BF16, rng)
    dev = _dev16(host, BF16)
    ws = _ws(host.size)
    outs = set()
    for _ in range(3):
        res = _res_tensor()
        Z.zero_unscale_check_norm(dev, 1.0, res, ws)
        outs.add(Z.read_result(res).sumsq)
    assert len(outs) == 1


# -------------------------------------------------------------- AdamW ------
def _state(count, rng):
    master = (rng.standard_normal(count) * 0.02).astype(np.float32)
    m = (rng.standard_normal(count) * 1e-4).astype(np.float32)
    v = (rng.random(count) * 1e-8).astype(np.float32)
    return master, m, v


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("count", COUNTS)
@pytest.mark.parametrize("offset", [0, 1, 6])
@pytest.mark.parametrize("clip,t", [(0.0, 1), (1.0, 7), (1e-3, 3)])
def test_adamw_parity(dtype, count, offset, clip, t):
    rng = np.random.default_rng(count * 7 + offset + int(clip * 1000) + t)
    master, m, v = _state(count, rng)
    p16 = oracle.encode16(master, dtype)
    scale = 2.0 ** 10 if dtype == FP16 else 1.0
    grad = _rand16(count, dtype, rng, sigma=1e-3, scale=scale)
    inv = 1.0 / scale
    hp = oracle.HParams(max_grad_norm=clip)
    # device: check then step
    d_master, d_m, d_v = _dev32(master, offset), _dev32(m, offset), _dev32(v, offset)
    d_p16, d_g = _dev16(p16, dtype, offset), _dev16(grad, dtype, offset)
    res = _res_tensor()
    Z.zero_unscale_check_norm(d_g, inv, res, _ws(count))
    Z.zero_adamw_step(d_master, d_m, d_v, d_p16, d_g,
                      Z.zero_adamw_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                                           hp.max_grad_norm, t), res)
    torch.cuda.synchronize()
    # oracle
    flag, sumsq = oracle.check(grad, dtype, inv)
    oracle.adamw(master, m, v, p16, grad, dtype, inv, sumsq, flag, hp, t)
    assert_f32_close(to_np32(d_master), master, "master")
    assert_f32_close(to_np32(d_m), m, "exp_avg")
    assert_f32_close(to_np32(d_v), v, "exp_avg_sq")
    assert_p16_close(to_np16(d_p16), p16, dtype, "param16")


# Lane l of an AdamW block takes the element quads at 4l and 1024 + 4l of the
# block's 2048 elements: these sizes end the vector body exactly at, just
# before and just after the half-block boundary of the last block, and in the
# middle of either half, so lanes with both quads, only the first, and none
# all occur (with the misaligned offsets also through the head path).
@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("count", [2048 + 1024, 2048 + 1020, 2048 + 1028, 3 * 2048 + 500 + 5,
                                   5 * 2048 + 1600 + 7])
@pytest.mark.parametrize("offset", [0, 1, 6])
def test_adamw_half_block_edges(dtype, count, offset):
    rng = np.random.default_rng(count + 31 * offset)
    master, m, v = _state(count, rng)
    p16 = oracle.encode16(master, dtype)
    grad = _rand16(count, dtype, rng, sigma=1e-3, scale=1.0)
    hp = oracle.HParams(max_grad_norm=1.0)
    d_master, d_m, d_v = _dev32(master, offset), _dev32(m, offset), _dev32(v, offset)
    d_p16, d_g = _dev16(p16, dtype, offset), _dev16(grad, dtype, offset)
    res = _res_tensor()
    Z.zero_unscale_check_norm(d_g, 1.0, res, _ws(count))
    Z.zero_adamw_step(d_master, d_m, d_v, d_p16, d_g,
                      Z.zero_adamw_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                                           hp.max_grad_norm, 2), res)
    torch.cuda.synchronize()
    flag, sumsq = oracle.check(grad, dtype, 1.0)
    oracle.adamw(master, m, v, p16, grad, dtype, 1.0, sumsq, flag, hp, 2)
    assert_f32_close(to_np32(d_master), master, "master")
    assert_f32_close(to_np32(d_m), m, "exp_avg")
    assert_f32_close(to_np32(d_v), v, "exp_avg_sq")
    assert_p16_close(to_np16(d_p16), p16, dtype, "param16")


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_adamw_bit_exact_large(dtype):
    """On a large aligned shard the fp32 results are expected to be bit-equal."""
    rng = np.random.default_rng(99)
    count = 2_000_003
    master, m, v = _state(count, rng)
    p16 = oracle.encode16(master, dtype)
    grad = _rand16(count, dtype, rng, sigma=1e-4, scale=1.0)
    hp = oracle.HParams(max_grad_norm=1.0)
    d = [_dev32(master), _dev32(m), _dev32(v)]
    d_p16, d_g = _dev16(p16, dtype), _dev16(grad, dtype)
    res = _res_tensor()
    Z.zero_unscale_check_norm(d_g, 1.0, res, _ws(count))
    Z.zero_adamw_step(*d, d_p16, d_g, Z.zero_adamw_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps,
                                                           hp.weight_decay, 1.0, 4), res)
    torch.cuda.synchronize()
    flag, sumsq = oracle.check(grad, dtype, 1.0)
    oracle.adamw(master, m, v, p16, grad, dtype, 1.0, sumsq, flag, hp, 4)
    for dev, want in zip(d, (master, m, v)):
        assert assert_f32_close(to_np32(dev), want) == 0
    assert np.array_equal(to_np16(d_p16), p16)


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_adamw_skips_on_overflow(dtype):
    rng = np.random.default_rng(5)
    count = 70001
    master, m, v = _state(count, rng)
    p16 = oracle.encode16(master, dtype)
    grad = _rand16(count, dtype, rng, specials=0.0)
    grad[12345] = synth.QNAN[dtype]
    d = [_dev32(master), _dev32(m), _dev32(v)]
    d_p16, d_g = _dev16(p16, dtype), _dev16(grad, dtype)
    res = _res_tensor()
    Z.zero_unscale_check_norm(d_g, 1.0, res, _ws(count))
    Z.zero_adamw_step(*d, d_p16, d_g, Z.zero_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1),
                      res)
    torch.cuda.synchronize()
    assert Z.read_result(res).overflow == 1
    for dev, want in zip(d, (master, m, v)):
        assert np.array_equal(to_np32(dev).view(np.uint32), want.view(np.uint32))
    assert np.array_equal(to_np16(d_p16), p16)


# -------------------------------------------------------------- errors -----
def test_invalid_arguments_launch_nothing():
    L = Z.lib()
    dst = torch.zeros(16, dtype=torch.float16, device="cuda")
    ptrs = (ctypes.c_void_p * 1)(dst.data_ptr())
    assert L.zero_reduce_owned(dst.data_ptr(), ptrs, 0, 16, FP16, None) == Z.ZERO_EINVAL
    assert L.zero_reduce_owned(dst.data_ptr(), ptrs, 17, 16, FP16, None) == Z.ZERO_EINVAL
    assert L.zero_reduce_owned(dst.data_ptr(), ptrs, 1, -1, FP16, None) == Z.ZERO_EINVAL
    assert L.zero_reduce_owned(dst.data_ptr(), ptrs, 1, 16, 7, None) == Z.ZERO_EINVAL
    assert L.zero_reduce_owned(dst.data_ptr(), None, 1, 16, FP16, None) == Z.ZERO_EINVAL
    ws = _ws(16)
    assert L.zero_unscale_check_norm(dst.data_ptr(), 16, FP16, 1.0, None, ws.data_ptr(), 8 * ws.numel(),
                                     0, None) == Z.ZERO_EINVAL
    res = _res_tensor()
    assert L.zero_unscale_check_norm(dst.data_ptr(), 16, FP16, 1.0, res.data_ptr(), ws.data_ptr(), 0,
                                     0, None) == Z.ZERO_EINVAL
    hp = Z.zero_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 0.0, 0)
    f = torch.zeros(16, device="cuda")
    assert L.zero_adamw_step(f.data_ptr(), f.data_ptr(), f.data_ptr(), dst.data_ptr(), dst.data_ptr(),
                             16, FP16, ctypes.byref(hp), res.data_ptr(), None) == Z.ZERO_EINVAL
    torch.cuda.synchronize()
    assert (dst == 0).all()


def test_step_control_update_matches_host_rules():
    """zero_step_control_update against the host loss scaler and the oracle's
    constants over 300 steps with random overflow flags, a 3-step doubling
    window and a floor: scale, counters and t exact; inv_scale exact; the
    bias corrections for the next step equal the host's fp64 pow rounded to
    fp32 (device pow: allowed 1 ulp, counted)."""
    rng = np.random.default_rng(5)
    ctl_h = Z.zero_step_control_init(64.0, 2.0, 3, 2.0, 0.9, 0.999)
    ctl = Z.control_to_device(ctl_h)
    scaler = Z.zero_loss_scaler(64.0, 2.0, 3, 0, 0)
    t = 0
    res = _res_tensor()
    exact = 0
    for k in range(300):
        flag = int(rng.random() < 0.35)
        res.zero_()
        res[2] = flag                                     # zero_step_result.overflow
        Z.zero_step_control_update(ctl, res)
        c = Z.read_control(ctl)
        Z.zero_loss_scaler_update(scaler, flag)
        t += 1 - flag
        assert (c.scale, c.clean, c.skipped, c.t) == (scaler.scale, scaler.clean, scaler.skipped, t)
        assert c.inv_scale == float(np.float32(1.0 / (scaler.scale * 2.0)))
        want = oracle.adam_consts(oracle.HParams(), t + 1)
        for got, w in ((c.bc1, want["bc1"]), (c.bc2, want["bc2"])):
            d = abs(int(np.float32(got).view(np.int32)) - int(np.float32(w).view(np.int32)))
            assert d <= 1, (k, got, w)
            exact += d == 0
    print(f"bias corrections equal to the host's in {exact} of 600", flush=True)
