"""The range-list calls on the GPU against the oracle, every element:
zero_reduce_check_ranges and zero_adamw_step_ranges over disjoint ranges of
random sizes and alignments (empty ranges, ranges one element apart, ranges
that touch and are merged into one launch, touching ranges that tile the whole
buffer, lists of up to 70 ranges sharing one fold of the norm), with
the result and inv_scale given on the host or read from a device step
control; elements outside the ranges untouched.

Tolerances as everywhere: reduced values, flags bit-exact; the norm within
1e-12 of the oracle's exact fp64 sum (the fold order differs from a chain of
single-range calls only in the last bits); fp32 state bit-equal or within
2e-6 relative; the 16-bit copy within 1 ulp."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_partitioned_mixed_shard_amd as Z
from _common import (assert_bits16_equal, assert_f32_close, assert_p16_close, to_np16,
                     to_np32)

pytestmark = pytest.mark.gpu

FP16, BF16 = 1, 2


def _rand16(n, dtype, rng, sigma=1e-3, scale=2.0 ** 10):
    spec = synth.normal_spec(sigma, dtype)
    if dtype == FP16:
        spec = synth.scaled(spec, scale)
    a = np.empty(n, np.uint16)
    synth.fill_host(a, int(rng.integers(0, 2 ** 40)), int(rng.integers(0, 2 ** 63)), spec)
    return a


def _dev16(a, dtype, offset=0):
    base = torch.zeros(a.size + offset + 8, dtype=torch.int16, device="cuda")
    base[offset:offset + a.size] = torch.from_numpy(a.view(np.int16)).cuda()
    return base.view(torch.float16 if dtype == FP16 else torch.bfloat16)[offset:offset + a.size]


def _dev32(a, offset=0):
    base = torch.zeros(a.size + offset + 8, dtype=torch.float32, device="cuda")
    base[offset:offset + a.size] = torch.from_numpy(a).cuda()
    return base[offset:offset + a.size]


def _random_ranges(total, k, rng):
    """k disjoint ranges in [0, total) in random order: random gaps (about a
    third of the ranges touch the one before, which the library merges into
    one launch), random lengths, a few empty ranges."""
    cuts = np.sort(rng.choice(np.arange(1, total), size=2 * k, replace=False))
    rs = []
    for j in range(k):
        a, b = int(cuts[2 * j]), int(cuts[2 * j + 1])
        if j > 0 and rng.random() < 0.3:
            a = int(cuts[2 * j - 1])               # starts where the previous ends
        if rng.random() < 0.1:
            b = a                                  # empty
        rs.append((a, b - a))
    order = rng.permutation(len(rs))
    return [rs[i] for i in order]


def _tiling_ranges(total, k, rng):
    """k ranges that cover [0, total) exactly, each touching the next, in
    random order (a few empty)."""
    cuts = np.concatenate([[0], np.sort(rng.choice(np.arange(1, total), size=k - 1,
                                                   replace=False)), [total]])
    rs = [(int(cuts[j]), int(cuts[j + 1] - cuts[j])) for j in range(k)]
    rs += [(int(rng.integers(0, total)), 0) for _ in range(2)]
    order = rng.permutation(len(rs))
    return [rs[i] for i in order]


def _mask(total, ranges):
    m = np.zeros(total, bool)
    for a, c in ranges:
        m[a:a + c] = True
    return m


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("n_ranks", [1, 3, 8, 16])
@pytest.mark.parametrize("k", [1, 5, 33, 70])
@pytest.mark.parametrize("offset,in_place", [(0, False), (3, False), (0, True)])
@pytest.mark.parametrize("control", ["host", "device"])
def test_reduce_check_ranges_parity(dtype, n_ranks, k, offset, in_place, control):
    total = 600_003
    rng = np.random.default_rng(100 * dtype + 7 * n_ranks + k + offset + int(in_place))
    host = [_rand16(total, dtype, rng) for _ in range(n_ranks)]
    srcs = [_dev16(h, dtype, offset) for h in host]
    sentinel = np.full(total, 0x1234, np.uint16)
    dst = srcs[0] if in_place else _dev16(sentinel, dtype, offset)
    ranges = _random_ranges(total, k, rng)
    inv = 2.0 ** -10 if dtype == FP16 else 1.0
    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(Z.zero_range_workspace_bytes(ranges) // 8 + 1, dtype=torch.float64,
                     device="cuda")
    ctl = None
    if control == "device":
        # scale S with 1 / (S * D) = inv: the step control reads the same factor
        c = Z.zero_step_control_init(1.0 / inv, 1.0, 1000, 1.0, 0.9, 0.999)
        ctl = Z.control_to_device(c)
    Z.zero_reduce_check_ranges(dst, srcs, ranges, inv, res, ws, ctl_dev=ctl)
    r = Z.read_result(res)
    got = to_np16(dst)
    m = _mask(total, ranges)
    want_red = oracle.reduce([h[m] for h in host], dtype) if m.any() else np.zeros(0, np.uint16)
    assert_bits16_equal(got[m], want_red, dtype, "reduce in ranges")
    outside = host[0][~m] if in_place else sentinel[~m]
    assert np.array_equal(got[~m], outside), "an element outside every range changed"
    flag, sumsq = oracle.check(want_red, dtype, inv)
    assert r.overflow == flag and r.inv_scale == np.float32(inv)
    if not flag:
        assert r.sumsq == pytest.approx(sumsq, rel=1e-12, abs=0)


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("n_ranks", [8, 16])
@pytest.mark.parametrize("k", [2, 18])
@pytest.mark.parametrize("offset", [0, 5])
def test_ranges_tiling_whole_buffer(dtype, n_ranks, k, offset):
    """Touching ranges that cover the whole buffer (a bucket group's windows
    with every owner on one GPU): merged into one launch per call; reduce,
    flag, norm and AdamW equal the oracle over the whole buffer."""
    total = 900_017
    rng = np.random.default_rng(1000 + 10 * dtype + n_ranks + k + offset)
    host = [_rand16(total, dtype, rng) for _ in range(n_ranks)]
    srcs = [_dev16(h, dtype, offset) for h in host]
    dst = _dev16(np.zeros(total, np.uint16), dtype, offset)
    ranges = _tiling_ranges(total, k, rng)
    inv = 2.0 ** -10 if dtype == FP16 else 1.0
    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(Z.zero_range_workspace_bytes(ranges) // 8 + 1, dtype=torch.float64,
                     device="cuda")
    Z.zero_reduce_check_ranges(dst, srcs, ranges, inv, res, ws)
    want_red = oracle.reduce(host, dtype)
    assert_bits16_equal(to_np16(dst), want_red, dtype, "reduce over the tiling")
    flag, sumsq = oracle.check(want_red, dtype, inv)
    r = Z.read_result(res)
    assert r.overflow == flag == 0
    assert r.sumsq == pytest.approx(sumsq, rel=1e-12, abs=0)
    master = (rng.standard_normal(total) * 0.02).astype(np.float32)
    p16 = oracle.encode16(master, dtype)
    d = [_dev32(x, offset) for x in (master, np.zeros(total, np.float32),
                                     np.zeros(total, np.float32))]
    d_p16 = _dev16(p16, dtype, offset)
    hp = oracle.HParams(max_grad_norm=1.0)
    Z.zero_adamw_step_ranges(*d, d_p16, dst, ranges,
                             Z.zero_adamw_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps,
                                                  hp.weight_decay, hp.max_grad_norm, 1), res)
    torch.cuda.synchronize()
    want = [master.copy(), np.zeros(total, np.float32), np.zeros(total, np.float32), p16.copy()]
    oracle.adamw(*want, want_red, dtype, inv, sumsq, flag, hp, 1)
    for dev, w, kk in zip(d, want, ("master", "exp_avg", "exp_avg_sq")):
        assert_f32_close(to_np32(dev), w, kk)
    assert_p16_close(to_np16(d_p16), want[3], dtype, "param16")


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("k", [1, 4, 40])
@pytest.mark.parametrize("offset", [0, 1, 6])
@pytest.mark.parametrize("control", ["host", "device"])
def test_adamw_ranges_parity(dtype, k, offset, control):
    total = 1_000_003
    rng = np.random.default_rng(11 * dtype + k + 3 * offset)
    master = (rng.standard_normal(total) * 0.02).astype(np.float32)
    m_ = (rng.standard_normal(total) * 1e-4).astype(np.float32)
    v = (rng.random(total) * 1e-8).astype(np.float32)
    p16 = oracle.encode16(master, dtype)
    scale = 2.0 ** 10 if dtype == FP16 else 1.0
    grad = _rand16(total, dtype, rng, scale=scale)
    inv = 1.0 / scale
    ranges = _random_ranges(total, k, rng)
    msk = _mask(total, ranges)
    hp = oracle.HParams(max_grad_norm=1.0)
    t = 3
    d = [_dev32(x, offset) for x in (master, m_, v)]
    d_p16, d_g = _dev16(p16, dtype, offset), _dev16(grad, dtype, offset)
    # the check over the same ranges gives the flag and the global norm
    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(Z.zero_range_workspace_bytes(ranges) // 8 + 1, dtype=torch.float64,
                     device="cuda")
    zhp = Z.zero_adamw_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                               hp.max_grad_norm, t)
    ctl = None
    if control == "device":
        c = Z.zero_step_control_init(scale, 1.0, 1000, 1.0, hp.beta1, hp.beta2)
        c.t = t - 1                                   # the next step is step t
        # bias corrections of step t from the fp32 betas, fp64, rounded once
        # (as the control update derives them)
        c.bc1 = float(np.float32(1.0 - float(np.float32(hp.beta1)) ** t))
        c.bc2 = float(np.float32(1.0 - float(np.float32(hp.beta2)) ** t))
        ctl = Z.control_to_device(c)
    # a one-rank "reduce" writes the gradient to a scratch copy and checks it
    scratch = d_g.clone()
    Z.zero_reduce_check_ranges(scratch, [d_g], ranges, inv, res, ws, ctl_dev=ctl)
    Z.zero_adamw_step_ranges(*d, d_p16, d_g, ranges, zhp, res, ctl_dev=ctl)
    torch.cuda.synchronize()
    flag, sumsq = oracle.check(grad[msk], dtype, inv)
    want = {"master": master.copy(), "exp_avg": m_.copy(), "exp_avg_sq": v.copy(),
            "param16": p16.copy()}
    sel = {kk: x[msk].copy() for kk, x in want.items()}
    oracle.adamw(sel["master"], sel["exp_avg"], sel["exp_avg_sq"], sel["param16"], grad[msk],
                 dtype, inv, sumsq, flag, hp, t)
    for kk in ("master", "exp_avg", "exp_avg_sq"):
        want[kk][msk] = sel[kk]
    want["param16"][msk] = sel["param16"]
    for dev, kk in zip(d, ("master", "exp_avg", "exp_avg_sq")):
        got = to_np32(dev)
        assert_f32_close(got[msk], want[kk][msk], kk)
        assert np.array_equal(got[~msk].view(np.uint32), want[kk][~msk].view(np.uint32)), kk
    got16 = to_np16(d_p16)
    assert_p16_close(got16[msk], want["param16"][msk], dtype, "param16")
    assert np.array_equal(got16[~msk], p16[~msk])


def test_adamw_ranges_skip_on_overflow():
    """An inf in one range's gradient: the flag is set and no range changes."""
    dtype, total = BF16, 200_003
    rng = np.random.default_rng(5)
    grad = _rand16(total, dtype, rng, sigma=1e-4, scale=1.0)
    ranges = [(10, 5000), (90_000, 7000), (150_000, 40_000)]
    grad[152_345] = 0x7F80                           # +inf inside the last range
    master = (rng.standard_normal(total) * 0.02).astype(np.float32)
    d_g = _dev16(grad, dtype)
    d = [_dev32(master), _dev32(np.zeros(total, np.float32)), _dev32(np.zeros(total, np.float32))]
    p16 = _dev16(oracle.encode16(master, dtype), dtype)
    before = [x.clone() for x in d] + [p16.clone()]
    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(Z.zero_range_workspace_bytes(ranges) // 8 + 1, dtype=torch.float64,
                     device="cuda")
    Z.zero_reduce_check_ranges(d_g.clone(), [d_g], ranges, 1.0, res, ws)
    Z.zero_adamw_step_ranges(*d, p16, d_g, ranges,
                             Z.zero_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1), res)
    assert Z.read_result(res).overflow == 1
    for a, b in zip(d + [p16], before):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))
