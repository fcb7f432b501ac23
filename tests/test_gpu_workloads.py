"""End-to-end owner-shard steps on the GPU against the oracle, every element,
every step: the ToyModel flat buffer (10 steps), the BERT-base-shaped buffer
(20 steps, clip 1.0) and a fragmented-bucket buffer with all 16 owners,
bucket windows, dynamic loss scaling and an inf/NaN every 4th step (40 steps).

Per step: the reduced gradient bit-exact, the overflow flag and the skip
decision bit-exact, the norm within 1e-5 relative, the fp32 master / m / v
bit-equal or within 2e-6 relative, the 16-bit copy within 1 ulp, and the loss
scale and step count equal.  Inputs are regenerated on each side from the
same seeded generator.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import inputs as I
from synth import workloads as W
import zero_partitioned_mixed_shard_amd as Z
from zero_partitioned_mixed_shard_amd.shard import ARENA_ORDERS, ShardStep
from _common import (REL_TOL_NORM, assert_bits16_equal, assert_f32_close, assert_p16_close,
                     to_np16, to_np32)

pytestmark = pytest.mark.gpu


def round_robin_ranges(wl, offs, owner):
    """Tensors i with i mod N == owner, whole (ZeRO 优化器, "参数分配策略")."""
    return [(int(offs[i]), int(offs[i]) + int(n)) for i, n in enumerate(wl.numels)
            if i % wl.world == owner and n > 0]


def _setup(wl, owner_ids, round_robin=False):
    offs, parts, padded = oracle.layout(wl.numels, wl.world, wl.align)
    d_offs, d_parts, d_padded = Z.zero_partition_layout(wl.numels, wl.world, wl.align)
    assert np.array_equal(offs, d_offs) and np.array_equal(parts, d_parts) and padded == d_padded
    if round_robin:
        owners = [r for p in owner_ids for r in round_robin_ranges(wl, offs, p)]
        owners.sort()
        return offs, padded, owners, 0, wl.phi, None
    owners = [(int(parts[p]), int(parts[p + 1])) for p in owner_ids]
    begin, end = owners[0][0], owners[-1][1]
    windows = None
    if wl.bucket_cap:
        first = oracle.buckets(wl.numels, wl.bucket_cap)
        assert np.array_equal(first, Z.zero_bucket_layout(wl.numels, wl.bucket_cap))
        windows = W.bucket_windows(wl, offs, padded, first)
    return offs, padded, owners, begin, end, windows


def run_parity(name, owner_ids, steps=None, threads=4, fused=True, round_robin=False,
               device_control=False, placement=None, in_place_rank=None, arena_slack=0,
               batched=True, rank_layout="flat", bucket_cap=None):
    """placement: None for separate rank buffers handed to each step, else
    the arena order of a step that holds its own rank data.  rank_layout
    "bucket": the step holds its own rank data, each reduce window's N slices
    back to back (reduce windows from the workload's buckets, or from
    bucket_cap)."""
    wl = W.WORKLOADS[name]
    if bucket_cap is not None:
        wl = dataclasses.replace(wl, bucket_cap=bucket_cap)
    steps = wl.steps if steps is None else steps
    offs, padded, owners, begin, end, windows = _setup(wl, owner_ids, round_robin)
    bucket = rank_layout == "bucket"
    arena = placement is not None
    shard = ShardStep(begin, end, owners, wl.dtype, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                      eps=wl.eps, weight_decay=wl.weight_decay, max_grad_norm=wl.clip,
                      scale0=wl.scale0, min_scale=wl.min_scale, window=wl.window, windows=windows,
                      fused=fused, device_control=device_control, own_ranks=arena or bucket,
                      world=wl.world if arena or bucket else 0, arena=arena,
                      placement=placement or "interleaved", in_place_rank=in_place_rank,
                      arena_slack=arena_slack, batched=batched, rank_layout=rank_layout)
    # initial state: device generator on the GPU, host generator for the oracle
    d_p16 = I.device_param16(wl, offs, begin, end)
    h_p16 = I.host_param16(wl, offs, begin, end, threads)
    assert np.array_equal(to_np16(d_p16), h_p16)
    shard.load_param16(d_p16)
    states = [oracle.OwnerState.from_param16(h_p16[a - begin:b - begin], wl.dtype)
              for a, b in owners]
    scaler = oracle.Scaler(wl.scale0, wl.min_scale, wl.window)
    t = 0
    if bucket:
        rank_bufs = None
    else:
        rank_bufs = shard.rank_bufs if arena else \
            [torch.empty(end - begin, dtype=shard.tdtype, device="cuda") for _ in range(wl.world)]
    skipped = 0
    for s in range(1, steps + 1):
        assert shard.scale == scaler.scale
        if bucket:
            shard.fill_ranks(lambda r, a, b, out: I.device_rank_grad(
                wl, s, scaler.scale, r, begin + a, begin + b, padded, out=out))
        else:
            for r in range(wl.world):
                I.device_rank_grad(wl, s, scaler.scale, r, begin, end, padded, out=rank_bufs[r])
        info = shard.step(rank_bufs)
        host = I.host_rank_grads(wl, s, scaler.scale, begin, end, padded, threads)
        per_owner = [[g[a - begin:b - begin] for g in host] for a, b in owners]
        res, t = oracle.step(states, per_owner, wl.dtype, oracle.HParams(
            wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, wl.clip), scaler, t)
        where = f"{name} step {s}"
        assert info.overflow == res.overflow, where
        assert info.applied == res.applied and info.t == t, where
        skipped += not res.applied
        if not res.overflow:
            assert np.sqrt(info.sumsq) == pytest.approx(np.sqrt(res.sumsq), rel=REL_TOL_NORM), where
        sel = np.concatenate([np.arange(a - begin, b - begin) for a, b in owners])
        red = to_np16(shard.reduced(rank_bufs))[sel]
        assert_bits16_equal(red, np.concatenate(res.reduced), wl.dtype, where + " reduce")
        want = {k: np.concatenate([getattr(st, k) for st in states])
                for k in ("master", "exp_avg", "exp_avg_sq", "param16")}
        ulps = [assert_f32_close(to_np32(shard.master)[sel], want["master"], where + " master"),
                assert_f32_close(to_np32(shard.exp_avg)[sel], want["exp_avg"],
                                 where + " exp_avg"),
                assert_f32_close(to_np32(shard.exp_avg_sq)[sel], want["exp_avg_sq"],
                                 where + " exp_avg_sq")]
        assert_p16_close(to_np16(shard.param16)[sel], want["param16"], wl.dtype,
                         where + " param16")
        print(f"{where}: overflow={info.overflow} norm={np.sqrt(info.sumsq):.6g} "
              f"max-ulp(master,m,v)={ulps}", flush=True)
    assert shard.scale == scaler.scale and shard.scaler.skipped == scaler.skipped == skipped
    return shard, scaler, skipped, t


def test_toy_owner0_all_steps():
    run_parity("toy", [0])


def test_toy_last_owner_with_padding():
    # the last partition holds the 6 padding elements of the ToyModel layout
    run_parity("toy", [7], steps=3)


def test_bert_owner0_all_steps_clip():
    run_parity("bert", [0])


def _fp32_inexact_fraction(wl, step, scale, begin, n):
    """Fraction of the first n columns whose rank-order fp32 sum differs from
    the exact sum (the reduce's rounding then matters)."""
    _, _, padded = oracle.layout(wl.numels, wl.world, wl.align)
    host = I.host_rank_grads(wl, step, scale, begin, begin + n, padded)
    vals = [oracle.decode16(g, wl.dtype).astype(np.float64) for g in host]
    acc = np.zeros(n, np.float32)
    for v in vals:
        acc = (acc + v.astype(np.float32)).astype(np.float32)
    exact = np.sum(vals, axis=0)            # exact: binary16 values, 8 ranks, 32 binades
    return float(np.mean(acc.astype(np.float64) != exact))


def test_toy_offgrid_owner0_rank_order_rounding():
    """The ranks' gradients on grids 3 binades apart (rank 7's values 2^-21
    times rank 0's): most fp32 sums of the reduce round, so the rank order
    and the fp32 reading of the reduce are exercised on every element of a
    whole workload run, whose results still match the oracle's bit for bit
    (reduced gradient) and to the usual tolerances."""
    wl = W.WORKLOADS["toy_offgrid"]
    assert _fp32_inexact_fraction(wl, 1, wl.scale0, 0, 1 << 16) > 0.5
    run_parity("toy_offgrid", [0])


@pytest.mark.parametrize("name,owners,cap,placement", [
    ("toy", [0], 3_000_000, None), ("toy", [0], 3_000_000, "spread"),
    ("toy_offgrid", [2], 5_000_000, "spread"),
    ("buckets_small", list(range(16)), None, "spread")])
def test_bucket_rank_layout(name, owners, cap, placement):
    """The ranks' gradients held bucket by bucket (each reduce window's N
    slices back to back) and reduced with one zero_reduce_check_buckets call:
    tensor-aligned buckets of the ToyModel (8 ranks, the LDS-staged reduce)
    and the fragmented 400-tensor group with all 16 owners and inf/NaN steps,
    in separate allocations and in the spread arena."""
    run_parity(name, owners, steps=4, placement=placement, rank_layout="bucket", bucket_cap=cap,
               device_control=name == "buckets_small")


@pytest.mark.parametrize("name,owner,batched", [("toy", 0, True), ("toy", 5, True),
                                                ("bert", 3, True), ("bert", 3, False)])
def test_round_robin_ownership(name, owner, batched):
    """Whole tensors i with i mod N == owner (ZeRO 优化器, "参数分配策略"):
    every owned tensor is its own reduce window and AdamW range -- one
    range-list call each (batched), or one reduce+check call per tensor,
    accumulated into one norm, and one AdamW call per tensor."""
    run_parity(name, [owner], steps=4, round_robin=True, batched=batched)


def test_round_robin_all_owners_equals_flat_union():
    """Every owner under round-robin ownership together updates every tensor
    exactly once: the same result as all owners of the flat layout."""
    run_parity("toy_tiny", list(range(8)), steps=3, round_robin=True)


@pytest.mark.parametrize("placement", sorted(ARENA_ORDERS) + ["auto"])
@pytest.mark.parametrize("in_place_rank", [None, 0, 5])
def test_arena_orders_parity(placement, in_place_rank):
    """The step holds its rank buffers in one arena, in every buffer order
    and with the order measured at construction: the results do not depend
    on where the buffers sit (in place: the reduced gradient overwrites that
    rank's buffer).  The small ToyModel for the fixed orders, the full one's
    partition 2 for the measured order."""
    name = "toy" if placement == "auto" else "toy_tiny"
    shard, _, _, _ = run_parity(name, [2], steps=3, placement=placement,
                                in_place_rank=in_place_rank)
    assert shard.placement in ARENA_ORDERS
    if placement == "auto":
        assert set(shard.placement_ms) == set(ARENA_ORDERS)
        fin = shard.placement_finalists_ms
        assert len(fin) == min(6, len(ARENA_ORDERS)) and set(fin) <= set(shard.placement_ms)
        assert shard.placement == min(fin, key=fin.get)
    else:
        assert shard.placement == placement and not shard.placement_ms


def test_arena_slack_parity():
    """With slack every order is also tried shifted to the arena's end; the
    chosen one (either) gives the oracle's results."""
    shard, _, _, _ = run_parity("toy", [1], steps=3, placement="auto", in_place_rank=3,
                                arena_slack=1 << 30)
    assert shard.arena_slack == 1 << 30
    assert len(shard.placement_ms) == 2 * len(ARENA_ORDERS)
    assert shard.placement in shard.placement_ms
    assert shard.arena.numel() >= shard.arena_slack + 4 * shard.count


def test_arena_auto_buckets_all_owners():
    """Measured placement with 16 owners, bucket windows and an overflow
    every 4th step."""
    shard, scaler, skipped, t = run_parity("buckets_small", list(range(16)), steps=8,
                                           placement="auto")
    assert skipped == 2 and t == 6


@pytest.mark.parametrize("fused,batched", [(True, True), (True, False), (False, True)])
def test_buckets_small_all_owners_dynamic_scaling(fused, batched):
    """Fused and batched: one range-list reduce+check call over all
    bucket-x-owner windows and one range-list AdamW over all owners.  Fused,
    not batched: one reduce+check call per window, accumulated, and one AdamW
    per owner.  Unfused: reduce per window, then check per owner."""
    shard, scaler, skipped, t = run_parity("buckets_small", list(range(16)), fused=fused,
                                           batched=batched)
    # ten inf/NaN injections in 40 steps: ten halvings of 2^16, t = 30
    assert skipped == 10 and t == 30 and scaler.scale == 64.0


@pytest.mark.parametrize("name,owners,fused", [("buckets_small", list(range(16)), True),
                                               ("buckets_small", list(range(16)), False),
                                               ("bert", [0], True)])
def test_device_step_control(name, owners, fused):
    """The loss scaler and the step count on the device (zero_step_control):
    the *_ctl calls read the unscale factor, betas and bias corrections there
    and zero_step_control_update advances them; every step matches the oracle
    as the host-driven step does (scale, skips and t read back from the
    device)."""
    shard, scaler, skipped, t = run_parity(name, owners, fused=fused, device_control=True)
    if name == "buckets_small":
        assert skipped == 10 and t == 30 and scaler.scale == 64.0
    c = Z.read_control(shard.ctl)
    assert (c.scale, c.skipped, c.t) == (scaler.scale, scaler.skipped, t)

