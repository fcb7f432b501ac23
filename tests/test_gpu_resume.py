"""Checkpoint and resume of the owner-shard step state.

The state is {master, m, v, the 16-bit copy, t, loss scale, clean-step count,
skipped count} (with the device step control: the zero_step_control block).
A run of the fragmented-bucket group (16 owners, dynamic loss scaling, an
inf/NaN every 4th step) is saved to host memory after step 9, restored into a
freshly built step and continued to step 20; every later step must equal the
uninterrupted run bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import inputs as I
from synth import workloads as W
import zero_partitioned_mixed_shard_amd as Z
from zero_partitioned_mixed_shard_amd.shard import ShardStep

pytestmark = pytest.mark.gpu

STATE = ("master", "exp_avg", "exp_avg_sq", "param16")


def _build(wl, offs, parts, padded, windows, device_control):
    owners = [(int(parts[p]), int(parts[p + 1])) for p in range(wl.world)]
    shard = ShardStep(0, padded, owners, wl.dtype, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                      eps=wl.eps, weight_decay=wl.weight_decay, max_grad_norm=wl.clip,
                      scale0=wl.scale0, min_scale=wl.min_scale, window=wl.window,
                      windows=windows, own_ranks=True, world=wl.world,
                      device_control=device_control)
    shard.load_param16(I.device_param16(wl, offs, 0, padded, out=shard.param16))
    return shard


def _step(shard, wl, s, padded):
    for r, buf in enumerate(shard.rank_bufs):
        I.device_rank_grad(wl, s, shard.scale, r, 0, padded, padded, out=buf)
    return shard.step()


def save(shard):
    ck = {k: getattr(shard, k).detach().cpu().clone() for k in STATE}
    if shard.ctl is not None:
        ck["ctl"] = shard.ctl.detach().cpu().clone()
    ck["host"] = (shard.t, shard.scaler.scale, shard.scaler.clean, shard.scaler.skipped)
    return ck


def restore(shard, ck):
    for k in STATE:
        getattr(shard, k).copy_(ck[k])
    if shard.ctl is not None:
        shard.ctl.copy_(ck["ctl"])
    shard.t, shard.scaler.scale, shard.scaler.clean, shard.scaler.skipped = ck["host"]


@pytest.mark.parametrize("device_control", [False, True])
def test_resume_continues_bit_for_bit(device_control):
    wl = W.WORKLOADS["buckets_small"]
    offs, parts, padded = oracle.layout(wl.numels, wl.world, wl.align)
    windows = W.bucket_windows(wl, offs, padded, oracle.buckets(wl.numels, wl.bucket_cap))
    ref = _build(wl, offs, parts, padded, windows, device_control)
    run = _build(wl, offs, parts, padded, windows, device_control)
    for s in range(1, 10):
        _step(ref, wl, s, padded)
        _step(run, wl, s, padded)
    ck = save(run)
    del run
    torch.cuda.empty_cache()
    resumed = _build(wl, offs, parts, padded, windows, device_control)
    restore(resumed, ck)
    for s in range(10, 21):
        a = _step(ref, wl, s, padded)
        b = _step(resumed, wl, s, padded)
        assert (a.overflow, a.applied, a.t, a.scale_used) == (b.overflow, b.applied, b.t,
                                                              b.scale_used), s
        assert torch.equal(ref.res, resumed.res), s          # result bits, NaN norm included
        for k in STATE:
            x, y = getattr(ref, k), getattr(resumed, k)
            assert torch.equal(x.view(torch.int16 if x.element_size() == 2 else torch.int32),
                               y.view(torch.int16 if y.element_size() == 2 else torch.int32)), \
                f"step {s} {k}"
    assert ref.scaler.skipped == resumed.scaler.skipped == 5 and ref.t == resumed.t == 15
