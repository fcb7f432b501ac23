"""One owner-shard step captured in a HIP graph and replayed, step after step.

With the device-resident step control every per-step scalar (unscale factor,
bias corrections, the skip decision, the loss-scale update) is read or
written on the device, so one captured step serves every later step.  The
fragmented-bucket group (16 owners, 3 bucket windows, dynamic loss scaling,
inf/NaN every 4th step) runs 16 steps twice from the same start: eagerly,
and as replays of one captured graph, with the program's own eager work (the
next step's gradient generation) and a synchronisation between replays.
Every replay must equal the eager step bit for bit: reduced gradient, result,
control, master, m, v and the 16-bit copy.  (The eager device-control path
itself is checked against the oracle in test_gpu_workloads.py.)
"""
import numpy as np
import pytest
import torch

import oracle
from synth import inputs as I
from synth import workloads as W
import zero_partitioned_mixed_shard_amd as Z
from zero_partitioned_mixed_shard_amd.shard import ShardStep
from _common import to_np16

pytestmark = pytest.mark.gpu


def _shard(wl, offs, parts, padded, windows):
    owners = [(int(parts[p]), int(parts[p + 1])) for p in range(wl.world)]
    shard = ShardStep(0, padded, owners, wl.dtype, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                      eps=wl.eps, weight_decay=wl.weight_decay, max_grad_norm=wl.clip,
                      scale0=wl.scale0, min_scale=wl.min_scale, window=wl.window,
                      windows=windows, own_ranks=True, world=wl.world, device_control=True)
    shard.load_param16(I.device_param16(wl, offs, 0, padded, out=shard.param16))
    return shard


def _bits(t):
    return t.detach().view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy()


@pytest.mark.parametrize("fused", [True, False])
def test_graph_replays_equal_eager_steps(fused):
    wl = W.WORKLOADS["buckets_small"]
    offs, parts, padded = oracle.layout(wl.numels, wl.world, wl.align)
    windows = W.bucket_windows(wl, offs, padded, oracle.buckets(wl.numels, wl.bucket_cap))
    eager = _shard(wl, offs, parts, padded, windows)
    graphed = _shard(wl, offs, parts, padded, windows)
    eager.fused = graphed.fused = fused
    torch.cuda.synchronize()
    graph = graphed.capture()                    # records launches only; nothing runs yet
    torch.cuda.synchronize()
    skipped = 0
    for s in range(1, 17):
        for shard in (eager, graphed):
            shard.sync_control()
            for r, buf in enumerate(shard.rank_bufs):
                I.device_rank_grad(wl, s, shard.scale, r, 0, padded, padded, out=buf)
        eager.launch()
        graph.replay()
        torch.cuda.synchronize()
        where = f"step {s}"
        assert np.array_equal(_bits(eager.res), _bits(graphed.res)), where
        assert np.array_equal(_bits(eager.ctl), _bits(graphed.ctl)), where
        for k in ("master", "exp_avg", "exp_avg_sq", "param16"):
            assert np.array_equal(_bits(getattr(eager, k)), _bits(getattr(graphed, k))), \
                f"{where} {k}"
        assert np.array_equal(to_np16(eager.reduced()), to_np16(graphed.reduced())), where
        skipped += Z.read_result(graphed.res).overflow
    c = Z.read_control(graphed.ctl)
    assert skipped == 4 and c.skipped == 4 and c.t == 12 and c.scale == wl.scale0 / 16
