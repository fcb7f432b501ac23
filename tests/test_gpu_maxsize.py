"""Passes longer than one launch can hold.

A launch's grid holds at most 2^32 - 1 work-items (16,777,215 blocks of 256),
i.e. 34,359,736,320 elements at one 8-element lane tile per lane, or twice
that for the reduce (two lane tiles per lane).  Longer passes are issued as
several launches in order on the stream.  These tests run the check and the
fused reduce+check just past those limits and pin the results with closed
forms that hold at any size: a buffer of ones has squared norm equal to its
length (exact in fp64 below 2^53), a few planted values add known amounts,
an inf anywhere sets the flag, and an in-place one-rank reduce turns every -0
into +0 (the sum starts from +0), so every element must read back as +0.

They need 69 GB and 137 GB of device memory and are skipped when that much is
not free.
"""
import gc

import numpy as np
import pytest
import torch

import zero_partitioned_mixed_shard_amd as Z

pytestmark = pytest.mark.gpu

BF16 = Z.ZERO_BF16
GRID_BLOCKS = (1 << 32) // 256 - 1          # blocks one launch can hold
LANE_TILE = 8


def _free_gb():
    gc.collect()
    torch.cuda.empty_cache()
    return torch.cuda.mem_get_info()[0] / 1e9


def _bf16(x: float) -> torch.Tensor:
    return torch.tensor([x], dtype=torch.bfloat16, device="cuda")


def _all_zero_bits(buf: torch.Tensor, chunk: int = 1 << 30) -> bool:
    bits = buf.view(torch.int16)
    for a in range(0, bits.numel(), chunk):
        if int(torch.count_nonzero(bits[a:a + chunk])) != 0:
            return False
    return True


def test_check_past_one_launch():
    # one block per 256 lane tiles: the second launch gets 3 blocks and the
    # 13 trailing elements go to block 0's tail lanes
    count = (GRID_BLOCKS + 2) * 256 * LANE_TILE + 13
    need = count * 2 / 1e9 + 1
    if _free_gb() < need:
        pytest.skip(f"needs {need:.0f} GB of free device memory")
    print(f"check over {count} bf16 elements ({count * 2 / 1e9:.1f} GB)", flush=True)
    g = torch.ones(count, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((Z.zero_check_workspace_bytes(count) + 7) // 8, dtype=torch.float64,
                     device="cuda")
    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    try:
        Z.zero_unscale_check_norm(g, 1.0, res, ws)
        r = Z.read_result(res)
        assert r.overflow == 0 and r.sumsq == float(count)
        # planted values: first element of the second launch, the last vector
        # lane, the last (tail) element
        first2 = GRID_BLOCKS * 256 * LANE_TILE
        last_vec = (count // LANE_TILE) * LANE_TILE - 1
        g[first2:first2 + 1] = _bf16(2.0)       # +3
        g[last_vec:last_vec + 1] = _bf16(0.5)   # -0.75
        g[count - 1:count] = _bf16(3.0)         # +8
        Z.zero_unscale_check_norm(g, 1.0, res, ws)
        r = Z.read_result(res)
        assert r.overflow == 0 and r.sumsq == float(count) + 3.0 - 0.75 + 8.0
        g[count - 5:count - 4] = _bf16(float("inf"))
        Z.zero_unscale_check_norm(g, 1.0, res, ws)
        assert Z.read_result(res).overflow == 1
    finally:
        del g, ws, res
        _free_gb()


def test_reduce_check_in_place_past_one_launch():
    # the reduce takes two lane tiles per lane: past 2 x GRID_BLOCKS x 256 tiles
    count = (GRID_BLOCKS + 1) * 2 * 256 * LANE_TILE + 7
    need = count * 2 / 1e9 + 1
    if _free_gb() < need:
        pytest.skip(f"needs {need:.0f} GB of free device memory")
    print(f"in-place 1-rank reduce+check over {count} bf16 elements ({count * 2 / 1e9:.1f} GB)",
          flush=True)
    buf = torch.empty(count, dtype=torch.bfloat16, device="cuda")
    buf.view(torch.int16).fill_(-32768)                 # 0x8000: bfloat16 -0
    ws = torch.empty((Z.zero_check_workspace_bytes(count) + 7) // 8, dtype=torch.float64,
                     device="cuda")
    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    try:
        Z.zero_reduce_check_owned(buf, [buf], 1.0, res, ws)
        r = Z.read_result(res)
        assert r.overflow == 0 and r.sumsq == 0.0
        assert _all_zero_bits(buf), "some -0 was not rewritten as +0"
        first2 = GRID_BLOCKS * 2 * 256 * LANE_TILE
        for e, x in ((0, 1.0), (first2 - 1, 2.0), (first2, 4.0), (count - 8, 0.5), (count - 1, 8.0)):
            buf[e:e + 1] = _bf16(x)
        Z.zero_reduce_check_owned(buf, [buf], 1.0, res, ws)
        r = Z.read_result(res)
        assert r.overflow == 0 and r.sumsq == 1.0 + 4.0 + 16.0 + 0.25 + 64.0
        got = [float(buf[e]) for e in (0, first2 - 1, first2, count - 8, count - 1, first2 + 1)]
        assert got == [1.0, 2.0, 4.0, 0.5, 8.0, 0.0]
    finally:
        del buf, ws, res
        _free_gb()
