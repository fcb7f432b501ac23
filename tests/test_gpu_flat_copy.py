"""Bucket copy-in (zero_flat_gather) and write-back (zero_flat_scatter) on the
GPU against the oracle, bit for bit.

Ragged tensors (0, 1, 2, 3 ... 2049, 70001 elements), runs of 1-element
tensors that put dozens of tensor boundaries inside one 2048-element block,
gaps between tensors and a padded tail (zero-filled on gather), flat sizes
that are not multiples of the block size, an empty table; then the
10,000-tensor fragmented group copied into its three 5e8-element reduce
buckets (ZeRO-2 source walkthrough sections 2.4 and 4.2) and written back.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W
import zero_partitioned_mixed_shard_amd as Z
from _common import to_np16

pytestmark = pytest.mark.gpu


def _rand_tensors(sizes, rng):
    host = [rng.integers(0, 65536, n).astype(np.uint16) for n in sizes]
    dev = [torch.from_numpy(h.view(np.int16)).cuda().view(torch.bfloat16) for h in host]
    return host, dev


def _layout_with_gaps(sizes, rng, gap_max):
    offs, cur = [], int(rng.integers(0, gap_max + 1))
    for n in sizes:
        offs.append(cur)
        cur += n + int(rng.integers(0, gap_max + 1))
    return offs, cur + int(rng.integers(0, 3000))


@pytest.mark.parametrize("case", ["ragged", "tiny_runs", "no_gaps", "empty_table", "one_big"])
def test_gather_scatter_parity(case):
    rng = np.random.default_rng(hash(case) % 1000)
    if case == "ragged":
        sizes = [0, 1, 2, 3, 7, 8, 9, 64, 1000, 2047, 2048, 2049, 4095, 70001, 5, 0, 333]
        gap = 40
    elif case == "tiny_runs":
        sizes = [1] * 700 + [3] * 300 + [2] * 500 + [17, 1, 1, 4099]
        gap = 2
    elif case == "no_gaps":
        sizes = list(rng.integers(1, 5000, 300))
        gap = 0
    elif case == "empty_table":
        sizes = []
        gap = 0
    else:
        sizes = [3_000_001]
        gap = 9
    host, dev = _rand_tensors(sizes, rng)
    offs, count = _layout_with_gaps(sizes, rng, gap)
    count = max(count, 1)
    descs = Z.tensor_descs(dev, offs)
    flat = torch.full((count,), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    Z.zero_flat_gather(flat, descs)
    want = oracle.flat_gather(host, offs, count)
    assert np.array_equal(to_np16(flat), want)
    # write-back: a fresh flat buffer scattered into zeroed tensors
    new_flat = rng.integers(0, 65536, count).astype(np.uint16)
    d_flat = torch.from_numpy(new_flat.view(np.int16)).cuda().view(torch.bfloat16)
    for t in dev:
        t.zero_()
    Z.zero_flat_scatter(d_flat, descs)
    back = oracle.flat_scatter(new_flat, offs, sizes)
    for t, w in zip(dev, back):
        assert np.array_equal(to_np16(t), w)


def test_invalid_arguments():
    flat = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    L = Z.lib()
    assert L.zero_flat_gather(flat.data_ptr(), -1, None, 0, None) == Z.ZERO_EINVAL
    assert L.zero_flat_gather(flat.data_ptr(), 16, None, 3, None) == Z.ZERO_EINVAL
    assert L.zero_flat_gather(None, 16, None, 0, None) == Z.ZERO_EINVAL
    assert L.zero_flat_scatter(flat.data_ptr(), 16, None, -2, None) == Z.ZERO_EINVAL


def test_fragmented_group_into_buckets_and_back():
    """The 10,000-tensor group: every tensor its own allocation, gathered
    into the three reduce buckets (one call per bucket, the last bucket taking
    the alignment padding), compared with the oracle element by element, then
    written back from the flat buffer into the tensors."""
    wl = W.WORKLOADS["buckets"]
    offs, parts, padded = oracle.layout(wl.numels, wl.world, wl.align)
    first = oracle.buckets(wl.numels, wl.bucket_cap)
    windows = W.bucket_windows(wl, offs, padded, first)
    spec = wl.grad_spec(wl.scale0)
    key = wl.grad_key(1, 0)
    host = np.empty(padded, np.uint16)
    synth.fill_host(host[:wl.phi], 0, key, spec, threads=16)
    host[wl.phi:] = 0
    tensors = [torch.from_numpy(host[o:o + n].view(np.int16)).cuda().view(torch.float16)
               for o, n in zip(offs, wl.numels)]
    flat = torch.full((padded,), 1, dtype=torch.int16, device="cuda").view(torch.float16)
    for b, (a, z) in enumerate(windows):
        ks = range(int(first[b]), int(first[b + 1]))
        descs = Z.tensor_descs([tensors[k] for k in ks], [int(offs[k]) - a for k in ks])
        Z.zero_flat_gather(flat[a:z], descs)
    # the oracle's gather of the same per-tensor data
    want = oracle.flat_gather([host[o:o + n] for o, n in zip(offs, wl.numels)], offs, padded)
    assert np.array_equal(to_np16(flat), want)
    # write-back into the tensors from a different flat buffer
    flat2 = torch.flip(flat, [0]).contiguous()
    descs = Z.tensor_descs(tensors, offs)
    Z.zero_flat_scatter(flat2, descs)
    f2 = to_np16(flat2)
    back = oracle.flat_scatter(f2, offs, wl.numels)
    for k in np.random.default_rng(1).choice(len(tensors), 300, replace=False):
        assert np.array_equal(to_np16(tensors[k]), back[k])
    got = np.concatenate([to_np16(t) for t in tensors])
    assert np.array_equal(got, np.concatenate(back))
