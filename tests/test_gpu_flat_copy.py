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


@pytest.mark.parametrize("mem_gap_max", [0, 3, 9])
def test_views_of_one_buffer(mem_gap_max):
    """Tensors that are views into one device buffer at arbitrary element
    offsets, some back to back in memory with different misalignments: the
    copy kernels share 16-byte chunks between lanes whose tiles are
    consecutive in memory, whichever tensor they belong to.  The scatter must
    write every view's elements exactly and leave the elements between views
    untouched."""
    rng = np.random.default_rng(100 + mem_gap_max)
    sizes = [int(x) for x in rng.integers(1, 3000, 300)] + [1] * 40 + [9, 17, 2049, 5000]
    rng.shuffle(sizes)
    pos, cur = [], int(rng.integers(0, 8))
    for n in sizes:
        pos.append(cur)
        cur += n + int(rng.integers(0, mem_gap_max + 1))
    backing_host = rng.integers(0, 65536, cur + 8).astype(np.uint16)
    backing = torch.from_numpy(backing_host.view(np.int16)).cuda().view(torch.bfloat16)
    dev = [backing[p:p + n] for p, n in zip(pos, sizes)]
    host = [backing_host[p:p + n].copy() for p, n in zip(pos, sizes)]
    offs, count = _layout_with_gaps(sizes, rng, 5)
    descs = Z.tensor_descs(dev, offs)
    flat = torch.full((count,), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    Z.zero_flat_gather(flat, descs)
    assert np.array_equal(to_np16(flat), oracle.flat_gather(host, offs, count))
    new_flat = rng.integers(0, 65536, count).astype(np.uint16)
    d_flat = torch.from_numpy(new_flat.view(np.int16)).cuda().view(torch.bfloat16)
    Z.zero_flat_scatter(d_flat, descs)
    back = oracle.flat_scatter(new_flat, offs, sizes)
    want = backing_host.copy()
    for p, n, w in zip(pos, sizes, back):
        want[p:p + n] = w
    assert np.array_equal(to_np16(backing), want)


def test_one_tensor_every_misalignment():
    """One tensor spanning several blocks at every flat offset 0..7 and
    memory offsets 0, 1 and 5 inside a larger buffer: the tensor side sits
    0..7 elements off the flat side's 16-byte grid, so every lane, row and
    wave edge of the copy kernels shares a misaligned chunk with the next
    tile (within a row, from lane 63 to the next row, and across waves and
    blocks).  The scatter must leave the buffer around the tensor untouched."""
    rng = np.random.default_rng(77)
    n = 3 * 8192 + 2048 + 13
    for f in range(8):
        for p in (0, 1, 5):
            backing_host = rng.integers(0, 65536, n + 24).astype(np.uint16)
            backing = torch.from_numpy(backing_host.view(np.int16)).cuda().view(torch.bfloat16)
            t = backing[p:p + n]
            count = f + n + 11
            descs = Z.tensor_descs([t], [f])
            flat = torch.full((count,), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            Z.zero_flat_gather(flat, descs)
            want = oracle.flat_gather([backing_host[p:p + n].copy()], [f], count)
            assert np.array_equal(to_np16(flat), want), (f, p)
            new_flat = rng.integers(0, 65536, count).astype(np.uint16)
            d_flat = torch.from_numpy(new_flat.view(np.int16)).cuda().view(torch.bfloat16)
            Z.zero_flat_scatter(d_flat, descs)
            want_b = backing_host.copy()
            want_b[p:p + n] = oracle.flat_scatter(new_flat, [f], [n])[0]
            assert np.array_equal(to_np16(backing), want_b), (f, p)


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



LLAMA_PER_LAYER = 9          # q, k, v, o, gate, up, down, two norm gains


def _layer_range(wl, offs, layer):
    k0 = 1 + LLAMA_PER_LAYER * layer                 # tensor 0 is the embedding
    k1 = k0 + LLAMA_PER_LAYER - 1
    return k0, k1, int(offs[k0]), int(offs[k1] + wl.numels[k1])


def _time_gather(out, descs, reps=5):
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        Z.zero_flat_gather(out, descs)
    ev[1].record()
    ev[1].synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


@pytest.mark.parametrize("ownership", ["flat_partition", "whole_tensor"])
def test_zero3_layer_gather(ownership):
    """Stage 3 keeps each parameter only with its owner and assembles a layer's
    full 16-bit parameters just before the layer runs, dropping them after
    (wmrh.cn ZeRO article, section 2.2.3; ZeRO 优化器, "ZeRO Stage 3").  On one
    GPU the owners' stores are separate allocations and the assembly is
    zero_flat_gather into one layer buffer:

    * flat_partition: owner p holds [p*P, (p+1)*P) of the flat buffer (ZeRO-2
      source walkthrough, section 2.1); a layer's range takes one descriptor per
      overlapping partition piece, cutting through tensors;
    * whole_tensor: tensor i belongs to owner i mod N, which keeps its tensors
      packed back to back (ZeRO 优化器, "ZeRO Stage 3", inter-tensor split).

    LLaMA-7B shapes, N = 8, bf16; layers 0 and 31 and two layers that straddle a
    partition boundary (3 and 16).  The gathered layer must
    equal the oracle's gather of the same pieces and the layer's parameters as
    generated directly for that flat range."""
    from synth import inputs as I
    wl = W.WORKLOADS["llama7b"]
    offs, parts, padded = oracle.layout(wl.numels, wl.world, wl.align)
    n = wl.world
    if ownership == "flat_partition":
        stores = [I.device_param16(wl, offs, int(parts[p]), int(parts[p + 1])) for p in range(n)]
    else:
        # owner p packs tensors p, p+N, ... ; where[i] = (owner, offset in its store)
        where, sizes = {}, [0] * n
        for i, m in enumerate(wl.numels):
            where[i] = (i % n, sizes[i % n])
            sizes[i % n] += int(m)
        stores = [torch.empty(sizes[p], dtype=torch.bfloat16, device="cuda") for p in range(n)]
        for i, m in enumerate(wl.numels):
            p, o = where[i]
            I.device_param16(wl, offs, int(offs[i]), int(offs[i] + m), out=stores[p][o:o + int(m)])
    biggest = max(_layer_range(wl, offs, 0)[3] - _layer_range(wl, offs, 0)[2], 1)
    layer_buf = torch.empty(biggest, dtype=torch.bfloat16, device="cuda")
    for layer in (0, 3, 16, 31):
        k0, k1, a, b = _layer_range(wl, offs, layer)
        pieces, poffs = [], []
        if ownership == "flat_partition":
            for p in range(n):
                lo, hi = max(a, int(parts[p])), min(b, int(parts[p + 1]))
                if lo < hi:
                    pieces.append(stores[p][lo - int(parts[p]):hi - int(parts[p])])
                    poffs.append(lo - a)
        else:
            for i in range(k0, k1 + 1):
                p, o = where[i]
                pieces.append(stores[p][o:o + int(wl.numels[i])])
                poffs.append(int(offs[i]) - a)
        if ownership == "flat_partition":
            assert len(pieces) == (2 if layer in (3, 16) else 1)
        descs = Z.tensor_descs(pieces, poffs)
        out = layer_buf[:b - a]
        out.fill_(float("nan"))
        Z.zero_flat_gather(out, descs)
        torch.cuda.synchronize()
        got = to_np16(out)
        want = oracle.flat_gather([to_np16(t) for t in pieces], poffs, b - a)
        assert np.array_equal(got, want), (ownership, layer)
        assert np.array_equal(got, I.host_param16(wl, offs, a, b, threads=8)), (ownership, layer)
        ms = _time_gather(out, descs)
        print(f"{ownership} layer {layer}: {b - a} elements from {len(pieces)} pieces, "
              f"{ms:.3f} ms, {4 * (b - a) / ms / 1e6:.0f} GB/s", flush=True)
