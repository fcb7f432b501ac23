"""Pins for the oracle's layout, bucketing and memory closed forms (not GPU).

* Brute force on tiny groups: every composition of Phi <= 10 elements into at
  most four tensors, every N in 1..10, alignment 1, 2 and 8.  The partitions
  must be equal, contiguous, cover the padded buffer exactly once and the real
  elements [0, Phi) exactly once (ZeRO-2 source walkthrough, sections 2.1 and
  4.1: flatten, align, split into as many near-equal partitions as ranks).
* Bucket copy-in / write-back (ZeRO-2 source walkthrough, sections 2.4, 4.2
  and 4.4): a worked example by hand, then invariants on random tables --
  write-back of a copy-in returns every tensor, elements no tensor covers
  are 0 even in a buffer that held other bits, and the copy-in of the
  write-back of a buffer keeps exactly the covered elements.
* The pages' memory formulas and worked examples (tests/golden/pages_values.json).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def _compositions(total, parts):
    if parts == 1:
        yield (total,)
        return
    for first in range(total + 1):
        for rest in _compositions(total - first, parts - 1):
            yield (first,) + rest


def test_layout_brute_force_tiny():
    cases = 0
    for phi in range(0, 11):
        for nt in range(1, 5):
            for numels in _compositions(phi, nt):
                for world in range(1, 11):
                    for align in (1, 2, 8):
                        offs, parts, padded = oracle.layout(numels, world, align)
                        # offsets are the running sums: tensors sit back to back
                        assert list(offs) == [sum(numels[:k]) for k in range(nt)]
                        # padding: smallest multiple of N*A that holds Phi
                        assert padded % (world * align) == 0
                        assert 0 <= padded - phi < world * align
                        # N equal contiguous partitions covering [0, padded)
                        assert parts[0] == 0 and parts[-1] == padded
                        sizes = np.diff(parts)
                        assert (sizes == padded // world).all()
                        assert sizes[0] % align == 0
                        # every index lies in exactly one partition
                        owner = np.full(padded, -1)
                        for p in range(world):
                            assert (owner[parts[p]:parts[p + 1]] == -1).all()
                            owner[parts[p]:parts[p + 1]] = p
                        assert (owner >= 0).all()
                        # every real element of every tensor has exactly one owner
                        for k in range(nt):
                            for i in range(offs[k], offs[k] + numels[k]):
                                assert 0 <= owner[i] < world
                        cases += 1
    assert cases > 20000


def test_layout_errors():
    with pytest.raises(ValueError):
        oracle.layout([4, 4], 0, 2)
    with pytest.raises(ValueError):
        oracle.layout([4, 4], 2, 0)
    with pytest.raises(ValueError):
        oracle.layout([4, -1], 2, 2)
    with pytest.raises(ValueError):  # sum overflows int64
        oracle.layout([2 ** 62, 2 ** 62, 2 ** 62], 2, 2)


@pytest.mark.parametrize("name,phi,part", [
    ("toy", 100_734_986, 12_591_874),
    ("bert", 109_482_240, 13_685_280),
    ("llama7b", 6_738_415_616, 842_301_952),
    ("llama70b", 68_976_648_192, 8_622_081_024),
    ("buckets", 1_084_742_524, 67_796_408),
])
def test_workload_layouts(name, phi, part):
    wl = W.WORKLOADS[name]
    assert wl.phi == phi
    offs, parts, padded = oracle.layout(wl.numels, wl.world, wl.align)
    assert parts[1] - parts[0] == part
    assert padded == part * wl.world
    assert padded - phi < wl.world * wl.align


def test_workload_shapes():
    # ToyModel of the wmrh.cn article, section 3.1 (hidden 1024, 12 layers, 10 classes)
    assert len(W.WORKLOADS["toy"].tensors) == 50
    assert len(W.WORKLOADS["bert"].tensors) == 199
    assert len(W.WORKLOADS["llama7b"].tensors) == 291
    assert len(W.WORKLOADS["llama70b"].tensors) == 723
    b = W.WORKLOADS["buckets"]
    sizes = b.numels
    assert sizes.size == 10_000 and sizes.min() >= 64 and sizes.max() <= 1 << 20
    # log-uniform: log2 of the sizes is roughly uniform on [6, 20]
    h, _ = np.histogram(np.log2(sizes), bins=7, range=(6, 20))
    assert h.min() > 0.8 * 10_000 / 7 and h.max() < 1.2 * 10_000 / 7


def test_buckets_brute_force():
    rng = np.random.default_rng(11)
    for trial in range(300):
        n = int(rng.integers(1, 12))
        numels = rng.integers(0, 20, n)
        cap = int(rng.integers(1, 40))
        first = oracle.buckets(numels, cap)
        assert first[0] == 0 and first[-1] == n
        assert (np.diff(first) > 0).all()
        for b in range(first.size - 1):
            lo, hi = first[b], first[b + 1]
            fill = int(numels[lo:hi].sum())
            # a bucket exceeds the cap only if it holds one non-empty tensor
            assert fill <= cap or int((numels[lo:hi] > 0).sum()) == 1
            # greedy: the next tensor would not have fitted
            if hi < n and fill > 0:
                assert fill + numels[hi] > cap
    # the fragmented workload at the pages' bucket size
    b = W.WORKLOADS["buckets"]
    cap = GOLDEN["reduce_bucket_size"]["value"]
    first = oracle.buckets(b.numels, cap)
    fills = [int(b.numels[first[k]:first[k + 1]].sum()) for k in range(first.size - 1)]
    assert len(fills) == 3 and max(fills) <= cap


# ------------------------------------------------------ copy-in / write-back
def test_flat_copy_worked_example():
    # tensors [1 2 3] at offset 1 and [4] at offset 5 of a 7-element buffer
    t0 = np.array([1, 2, 3], np.uint16)
    t1 = np.array([4], np.uint16)
    poisoned = np.full(7, 0xFFFF, np.uint16)
    flat = oracle.flat_gather([t0, t1], [1, 5], 7, out=poisoned)
    assert flat.tolist() == [0, 1, 2, 3, 0, 4, 0]
    back = oracle.flat_scatter(np.array([9, 8, 7, 6, 5, 4, 3], np.uint16), [1, 5], [3, 1])
    assert [b.tolist() for b in back] == [[8, 7, 6], [4]]
    assert oracle.flat_gather([], [], 3, out=np.full(3, 7, np.uint16)).tolist() == [0, 0, 0]


def test_flat_copy_invariants():
    rng = np.random.default_rng(17)
    for trial in range(200):
        n = int(rng.integers(0, 9))
        sizes = rng.integers(0, 13, n)
        offs, cur = [], int(rng.integers(0, 4))
        for m in sizes:                                   # sorted, gaps of 0..3
            offs.append(cur)
            cur += int(m) + int(rng.integers(0, 4))
        count = cur + int(rng.integers(0, 4))
        ts = [rng.integers(1, 65536, int(m)).astype(np.uint16) for m in sizes]
        covered = np.zeros(count, bool)
        for o, m in zip(offs, sizes):
            covered[o:o + m] = True
        flat = oracle.flat_gather(ts, offs, count,
                                  out=rng.integers(1, 65536, count).astype(np.uint16))
        assert (flat[~covered] == 0).all()
        for t, b in zip(ts, oracle.flat_scatter(flat, offs, sizes)):
            assert np.array_equal(t, b)
        src = rng.integers(0, 65536, count).astype(np.uint16)
        again = oracle.flat_gather(oracle.flat_scatter(src, offs, sizes), offs, count)
        assert np.array_equal(again, np.where(covered, src, 0))


# ---------------------------------------------------------------- memory
def test_memory_closed_forms_match_pages():
    coef = GOLDEN["stage_memory_coefficients"]["value"]
    for phi in (16, 1_000_000, 110_000_000, 6_738_415_616):
        for world in (1, 2, 4, 8, 16):
            if phi % world:
                continue
            for stage in range(4):
                a, b = coef[str(stage)]
                assert oracle.memory_bytes(stage, phi, world) == a * phi + Fraction(b * phi, world)
    per = GOLDEN["bytes_per_param"]["value"]
    assert oracle.memory_bytes(0, 1, 1) == per["total"]
    assert per["param16"] + per["grad16"] + per["master32"] + per["exp_avg"] + per["exp_avg_sq"] \
        == per["total"]
    opt = per["master32"] + per["exp_avg"] + per["exp_avg_sq"]
    assert Fraction(opt, per["total"]) == Fraction(per["optimizer_share"]).limit_denominator()


def test_memory_worked_examples():
    # optimizer memory saving: 1 - 1/N (75% at N=4, 87.5% at N=8)
    for key in ("optimizer_saving_n4", "optimizer_saving_n8"):
        g = GOLDEN[key]["value"]
        phi = 1_000_000
        full = oracle.memory_bytes(0, phi, g["world"]) - oracle.memory_bytes(1, phi, g["world"])
        # stage 1 keeps 12*Phi/N of the 12*Phi optimizer bytes
        assert full / (12 * phi) == Fraction(g["saving"]).limit_denominator()
    # BERT-base: 2-byte params and grads, 4-byte m and v
    g = GOLDEN["bert_base_bytes"]["value"]
    phi = g["params"]
    assert 2 * phi == g["param16_MB"] * 10 ** 6
    assert 2 * phi == g["grad16_MB"] * 10 ** 6
    assert 8 * phi == g["exp_avg_plus_sq_MB"] * 10 ** 6
    # 70B parameters on 8 ranks under stage 3: 140 GB -> 17.5 GB of 16-bit params
    g = GOLDEN["llama70b_param_bytes"]["value"]
    phi, n = g["params"], g["world"]
    assert 2 * phi == g["full_GB"] * 10 ** 9
    # going from stage 2 to stage 3 shards exactly the 16-bit parameters
    saved = oracle.memory_bytes(2, phi, n) - oracle.memory_bytes(3, phi, n)
    assert 2 * phi - saved == Fraction(g["per_rank_GB"]).limit_denominator() * 10 ** 9


def test_memory_with_padding_equals_closed_form_when_divisible():
    for name in ("bert", "llama7b", "llama70b"):
        wl = W.WORKLOADS[name]
        _, _, padded = oracle.layout(wl.numels, wl.world, wl.align)
        assert padded == wl.phi
        for stage in range(4):
            assert oracle.memory_bytes(stage, wl.phi, wl.world, padded) == \
                oracle.memory_bytes(stage, wl.phi, wl.world)
    wl = W.WORKLOADS["toy"]  # pads 6 elements: the sharded parts hold P each
    _, parts, padded = oracle.layout(wl.numels, wl.world, wl.align)
    assert oracle.memory_bytes(3, wl.phi, wl.world, padded) == 16 * int(parts[1])
