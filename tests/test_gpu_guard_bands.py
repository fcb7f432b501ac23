"""Guard bands: every device call writes only inside its buffers.

Each buffer is the interior of a larger allocation whose 4 KiB on either side
(plus the bytes a misaligned start leaves) hold a canary byte pattern; after
every call all canaries must be intact.  Ragged counts, misaligned starts
(the vector path with a head, and the element-by-element path when the
pointers disagree modulo 16 bytes), in-place reduce into a rank's own buffer,
1 to 16 ranks, copy-in / write-back with tensors in guarded buffers, and the
device step control.
"""
import numpy as np
import pytest
import torch

import zero_partitioned_mixed_shard_amd as Z

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0xA5
FP16, BF16 = Z.ZERO_FP16, Z.ZERO_BF16
_tracked = []


def guarded(n, dtype, offset=0, fill=None):
    """A device tensor of n elements at `offset` elements past a 4 KiB guard."""
    eb = torch.tensor([], dtype=dtype).element_size()
    whole = torch.full((2 * GUARD + (n + offset) * eb,), CANARY, dtype=torch.uint8, device="cuda")
    lo = GUARD + offset * eb
    inner = whole[lo:lo + n * eb].view(dtype)
    if fill is not None:
        inner.copy_(fill)
    _tracked.append((whole, lo, lo + n * eb))
    return inner


def check_guards(where):
    torch.cuda.synchronize()
    for whole, lo, hi in _tracked:
        for part in (whole[:lo], whole[hi:]):
            if part.numel():
                bad = int((part != CANARY).sum())
                assert bad == 0, f"{where}: {bad} guard bytes overwritten"


@pytest.fixture(autouse=True)
def _reset():
    _tracked.clear()
    yield
    _tracked.clear()


def _rand16(n, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = (torch.randn(n, generator=g) * 1e-2).to(torch.float16 if dtype == FP16 else torch.bfloat16)
    return x.cuda()


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("count", [1, 7, 4097, 100_003, 1_000_003])
@pytest.mark.parametrize("offsets", [(0, 0), (3, 3), (1, 4)])
def test_check_paths_stay_inside(dtype, count, offsets):
    tdt = torch.float16 if dtype == FP16 else torch.bfloat16
    o_src, o_dst = offsets
    for n_ranks in (1, 3, 8, 16):
        srcs = [guarded(count, tdt, o_src, _rand16(count, dtype, r)) for r in range(n_ranks)]
        dst = guarded(count, tdt, o_dst)
        Z.zero_reduce_owned(dst, srcs)
        check_guards(f"reduce N={n_ranks}")
        res = guarded(4, torch.int32)
        ws = guarded((Z.zero_check_workspace_bytes(count) + 7) // 8, torch.float64)
        Z.zero_reduce_check_owned(dst, srcs, 2.0 ** -8, res, ws)
        check_guards(f"fused N={n_ranks}")
        Z.zero_reduce_check_owned(srcs[0], srcs, 2.0 ** -8, res, ws)      # in place
        check_guards(f"fused in place N={n_ranks}")
        Z.zero_unscale_check_norm(dst, 1.0, res, ws, accumulate=True)
        check_guards("check")
        _tracked.clear()


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("count", [1, 9, 2049, 300_001])
@pytest.mark.parametrize("offsets", [(0, 0, 0), (1, 2, 2), (3, 1, 5)])
def test_adamw_and_control_stay_inside(dtype, count, offsets):
    tdt = torch.float16 if dtype == FP16 else torch.bfloat16
    o32, o16, og = offsets
    p16 = guarded(count, tdt, o16, _rand16(count, dtype, 7))
    master = guarded(count, torch.float32, o32)
    m = guarded(count, torch.float32, o32, torch.zeros(count))
    v = guarded(count, torch.float32, o32, torch.zeros(count))
    g16 = guarded(count, tdt, og, _rand16(count, dtype, 8))
    Z.zero_init_master(master, p16)
    check_guards("init_master")
    res = guarded(4, torch.int32)
    ws = guarded((Z.zero_check_workspace_bytes(count) + 7) // 8, torch.float64)
    Z.zero_unscale_check_norm(g16, 1.0, res, ws)
    hp = Z.zero_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    Z.zero_adamw_step(master, m, v, p16, g16, hp, res)
    check_guards("adamw")
    ctl = guarded(Z.CONTROL_BYTES, torch.uint8)
    Z.control_to_device(Z.zero_step_control_init(1024.0, 1.0, 3, 1.0, 0.9, 0.999), out=ctl)
    Z.zero_unscale_check_norm_ctl(g16, ctl, res, ws)
    Z.zero_adamw_step_ctl(master, m, v, p16, g16, hp, ctl, res)
    Z.zero_step_control_update(ctl, res)
    check_guards("device step control")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_flat_copies_stay_inside(seed):
    rng = np.random.default_rng(seed)
    sizes = [int(x) for x in rng.integers(1, 5000, 60)] + [1, 2, 3, 8, 9]
    tensors = [guarded(n, torch.bfloat16, int(rng.integers(0, 8)), _rand16(n, BF16, k))
               for k, n in enumerate(sizes)]
    offs, cur = [], int(rng.integers(0, 9))
    for n in sizes:
        offs.append(cur)
        cur += n + int(rng.integers(0, 5))
    count = cur + 3
    flat = guarded(count, torch.bfloat16, int(rng.integers(0, 8)))
    descs = Z.tensor_descs(tensors, offs)
    Z.zero_flat_gather(flat, descs)
    check_guards("gather")
    Z.zero_flat_scatter(flat, descs)
    check_guards("scatter")
    for t, o in zip(tensors, offs):                 # the round trip is the identity
        assert torch.equal(t.view(torch.int16), flat[o:o + t.numel()].view(torch.int16))
