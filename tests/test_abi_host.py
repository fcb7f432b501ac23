"""The C-ABI library on the CPU (no GPU calls): it loads, exports every
function include/zero_shard.h declares, and its host-side logic (layout,
bucket windows, memory bytes, loss scaler) agrees with the oracle exactly."""
import os
import re

import numpy as np
import pytest

import oracle
from synth import workloads as W
import zero_partitioned_mixed_shard_amd as Z

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "zero_shard.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    lib = Z.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(Z.EXPORTS)


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_layout_matches_oracle_on_workloads(name):
    wl = W.WORKLOADS[name]
    a = Z.zero_partition_layout(wl.numels, wl.world, wl.align)
    b = oracle.layout(wl.numels, wl.world, wl.align)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_layout_matches_oracle_random():
    rng = np.random.default_rng(2)
    for _ in range(2000):
        n = int(rng.integers(0, 8))
        numels = rng.integers(0, 1 << int(rng.integers(1, 30)), n)
        world = int(rng.integers(1, 17))
        align = int(rng.choice([1, 2, 4, 8]))
        a = Z.zero_partition_layout(numels, world, align)
        b = oracle.layout(numels, world, align)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_layout_errors():
    for args in (([1, 2], 0, 2), ([1, 2], 2, 0), ([1, -2], 2, 2)):
        with pytest.raises(Z.ZeroError):
            Z.zero_partition_layout(*args)
    with pytest.raises(Z.ZeroError, match="range"):
        Z.zero_partition_layout([2 ** 62, 2 ** 62, 2 ** 62], 2, 2)


def test_buckets_match_oracle():
    rng = np.random.default_rng(3)
    for _ in range(2000):
        n = int(rng.integers(1, 20))
        numels = rng.integers(0, 50, n)
        cap = int(rng.integers(1, 80))
        assert np.array_equal(Z.zero_bucket_layout(numels, cap), oracle.buckets(numels, cap))
    wl = W.WORKLOADS["buckets"]
    assert np.array_equal(Z.zero_bucket_layout(wl.numels, wl.bucket_cap),
                          oracle.buckets(wl.numels, wl.bucket_cap))


def test_memory_bytes_match_oracle():
    for name, wl in W.WORKLOADS.items():
        _, _, padded = oracle.layout(wl.numels, wl.world, wl.align)
        for stage in range(4):
            assert Z.zero_memory_bytes(stage, wl.phi, padded, wl.world) == \
                oracle.memory_bytes(stage, wl.phi, wl.world, padded)
    with pytest.raises(Z.ZeroError):
        Z.zero_memory_bytes(4, 10, 10, 1)
    with pytest.raises(Z.ZeroError):
        Z.zero_memory_bytes(1, 10, 9, 1)


def test_loss_scaler_matches_oracle():
    rng = np.random.default_rng(4)
    for window in (1, 2, 3, 1000):
        a = Z.zero_loss_scaler(2.0 ** 16, 1.0, window, 0, 0)
        b = oracle.Scaler(2.0 ** 16, 1.0, window)
        for f in (rng.random(3000) < 0.3).astype(int):
            Z.zero_loss_scaler_update(a, int(f))
            b.update(int(f))
            assert (a.scale, a.clean, a.skipped) == (b.scale, b.clean, b.skipped)


def test_status_strings():
    assert Z.zero_status_str(Z.ZERO_OK) == "ok"
    assert "invalid" in Z.zero_status_str(Z.ZERO_EINVAL)
    assert Z.zero_check_workspace_bytes(0) >= 16
    # one 12-byte partial per 2048 elements plus the fold levels
    for n in (1, 2047, 2048, 10 ** 6, 842_301_952, 8_622_081_024, 10 ** 12):
        ws = Z.zero_check_workspace_bytes(n)
        assert 12 * (n // 2048) <= ws <= n / 170 + 1024
    assert Z.zero_check_workspace_bytes(8_622_081_024) < 51e6


@pytest.mark.parametrize("scale0,divisor,betas", [(2.0 ** 16, 1.0, (0.9, 0.999)),
                                                  (1.0, 8.0, (0.9, 0.95)),
                                                  (3.0, 3.0, (0.0, 0.5))])
def test_step_control_init_matches_oracle_constants(scale0, divisor, betas):
    """The device step control's first-step scalars are the oracle's: the
    unscale factor fp32(1/(S*D)) and AdamW's bias corrections for t = 1."""
    import ctypes
    c = Z.zero_step_control_init(scale0, 1.0, 1000, divisor, *betas)
    assert (c.scale, c.min_scale, c.window, c.clean, c.skipped, c.t) == (scale0, 1.0, 1000, 0, 0, 0)
    assert c.inv_scale == float(np.float32(1.0 / (scale0 * divisor)))
    want = oracle.adam_consts(oracle.HParams(1e-3, betas[0], betas[1], 1e-8, 0.01, 0.0), 1)
    assert (c.bc1, c.bc2) == (want["bc1"], want["bc2"])
    assert (c.beta1, c.beta2) == (want["b1"], want["b2"])
    assert ctypes.sizeof(c) == 72


def test_step_control_init_errors():
    for args in ((0.0,), (1.0, 0.0), (1.0, 1.0, 0), (1.0, 1.0, 10, 0.0), (1.0, 1.0, 10, 1.0, 1.0),
                 (1.0, 1.0, 10, 1.0, 0.9, -0.1), (float("inf"),)):
        with pytest.raises(Z.ZeroError):
            Z.zero_step_control_init(*args)


def test_device_control_calls_reject_null_pointers_before_launching():
    """Argument checks run on the host before anything is launched, so they
    need no GPU: a NULL control block, result or buffer is ZERO_EINVAL."""
    import ctypes
    L = Z.lib()
    hp = Z.zero_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    fake = ctypes.c_void_p(0x10000)          # never dereferenced: every call fails first
    srcs = (ctypes.c_void_p * 1)(fake)
    assert L.zero_step_control_update(None, fake, None) == Z.ZERO_EINVAL
    assert L.zero_step_control_update(fake, None, None) == Z.ZERO_EINVAL
    assert L.zero_reduce_check_owned_ctl(fake, srcs, 1, 16, Z.ZERO_BF16, None, fake, fake, 1 << 20,
                                         0, None) == Z.ZERO_EINVAL
    assert L.zero_unscale_check_norm_ctl(fake, 16, Z.ZERO_BF16, None, fake, fake, 1 << 20, 0,
                                         None) == Z.ZERO_EINVAL
    assert L.zero_adamw_step_ctl(fake, fake, fake, fake, fake, 16, Z.ZERO_BF16, ctypes.byref(hp),
                                 None, fake, None) == Z.ZERO_EINVAL
    assert L.zero_adamw_step_ctl(fake, fake, fake, fake, fake, 16, 7, ctypes.byref(hp), fake, fake,
                                 None) == Z.ZERO_EINVAL
    assert L.zero_adamw_step_ctl(fake, fake, fake, fake, fake, 16, Z.ZERO_BF16, None, fake, fake,
                                 None) == Z.ZERO_EINVAL


def test_builder_loads_without_the_package():
    """build() must work on a tree where nothing is built yet: loading the
    build module may not import the package, whose import needs the library."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(HEADER))
    code = ("import sys, __graft_entry__ as g; m = g._load_builder(); "
            "assert callable(m.build) and m.LIB.endswith('libzero_shard.so'); "
            "assert 'zero_partitioned_mixed_shard_amd' not in sys.modules, sorted(sys.modules)")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr


@pytest.mark.parametrize("n_ranks,in_place,bucket", [(0, None, False), (1, 0, False),
                                                     (8, None, False), (8, 0, False),
                                                     (8, 5, False), (16, None, False),
                                                     (16, 15, False), (8, None, True)])
def test_arena_orders_place_every_buffer_once(n_ranks, in_place, bucket):
    """Every arena order is a permutation of the step's buffers, and the
    placement gives each one a 64 KiB aligned, non-overlapping range, with
    master, m and v at least min_gap apart.  With the bucket layout the
    rank data are blocks of different sizes, one per reduce window, kept in
    window order."""
    from zero_partitioned_mixed_shard_amd.shard import ARENA_ORDERS, FP32_ARRAYS, ShardStep
    n = 1_000_003
    names = ["master", "exp_avg", "exp_avg_sq", "param16"] + (["red"] if in_place is None else [])
    sizes = {nm: n * (4 if nm in FP32_ARRAYS else 2) for nm in names}
    rank_names = ([f"rankw{w}" for w in range(12)] if bucket else
                  [f"rank{r}" for r in range(n_ranks)])
    for k, nm in enumerate(rank_names):
        sizes[nm] = n_ranks * (1000 + 77777 * k) * 2 if bucket else 2 * n
    names += rank_names
    streams = set(names[:4]) | ({"red"} if in_place is None else {f"rank{in_place}"})
    for name, order in ARENA_ORDERS.items():
        seq = order(names, streams, in_place)
        assert sorted(seq) == sorted(names), name
        if bucket:
            assert [nm for nm in seq if nm.startswith("rank")] == rank_names, name
        gap_set = set(FP32_ARRAYS)
        for gap in (0, 3 << 20):
            offs, end = ShardStep._place(seq, sizes, gap_set, gap)
            spans = sorted((offs[nm], offs[nm] + sizes[nm]) for nm in names)
            assert all(a % (1 << 16) == 0 for a, _ in spans)
            assert all(b <= c for (_, b), (c, _) in zip(spans, spans[1:])), name
            assert spans[-1][1] == end
            st = sorted(offs[nm] for nm in gap_set)
            assert all(b - a >= gap for a, b in zip(st, st[1:])), name


def test_range_lists_are_checked_before_launching():
    """The *_ranges calls reject a bad range list on the host, before any
    launch (no GPU needed): negative offsets or counts, overlapping ranges
    (ZERO_EINVAL) and offset + count beyond int64 (ZERO_ERANGE).  The
    workspace bound over a list is the single-range bound's fold of the
    summed block counts."""
    import ctypes
    L = Z.lib()
    hp = Z.zero_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    fake = ctypes.c_void_p(0x10000)          # never dereferenced: every call fails first
    srcs = (ctypes.c_void_p * 2)(fake, fake)
    bad = {
        "negative offset": ([(-1, 4)], Z.ZERO_EINVAL),
        "negative count": ([(0, -4)], Z.ZERO_EINVAL),
        "overlap": ([(0, 100), (99, 10)], Z.ZERO_EINVAL),
        "overlap, unsorted": ([(500, 10), (0, 100), (95, 3)], Z.ZERO_EINVAL),
        "overflow": ([(2 ** 62, 2 ** 62)], Z.ZERO_ERANGE),
    }
    for what, (rs, want) in bad.items():
        arr = Z._ranges(rs)
        got = L.zero_reduce_check_ranges(fake, srcs, 2, arr, len(rs), Z.ZERO_BF16, 1.0, None, fake,
                                         fake, 1 << 30, 0, None)
        assert got == want, what
        got = L.zero_adamw_step_ranges(fake, fake, fake, fake, fake, arr, len(rs), Z.ZERO_BF16,
                                       ctypes.byref(hp), None, fake, None)
        assert got == want, what
        assert L.zero_range_workspace_bytes(arr, len(rs)) == 0, what
    # NULL list with entries, NULL result, unknown dtype
    assert L.zero_reduce_check_ranges(fake, srcs, 2, None, 3, Z.ZERO_BF16, 1.0, None, fake, fake,
                                      1 << 30, 0, None) == Z.ZERO_EINVAL
    ok = Z._ranges([(0, 10), (10, 5)])
    assert L.zero_reduce_check_ranges(fake, srcs, 2, ok, 2, Z.ZERO_BF16, 1.0, None, None, fake,
                                      1 << 30, 0, None) == Z.ZERO_EINVAL
    assert L.zero_adamw_step_ranges(fake, fake, fake, fake, fake, ok, 2, 9, ctypes.byref(hp), None,
                                    fake, None) == Z.ZERO_EINVAL
    # too small a workspace
    assert L.zero_reduce_check_ranges(fake, srcs, 2, ok, 2, Z.ZERO_BF16, 1.0, None, fake, fake, 8,
                                      0, None) == Z.ZERO_EINVAL
    # workspace bound: one range is the single-range bound; touching ranges are fine
    assert Z.zero_range_workspace_bytes([(0, 10_000_019)]) == \
        Z.zero_check_workspace_bytes(10_000_019)
    assert Z.zero_range_workspace_bytes([(0, 4096), (4096, 4096)]) >= \
        Z.zero_check_workspace_bytes(8192)


def test_bucket_windows_are_checked_before_launching():
    """zero_reduce_check_buckets rejects bad windows on the host like the
    range-list calls, and a missing rank pointer of a non-empty window
    (ZERO_EINVAL); the pointers of an empty window are not read."""
    import ctypes
    L = Z.lib()
    fake = ctypes.c_void_p(0x10000)          # never dereferenced: every call fails first
    bad = {
        "negative offset": ([(-1, 4)], Z.ZERO_EINVAL),
        "negative count": ([(0, -4)], Z.ZERO_EINVAL),
        "overlap": ([(0, 100), (99, 10)], Z.ZERO_EINVAL),
        "overflow": ([(2 ** 62, 2 ** 62)], Z.ZERO_ERANGE),
    }
    for what, (rs, want) in bad.items():
        srcs = (ctypes.c_void_p * (2 * len(rs)))(*([fake] * (2 * len(rs))))
        got = L.zero_reduce_check_buckets(fake, srcs, 2, Z._ranges(rs), len(rs), Z.ZERO_BF16, 1.0,
                                          None, fake, fake, 1 << 30, 0, None)
        assert got == want, what
    ok = Z._ranges([(0, 10), (10, 0), (20, 5)])
    # window 2's second rank is missing
    srcs = (ctypes.c_void_p * 6)(fake, fake, None, None, fake, None)
    assert L.zero_reduce_check_buckets(fake, srcs, 2, ok, 3, Z.ZERO_BF16, 1.0, None, fake, fake,
                                       1 << 30, 0, None) == Z.ZERO_EINVAL
    srcs = (ctypes.c_void_p * 6)(fake, fake, None, None, fake, fake)
    for args, what in (((None, srcs, 2, ok, 3, Z.ZERO_BF16, 1.0, None, fake, fake, 1 << 30),
                        "no dst"),
                       ((fake, None, 2, ok, 3, Z.ZERO_BF16, 1.0, None, fake, fake, 1 << 30),
                        "no rank pointers"),
                       ((fake, srcs, 0, ok, 3, Z.ZERO_BF16, 1.0, None, fake, fake, 1 << 30),
                        "no ranks"),
                       ((fake, srcs, 2, ok, 3, 7, 1.0, None, fake, fake, 1 << 30), "dtype"),
                       ((fake, srcs, 2, ok, 3, Z.ZERO_BF16, 0.0, None, fake, fake, 1 << 30),
                        "inv_scale"),
                       ((fake, srcs, 2, ok, 3, Z.ZERO_BF16, 1.0, None, None, fake, 1 << 30),
                        "no result"),
                       ((fake, srcs, 2, ok, 3, Z.ZERO_BF16, 1.0, None, fake, fake, 8),
                        "workspace too small")):
        assert L.zero_reduce_check_buckets(*args, 0, None) == Z.ZERO_EINVAL, what


def test_header_compiles_as_c(tmp_path):
    """include/zero_shard.h is a C header: a C11 translation unit that uses
    its types and a declaration compiles, with no diagnostic from the header
    itself (HIP's runtime API header supplies hipStream_t)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    src = tmp_path / "use_header.c"
    src.write_text('#include "zero_shard.h"\n'
                   "int main(void) {\n"
                   "    zero_range r = {0, 1};\n"
                   "    zero_tensor_desc d = {0, 0, 0, 0};\n"
                   "    zero_step_result s;\n"
                   "    (void)d; (void)s;\n"
                   "    return (int)zero_range_workspace_bytes(&r, 1) * 0;\n"
                   "}\n")
    r = subprocess.run([gcc, "-x", "c", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.dirname(HEADER), "-I", "/opt/rocm/include", "-fsyntax-only",
                        str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    own = [l for l in r.stderr.splitlines() if "zero_shard.h:" in l and "included from" not in l]
    assert not own, own


def test_noalloc_scratch_covers_its_largest_count():
    """The allocation-free reduce+check keeps its check partials in an array
    inside the library of 25,178,368 bytes (the workspace of 2^32 elements,
    rounded up to 256 bytes) and accepts counts up to 2^32: the workspace the
    workspace call needs for every count up to that limit fits in it, so a
    count the call accepts is never refused for lack of scratch."""
    limit, scratch = 1 << 32, 25_178_368
    L = Z.lib()
    for count in (limit, limit - 1, limit - 4095, 3 * (1 << 30) + 7, 1 << 20, 1):
        need = L.zero_check_workspace_bytes(count)
        assert 0 < need <= scratch, (count, need)
    # the requirement grows with the count, so the largest count bounds them all
    assert L.zero_check_workspace_bytes(limit) >= L.zero_check_workspace_bytes(limit // 2)
