"""Benchmark of the ZeRO-1/2 owner-shard step on one MI355X.

One step = the whole owner-shard path over one batch of synthetic gradients
already resident in HBM:
  layout (host) -> reduce N ranks' 16-bit gradients to the owner fused with
  unscale + overflow check + squared norm (HIP) -> fused AdamW + 16-bit copy
  (HIP) -> loss-scale update and step count (HIP, device-resident step
  control: no host round trip between steps; --host-control reads the
  16-byte result back and updates the scaler on the host instead)
Algorithmic HBM bytes per owned element: 2N + 2 for reduce+check (2N + 4 with
--unfused, which re-reads the reduced gradient), 28 for AdamW.

Default workload: owner 0's partition of the LLaMA-70B-shaped flat buffer
(68,976,648,192 parameters, N = 8 ranks, 8,622,081,024 owned elements, bf16
gradients N(0, 1e-4), AdamW lr 1e-3, betas (0.9, 0.999), eps 1e-8, wd 0.01,
clip 1.0), the largest configuration that fits one GPU: 275.9 GB resident
with the reduced gradient in a buffer of its own (258.7 GB with
--in-place-reduce, the reduce then writing into rank 0's buffer).  The
ranks' gradients arrive bucket by bucket (5e8-element, tensor-aligned reduce
buckets; each bucket's 8 slices back to back), and the buffers sit in one
arena in a fixed order (ranks_first, master / m / v at least 32 GiB apart):
no placement search unless --placement auto.  After the 70B shard is freed
the LLaMA-7B-shaped shard (842,301,952 owned elements) is timed the same way
and reported as the "secondary" object, then once more with its placement
measured at setup ("secondary_tuned": every arena order at base offsets 4 GiB
apart in 64 GiB of slack; the 7B shard's rate follows the physical addresses
its arrays land on, which vary between allocations and boxes).
--secondary none skips both; --workload llama7b runs the 7B shard alone.

Prints one JSON line: params updated per second (owned elements x applied
steps / time), per-phase times measured with HIP events on the stream the
kernels run on (timing-only events without the system-scope fence; the two
events around the timed steps are default ones), the AdamW kernel's achieved HBM bandwidth against the 8 TB/s
peak, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# the sources the reduce and AdamW kernels are built from (the flat copy
# kernels live in csrc/zero_flat.hip and do not affect their counters)
KERNEL_SRCS = [os.path.join(ROOT, "zero_partitioned_mixed_shard_amd", "csrc", f)
               for f in ("zero_common.h", "zero_shard.hip")]
COUNTERS = {w: os.path.join(ROOT, "profiles", f"adamw_reduce_{w}_hbm_counters.md")
            for w in ("toy", "bert", "llama7b", "llama70b", "buckets")}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary, or None when there is none or the kernel source changed
    since the counters were taken."""
    import hashlib
    import re
    try:
        h = hashlib.sha256()
        for f in KERNEL_SRCS:
            h.update(open(f, "rb").read())
        src = h.hexdigest()[:16]
        text = open(COUNTERS[workload]).read()
    except (OSError, KeyError):
        return None
    m = re.search(rf"machine-readable: {kernel} traffic_bytes=(\d+) source_sha256_16=(\w+)", text)
    if not m or m.group(2) != src:
        return None
    return int(m.group(1))


class TimingEvent:
    """A HIP event used only to time work on torch's current stream, created
    with hipEventDisableSystemFence: recording it skips the system-scope
    fence (cache write-back and invalidation) that a default event performs,
    which on MI355X costs the stream about 5.7 us per record.  The timed
    region's two outer events stay default torch events, and every read of
    these follows a device synchronize.  Same record() / elapsed_time() as
    torch.cuda.Event."""
    FLAGS = 0x20000000                       # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def runtime(cls):
        """The HIP runtime torch loaded (the only one in the process)."""
        import ctypes
        if cls._hip is None:
            paths = [ln.split()[-1] for ln in open("/proc/self/maps")
                     if len(ln.split()) >= 6 and "libamdhip64" in ln.split()[-1]]
            if not paths:
                raise RuntimeError("the HIP runtime is not loaded")
            hip = ctypes.CDLL(paths[0])
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        if self.runtime().hipEventCreateWithFlags(ctypes.byref(self._ev), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self):
        import torch
        if self.runtime().hipEventRecord(self._ev, torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        if self.runtime().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self):
        if self._ev:
            self.runtime().hipEventDestroy(self._ev)
            self._ev = None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 40 for the buckets workload)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama70b",
                    choices=["toy", "bert", "llama7b", "llama70b", "buckets"])
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (e.g. under a profiler)")
    ap.add_argument("--cpu-seconds", type=float, default=1.5,
                    help="wall-clock budget of the CPU oracle leg")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="also run a plain device copy of this size (for HBM counter scaling)")
    ap.add_argument("--unfused", action="store_true",
                    help="separate reduce and check calls instead of the fused one")
    ap.add_argument("--round-robin-owner", type=int, default=None,
                    help="instead of flat partition 0, own the whole tensors i with "
                         "i mod N == this owner (packed; one reduce window per tensor)")
    ap.add_argument("--no-arena", action="store_true",
                    help="separate allocations instead of one arena with spread placement")
    ap.add_argument("--placement", default="ranks_first",
                    choices=["auto", "spread", "interleaved", "rank_block", "rank_block_b",
                             "master_ranks", "streams_first", "ranks_first"],
                    help="order of the buffers in the arena (default ranks_first: the rank "
                         "data, then master, m, v, the 16-bit copy and the reduced gradient, "
                         "with --min-gap-gib between master, m and v); auto times every order "
                         "at setup (outside the timed steps) and keeps the fastest")
    ap.add_argument("--secondary", default=None,
                    help="a second workload timed in the same run after the first is freed, "
                         "reported as the 'secondary' object (default: llama7b after llama70b; "
                         "'none' to skip)")
    ap.add_argument("--secondary-steps", type=int, default=20)
    ap.add_argument("--no-secondary-tuned", action="store_true",
                    help="skip the secondary shard's second run with its placement measured at "
                         "setup ('secondary_tuned')")
    ap.add_argument("--arena-slack-gib", type=float, default=0.0,
                    help="allocate the arena up to this much larger (never more than is free, "
                         "less 4 GiB) and let --placement auto also try every order at base "
                         "offsets 4 GiB apart inside it, i.e. at other physical addresses; 0 = "
                         "an arena of exactly the working set")
    ap.add_argument("--min-gap-gib", type=float, default=32.0,
                    help="minimum distance between the bases of master, m and v in the arena "
                         "(halved, down to 0, where the device cannot hold it)")
    ap.add_argument("--bucket-cap", type=float, default=None,
                    help="reduce bucket size in elements for the LLaMA shards (default 5e8, "
                         "the pages' reduce_bucket_size)")
    ap.add_argument("--flush-gib", type=float, default=0.0,
                    help="write this much scratch memory between timed steps (untimed), so that "
                         "no step finds its inputs in the 256 MB Infinity Cache or the L2; "
                         "value and ms_per_step then come from the per-step events")
    ap.add_argument("--inject-every", type=int, default=None,
                    help="every K-th timed step, one rank's gradient holds +inf (odd "
                         "occurrences) or NaN (even) at a seeded index: the step is skipped "
                         "and the loss scale halves; 0 = off (default 4 for the buckets "
                         "workload, whose protocol has an overflow every 4th step; else 0)")
    ap.add_argument("--in-place-reduce", action="store_true",
                    help="LLaMA-70B / 7B shard: reduce into rank 0's buffer instead of a reduced "
                         "buffer of its own (17.2 GB less at the 70B size; the separate buffer "
                         "measured 0.5-1 %% faster there)")
    ap.add_argument("--no-batch", action="store_true",
                    help="one reduce+check call per reduce window and one AdamW call per owner, "
                         "instead of one range-list call each (bucket group, round-robin owner)")
    ap.add_argument("--host-control", action="store_true",
                    help="keep the loss scaler and step count on the host: every step ends with "
                         "a 16-byte result readback (the GPU idles while the host updates the "
                         "scaler and enqueues the next step); default: device-resident step "
                         "control, no per-step round trip")
    ap.add_argument("--fenced-events", action="store_true",
                    help="time the phases with default events (each record adds a system-scope "
                         "fence, about 5.7 us of the step) instead of fence-free timing events")
    ap.add_argument("--graph", action="store_true",
                    help="keep the loss scaler and step count on the device and replay one "
                         "captured HIP graph per step (no host round trip between steps)")
    ap.add_argument("--write-back", action="store_true",
                    help="buckets workload: also scatter the updated 16-bit flat buffer into "
                         "per-parameter tensors after AdamW (zero_flat_scatter), timed as a phase")
    args = ap.parse_args()
    if args.secondary is None:
        args.secondary = ("llama7b" if args.workload == "llama70b" and args.round_robin_owner is None
                          else "none")
    if args.secondary == "none":
        args.secondary = None
    return args


def cpu_baseline(wl, begin: int, seconds: float) -> dict:
    """The oracle, as it is, on the first 2^22 owned elements of the same
    workload, chunked over all host cores (ctypes releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from synth import inputs as I

    n = 1 << 22
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(threads, 64))
    offs, parts, padded = oracle.layout(wl.numels, wl.world, wl.align)
    p16 = I.host_param16(wl, offs, begin, begin + n, threads)
    grads = I.host_rank_grads(wl, 1, wl.scale0, begin, begin + n, padded, threads)
    state = oracle.OwnerState.from_param16(p16, wl.dtype)
    hp = oracle.HParams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, wl.clip)
    inv = 1.0 / wl.scale0
    chunk = (n + threads - 1) // threads
    bounds = [(k * chunk, min(n, (k + 1) * chunk)) for k in range(threads)]
    red = np.empty(n, np.uint16)

    def reduce_part(b):
        a, z = b
        red[a:z] = oracle.reduce([g[a:z] for g in grads], wl.dtype)

    def check_part(b):
        a, z = b
        return oracle.check(red[a:z], wl.dtype, inv)

    def adam_part(args):
        (a, z), sumsq, t = args
        v = [x[a:z] for x in (state.master, state.exp_avg, state.exp_avg_sq, state.param16)]
        oracle.adamw(*v, red[a:z], wl.dtype, inv, sumsq, 0, hp, t)

    steps = 0
    phase = {"reduce": 0.0, "check": 0.0, "adamw": 0.0}
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        while True:
            ta = time.perf_counter()
            list(ex.map(reduce_part, bounds))
            tb = time.perf_counter()
            parts_ = list(ex.map(check_part, bounds))
            flag = max(p[0] for p in parts_)
            sumsq = sum(p[1] for p in parts_)
            tc = time.perf_counter()
            steps += 1
            list(ex.map(adam_part, [(b, sumsq, steps) for b in bounds]))
            td = time.perf_counter()
            phase["reduce"] += tb - ta
            phase["check"] += tc - tb
            phase["adamw"] += td - tc
            assert flag == 0
            if time.perf_counter() - t0 >= seconds and steps >= 2:
                break
    dt = time.perf_counter() - t0
    return {"value": n * steps / dt, "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} owned elements of the same workload (N={wl.world} ranks), "
                      f"{steps} full oracle steps (reduce, check, AdamW) in {dt:.2f} s wall "
                      f"on {threads} threads (about {dt * threads:.0f} core-seconds)",
            "phase_params_per_s": {k: round(n * steps / v, 1) for k, v in phase.items()}}


def build_shard(wl, arena: bool = True, min_gap: int = 32 << 30, fused: bool = True,
                device_control: bool = False, placement: str = "ranks_first",
                arena_slack: int = 0, batched: bool = True, in_place: bool = False,
                bucket_cap=None):
    """Owner 0's shard of `wl` as the bench runs it: state, reduced gradient
    (a buffer of its own, or with in_place -- or when the device cannot hold
    a separate one -- rank 0's buffer), the N ranks' gradients, initial
    16-bit weights and one gradient batch generated on the device.  With a
    reduced buffer of its own and the fused reduce+check, the ranks'
    gradients arrive bucket by bucket (ZeRO-2 source walkthrough section
    4.2: reduce buckets of reduce_bucket_size = 5e8 elements, tensor-aligned):
    each bucket's N slices of the owner's partition lie back to back, and one
    zero_reduce_check_buckets call reduces every bucket.  Otherwise each rank
    has one flat buffer.  Returns (shard, begin, end, padded, in_place)."""
    import torch

    from synth import inputs as I
    from synth import workloads as W
    import zero_partitioned_mixed_shard_amd as Z
    from zero_partitioned_mixed_shard_amd.shard import ShardStep

    offs, parts, padded = Z.zero_partition_layout(wl.numels, wl.world, wl.align)
    begin, end = int(parts[0]), int(parts[1])
    if not in_place:
        # a reduced buffer of its own needs 2 B per element more; where the
        # device cannot hold it (with 4 GiB to spare), reduce into rank 0's
        # buffer instead (reported as config.in_place_reduce)
        need = (end - begin) * (12 + 2 + 2 + 2 * wl.world) + (4 << 30)
        in_place = torch.cuda.mem_get_info()[0] < need
    cap = int(bucket_cap or wl.bucket_cap or 0)
    layout = "bucket" if fused and not in_place and cap else "flat"
    windows = None
    if layout == "bucket":
        windows = W.bucket_windows(wl, offs, padded, Z.zero_bucket_layout(wl.numels, cap))
    shard = ShardStep(begin, end, [(begin, end)], wl.dtype, lr=wl.lr, beta1=wl.beta1,
                      beta2=wl.beta2, eps=wl.eps, weight_decay=wl.weight_decay,
                      max_grad_norm=wl.clip, scale0=wl.scale0, min_scale=wl.min_scale,
                      window=wl.window, windows=windows, in_place_rank=0 if in_place else None,
                      fused=fused, own_ranks=True, world=wl.world, arena=arena, min_gap=min_gap,
                      device_control=device_control, placement=placement,
                      arena_slack=arena_slack, batched=batched, rank_layout=layout)
    shard.load_param16(I.device_param16(wl, offs, begin, end, out=shard.param16))
    shard.fill_ranks(lambda r, a, b, out: I.device_rank_grad(wl, 1, wl.scale0, r, begin + a,
                                                             begin + b, padded, out=out))
    torch.cuda.synchronize()
    return shard, begin, end, padded, in_place


def build_buckets(wl, arena: bool = True, min_gap: int = 0, fused: bool = True,
                  write_back: bool = False, device_control: bool = False,
                  placement: str = "auto", arena_slack: int = 0, batched: bool = True):
    """The 10,000-tensor group with all N owners on this GPU, as the bench runs
    it: rank 0's gradient arrives as one separate device tensor per parameter
    (10,000 allocations) and is copied into rank 0's flat buffer bucket by
    bucket (zero_flat_gather, ZeRO-2 source walkthrough section 2.4
    contiguous_gradients); ranks 1..N-1 arrive already flat.  With write_back,
    the parameters also live as one device tensor each (10,000 allocations)
    and the updated flat 16-bit buffer is scattered into them after the step
    (zero_flat_scatter, ZeRO-2 source walkthrough section 4.4).  Returns
    (shard, copy_in, padded, write_back) where copy_in() / write_back()
    enqueue the copies (write_back is None without the option)."""
    import torch

    from synth import inputs as I
    from synth import workloads as W
    import zero_partitioned_mixed_shard_amd as Z
    from zero_partitioned_mixed_shard_amd.shard import ShardStep

    offs, parts, padded = Z.zero_partition_layout(wl.numels, wl.world, wl.align)
    first = Z.zero_bucket_layout(wl.numels, wl.bucket_cap)
    windows = W.bucket_windows(wl, offs, padded, first)
    owners = [(int(parts[p]), int(parts[p + 1])) for p in range(wl.world)]
    shard = ShardStep(0, padded, owners, wl.dtype, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                      eps=wl.eps, weight_decay=wl.weight_decay, max_grad_norm=wl.clip,
                      scale0=wl.scale0, min_scale=wl.min_scale, window=wl.window,
                      windows=windows, fused=fused, own_ranks=True, world=wl.world,
                      arena=arena, min_gap=min_gap, device_control=device_control,
                      placement=placement, arena_slack=arena_slack, batched=batched)
    shard.load_param16(I.device_param16(wl, offs, 0, padded, out=shard.param16))
    for r, buf in enumerate(shard.rank_bufs):
        I.device_rank_grad(wl, 1, wl.scale0, r, 0, padded, padded, out=buf)
    # rank 0's gradient as per-parameter tensors (one allocation each) holding
    # the same values, written by the seeded generator straight into each
    # tensor: the setup makes no device-to-device copies
    flat0 = shard.rank_bufs[0]
    grads = []
    for o, n in zip(offs, wl.numels):
        o, n = int(o), int(n)
        grads.append(I.device_rank_grad(wl, 1, wl.scale0, 0, o, o + n, padded))
    flat0.fill_(-1.0)                       # the copy-in must rewrite every element
    tables = []
    for b, (a, z) in enumerate(windows):
        ks = range(int(first[b]), int(first[b + 1]))
        tables.append((a, z, Z.tensor_descs([grads[k] for k in ks], [int(offs[k]) - a for k in ks])))

    def copy_in():
        for a, z, descs in tables:
            Z.zero_flat_gather(flat0[a:z], descs)

    copy_in()
    wb = None
    if write_back:
        params = [torch.empty(int(n), dtype=shard.param16.dtype, device="cuda") for n in wl.numels]
        wb_descs = Z.tensor_descs(params, [int(o) for o in offs])

        def wb():
            Z.zero_flat_scatter(shard.param16, wb_descs)

        wb()
        shard.per_tensor_params = params
    torch.cuda.synchronize()
    shard.per_tensor_grads = grads
    return shard, copy_in, padded, wb


def build_round_robin(wl, owner: int, arena: bool = True, min_gap: int = 0, fused: bool = True,
                      device_control: bool = False, placement: str = "auto",
                      arena_slack: int = 0, batched: bool = True):
    """Round-robin inter-tensor ownership (ZeRO 优化器, "参数分配策略"): this
    owner holds the whole tensors i with i mod N == owner, packed back to back
    (state only for what it owns); each tensor is reduced to it on its own
    (one reduce window per tensor, as the per-parameter reduce of that page's
    training loop).  Returns (shard, owned_elems, n_tensors, imbalance) where
    imbalance = the largest owner's elements / the mean."""
    import torch

    from synth import inputs as I
    from zero_partitioned_mixed_shard_amd.shard import ShardStep
    import zero_partitioned_mixed_shard_amd as Z

    offs, parts, padded = Z.zero_partition_layout(wl.numels, wl.world, wl.align)
    owned = [i for i, n in enumerate(wl.numels) if i % wl.world == owner and n > 0]
    sizes = [int(wl.numels[i]) for i in owned]
    packed = [0]
    for n in sizes:
        packed.append(packed[-1] + n)
    count = packed[-1]
    per_owner = [sum(int(n) for i, n in enumerate(wl.numels) if i % wl.world == p)
                 for p in range(wl.world)]
    windows = [(packed[k], packed[k + 1]) for k in range(len(owned))]
    shard = ShardStep(0, count, [(0, count)], wl.dtype, lr=wl.lr, beta1=wl.beta1,
                      beta2=wl.beta2, eps=wl.eps, weight_decay=wl.weight_decay,
                      max_grad_norm=wl.clip, scale0=wl.scale0, min_scale=wl.min_scale,
                      window=wl.window, windows=windows, fused=fused, own_ranks=True,
                      world=wl.world, arena=arena, min_gap=min_gap,
                      device_control=device_control, placement=placement,
                      arena_slack=arena_slack, batched=batched)
    for k, i in enumerate(owned):
        a, b = packed[k], packed[k + 1]
        g0 = int(offs[i])
        I.device_param16(wl, offs, g0, g0 + sizes[k], out=shard.param16[a:b])
        for r, buf in enumerate(shard.rank_bufs):
            I.device_rank_grad(wl, 1, wl.scale0, r, g0, g0 + sizes[k], padded, out=buf[a:b])
    shard.load_param16(shard.param16)
    torch.cuda.synchronize()
    return shard, count, len(owned), max(per_owner) / (sum(per_owner) / wl.world)


def run_workload(args, workload: str, steps: int, inject_every: int,
                 calibrate: bool = False) -> dict:
    """Builds `workload` as the bench runs it, does the warm-up steps, times
    `steps` steps and returns the measured fields (and the owned range under
    "_begin"), then frees the device memory it used."""
    import numpy as np
    import torch

    from synth import workloads as W
    import zero_partitioned_mixed_shard_amd as Z

    wl = W.WORKLOADS[workload]
    torch.cuda.set_device(0)
    if calibrate and args.copy_calibration_gib > 0:
        # one elementwise kernel that reads and writes exactly `nbytes` each:
        # the reference for scaling the HBM byte counters
        nbytes = int(args.copy_calibration_gib * 2 ** 30)
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    copy_in = None
    write_back = None
    rr_info = None
    slack = int(args.arena_slack_gib * 2 ** 30)
    flush = None
    if args.flush_gib > 0:
        # allocated before the shard: the arena's slack is clamped to what is left
        flush = torch.empty(int(args.flush_gib * 2 ** 30) // 4, dtype=torch.float32, device="cuda")
    if args.round_robin_owner is not None and workload == args.workload:
        shard, count_rr, n_owned, imbalance = build_round_robin(
            wl, args.round_robin_owner, arena=not args.no_arena,
            min_gap=int(args.min_gap_gib * 2 ** 30), fused=not args.unfused,
            device_control=not args.host_control, placement=args.placement,
            arena_slack=slack, batched=not args.no_batch)
        begin, end, padded, in_place = 0, count_rr, 0, False
        rr_info = {"owner": args.round_robin_owner, "owned_tensors": n_owned,
                   "owned_elems": count_rr, "largest_over_mean_owner": round(imbalance, 4)}
    elif workload == "buckets":
        shard, copy_in, padded, write_back = build_buckets(
            wl, arena=not args.no_arena, min_gap=int(args.min_gap_gib * 2 ** 30),
            fused=not args.unfused, write_back=args.write_back,
            device_control=not args.host_control, placement=args.placement, arena_slack=slack,
            batched=not args.no_batch)
        begin, end, in_place = 0, padded, False
    else:
        shard, begin, end, padded, in_place = build_shard(
            wl, arena=not args.no_arena, min_gap=int(args.min_gap_gib * 2 ** 30),
            fused=not args.unfused, device_control=not args.host_control, placement=args.placement,
            arena_slack=slack, batched=not args.no_batch, in_place=args.in_place_reduce,
            bucket_cap=args.bucket_cap)
    count = end - begin
    bufs = shard.rank_bufs if shard.rank_layout == "flat" else None

    def one_step(marks=None):
        """Enqueue one step.  With device-resident control nothing is read
        back (the loss scale and step count advance on the device); with
        host control the 16-byte result is read and the scaler updated."""
        shard.launch(bufs, marks)
        if write_back:
            write_back()
            if marks:
                marks[5].record()
        if shard.ctl is not None:
            return None
        return shard.finish()

    for _ in range(args.warmup):
        Z.zero_partition_layout(wl.numels, wl.world, wl.align)
        if copy_in:
            copy_in()
        one_step()
    torch.cuda.synchronize()

    # the values the inf/NaN injections overwrite, read before the timed steps
    originals = {}
    for k in range(steps):
        if inject_every and (k + 1) % inject_every == 0:
            r = 1 + (k % (shard.n_ranks - 1)) if shard.n_ranks > 1 else 0
            originals[k] = float(shard.rank_element(r, (k * 2654435761 + 12345) % count).item())
    # per step, only the events the phases need (fence-free timing events;
    # with --fenced-events each record adds about 5.7 us to the step): [0]
    # before the reduce, [1] before the separate check (--unfused), [2] before
    # AdamW, [3] after AdamW, [4] before the copy-in, [5] after the write-back
    def events():
        need = {0, 2, 3} | ({1} if args.unfused else set()) | ({4} if copy_in else set()) \
            | ({5} if write_back else set())
        make = ((lambda: torch.cuda.Event(enable_timing=True)) if fenced else TimingEvent)
        return [make() if i in need else None for i in range(6)]

    fenced = args.fenced_events
    if not fenced:
        try:
            TimingEvent.runtime()
        except (OSError, RuntimeError, AttributeError):
            fenced = True               # no handle on torch's HIP runtime: default events

    ev = [events() for _ in range(steps)]
    applied = 0
    infos = []
    last_sumsq = None
    graph = None
    t_before = None
    if shard.ctl is not None:
        shard.sync_control()
        t_before = shard.t
    if args.graph:
        # one captured step (copy-in, reduce+check windows, AdamW per owner,
        # control update, write-back), replayed: per-step events bracket each
        # replay, phases inside the graph are not separated
        graph = shard.capture(bufs, before=copy_in, after=write_back)
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    injections = 0
    for k in range(steps):
        Z.zero_partition_layout(wl.numels, wl.world, wl.align)
        if flush is not None:
            flush.fill_(float(k))                  # evicts the caches; outside the step's events
        planted = None
        if inject_every and (k + 1) % inject_every == 0:
            # a rank whose data the copy-in does not rewrite; seeded index.
            # After the step a fill restores the element (no device-to-device
            # copy)
            injections += 1
            r = 1 + (k % (shard.n_ranks - 1)) if shard.n_ranks > 1 else 0
            idx = (k * 2654435761 + 12345) % count
            bad = float("inf") if injections % 2 else float("nan")
            cell = shard.rank_element(r, idx)
            planted = (cell, originals[k])
            cell.fill_(bad)
        if graph is not None:
            ev[k][0].record()
            graph.replay()
            ev[k][3].record()
        else:
            if copy_in:
                ev[k][4].record()
                copy_in()
            info = one_step(marks=ev[k])
            if info is not None:
                applied += info.applied
                infos.append(info)
        if planted is not None:
            cell, value = planted
            cell.fill_(value)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    if shard.ctl is not None:
        shard.sync_control()
        applied = shard.t - t_before
        last_sumsq = Z.read_result(shard.res).sumsq

    if graph is not None:
        ms = {"step_graph": [e[0].elapsed_time(e[3]) for e in ev]}
        bytes_per = {"step_graph": 2 * wl.world + 30 + (2 if args.unfused else 0)
                     + (4 if copy_in else 0) + (4 if write_back else 0)}
    elif args.unfused:
        ms = {"reduce": [], "check": [], "adamw": []}
        for e in ev:
            ms["reduce"].append(e[0].elapsed_time(e[1]))
            ms["check"].append(e[1].elapsed_time(e[2]))
            ms["adamw"].append(e[2].elapsed_time(e[3]))
        bytes_per = {"reduce": 2 * wl.world + 2, "check": 2, "adamw": 28}
    else:
        ms = {"reduce_check": [], "adamw": []}
        for e in ev:
            ms["reduce_check"].append(e[0].elapsed_time(e[2]))
            ms["adamw"].append(e[2].elapsed_time(e[3]))
        bytes_per = {"reduce_check": 2 * wl.world + 2, "adamw": 28}
    if copy_in and graph is None:
        ms["copy_in"] = [e[4].elapsed_time(e[0]) for e in ev]
        bytes_per["copy_in"] = 4
    if write_back and graph is None:
        ms["write_back"] = [e[3].elapsed_time(e[5]) for e in ev]
        bytes_per["write_back"] = 4
    # steps that ran whole: an injected overflow makes AdamW return early, so
    # phase rates, the roofline and step_GBps average over the other steps only
    whole = [k for k in range(steps) if not (inject_every and (k + 1) % inject_every == 0)]
    phases = {}
    for k, v in ms.items():
        avg = float(np.mean([v[i] for i in whole]))
        phases[k] = {"ms": round(avg, 4), "bytes_per_elem": bytes_per[k],
                     "GBps": round(bytes_per[k] * count / (avg * 1e-3) / 1e9, 1)}
    # each step's own device time: from its first event (copy-in or reduce)
    # to its last (AdamW, or the write-back)
    first = 0 if (graph is not None or not copy_in) else 4
    last = 5 if (write_back and graph is None) else 3
    per_step = [e[first].elapsed_time(e[last]) for e in ev]
    if flush is not None:                          # the flushes sit between the steps' events
        total_ms = float(sum(per_step))
    step_ms = total_ms / steps
    whole_ms = step_ms if not inject_every else float(np.mean([per_step[i] for i in whole]))
    step_bytes = sum(bytes_per.values()) * count
    # the roofline entry is for the step's dominant kernel: AdamW on the LLaMA
    # shards (28 of 46 B per element), the fused reduce+check on the 16-rank
    # bucket group (34 of 62 B)
    roofline = None
    kernels = {"adamw": ("adamw_kernel", "adamw_kernel (zero_adamw_step)"),
               "reduce_check": ("reduce_kernel", "reduce_kernel (fused reduce+check; the phase "
                                                 "includes its fold and final pass)")}
    timed = {k: float(np.mean([ms[k][i] for i in whole])) for k in kernels if k in ms}
    if timed:
        dom = max(timed, key=timed.get)
        achieved = bytes_per[dom] * count / (timed[dom] * 1e-3) / 1e9
        roofline = {
            "bound": "hbm",
            "kernel": kernels[dom][1],
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(kernels[dom][0], workload),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, "
                            "factors from a known-size elementwise kernel)",
        }

    if shard.ctl is not None:
        shard.sync_control()
    shard_scale = shard.scale
    last = infos[-1].sumsq if infos else last_sumsq
    final_norm = float(np.sqrt(last)) if last is not None and np.isfinite(last) else None
    layout = ("separate allocations" if args.no_arena else
              f"one arena, buffer order {shard.placement}"
              + (" (fastest of the orders timed at setup)" if args.placement == "auto" else "")
              + (f", master / m / v at least {shard.fp32_gap / 2 ** 30:g} GiB apart"
                 if shard.fp32_gap else ""))
    rank_data = ("each reduce bucket's N rank slices back to back" if shard.rank_layout == "bucket"
                 else "one flat buffer per rank")
    reduced = "in place, in rank 0's buffer" if in_place else "a buffer of its own"
    out = {
        "value": count * applied / (total_ms * 1e-3),
        "ms_per_step": round(step_ms, 4),
        "config": {
            "workload": (f"{wl.name}-shaped owner-0 shard" if workload != "buckets" else
                         "10,000-tensor group, all owners, copy-in + bucketed reduce + AdamW"
                         + (" + write-back" if write_back else ""))
                        if rr_info is None else
                        f"{wl.name}-shaped, round-robin owner {rr_info['owner']} (whole tensors)",
            "round_robin": rr_info,
            "description": f"{wl.description}; rank data: {rank_data}; reduced gradient: "
                           f"{reduced}",
            "owned_elems": count,
            "ranks": wl.world,
            "grad_dtype": "bf16" if wl.dtype == Z.ZERO_BF16 else "fp16",
            "clip": wl.clip,
            "in_place_reduce": in_place,
            "rank_layout": shard.rank_layout,
            "reduce_windows": len(shard.reduce_ranges),
            "fused_reduce_check": not args.unfused,
            "range_list_calls": not args.no_batch,
            "step_control": "host (16-byte readback per step)" if args.host_control else
                            "device-resident (no per-step readback)",
            "graph": bool(args.graph),
            "phase_events": ("default (system-scope fence per record)" if fenced
                             else "fence-free timing events (hipEventDisableSystemFence)"),
            "flush_between_steps_gib": args.flush_gib,
            "inf_nan_every": inject_every,
            "placement": layout,
            "placement_search": args.placement == "auto",
            "placement_candidates": len(shard.placement_ms) or None,
            # the finalists' medians of three timed steps (the choice is their minimum)
            "placement_setup_ms": dict(sorted(getattr(shard, "placement_finalists_ms", {}).items(),
                                              key=lambda kv: kv[1])) or None,
            "arena_slack_gib": round(getattr(shard, "arena_slack", 0) / 2 ** 30, 3),
            "parallelism": "one owner partition on one GPU (N ranks simulated in HBM)",
        },
        "step_GBps": round(step_bytes / (whole_ms * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(step_bytes / (whole_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "phases": phases,
        "applied_steps": applied,
        "skipped_steps": steps - applied,
        "final_loss_scale": shard_scale,
        "per_step_ms": [round(x, 4) for x in per_step],
        "median_step_ms": round(float(np.median(per_step)), 4),
        # the last step's norm; null when that step overflowed (no finite norm)
        "final_norm": final_norm,
        "host_wall_s": round(wall, 4),
        "roofline": roofline,
        "_begin": begin,
    }
    for e in ev:
        for x in e:
            if isinstance(x, TimingEvent):
                x.destroy()
    # drop every reference to the shard's device memory before the next run
    planted = None
    del bufs, shard, flush, graph, planted, copy_in, write_back, one_step
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "runs on one GPU only: the owner-shard step is "
                          "measured on one GPU's partition; run with --gpus 1"}), file=sys.stderr)
        sys.exit(2)
    if args.steps is None:
        args.steps = 40 if args.workload == "buckets" else 20
    if args.inject_every is None:
        args.inject_every = 4 if args.workload == "buckets" else 0
    if args.inject_every < 0 or args.inject_every == 1:
        print(json.dumps({"error": "--inject-every takes 0 (off) or K >= 2, so that some "
                          "steps run whole"}), file=sys.stderr)
        sys.exit(2)
    if args.graph and args.host_control:
        print(json.dumps({"error": "--graph replays a step with device-resident control; it "
                          "cannot be combined with --host-control"}), file=sys.stderr)
        sys.exit(2)
    if args.write_back and args.workload != "buckets":
        print(json.dumps({"error": "--write-back applies to --workload buckets"}), file=sys.stderr)
        sys.exit(2)
    from synth import workloads as W

    run = run_workload(args, args.workload, args.steps, args.inject_every, calibrate=True)
    begin = run.pop("_begin")
    result = {
        "metric": "params updated/s per GPU (ZeRO shard AdamW step) + achieved HBM GB/s % of peak",
        "value": run.pop("value"),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": run.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
    }
    result.update(run)
    if args.secondary and args.secondary != args.workload:
        # a second shard in the same run, same options, its own JSON object;
        # then the same shard with its placement measured at setup (every
        # arena order at base offsets 4 GiB apart in 64 GiB of slack), which
        # finds physical addresses that suit it on the box at hand
        keep = ("value", "ms_per_step", "median_step_ms", "step_GBps", "step_frac_of_peak",
                "phases", "roofline", "applied_steps", "final_norm", "per_step_ms")

        def entry(sec):
            sec.pop("_begin")
            return {"workload": sec["config"]["workload"], "steps": args.secondary_steps,
                    "unit": "params/s", **{k: sec[k] for k in keep},
                    "config": {k: sec["config"][k] for k in
                               ("description", "owned_elems", "ranks", "placement", "rank_layout",
                                "reduce_windows", "in_place_reduce", "placement_search",
                                "placement_candidates", "arena_slack_gib")}}

        result["secondary"] = entry(run_workload(args, args.secondary, args.secondary_steps, 0))
        if not args.no_secondary_tuned and args.placement != "auto":
            fixed = (args.placement, args.arena_slack_gib)
            args.placement, args.arena_slack_gib = "auto", 64.0
            result["secondary_tuned"] = entry(run_workload(args, args.secondary,
                                                           args.secondary_steps, 0))
            args.placement, args.arena_slack_gib = fixed
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(W.WORKLOADS[args.workload], begin, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
