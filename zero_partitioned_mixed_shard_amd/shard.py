"""Owner-shard step driver: device buffers plus the ABI calls in order.

Holds the fp32 master / m / v, the 16-bit parameter copy, the reduced
gradient, the 16-byte step result and the check workspace for one simulated
region of the flat buffer (one owner's partition, or several owners'), and
runs one step as the library's calls:

  for each reduce window (bucket x owner)   zero_reduce_check_owned (windows after
                                            the first accumulate: one global
                                            flag and norm)
  for each owner                            zero_adamw_step (skips on overflow,
                                            on the device)
  16-byte readback                          zero_loss_scaler_update, t

With several reduce windows or owners (a bucketed group with all owners on
one GPU, round-robin ownership with one window per owned tensor) the fused
step makes one range-list call for all windows (zero_reduce_check_ranges)
and one for all owners (zero_adamw_step_ranges); the library merges ranges
that touch into one launch and folds the norm once.  batched=False keeps one
call per window and per owner.

With fused=False the reduce and the check are separate calls
(zero_reduce_owned per window, then zero_unscale_check_norm per owner).

Rank data.  With own_ranks=True the step holds the N ranks' 16-bit
gradients itself, in one of two layouts (`rank_layout`):
  flat    one buffer of the step's whole range per rank (rank_bufs);
  bucket  one block per reduce window holding that window's N rank slices
          back to back (rank_slices[w][r]), as the owner receives them bucket
          by bucket (ZeRO-2 source walkthrough section 4.2), reduced with one
          zero_reduce_check_buckets call.  On MI355X the 8-rank reduce over
          the LLaMA-70B shard ran at 6.42 TB/s on every base offset tried
          with 5e8-element buckets laid out this way, against 5.98-6.40 TB/s
          with eight whole-shard rank buffers.
fill_ranks() and rank_element() reach the rank data in either layout.

With device_control=True the loss scaler and the step count live on the
device (zero_step_control): the step runs the *_ctl calls and ends with
zero_step_control_update, so it needs no host round trip and can be
captured once in a HIP graph (capture()) and replayed; finish() only reads
the result and the control back for reporting.

Placement.  With own_ranks=True the step also holds the N simulated rank
buffers.  With arena=True every large buffer is carved from one device
allocation, in one of the orders of ARENA_ORDERS (`placement`):
  interleaved   the arrays AdamW streams (master, m, v, the 16-bit copy, the
                reduced gradient) with rank buffers between them;
  rank_block    16-bit copy, master, m, then all rank buffers in rank order
                (the reduced gradient right after them), then v;
  rank_block_b  master, m, 16-bit copy, rank buffers, reduced gradient, v;
  master_ranks  master, rank buffers, reduced gradient, m, v, 16-bit copy;
  streams_first the AdamW arrays, then the rank buffers;
  ranks_first   the rank buffers, then the AdamW arrays;
  spread        master, the rank data, the reduced gradient and the 16-bit
                copy, then m and v.
`min_gap` bytes additionally keeps the bases of master, m and v at least
that far apart (halved, down to 0, where the device cannot hold the arena):
over the LLaMA-7B shard AdamW ran at 6.3-6.4 TB/s with them 32 GiB apart in
every order, against 5.9-6.0 TB/s packed.  On MI355X the HBM bandwidth of both passes depends on where
the arrays sit in physical memory, which a process cannot see: the same
buffers at the same offsets run at different rates in arenas of different
sizes, and shifting the LLaMA-7B shard's whole layout by 4 GiB steps moves
its step between 5.9 and 6.4 ms.  With placement="auto" the step therefore
measures: it zeroes the arena, times one step of the real call sequence in
every candidate placement, then three more for each of the six fastest,
and keeps the one with the shortest median of those three
(`placement_ms` holds the first stage's times, `placement_finalists_ms` the
medians).  The candidates are the orders of
ARENA_ORDERS at the arena's start and, with `arena_slack` bytes (at most
what the device has free, less 4 GiB; the arena is that much larger), at
every PLACEMENT_STEP into the slack and at its end.  The cost is two steps
per candidate and 24 more at construction; the slack holds nothing.

Nothing here computes on the data; it sequences calls and keeps host scalars.
"""
from __future__ import annotations

import re
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import (RESULT_BYTES, ZERO_BF16, ZERO_FP16, control_to_device, read_control,
               read_result, zero_adamw_hparams, zero_adamw_step, zero_adamw_step_ctl,
               zero_check_workspace_bytes, zero_init_master, zero_loss_scaler,
               zero_loss_scaler_update, zero_reduce_check_owned, zero_reduce_check_owned_ctl,
               zero_reduce_owned, zero_step_control_init, zero_step_control_update,
               zero_unscale_check_norm, zero_unscale_check_norm_ctl, zero_adamw_step_ranges,
               zero_range_workspace_bytes, zero_reduce_check_buckets, zero_reduce_check_ranges)


def _interleaved(names, streams, in_place):
    """AdamW arrays with rank buffers between them (remaining ranks last)."""
    st = [nm for nm in names if nm in streams]
    rk = [nm for nm in names if nm not in streams]
    seq = []
    for k, nm in enumerate(st):
        seq.append(nm)
        if k < len(rk):
            seq.append(rk[k])
    return seq + rk[len(st):]


def _rank_block(head):
    """`head` arrays, all rank buffers in rank order, the separate reduced
    gradient, then the AdamW arrays not yet placed."""
    def order(names, streams, in_place):
        rk = _rank_names(names)
        first = [nm for nm in head if nm in names]
        red = ["red"] if "red" in names else []
        rest = [nm for nm in names if nm not in first and nm not in rk and nm not in red]
        return first + rk + red + rest
    return order


def _rank_names(names):
    """The rank-data buffers (one per rank, or one per reduce window) in order."""
    return sorted((nm for nm in names if nm.startswith("rank")),
                  key=lambda x: int(re.search(r"\d+$", x).group()))


def _streams_first(names, streams, in_place):
    """The AdamW arrays (and a separate reduced gradient), then the ranks."""
    return [nm for nm in names if not nm.startswith("rank")] + _rank_names(names)


def _ranks_first(names, streams, in_place):
    """The rank buffers, then the AdamW arrays."""
    return _rank_names(names) + [nm for nm in names if not nm.startswith("rank")]


def _spread(names, streams, in_place):
    """master, the rank data, the reduced gradient and the 16-bit copy, then
    m and v (with a min_gap, the space between master and m holds the rank
    data)."""
    head = [nm for nm in ("master",) if nm in names]
    mid = [nm for nm in ("red", "param16") if nm in names]
    tail = [nm for nm in ("exp_avg", "exp_avg_sq") if nm in names]
    return head + _rank_names(names) + mid + tail


# Spacing of the base offsets at which a measured placement tries each
# order inside the arena's slack.
PLACEMENT_STEP = 4 << 30

# The arrays a min_gap keeps apart: AdamW's fp32 state.  On MI355X AdamW over
# a LLaMA-7B-sized shard ran at 6.22-6.41 TB/s with master, m and v 24-48 GiB
# apart at any base offset tried, against 5.5-6.0 TB/s with them 3-12 GiB
# apart (most bases); the reduce's rank data ran fastest packed together.
FP32_ARRAYS = ("master", "exp_avg", "exp_avg_sq")

# Buffer orders an arena can be laid out in (see the module docstring).
ARENA_ORDERS = {
    "interleaved": _interleaved,
    "rank_block": _rank_block(["param16", "master", "exp_avg"]),
    "rank_block_b": _rank_block(["master", "exp_avg", "param16"]),
    "master_ranks": _rank_block(["master"]),
    "streams_first": _streams_first,
    "ranks_first": _ranks_first,
    "spread": _spread,
}


@dataclass
class StepInfo:
    overflow: int
    sumsq: float
    applied: bool
    scale_used: float
    t: int


class ShardStep:
    """State and step of the owners whose partitions lie in [begin, end)."""

    def __init__(self, begin: int, end: int, owners: Sequence[Tuple[int, int]], dtype: int,
                 lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=0.0,
                 scale0=1.0, min_scale=1.0, window=1000, windows: Optional[Sequence[Tuple[int, int]]] = None,
                 divisor: int = 1, in_place_rank: Optional[int] = None, fused: bool = True,
                 own_ranks: bool = False, world: int = 0, arena: bool = False,
                 min_gap: int = 0, device_control: bool = False, placement: str = "interleaved",
                 arena_slack: int = 0, batched: bool = True, rank_layout: str = "flat",
                 device="cuda"):
        self.begin, self.end = begin, end
        self.count = end - begin
        self.owners = [(a - begin, b - begin) for a, b in owners]
        for a, b in self.owners:
            assert 0 <= a <= b <= self.count
        self.dtype = dtype
        self.tdtype = torch.float16 if dtype == ZERO_FP16 else torch.bfloat16
        self.hp = zero_adamw_hparams(lr, beta1, beta2, eps, weight_decay, max_grad_norm, 0)
        self.scaler = zero_loss_scaler(scale0, min_scale, window, 0, 0)
        self.divisor = divisor
        self.t = 0
        self.in_place_rank = in_place_rank
        self.fused = fused
        # reduce windows = buckets intersected with owner partitions
        bounds = [(begin, end)] if windows is None else windows
        self.reduce_ranges = []
        for a, b in self.owners:
            for wa, wb in bounds:
                lo, hi = max(a, wa - begin), min(b, wb - begin)
                if lo < hi:
                    self.reduce_ranges.append((lo, hi))
        n = self.count
        n_ranks = world if own_ranks else 0
        if own_ranks and world < 1:
            raise ValueError("own_ranks needs world >= 1")
        if placement != "auto" and placement not in ARENA_ORDERS:
            raise ValueError(f"placement: one of {sorted(ARENA_ORDERS)} or 'auto'")
        if rank_layout not in ("flat", "bucket"):
            raise ValueError("rank_layout: 'flat' or 'bucket'")
        if rank_layout == "bucket" and (not own_ranks or in_place_rank is not None or not fused):
            raise ValueError("the bucket rank layout needs own_ranks, a reduced buffer of its own "
                             "and the fused reduce+check")
        self.rank_layout = rank_layout
        self.n_ranks = n_ranks
        self.res = torch.zeros(RESULT_BYTES // 4, dtype=torch.int32, device=device)
        self.ctl = None
        # several reduce windows / owners: one range-list call each instead
        # of one call per range (fused path)
        self.batched = batched
        self._reduce_list = [(a, b - a) for a, b in self.reduce_ranges]
        self._owner_list = [(a, b - a) for a, b in self.owners]
        spans = [b - a for a, b in self.owners] + [b - a for a, b in self.reduce_ranges]
        ws = max(zero_check_workspace_bytes(n) for n in spans) if spans else 64
        if batched and (len(self._reduce_list) > 1 or rank_layout == "bucket"):
            ws = max(ws, zero_range_workspace_bytes(self._reduce_list))
        self.workspace = torch.empty((ws + 7) // 8, dtype=torch.float64, device=device)
        self.placement = placement if arena else "separate"
        self.placement_ms = {}                  # first stage: one timed step per candidate
        self.placement_finalists_ms = {}        # second stage: median of three, six fastest
        self.arena_slack = 0
        self.fp32_gap = 0                       # distance kept between master, m and v
        self._allocate(n, n_ranks, in_place_rank is None, arena, min_gap, placement,
                       arena_slack, device)
        self.exp_avg.zero_()
        self.exp_avg_sq.zero_()
        if device_control:
            self.ctl = control_to_device(zero_step_control_init(
                scale0, min_scale, window, float(divisor), beta1, beta2), device=device)

    # ----------------------------------------------------------- placement
    def _allocate(self, n, n_ranks, separate_red, arena, min_gap, placement, slack, device):
        f32, b16 = torch.float32, self.tdtype
        # name -> (dtype, elements)
        streams = {"master": (f32, n), "exp_avg": (f32, n), "exp_avg_sq": (f32, n),
                   "param16": (b16, n)}
        if separate_red:
            streams["red"] = (b16, n)
        ranks = {}
        self._rank_geom = []
        if self.rank_layout == "bucket":
            # one block per reduce window holding its N rank slices back to
            # back; slice r starts at r*stride + lead, with lead = the window's
            # offset mod 8, so that every slice has the reduced buffer's
            # 16-byte phase at that offset (the vector path needs a common one)
            for w, (a, b) in enumerate(self.reduce_ranges):
                lead = a % 8
                stride = (lead + (b - a) + 7) // 8 * 8
                self._rank_geom.append((lead, stride))
                ranks[f"rankw{w}"] = (b16, n_ranks * stride)
        else:
            for r in range(n_ranks):
                ranks[f"rank{r}"] = (b16, n)
        kinds = {**streams, **ranks}
        if not arena:
            self._set_views({name: torch.empty(cnt, dtype=dt, device=device)
                             for name, (dt, cnt) in kinds.items()})
            return
        sizes = {name: cnt * torch.tensor([], dtype=dt).element_size()
                 for name, (dt, cnt) in kinds.items()}
        names = list(kinds)
        stream_set = set(streams)
        if self.in_place_rank is not None and self.in_place_rank < n_ranks:
            # the reduced gradient lives in the owner's own rank buffer: an AdamW stream
            stream_set.add(f"rank{self.in_place_rank}")
        free, _ = torch.cuda.mem_get_info(device)
        orders = ARENA_ORDERS if placement == "auto" else {placement: ARENA_ORDERS[placement]}
        plans = {}
        gaps = {}
        for name, order_fn in orders.items():
            seq = order_fn(names, stream_set, self.in_place_rank)
            assert sorted(seq) == sorted(names), (name, seq)
            # the widest of min_gap, min_gap / 2, min_gap / 4 and 0 between
            # the bases of master, m and v that leaves 4 GiB of the device free
            for gap in (min_gap, min_gap // 2, min_gap // 4, 0):
                plan = self._place(seq, sizes, set(FP32_ARRAYS), gap)
                if plan[1] + (4 << 30) <= free or gap == 0:
                    break
            plans[name], gaps[name] = plan, gap
        size = max(end for _, end in plans.values())
        # slack: unused bytes at one end of the arena, up to what the device
        # has free (4 GiB kept back); the buffers start at the arena's start
        # or `slack` bytes in, which moves them to other physical addresses
        align = 1 << 16
        if slack > 0:
            slack = max(0, min(int(slack), free - size - (4 << 30))) // align * align
        self.arena_slack = slack
        if slack > 0:
            # every order also at bases every PLACEMENT_STEP bytes into the
            # slack, and at its end
            bases = list(range(PLACEMENT_STEP, slack, PLACEMENT_STEP)) + [slack]
            for name in list(plans):
                offs, end = plans[name]
                for b in bases:
                    plans[f"{name}@+{b / 2 ** 30:g}GiB"] = (
                        {k: v + b for k, v in offs.items()}, end + b)
        self.arena = torch.empty(max(size + slack, 1), dtype=torch.uint8, device=device)
        self._kinds, self._sizes = kinds, sizes
        if len(plans) == 1 or n_ranks == 0:
            best = next(iter(plans))
        else:
            best = self._tune(plans)
        self.placement = best
        self.fp32_gap = gaps[best.split("@")[0]]
        self.placement_offsets = dict(plans[best][0])
        self._set_views(self._carve(plans[best][0]))

    @staticmethod
    def _place(seq, sizes, gap_set, min_gap):
        """Byte offsets of the buffers laid out in `seq` order (64 KiB
        aligned), each buffer of `gap_set` at least `min_gap` after the base
        of the previous one; -> (offsets, end)."""
        align = 1 << 16
        offs, cur, last = {}, 0, None
        for name in seq:
            gapped = name in gap_set
            if gapped and last is not None:
                cur = max(cur, last + min_gap)
            cur = (cur + align - 1) // align * align
            offs[name] = cur
            if gapped:
                last = cur
            cur += sizes[name]
        return offs, cur

    def _carve(self, offs):
        return {name: self.arena[o:o + self._sizes[name]].view(self._kinds[name][0])
                for name, o in offs.items()}

    def _set_views(self, bufs):
        self.master, self.exp_avg, self.exp_avg_sq = bufs["master"], bufs["exp_avg"], bufs["exp_avg_sq"]
        self.param16 = bufs["param16"]
        self.red = bufs.get("red")
        if self.rank_layout == "bucket":
            self.rank_bufs = None
            self.rank_slices = []
            for w, (a, b) in enumerate(self.reduce_ranges):
                blk = bufs[f"rankw{w}"]
                lead, stride = self._rank_geom[w]
                self.rank_slices.append([blk[r * stride + lead:r * stride + lead + (b - a)]
                                         for r in range(self.n_ranks)])
        else:
            self.rank_bufs = [bufs[f"rank{r}"] for r in range(self.n_ranks)]
            self.rank_slices = None

    def _tune(self, plans) -> str:
        """Times the step's own calls (reduce windows, check, AdamW per owner)
        in every candidate placement on a zeroed arena and returns the
        fastest: one warm-up and one timed step each, then the median of
        three more for the six fastest.  Zero gradients raise no overflow, so every pass
        runs whole.  (On MI355X a zeroed arena runs the step 0.5-1 % faster
        than gradient data, in every placement alike: the choice is the
        same.)"""
        self.arena.zero_()
        for name, (offs, _) in plans.items():
            self._set_views(self._carve(offs))
            self.launch()
            self.placement_ms[name] = self._time_steps(1)
        # the shortest of many single samples is biased low: the finalists are
        # compared by the median of three fresh steps each
        finals = {}
        for name in sorted(self.placement_ms, key=self.placement_ms.get)[:6]:
            self._set_views(self._carve(plans[name][0]))
            self.launch()
            finals[name] = self._time_steps(3, median=True)
        self.placement_finalists_ms = finals
        return min(finals, key=finals.get)

    def _time_steps(self, k: int, median: bool = False) -> float:
        """Shortest (or median) of k timed launches of the step's calls (ms)."""
        times = []
        for _ in range(k):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            self.launch()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b))
        return round(float(np.median(times)) if median else min(times), 4)

    # ---------------------------------------------------------------- state
    def load_param16(self, param16: torch.Tensor) -> None:
        """Initial state: the 16-bit copy, fp32 master = its float, m = v = 0.
        `param16` may be self.param16 itself (filled in place)."""
        if param16.data_ptr() != self.param16.data_ptr():
            self.param16.copy_(param16)
        zero_init_master(self.master, self.param16)
        self.exp_avg.zero_()
        self.exp_avg_sq.zero_()

    @property
    def scale(self) -> float:
        return self.scaler.scale

    @property
    def inv_scale(self) -> float:
        return 1.0 / (self.scaler.scale * self.divisor)

    # ----------------------------------------------------------------- step
    def reduced(self, rank_bufs: Optional[Sequence[torch.Tensor]] = None) -> torch.Tensor:
        if rank_bufs is None:
            rank_bufs = self.rank_bufs
        return rank_bufs[self.in_place_rank] if self.red is None else self.red

    def fill_ranks(self, fill) -> None:
        """Write the step's own rank data: fill(r, a, b, out) stores rank r's
        gradient for shard elements [a, b) into the 16-bit tensor `out`.  It
        is called once per rank (flat layout) or once per rank and reduce
        window (bucket layout)."""
        if self.rank_layout == "bucket":
            for w, (a, b) in enumerate(self.reduce_ranges):
                for r in range(self.n_ranks):
                    fill(r, a, b, self.rank_slices[w][r])
        else:
            for r, buf in enumerate(self.rank_bufs):
                fill(r, 0, self.count, buf)

    def rank_element(self, r: int, i: int) -> torch.Tensor:
        """One-element view of rank r's gradient at shard element i (which must
        lie in a reduce window under the bucket layout)."""
        if self.rank_layout == "bucket":
            for w, (a, b) in enumerate(self.reduce_ranges):
                if a <= i < b:
                    return self.rank_slices[w][r][i - a:i - a + 1]
            raise IndexError(f"element {i} lies in no reduce window")
        return self.rank_bufs[r][i:i + 1]

    def launch(self, rank_bufs: Optional[Sequence[torch.Tensor]] = None,
               marks: Optional[List] = None) -> None:
        """Enqueue reduce -> check -> AdamW on the current stream (and, with
        device control, the control update).  `marks` (4 events, any of them
        None) are recorded before the reduce, before the separate check
        (fused=False only), before AdamW and after AdamW (before the control
        update).  Without rank_bufs the step's own rank data are used."""

        def mark(i):
            if marks and marks[i] is not None:
                marks[i].record()

        bucket = rank_bufs is None and self.rank_layout == "bucket"
        if rank_bufs is None:
            rank_bufs = self.rank_bufs
        red = self.reduced(rank_bufs)
        ctl = self.ctl
        inv = self.inv_scale
        mark(0)
        if bucket and self.batched:
            # every window's own rank slices, one call, one fold of the norm
            zero_reduce_check_buckets(red, self._reduce_list, self.rank_slices, inv, self.res,
                                      self.workspace, ctl_dev=ctl)
        elif self.fused and self.batched and not bucket and len(self._reduce_list) > 1:
            zero_reduce_check_ranges(red, rank_bufs, self._reduce_list, inv, self.res,
                                     self.workspace, ctl_dev=ctl)
        elif self.fused:
            for k, (a, b) in enumerate(self.reduce_ranges):
                srcs = self.rank_slices[k] if bucket else [r[a:b] for r in rank_bufs]
                if ctl is None:
                    zero_reduce_check_owned(red[a:b], srcs, inv, self.res, self.workspace,
                                            accumulate=k > 0)
                else:
                    zero_reduce_check_owned_ctl(red[a:b], srcs, ctl, self.res, self.workspace,
                                                accumulate=k > 0)
        else:
            for a, b in self.reduce_ranges:
                zero_reduce_owned(red[a:b], [r[a:b] for r in rank_bufs])
            mark(1)
            for k, (a, b) in enumerate(self.owners):
                if ctl is None:
                    zero_unscale_check_norm(red[a:b], inv, self.res, self.workspace,
                                            accumulate=k > 0)
                else:
                    zero_unscale_check_norm_ctl(red[a:b], ctl, self.res, self.workspace,
                                                accumulate=k > 0)
        mark(2)
        self.hp.step = self.t + 1
        if self.batched and len(self._owner_list) > 1:
            zero_adamw_step_ranges(self.master, self.exp_avg, self.exp_avg_sq, self.param16, red,
                                   self._owner_list, self.hp, self.res, ctl_dev=ctl)
        else:
            for a, b in self.owners:
                args = (self.master[a:b], self.exp_avg[a:b], self.exp_avg_sq[a:b],
                        self.param16[a:b], red[a:b], self.hp)
                if ctl is None:
                    zero_adamw_step(*args, self.res)
                else:
                    zero_adamw_step_ctl(*args, ctl, self.res)
        mark(3)
        if ctl is not None:
            zero_step_control_update(ctl, self.res)

    def finish(self) -> StepInfo:
        """Read the 16-byte result (synchronises) and update t and the scaler
        (with device control: read them back from the device)."""
        r = read_result(self.res)
        used = self.scaler.scale
        applied = not r.overflow
        if self.ctl is not None:
            self.sync_control()
        else:
            if applied:
                self.t += 1
            zero_loss_scaler_update(self.scaler, r.overflow)
        return StepInfo(int(r.overflow), float(r.sumsq), applied, used, self.t)

    def sync_control(self) -> None:
        """Host copies of the device control's scale, counters and t
        (synchronises the stream)."""
        c = read_control(self.ctl)
        self.scaler.scale, self.scaler.clean, self.scaler.skipped = c.scale, c.clean, c.skipped
        self.t = c.t

    def capture(self, rank_bufs: Optional[Sequence[torch.Tensor]] = None,
                before=None, after=None) -> "torch.cuda.CUDAGraph":
        """One whole step (optionally preceded by before(), e.g. a copy-in,
        and followed by after(), e.g. a write-back) captured in a HIP graph;
        each replay runs the next step.  Needs device_control=True: every
        per-step scalar is read on the device."""
        if self.ctl is None:
            raise ValueError("capture() needs device_control=True")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            if before is not None:
                before()
            self.launch(rank_bufs)
            if after is not None:
                after()
        return g

    def step(self, rank_bufs: Optional[Sequence[torch.Tensor]] = None,
             marks: Optional[List] = None) -> StepInfo:
        self.launch(rank_bufs, marks)
        return self.finish()
