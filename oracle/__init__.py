"""Plain CPU oracle for the ZeRO-1/2 owner-shard step.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` leg may import this package.  The product library
(``zero_partitioned_mixed_shard_amd``) never imports it, and it never imports
the product library: the two share no code.

The per-element work is in ``oracle.c`` (scalar C, built with gcc
``-O2 -ffp-contract=off``); this module loads it with ctypes, adds the
pages' memory closed forms and the step driver that strings the phases
together in the pages' order:

  reduce to the owner -> unscale + overflow check + norm -> clip -> AdamW on
  the fp32 partition -> 16-bit copy -> loss-scale update

Sources (cited by page title and section):
  * ZeRO 优化器 (cookllm.com): "训练状态的冗余分析" (16 bytes per parameter),
    "ZeRO Stage 1/2/3" memory tables, the reduce-to-owner training loop.
  * ZeRO / DeepSpeed 深度解读报告: section 2.1 (memory table), section 3.3
    (per-device memory formulas).
  * ZeRO-2 source walkthrough (discosf.com): sections 2.1, 4.1-4.4
    (flatten + align + partition, fp32 master clone, bucketed reduce,
    per-partition step, all-gather), section 三 (16-bit reduce-scatter).
  * wmrh.cn ZeRO article: section 2.1 (BERT-base byte counts), section 2.2
    (per-stage savings), section 3.1 (AdamW and fp16 loss-scale settings),
    section 3.3 (gradient_clipping).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from fractions import Fraction
from typing import List, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

FP16 = 1
BF16 = 2

OK, EINVAL, ERANGE = 0, -1, -2


def build() -> None:
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
         "-o", LIB, os.path.join(HERE, "oracle.c"), "-lm"],
        check=True)


class _HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("max_grad_norm", ctypes.c_float), ("step", ctypes.c_int64)]


class _Consts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_float) for n in
                ("decay", "b1", "omb1", "b2", "omb2", "bc1", "bc2", "lr", "eps")]


class _Scaler(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_double), ("min_scale", ctypes.c_double),
                ("window", ctypes.c_int64), ("clean", ctypes.c_int64),
                ("skipped", ctypes.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB)
        P, i64, i32, f32, f64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_float, ctypes.c_double)
        L.oracle_decode16.argtypes = [P, P, i64, i32]
        L.oracle_encode16_from_f32.argtypes = [P, P, i64, i32]
        L.oracle_encode16_from_f64.argtypes = [P, P, i64, i32]
        L.oracle_layout.argtypes = [P, i64, i32, i32, P, P, P]
        L.oracle_layout.restype = ctypes.c_int
        L.oracle_buckets.argtypes = [P, i64, i64, P, P]
        L.oracle_buckets.restype = ctypes.c_int
        L.oracle_reduce.argtypes = [P, P, i32, i64, i32]
        L.oracle_check.argtypes = [P, i64, i32, f32, P, P]
        L.oracle_clip_coef.argtypes = [f32, f64]
        L.oracle_clip_coef.restype = f32
        L.oracle_adam_consts_for.argtypes = [P, P]
        L.oracle_adamw.argtypes = [P, P, P, P, P, i64, i32, f32, f64, ctypes.c_uint32, P]
        L.oracle_adamw_f64.argtypes = [P, P, P, P, i64, i32, f64, f64, P, P, P, P]
        L.oracle_init_master.argtypes = [P, P, i64, i32]
        L.oracle_scaler_update.argtypes = [P, ctypes.c_uint32]
        L.oracle_flat_gather.argtypes = [P, i64, P, P, P, i64]
        L.oracle_flat_scatter.argtypes = [P, P, P, P, i64]
        for name in ("oracle_decode16", "oracle_encode16_from_f32", "oracle_encode16_from_f64",
                     "oracle_reduce", "oracle_check", "oracle_adam_consts_for", "oracle_adamw",
                     "oracle_adamw_f64", "oracle_init_master", "oracle_scaler_update",
                     "oracle_flat_gather", "oracle_flat_scatter"):
            getattr(L, name).restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


# --------------------------------------------------------------------------
# 16-bit converters (from the format definitions in oracle.c)
# --------------------------------------------------------------------------
def decode16(bits: np.ndarray, dtype: int) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    lib().oracle_decode16(_p(bits), _p(out), bits.size, dtype)
    return out


def encode16(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round fp32 or fp64 values to 16-bit patterns, ties to even."""
    x = np.ascontiguousarray(x)
    out = np.empty(x.shape, dtype=np.uint16)
    if x.dtype == np.float32:
        lib().oracle_encode16_from_f32(_p(x), _p(out), x.size, dtype)
    elif x.dtype == np.float64:
        lib().oracle_encode16_from_f64(_p(x), _p(out), x.size, dtype)
    else:
        raise TypeError(x.dtype)
    return out


# --------------------------------------------------------------------------
# Layout
# --------------------------------------------------------------------------
def layout(numels: Sequence[int], world: int, align: int):
    """-> (tensor_offsets[n], part_begin[world+1], padded_total)."""
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    offs = np.zeros(max(1, numels.size), dtype=np.int64)
    parts = np.zeros(world + 1 if world >= 1 else 1, dtype=np.int64)
    padded = np.zeros(1, dtype=np.int64)
    rc = lib().oracle_layout(_p(numels), numels.size, world, align, _p(offs), _p(parts),
                             _p(padded))
    if rc != OK:
        raise ValueError(f"oracle_layout: status {rc}")
    return offs[:numels.size].copy(), parts, int(padded[0])


def buckets(numels: Sequence[int], cap: int) -> np.ndarray:
    """-> bucket_first[n_buckets + 1] (first tensor of each bucket)."""
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    first = np.zeros(numels.size + 1, dtype=np.int64)
    nb = np.zeros(1, dtype=np.int64)
    rc = lib().oracle_buckets(_p(numels), numels.size, cap, _p(first), _p(nb))
    if rc != OK:
        raise ValueError(f"oracle_buckets: status {rc}")
    return first[:int(nb[0]) + 1].copy()


# --------------------------------------------------------------------------
# Bucket copy-in (gather into the flat buffer) and write-back (scatter out)
# --------------------------------------------------------------------------
def flat_gather(tensors: Sequence[np.ndarray], offsets: Sequence[int], flat_count: int,
                out: np.ndarray | None = None) -> np.ndarray:
    """Whole flat buffer (written into `out` when given): tensors at their
    offsets, 0 everywhere else."""
    ts = [np.ascontiguousarray(t, dtype=np.uint16) for t in tensors]
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    numel = np.array([t.size for t in ts], dtype=np.int64)
    assert offs.size == len(ts)
    assert all(o >= 0 and o + n <= flat_count for o, n in zip(offs, numel))
    ptrs = (ctypes.c_void_p * max(1, len(ts)))(*[_p(t) for t in ts])
    flat = np.empty(flat_count, dtype=np.uint16) if out is None else out
    assert flat.dtype == np.uint16 and flat.size == flat_count and flat.flags.c_contiguous
    lib().oracle_flat_gather(_p(flat), flat_count, ptrs, _p(offs), _p(numel), len(ts))
    return flat


def flat_scatter(flat: np.ndarray, offsets: Sequence[int], numels: Sequence[int]) -> list:
    flat = np.ascontiguousarray(flat, dtype=np.uint16)
    offs = np.ascontiguousarray(offsets, dtype=np.int64)
    numel = np.ascontiguousarray(numels, dtype=np.int64)
    assert all(o >= 0 and o + n <= flat.size for o, n in zip(offs, numel))
    outs = [np.empty(int(n), dtype=np.uint16) for n in numel]
    ptrs = (ctypes.c_void_p * max(1, len(outs)))(*[_p(t) for t in outs])
    lib().oracle_flat_scatter(_p(flat), ptrs, _p(offs), _p(numel), len(outs))
    return outs


# --------------------------------------------------------------------------
# Memory closed forms, bytes per rank (ZeRO 优化器 memory tables; ZeRO /
# DeepSpeed 深度解读报告 section 3.3).  16-bit parameters (2 B) and gradients
# (2 B), fp32 master + m + v (12 B).  Stage 0 is plain data parallelism.
# With a padded layout the sharded parts hold P = padded / N elements.
# --------------------------------------------------------------------------
def memory_bytes(stage: int, phi: int, world: int, padded: int | None = None) -> Fraction:
    if stage not in (0, 1, 2, 3):
        raise ValueError(stage)
    part = Fraction(phi if padded is None else padded, world)
    params = 2 * (part if stage >= 3 else phi)
    grads = 2 * (part if stage >= 2 else phi)
    optim = 12 * (part if stage >= 1 else phi)
    return params + grads + optim


# --------------------------------------------------------------------------
# The step phases
# --------------------------------------------------------------------------
def reduce(srcs: Sequence[np.ndarray], dtype: int, out: np.ndarray | None = None) -> np.ndarray:
    srcs = [np.ascontiguousarray(s, dtype=np.uint16) for s in srcs]
    n = srcs[0].size
    assert all(s.size == n for s in srcs)
    ptrs = (ctypes.c_void_p * len(srcs))(*[_p(s) for s in srcs])
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == n and out.flags.c_contiguous
    lib().oracle_reduce(_p(out), ptrs, len(srcs), n, dtype)
    return out


def check(red: np.ndarray, dtype: int, inv_scale: float, overflow: int = 0, sumsq: float = 0.0):
    """-> (overflow, sumsq), accumulated onto the given starting values.
    inv_scale is taken as an fp32 value."""
    red = np.ascontiguousarray(red, dtype=np.uint16)
    fl = np.array([overflow], dtype=np.uint32)
    ss = np.array([sumsq], dtype=np.float64)
    lib().oracle_check(_p(red), red.size, dtype, inv_scale, _p(fl), _p(ss))
    return int(fl[0]), float(ss[0])


def clip_coef(max_norm: float, sumsq: float) -> float:
    return float(lib().oracle_clip_coef(max_norm, sumsq))


@dataclass
class HParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_grad_norm: float = 0.0

    def c(self, step: int) -> _HParams:
        return _HParams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                        self.max_grad_norm, step)


def adam_consts(hp: HParams, step: int) -> dict:
    h = hp.c(step)
    c = _Consts()
    lib().oracle_adam_consts_for(ctypes.byref(h), ctypes.byref(c))
    return {n: getattr(c, n) for n, _ in _Consts._fields_}


def adamw(master, exp_avg, exp_avg_sq, param16, red, dtype, inv_scale, sumsq, overflow,
          hp: HParams, step: int) -> None:
    """In place.  `step` is t after this step's increment."""
    n = red.size
    for a in (master, exp_avg, exp_avg_sq):
        assert a.dtype == np.float32 and a.size == n and a.flags.c_contiguous
    assert param16.dtype == np.uint16 and param16.size == n
    red = np.ascontiguousarray(red, dtype=np.uint16)
    h = hp.c(step)
    lib().oracle_adamw(_p(master), _p(exp_avg), _p(exp_avg_sq), _p(param16), _p(red), n, dtype,
                       inv_scale, sumsq, overflow, ctypes.byref(h))


def adamw_f64(master, exp_avg, exp_avg_sq, red, dtype, inv_scale, coef, hp: HParams, step: int):
    n = red.size
    outs = [np.empty(n, dtype=np.float64) for _ in range(3)]
    h = hp.c(step)
    lib().oracle_adamw_f64(_p(master), _p(exp_avg), _p(exp_avg_sq),
                           _p(np.ascontiguousarray(red, dtype=np.uint16)), n, dtype, inv_scale,
                           coef, ctypes.byref(h), *[_p(o) for o in outs])
    return outs


def init_master(param16: np.ndarray, dtype: int) -> np.ndarray:
    param16 = np.ascontiguousarray(param16, dtype=np.uint16)
    out = np.empty(param16.size, dtype=np.float32)
    lib().oracle_init_master(_p(out), _p(param16), param16.size, dtype)
    return out


@dataclass
class Scaler:
    scale: float
    min_scale: float = 1.0
    window: int = 1000
    clean: int = 0
    skipped: int = 0

    def update(self, overflow: int) -> None:
        s = _Scaler(self.scale, self.min_scale, self.window, self.clean, self.skipped)
        lib().oracle_scaler_update(ctypes.byref(s), overflow)
        self.scale, self.clean, self.skipped = s.scale, s.clean, s.skipped


@dataclass
class OwnerState:
    """fp32 master / m / v and the 16-bit copy of one owner's partition."""
    master: np.ndarray
    exp_avg: np.ndarray
    exp_avg_sq: np.ndarray
    param16: np.ndarray

    @classmethod
    def from_param16(cls, param16: np.ndarray, dtype: int) -> "OwnerState":
        n = param16.size
        return cls(init_master(param16, dtype), np.zeros(n, np.float32), np.zeros(n, np.float32),
                   np.array(param16, dtype=np.uint16, copy=True))

    def copy(self) -> "OwnerState":
        return OwnerState(self.master.copy(), self.exp_avg.copy(), self.exp_avg_sq.copy(),
                          self.param16.copy())


@dataclass
class StepResult:
    overflow: int
    sumsq: float
    applied: bool
    scale_used: float
    reduced: List[np.ndarray] = field(default_factory=list)


def step(owners: Sequence[OwnerState], grads: Sequence[Sequence[np.ndarray]], dtype: int,
         hp: HParams, scaler: Scaler, t: int, divisor: int = 1):
    """One owner-shard step for one or more owners whose partitions are all
    simulated (grads[k] = the N ranks' gradient slices for owner k).

    Returns (StepResult, new t).  The norm and the overflow flag are global
    over the given owners, as the owners would agree on them before the
    update.  An overflow skips the update and leaves t unchanged.
    """
    inv = float(np.float32(1.0 / (scaler.scale * divisor)))   # fp32(1/(S*D))
    reduced = [reduce(g, dtype) for g in grads]
    overflow, sumsq = 0, 0.0
    for red in reduced:
        overflow, sumsq = check(red, dtype, inv, overflow, sumsq)
    applied = not overflow
    if applied:
        t = t + 1
        for st, red in zip(owners, reduced):
            adamw(st.master, st.exp_avg, st.exp_avg_sq, st.param16, red, dtype, inv, sumsq,
                  overflow, hp, t)
    res = StepResult(overflow, sumsq, applied, scaler.scale, reduced)
    scaler.update(overflow)
    return res, t
