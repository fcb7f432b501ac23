"""Seeded synthetic inputs, identical on host and device.

Test and benchmark infrastructure shared by the oracle side and the HIP side;
it holds none of the method's arithmetic.  The generator itself is defined
once in ``synth_core.h`` (SplitMix64 hash -> Irwin-Hall-4 integer draw ->
exact 16-bit encoding of ``x * 2**e``); ``libsynth_host.so`` runs it on the CPU
and ``libsynth_dev.so`` on the GPU, so any element of any rank's gradient at
any step can be regenerated anywhere without copying it between them.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth_host.so")
DEV_LIB = os.path.join(HERE, "libsynth_dev.so")

FP16 = 1
BF16 = 2
_FMT = {FP16: (5, 10), BF16: (8, 7)}

# stream kinds
KIND_INIT = 1
KIND_GRAD = 2
KIND_INJECT = 3
KIND_SIZES = 4

# standard deviation of the centred Irwin-Hall-4 sum of 16-bit uniforms
IH4_SD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)


def build(hipcc: str = "/opt/rocm/bin/hipcc", device: bool = True) -> None:
    """Compile the host generator (gcc) and, if asked, the device one (hipcc)."""
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", HOST_LIB,
         os.path.join(HERE, "synth_host.c")],
        check=True)
    if device:
        subprocess.run(
            [hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-o", DEV_LIB, os.path.join(HERE, "synth_dev.hip")],
            check=True)


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64] * 4
        lib.synth_hash64.restype = ctypes.c_uint64
        lib.synth_hash64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_fill.restype = None
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                   ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32]
        lib.synth_gather.restype = None
        lib.synth_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is missing: run __graft_entry__.build() first")
        import torch  # noqa: F401  (bind to the HIP runtime torch loaded)
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_dev_fill.restype = ctypes.c_int
        lib.synth_dev_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                       ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        _dev = lib
    return _dev


@dataclass(frozen=True)
class NormalSpec:
    """Values x * 2**e with x = (Irwin-Hall-4 draw) * mult >> 16; sd ~ sigma."""
    mult: int
    e: int
    dtype: int

    @property
    def sigma(self) -> float:
        return IH4_SD * self.mult / 65536.0 * 2.0 ** self.e

    @property
    def max_abs_int(self) -> int:
        return (131070 * self.mult) >> 16

    @property
    def max_abs(self) -> float:
        return self.max_abs_int * 2.0 ** self.e


def normal_spec(sigma: float, dtype: int) -> NormalSpec:
    """Pick (mult, e) so the draw's sd is close to ``sigma`` and every value is
    exactly representable in the 16-bit format (finest grid that fits)."""
    exp_bits, frac_bits = _FMT[dtype]
    bias = (1 << (exp_bits - 1)) - 1
    xmax = (1 << (frac_bits + 1)) - 1
    best = None
    for e in range(40, -200, -1):
        mult = int(round(sigma / 2.0 ** e / IH4_SD * 65536.0))
        if mult < 1:
            continue
        if (131070 * mult) >> 16 > xmax:
            break
        best = (mult, e)
    if best is None:
        raise ValueError(f"sigma {sigma} not representable")
    mult, e = best
    if e < 1 - bias - frac_bits:
        raise ValueError("grid finer than the smallest subnormal")
    if ((131070 * mult) >> 16) * 2.0 ** e >= 2.0 ** (bias + 1):
        raise ValueError("draw would overflow the format")
    return NormalSpec(mult, e, dtype)


def scaled(spec: NormalSpec, scale: float) -> NormalSpec:
    """The same draw multiplied by a power of two (the loss scale)."""
    k = math.log2(scale)
    if k != int(k):
        raise ValueError("scale must be a power of two")
    s = NormalSpec(spec.mult, spec.e + int(k), spec.dtype)
    exp_bits, frac_bits = _FMT[spec.dtype]
    bias = (1 << (exp_bits - 1)) - 1
    if s.e < 1 - bias - frac_bits or s.max_abs >= 2.0 ** (bias + 1):
        raise ValueError("scaled draw not exactly representable")
    return s


def stream_key(seed: int, kind: int, step: int, rank: int) -> int:
    return int(_host_lib().synth_key(seed, kind, step, rank))


def hash64(key: int, index: int) -> int:
    return int(_host_lib().synth_hash64(key, index))


def fill_host(out: np.ndarray, first: int, key: int, spec: NormalSpec, threads: int = 1) -> None:
    """out[j] = generated value at global index first + j (out is uint16)."""
    assert out.dtype == np.uint16 and out.flags.c_contiguous
    exp_bits, frac_bits = _FMT[spec.dtype]
    lib = _host_lib()
    n = out.size
    base = out.ctypes.data
    if threads <= 1 or n < (1 << 20):
        lib.synth_fill(base, n, first, key, spec.mult, spec.e, exp_bits, frac_bits)
        return
    chunk = (n + threads - 1) // threads

    def work(t):
        a = t * chunk
        b = min(n, a + chunk)
        if a < b:
            lib.synth_fill(base + 2 * a, b - a, first + a, key, spec.mult, spec.e,
                           exp_bits, frac_bits)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(threads)))


def gather_host(idx: np.ndarray, key: int, spec: NormalSpec) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.uint16)
    exp_bits, frac_bits = _FMT[spec.dtype]
    _host_lib().synth_gather(out.ctypes.data, idx.ctypes.data, idx.size, key, spec.mult, spec.e,
                             exp_bits, frac_bits)
    return out


def fill_device(ptr: int, n: int, first: int, key: int, spec: NormalSpec, stream: int = 0) -> None:
    """Device twin of fill_host: ptr is a device address of n uint16 slots."""
    exp_bits, frac_bits = _FMT[spec.dtype]
    rc = _dev_lib().synth_dev_fill(ptr, n, first, key, spec.mult, spec.e, exp_bits, frac_bits,
                                   stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill failed with {rc}")


# 16-bit patterns of a few constants used as inputs
ONE = {FP16: 0x3C00, BF16: 0x3F80}
POS_INF = {FP16: 0x7C00, BF16: 0x7F80}
QNAN = {FP16: 0x7E00, BF16: 0x7FC0}
