"""Workload inputs (16-bit initial parameters and per-rank gradients) for any
range of the flat buffer, on the host (numpy) or on the device (torch tensors
filled by libsynth_dev).  Both sides give identical bits for every index.

Initial values: weights N(0, 0.02), biases 0, normalisation gains 1.
Gradients of rank r at step s: N(0, sigma) times the loss scale (times
2^-(r * rank_shift) where a workload sets it), one stream per (step, rank)
over global flat indices; elements past the last tensor (the
alignment padding) are 0.  Injected inf/NaN go to the index the workload's
schedule names.
"""
from __future__ import annotations

import numpy as np

from . import FP16, BF16, ONE, POS_INF, QNAN, fill_device, fill_host
from .workloads import BIAS, NORM, WEIGHT, Workload, injections, tensor_segments


def host_param16(wl: Workload, offsets: np.ndarray, begin: int, end: int,
                 threads: int = 1) -> np.ndarray:
    out = np.zeros(end - begin, dtype=np.uint16)
    spec, key = wl.init_spec(), wl.init_key()
    for a, b, kind in tensor_segments(wl, offsets, begin, end):
        view = out[a - begin:b - begin]
        if kind == WEIGHT:
            fill_host(view, a, key, spec, threads)
        elif kind == NORM:
            view[:] = ONE[wl.dtype]
    return out


def host_rank_grads(wl: Workload, step: int, scale: float, begin: int, end: int,
                    padded: int, threads: int = 1, ranks=None, out_bufs=None) -> list:
    """The N ranks' gradients over [begin, end) of the flat buffer
    (written into `out_bufs` when given, one uint16 array per rank)."""
    phi = wl.phi
    inj = injections(wl, padded).get(step)
    out = []
    for k, r in enumerate(range(wl.world) if ranks is None else ranks):
        spec = wl.grad_spec(scale, r)
        if out_bufs is None:
            g = np.zeros(end - begin, dtype=np.uint16)
        else:
            g = out_bufs[k][:end - begin]
        stop = min(end, phi)
        if stop > begin:
            fill_host(g[:stop - begin], begin, wl.grad_key(step, r), spec, threads)
        if end > max(stop, begin):
            g[max(stop, begin) - begin:] = 0
        if inj is not None and inj[0] == r and begin <= inj[1] < end:
            g[inj[1] - begin] = POS_INF[wl.dtype] if inj[2] == "inf" else QNAN[wl.dtype]
        out.append(g)
    return out


def torch_dtype(dtype: int):
    import torch
    return torch.float16 if dtype == FP16 else torch.bfloat16


def device_param16(wl: Workload, offsets: np.ndarray, begin: int, end: int, out=None):
    import torch
    if out is None:
        out = torch.empty(end - begin, dtype=torch_dtype(wl.dtype), device="cuda")
    out.zero_()
    raw = out.view(torch.int16)
    spec, key = wl.init_spec(), wl.init_key()
    one = ONE[wl.dtype]
    one = one - 65536 if one >= 32768 else one
    stream = torch.cuda.current_stream().cuda_stream
    for a, b, kind in tensor_segments(wl, offsets, begin, end):
        if kind == WEIGHT:
            fill_device(raw[a - begin:b - begin].data_ptr(), b - a, a, key, spec, stream)
        elif kind == NORM:
            raw[a - begin:b - begin].fill_(one)
    return out


def device_rank_grad(wl: Workload, step: int, scale: float, rank: int, begin: int, end: int,
                     padded: int, out=None):
    """Rank `rank`'s gradient over [begin, end) into a device tensor."""
    import torch
    if out is None:
        out = torch.empty(end - begin, dtype=torch_dtype(wl.dtype), device="cuda")
    raw = out.view(torch.int16)
    stop = min(end, wl.phi)
    stream = torch.cuda.current_stream().cuda_stream
    if stop > begin:
        fill_device(raw.data_ptr(), stop - begin, begin, wl.grad_key(step, rank),
                    wl.grad_spec(scale, rank), stream)
    if end > max(stop, begin):
        raw[max(stop, begin) - begin:].zero_()
    inj = injections(wl, padded).get(step)
    if inj is not None and inj[0] == rank and begin <= inj[1] < end:
        bits = POS_INF[wl.dtype] if inj[2] == "inf" else QNAN[wl.dtype]
        raw[inj[1] - begin].fill_(bits - 65536 if bits >= 32768 else bits)
    return out
