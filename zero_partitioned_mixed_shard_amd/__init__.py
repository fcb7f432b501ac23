"""Python binding of the ZeRO-1/2 owner-shard step library (libzero_shard.so).

Argument marshalling only: every phase runs in the HIP kernels of
``csrc/zero_shard.hip`` and ``csrc/zero_flat.hip`` behind the C ABI of
``include/zero_shard.h``.  The functions keep the C names.  Device buffers are
torch tensors (device memory and streams are all torch is used for); 16-bit
data is passed as torch.float16 / torch.bfloat16 tensors, fp32 state as
torch.float32.  There is no fallback: if the library is missing, importing
this package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libzero_shard.so")

ZERO_OK, ZERO_EINVAL, ZERO_ERANGE, ZERO_EDEVICE = 0, -1, -2, -3
ZERO_FP16, ZERO_BF16 = 1, 2
ZERO_MAX_RANKS = 16


class zero_step_result(ctypes.Structure):
    _fields_ = [("sumsq", ctypes.c_double), ("overflow", ctypes.c_uint32),
                ("inv_scale", ctypes.c_float)]


class zero_adamw_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("max_grad_norm", ctypes.c_float), ("step", ctypes.c_int64)]


class zero_loss_scaler(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_double), ("min_scale", ctypes.c_double),
                ("window", ctypes.c_int64), ("clean", ctypes.c_int64),
                ("skipped", ctypes.c_int64)]


class zero_range(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("count", ctypes.c_int64)]


class zero_step_control(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_double), ("min_scale", ctypes.c_double),
                ("window", ctypes.c_int64), ("clean", ctypes.c_int64),
                ("skipped", ctypes.c_int64), ("t", ctypes.c_int64),
                ("divisor", ctypes.c_float), ("inv_scale", ctypes.c_float),
                ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("bc1", ctypes.c_float), ("bc2", ctypes.c_float)]


RESULT_BYTES = ctypes.sizeof(zero_step_result)   # 16
CONTROL_BYTES = ctypes.sizeof(zero_step_control)  # 72

EXPORTS = (
    "zero_partition_layout", "zero_bucket_layout", "zero_memory_bytes",
    "zero_loss_scaler_update", "zero_status_str", "zero_init_master", "zero_reduce_owned",
    "zero_check_workspace_bytes", "zero_unscale_check_norm", "zero_reduce_check_owned",
    "zero_adamw_step", "zero_flat_gather", "zero_flat_scatter",
    "zero_step_control_init", "zero_reduce_check_owned_ctl", "zero_unscale_check_norm_ctl",
    "zero_adamw_step_ctl", "zero_step_control_update",
    "zero_range_workspace_bytes", "zero_reduce_check_ranges", "zero_adamw_step_ranges",
    "zero_reduce_check_buckets", "zero_reduce_check_owned_noalloc",
)


class ZeroError(RuntimeError):
    pass


def _hip_runtimes() -> set:
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return set()


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    # torch brings its own HIP runtime; load it first so that this library
    # binds to the same one (two runtimes in one process do not share devices)
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    if len(_hip_runtimes()) > 1:
        raise ImportError(f"more than one HIP runtime is loaded: {sorted(_hip_runtimes())}")
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sig = {
        "zero_partition_layout": ([P, i64, i32, i32, P, P, P], ctypes.c_int),
        "zero_bucket_layout": ([P, i64, i64, P, P], ctypes.c_int),
        "zero_memory_bytes": ([i32, i64, i64, i32, P], ctypes.c_int),
        "zero_loss_scaler_update": ([P, ctypes.c_uint32], ctypes.c_int),
        "zero_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "zero_init_master": ([P, P, i64, i32, P], ctypes.c_int),
        "zero_reduce_owned": ([P, P, i32, i64, i32, P], ctypes.c_int),
        "zero_check_workspace_bytes": ([i64], ctypes.c_size_t),
        "zero_unscale_check_norm": ([P, i64, i32, f32, P, P, ctypes.c_size_t, i32, P],
                                    ctypes.c_int),
        "zero_reduce_check_owned": ([P, P, i32, i64, i32, f32, P, P, ctypes.c_size_t, i32, P],
                                    ctypes.c_int),
        "zero_adamw_step": ([P, P, P, P, P, i64, i32, P, P, P], ctypes.c_int),
        "zero_flat_gather": ([P, i64, P, i64, P], ctypes.c_int),
        "zero_flat_scatter": ([P, i64, P, i64, P], ctypes.c_int),
        "zero_step_control_init": ([P, ctypes.c_double, ctypes.c_double, i64, f32, f32, f32],
                                   ctypes.c_int),
        "zero_reduce_check_owned_ctl": ([P, P, i32, i64, i32, P, P, P, ctypes.c_size_t, i32, P],
                                        ctypes.c_int),
        "zero_unscale_check_norm_ctl": ([P, i64, i32, P, P, P, ctypes.c_size_t, i32, P],
                                        ctypes.c_int),
        "zero_adamw_step_ctl": ([P, P, P, P, P, i64, i32, P, P, P, P], ctypes.c_int),
        "zero_step_control_update": ([P, P, P], ctypes.c_int),
        "zero_range_workspace_bytes": ([P, i32], ctypes.c_size_t),
        "zero_reduce_check_ranges": ([P, P, i32, P, i32, i32, f32, P, P, P, ctypes.c_size_t, i32, P],
                                     ctypes.c_int),
        "zero_adamw_step_ranges": ([P, P, P, P, P, P, i32, i32, P, P, P, P], ctypes.c_int),
        "zero_reduce_check_buckets": ([P, P, i32, P, i32, i32, f32, P, P, P, ctypes.c_size_t, i32,
                                       P], ctypes.c_int),
        "zero_reduce_check_owned_noalloc": ([P, P, i32, i64, i32, f32, P, i32, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


_lib = _load()


def lib():
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != ZERO_OK:
        raise ZeroError(f"{what}: {_lib.zero_status_str(rc).decode()} ({rc})")


# ------------------------------------------------------------ marshalling --
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return ZERO_FP16
    if t.dtype == torch.bfloat16:
        return ZERO_BF16
    raise TypeError(f"16-bit tensor expected, got {t.dtype}")


def _dev(t, nbytes_per: int, count: int, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.element_size() != nbytes_per or t.numel() < count:
        raise ValueError(f"{name}: need {count} elements of {nbytes_per} bytes")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ host ---
def zero_partition_layout(numels: Sequence[int], world: int, align_elems: int = 2):
    """-> (tensor_offsets int64[n], part_begin int64[world+1], padded_total)."""
    n = np.ascontiguousarray(numels, dtype=np.int64)
    offs = np.zeros(max(1, n.size), dtype=np.int64)
    parts = np.zeros(max(1, world + 1), dtype=np.int64)
    padded = ctypes.c_int64(0)
    _check(_lib.zero_partition_layout(n.ctypes.data, n.size, world, align_elems, offs.ctypes.data,
                                      parts.ctypes.data, ctypes.byref(padded)),
           "zero_partition_layout")
    return offs[:n.size].copy(), parts, padded.value


def zero_bucket_layout(numels: Sequence[int], bucket_cap: int) -> np.ndarray:
    """-> bucket_first int64[n_buckets + 1]."""
    n = np.ascontiguousarray(numels, dtype=np.int64)
    first = np.zeros(n.size + 1, dtype=np.int64)
    nb = ctypes.c_int64(0)
    _check(_lib.zero_bucket_layout(n.ctypes.data, n.size, bucket_cap, first.ctypes.data,
                                   ctypes.byref(nb)), "zero_bucket_layout")
    return first[:nb.value + 1].copy()


def zero_memory_bytes(stage: int, numel_total: int, padded_total: int, world: int) -> int:
    out = ctypes.c_int64(0)
    _check(_lib.zero_memory_bytes(stage, numel_total, padded_total, world, ctypes.byref(out)),
           "zero_memory_bytes")
    return out.value


def zero_loss_scaler_update(scaler: zero_loss_scaler, overflow: int) -> zero_loss_scaler:
    _check(_lib.zero_loss_scaler_update(ctypes.byref(scaler), int(bool(overflow))),
           "zero_loss_scaler_update")
    return scaler


def zero_status_str(status: int) -> str:
    return _lib.zero_status_str(status).decode()


def zero_check_workspace_bytes(count: int) -> int:
    return int(_lib.zero_check_workspace_bytes(count))


# ---------------------------------------------------------------- device ---
def zero_init_master(master, param16, count: Optional[int] = None, stream=None) -> None:
    count = param16.numel() if count is None else count
    _check(_lib.zero_init_master(_dev(master, 4, count, "master"), _dev(param16, 2, count, "param16"),
                                 count, _dtype_code(param16), _stream(stream)), "zero_init_master")


def zero_reduce_owned(dst, srcs: Sequence, count: Optional[int] = None, stream=None) -> None:
    count = dst.numel() if count is None else count
    dt = _dtype_code(dst)
    if not 1 <= len(srcs) <= ZERO_MAX_RANKS:
        raise ValueError("1..16 rank buffers")
    for s in srcs:
        if _dtype_code(s) != dt:
            raise TypeError("rank buffers and dst must share the 16-bit type")
    ptrs = (ctypes.c_void_p * len(srcs))(*[_dev(s, 2, count, "src") for s in srcs])
    _check(_lib.zero_reduce_owned(_dev(dst, 2, count, "dst"), ptrs, len(srcs), count, dt,
                                  _stream(stream)), "zero_reduce_owned")


def zero_unscale_check_norm(grad16, inv_scale: float, res, workspace, accumulate: bool = False,
                            count: Optional[int] = None, stream=None) -> None:
    """res: a device tensor of >= 16 bytes holding one zero_step_result."""
    count = grad16.numel() if count is None else count
    ws_bytes = workspace.numel() * workspace.element_size()
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    _check(_lib.zero_unscale_check_norm(_dev(grad16, 2, count, "grad16"), count,
                                        _dtype_code(grad16), float(inv_scale), res.data_ptr(),
                                        _dev(workspace, workspace.element_size(), 0, "workspace"),
                                        ws_bytes, int(bool(accumulate)), _stream(stream)),
           "zero_unscale_check_norm")


def zero_reduce_check_owned(dst, srcs: Sequence, inv_scale: float, res, workspace,
                            accumulate: bool = False, count: Optional[int] = None,
                            stream=None) -> None:
    count = dst.numel() if count is None else count
    dt = _dtype_code(dst)
    if not 1 <= len(srcs) <= ZERO_MAX_RANKS:
        raise ValueError("1..16 rank buffers")
    for s in srcs:
        if _dtype_code(s) != dt:
            raise TypeError("rank buffers and dst must share the 16-bit type")
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    ptrs = (ctypes.c_void_p * len(srcs))(*[_dev(s, 2, count, "src") for s in srcs])
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.zero_reduce_check_owned(_dev(dst, 2, count, "dst"), ptrs, len(srcs), count, dt,
                                        float(inv_scale), res.data_ptr(),
                                        _dev(workspace, workspace.element_size(), 0, "workspace"),
                                        ws_bytes, int(bool(accumulate)), _stream(stream)),
           "zero_reduce_check_owned")


def zero_adamw_step(master, exp_avg, exp_avg_sq, param16, grad16, hp: zero_adamw_hparams, res,
                    count: Optional[int] = None, stream=None) -> None:
    count = master.numel() if count is None else count
    dt = _dtype_code(grad16)
    if _dtype_code(param16) != dt:
        raise TypeError("param16 and grad16 must share the 16-bit type")
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    _check(_lib.zero_adamw_step(_dev(master, 4, count, "master"), _dev(exp_avg, 4, count, "exp_avg"),
                                _dev(exp_avg_sq, 4, count, "exp_avg_sq"),
                                _dev(param16, 2, count, "param16"), _dev(grad16, 2, count, "grad16"),
                                count, dt, ctypes.byref(hp), res.data_ptr(), _stream(stream)),
           "zero_adamw_step")


def tensor_descs(tensors: Sequence, offsets: Sequence[int], device="cuda"):
    """Device table of zero_tensor_desc (int64 [n, 4]: ptr, offset, numel, 0)
    for 16-bit device tensors placed at `offsets` of a flat buffer."""
    import torch
    rows = []
    for t, off in zip(tensors, offsets):
        if t.numel() and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.numel() and t.element_size() != 2:
            raise ValueError("16-bit tensors expected")
        rows.append((t.data_ptr() if t.numel() else 0, int(off), t.numel(), 0))
    host = torch.tensor(rows if rows else [(0, 0, 0, 0)], dtype=torch.int64)
    return host[:len(rows)].to(device)


def zero_flat_gather(flat, descs, count: Optional[int] = None, stream=None) -> None:
    """descs: device int64 [n, 4] table from tensor_descs()."""
    count = flat.numel() if count is None else count
    _check(_lib.zero_flat_gather(_dev(flat, 2, count, "flat"), count,
                                 descs.data_ptr() if descs.numel() else None, descs.shape[0],
                                 _stream(stream)), "zero_flat_gather")


def zero_flat_scatter(flat, descs, count: Optional[int] = None, stream=None) -> None:
    count = flat.numel() if count is None else count
    _check(_lib.zero_flat_scatter(_dev(flat, 2, count, "flat"), count,
                                  descs.data_ptr() if descs.numel() else None, descs.shape[0],
                                  _stream(stream)), "zero_flat_scatter")


# ------------------------------------------------ device step control -------
def zero_step_control_init(scale0: float, min_scale: float = 1.0, window: int = 1000,
                           divisor: float = 1.0, beta1: float = 0.9,
                           beta2: float = 0.999) -> zero_step_control:
    """Host zero_step_control for the first step (copy it to the device with
    control_to_device)."""
    c = zero_step_control()
    _check(_lib.zero_step_control_init(ctypes.byref(c), float(scale0), float(min_scale),
                                       int(window), float(divisor), float(beta1), float(beta2)),
           "zero_step_control_init")
    return c


def control_to_device(ctl: zero_step_control, out=None, device="cuda"):
    """A device tensor (uint8, 72 bytes, 256-byte aligned by the allocator)
    holding `ctl`; written into `out` when given."""
    import torch
    host = torch.frombuffer(bytearray(bytes(ctl)), dtype=torch.uint8)
    if out is None:
        return host.to(device)
    out.copy_(host)
    return out


def read_control(ctl_dev) -> zero_step_control:
    """Copy a device zero_step_control to the host (synchronises the stream)."""
    raw = ctl_dev.detach().cpu().numpy().tobytes()[:CONTROL_BYTES]
    return zero_step_control.from_buffer_copy(raw)


def _ctl(ctl_dev) -> int:
    if not ctl_dev.is_cuda or ctl_dev.numel() * ctl_dev.element_size() < CONTROL_BYTES:
        raise ValueError("ctl must be a device tensor of at least 72 bytes")
    if ctl_dev.data_ptr() % 8:
        raise ValueError("ctl must be 8-byte aligned")
    return ctl_dev.data_ptr()


def zero_reduce_check_owned_ctl(dst, srcs: Sequence, ctl_dev, res, workspace,
                                accumulate: bool = False, count: Optional[int] = None,
                                stream=None) -> None:
    count = dst.numel() if count is None else count
    dt = _dtype_code(dst)
    if not 1 <= len(srcs) <= ZERO_MAX_RANKS:
        raise ValueError("1..16 rank buffers")
    for s in srcs:
        if _dtype_code(s) != dt:
            raise TypeError("rank buffers and dst must share the 16-bit type")
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    ptrs = (ctypes.c_void_p * len(srcs))(*[_dev(s, 2, count, "src") for s in srcs])
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.zero_reduce_check_owned_ctl(_dev(dst, 2, count, "dst"), ptrs, len(srcs), count, dt,
                                            _ctl(ctl_dev), res.data_ptr(),
                                            _dev(workspace, workspace.element_size(), 0,
                                                 "workspace"),
                                            ws_bytes, int(bool(accumulate)), _stream(stream)),
           "zero_reduce_check_owned_ctl")


def zero_unscale_check_norm_ctl(grad16, ctl_dev, res, workspace, accumulate: bool = False,
                                count: Optional[int] = None, stream=None) -> None:
    count = grad16.numel() if count is None else count
    ws_bytes = workspace.numel() * workspace.element_size()
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    _check(_lib.zero_unscale_check_norm_ctl(_dev(grad16, 2, count, "grad16"), count,
                                            _dtype_code(grad16), _ctl(ctl_dev), res.data_ptr(),
                                            _dev(workspace, workspace.element_size(), 0,
                                                 "workspace"),
                                            ws_bytes, int(bool(accumulate)), _stream(stream)),
           "zero_unscale_check_norm_ctl")


def zero_adamw_step_ctl(master, exp_avg, exp_avg_sq, param16, grad16, hp: zero_adamw_hparams,
                        ctl_dev, res, count: Optional[int] = None, stream=None) -> None:
    count = master.numel() if count is None else count
    dt = _dtype_code(grad16)
    if _dtype_code(param16) != dt:
        raise TypeError("param16 and grad16 must share the 16-bit type")
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    _check(_lib.zero_adamw_step_ctl(_dev(master, 4, count, "master"),
                                    _dev(exp_avg, 4, count, "exp_avg"),
                                    _dev(exp_avg_sq, 4, count, "exp_avg_sq"),
                                    _dev(param16, 2, count, "param16"),
                                    _dev(grad16, 2, count, "grad16"), count, dt,
                                    ctypes.byref(hp), _ctl(ctl_dev), res.data_ptr(),
                                    _stream(stream)),
           "zero_adamw_step_ctl")


def zero_step_control_update(ctl_dev, res, stream=None) -> None:
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    _check(_lib.zero_step_control_update(_ctl(ctl_dev), res.data_ptr(), _stream(stream)),
           "zero_step_control_update")


def read_result(res) -> zero_step_result:
    """Copy a device zero_step_result to the host (synchronises the stream)."""
    raw = res.detach().cpu().numpy().tobytes()[:RESULT_BYTES]
    return zero_step_result.from_buffer_copy(raw)


# ------------------------------------------------------------ range lists ---
def _ranges(ranges: Sequence) -> "ctypes.Array":
    """Host array of zero_range from (offset, count) pairs."""
    arr = (zero_range * max(1, len(ranges)))()
    for k, (a, c) in enumerate(ranges):
        arr[k].offset, arr[k].count = int(a), int(c)
    return arr


def zero_range_workspace_bytes(ranges: Sequence) -> int:
    return int(_lib.zero_range_workspace_bytes(_ranges(ranges), len(ranges)))


def _extent(ranges: Sequence) -> int:
    return max((int(a) + int(c) for a, c in ranges if int(c) > 0), default=0)


def zero_reduce_check_ranges(dst, srcs: Sequence, ranges: Sequence, inv_scale: float, res,
                             workspace, accumulate: bool = False, ctl_dev=None,
                             stream=None) -> None:
    """ranges: (offset, count) pairs of elements of dst and every src."""
    need = _extent(ranges)
    dt = _dtype_code(dst)
    if not 1 <= len(srcs) <= ZERO_MAX_RANKS:
        raise ValueError("1..16 rank buffers")
    for s in srcs:
        if _dtype_code(s) != dt:
            raise TypeError("rank buffers and dst must share the 16-bit type")
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    ptrs = (ctypes.c_void_p * len(srcs))(*[_dev(s, 2, need, "src") for s in srcs])
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.zero_reduce_check_ranges(
        _dev(dst, 2, need, "dst"), ptrs, len(srcs), _ranges(ranges), len(ranges), dt,
        float(inv_scale), _ctl(ctl_dev) if ctl_dev is not None else None, res.data_ptr(),
        _dev(workspace, workspace.element_size(), 0, "workspace"), ws_bytes,
        int(bool(accumulate)), _stream(stream)), "zero_reduce_check_ranges")


def zero_adamw_step_ranges(master, exp_avg, exp_avg_sq, param16, grad16, ranges: Sequence,
                           hp: zero_adamw_hparams, res, ctl_dev=None, stream=None) -> None:
    need = _extent(ranges)
    dt = _dtype_code(grad16)
    if _dtype_code(param16) != dt:
        raise TypeError("param16 and grad16 must share the 16-bit type")
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    _check(_lib.zero_adamw_step_ranges(
        _dev(master, 4, need, "master"), _dev(exp_avg, 4, need, "exp_avg"),
        _dev(exp_avg_sq, 4, need, "exp_avg_sq"), _dev(param16, 2, need, "param16"),
        _dev(grad16, 2, need, "grad16"), _ranges(ranges), len(ranges), dt, ctypes.byref(hp),
        _ctl(ctl_dev) if ctl_dev is not None else None, res.data_ptr(), _stream(stream)),
        "zero_adamw_step_ranges")


def zero_reduce_check_buckets(dst, windows: Sequence, srcs: Sequence[Sequence], inv_scale: float,
                              res, workspace, accumulate: bool = False, ctl_dev=None,
                              stream=None) -> None:
    """windows: (offset, count) pairs of elements of dst; srcs[w]: the N rank
    tensors of window w, each holding at least its count elements."""
    if len(srcs) != len(windows):
        raise ValueError("one list of rank tensors per window")
    n_ranks = len(srcs[0]) if srcs else 1
    if not 1 <= n_ranks <= ZERO_MAX_RANKS:
        raise ValueError("1..16 rank buffers")
    dt = _dtype_code(dst)
    flat = []
    for (a, c), ranks in zip(windows, srcs):
        if len(ranks) != n_ranks:
            raise ValueError("every window needs the same number of rank tensors")
        for t in ranks:
            if _dtype_code(t) != dt:
                raise TypeError("rank buffers and dst must share the 16-bit type")
            flat.append(_dev(t, 2, int(c), "src") if int(c) > 0 else None)
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    ptrs = (ctypes.c_void_p * max(1, len(flat)))(*flat)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.zero_reduce_check_buckets(
        _dev(dst, 2, _extent(windows), "dst"), ptrs, n_ranks, _ranges(windows), len(windows), dt,
        float(inv_scale), _ctl(ctl_dev) if ctl_dev is not None else None, res.data_ptr(),
        _dev(workspace, workspace.element_size(), 0, "workspace"), ws_bytes,
        int(bool(accumulate)), _stream(stream)), "zero_reduce_check_buckets")


def zero_reduce_check_owned_noalloc(dst, srcs: Sequence, inv_scale: float, res,
                                    accumulate: bool = False, count: Optional[int] = None,
                                    stream=None) -> None:
    """zero_reduce_check_owned with the library's own per-device scratch
    array instead of a workspace (nothing is allocated by the call)."""
    count = dst.numel() if count is None else count
    dt = _dtype_code(dst)
    if not 1 <= len(srcs) <= ZERO_MAX_RANKS:
        raise ValueError("1..16 rank buffers")
    for s in srcs:
        if _dtype_code(s) != dt:
            raise TypeError("rank buffers and dst must share the 16-bit type")
    if not res.is_cuda or res.numel() * res.element_size() < RESULT_BYTES:
        raise ValueError("res must be a device tensor of at least 16 bytes")
    ptrs = (ctypes.c_void_p * len(srcs))(*[_dev(s, 2, count, "src") for s in srcs])
    _check(_lib.zero_reduce_check_owned_noalloc(_dev(dst, 2, count, "dst"), ptrs, len(srcs), count,
                                                dt, float(inv_scale), res.data_ptr(),
                                                int(bool(accumulate)), _stream(stream)),
           "zero_reduce_check_owned_noalloc")
