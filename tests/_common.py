"""Shared helpers for the parity tests: comparisons to the tolerances the
owner-shard step is held to, and host/device conversions."""
import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None

REL_TOL_F32 = 2e-6      # fp32 master / m / v: relative, or bit-equal
REL_TOL_NORM = 1e-5     # grad-norm (sqrt of sumsq)
ULP_TOL_P16 = 1         # 16-bit parameter copy


def to_np16(t) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def to_np32(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def from_np16(a: np.ndarray, dtype: int, device="cuda"):
    tdt = torch.float16 if dtype == 1 else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(tdt)


def is_nan16(a: np.ndarray, dtype: int) -> np.ndarray:
    expo, frac = (0x7C00, 0x3FF) if dtype == 1 else (0x7F80, 0x7F)
    return ((a & expo) == expo) & ((a & frac) != 0)


def assert_bits16_equal(got: np.ndarray, want: np.ndarray, dtype: int, what=""):
    ok = (got == want) | (is_nan16(got, dtype) & is_nan16(want, dtype))
    if not ok.all():
        bad = np.flatnonzero(~ok)[:8]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} differ; first at {bad}: "
                             f"got {[hex(int(x)) for x in got[bad]]} "
                             f"want {[hex(int(x)) for x in want[bad]]}")


def _ordered16(a: np.ndarray) -> np.ndarray:
    a = a.astype(np.int64)
    return np.where(a & 0x8000, -(a & 0x7FFF), a)


def assert_p16_close(got: np.ndarray, want: np.ndarray, dtype: int, what=""):
    d = np.abs(_ordered16(got) - _ordered16(want))
    ok = (d <= ULP_TOL_P16) | (is_nan16(got, dtype) & is_nan16(want, dtype))
    if not ok.all():
        bad = np.flatnonzero(~ok)[:8]
        raise AssertionError(f"{what}: {int((~ok).sum())} 16-bit values beyond {ULP_TOL_P16} ulp; "
                             f"first {bad}")


def ulp_distance32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def assert_f32_close(got: np.ndarray, want: np.ndarray, what="") -> int:
    """Bit-equal, or within REL_TOL_F32 relative.  Returns the max ulp distance."""
    same = got.view(np.uint32) == want.view(np.uint32)
    close = np.abs(got.astype(np.float64) - want.astype(np.float64)) <= \
        REL_TOL_F32 * np.maximum(np.abs(got), np.abs(want)).astype(np.float64)
    ok = same | close
    if not ok.all():
        bad = np.flatnonzero(~ok)[:8]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} beyond {REL_TOL_F32}; "
                             f"first {bad}: got {got[bad]} want {want[bad]}")
    return int(ulp_distance32(got, want).max()) if got.size else 0
