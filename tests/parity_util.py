"""Comparison rules between a bf16 GEMM result and the fp64 oracle.

* rel-L2 = ||Y - Y_ref||_2 / ||Y_ref||_2 over the checked elements, bar 3e-3;
* per element |Y - Y_ref| <= 2e-2 * rms(Y_ref), or Y is one of the two bf16
  values that bracket Y_ref (a correctly rounded bf16 result can exceed the
  absolute bound where |Y_ref| >= 8 and half a bf16 ulp is 1/32);
* the error ratio (fraction of elements outside the absolute bound) is
  reported beside the other two.
"""
from __future__ import annotations

import numpy as np
import torch

REL_L2_BAR = 3e-3
MAX_ERR_FRACTION_OF_RMS = 2e-2


def bf16_to_f64(y) -> np.ndarray:
    if isinstance(y, torch.Tensor):
        return y.detach().to("cpu", torch.float32).numpy().astype(np.float64)
    return np.asarray(y, dtype=np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 (ties to even) -> fp64, in one rounding (normal range)."""
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)                          # x = f * 2**e, 0.5 <= |f| < 1
    return np.ldexp(np.rint(f * 256.0) / 256.0, e)   # np.rint rounds half to even


def bf16_brackets(ref: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The bf16 values lo <= ref <= hi adjacent to ref (lo == hi when ref is a bf16 value)."""
    f, e = np.frexp(ref)                        # ref = f * 2**e, 0.5 <= |f| < 1
    s = np.abs(f) * 256.0                        # 8 significant bits
    fl = np.floor(s)
    exact = fl == s
    lo_mag = np.ldexp(fl / 256.0, e)
    hi_mag = np.ldexp(np.where(exact, fl, fl + 1.0) / 256.0, e)
    neg = ref < 0
    lo = np.where(neg, -hi_mag, lo_mag)
    hi = np.where(neg, -lo_mag, hi_mag)
    return lo, hi


def compare(y, ref: np.ndarray) -> dict:
    y = bf16_to_f64(y)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    diff = y - ref
    nref = float(np.linalg.norm(ref))
    rel_l2 = float(np.linalg.norm(diff)) / nref if nref > 0 else float(np.linalg.norm(diff))
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = MAX_ERR_FRACTION_OF_RMS * rms
    absd = np.abs(diff)
    outside = absd > bound
    lo, hi = bf16_brackets(ref)
    neighbour = (y == lo) | (y == hi)
    failing = outside & ~neighbour
    finite = bool(np.all(np.isfinite(y)))
    return {
        "rel_l2": rel_l2,
        "max_abs_err": float(absd.max()) if absd.size else 0.0,
        "bound": bound,
        "error_ratio": float(outside.mean()) if outside.size else 0.0,
        "outside_count": int(outside.sum()),
        "failing_count": int(failing.sum()),
        "finite": finite,
    }


def assert_parity(y, ref: np.ndarray, what: str = "") -> dict:
    st = compare(y, ref)
    assert st["finite"], f"{what}: non-finite values in GPU output"
    assert st["rel_l2"] <= REL_L2_BAR, f"{what}: rel-L2 {st['rel_l2']:.3e} > {REL_L2_BAR}: {st}"
    assert st["failing_count"] == 0, f"{what}: {st['failing_count']} elements beyond max-error rule: {st}"
    return st
