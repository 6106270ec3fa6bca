"""Error metrics and tolerances for comparing the HIP path with the oracle.

Tolerances (the routing's stated bar):
  * fp32 I/O:  max |y - y*| / RMS(y*) <= 1e-5.
  * bf16 I/O with fp32 accumulation: max |y - y*| / RMS(y*) <= 2e-2, counting
    only the error beyond the output's own rounding to bfloat16, i.e.
    max_k max(0, |y_k - y*_k| - ulp_bf16(y*_k)/2) / RMS(y*).
    The exclusion is needed because on these inputs the exact result rounded
    once to bf16 already differs from y* by up to ~3% of RMS (outputs reach
    ~11x their RMS, where half a bf16 ulp is ~2^-8 of the value); no bf16
    output can do better than that rounding.
  * fp32 outputs computed from bf16 inputs (dw, dgain): plain max-abs / RMS
    <= 2e-2.
"""

from __future__ import annotations

import numpy as np

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def rms(y) -> float:
    y = np.asarray(y, np.float64)
    return float(np.sqrt(np.mean(y * y))) if y.size else 0.0


def max_abs_over_rms(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    if y.size == 0:
        return 0.0
    r = rms(ref)
    err = float(np.max(np.abs(y - ref)))
    return err / r if r > 0 else err


def half_ulp_bf16(ref) -> np.ndarray:
    """Half a bfloat16 ulp at |ref| (bf16 keeps 8 significant bits)."""
    a = np.abs(np.asarray(ref, np.float64))
    _, e = np.frexp(a)  # a = m * 2^e, m in [0.5, 1)
    return np.where(a > 0, np.ldexp(1.0, e - 9), 0.0)


def bf16_excess_over_rms(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    if y.size == 0:
        return 0.0
    excess = np.maximum(0.0, np.abs(y - ref) - half_ulp_bf16(ref))
    r = rms(ref)
    return float(np.max(excess)) / r if r > 0 else float(np.max(excess))


def check(y, ref, dtype: str, what: str = "") -> float:
    """Assert the tolerance for an output of the given I/O dtype; returns the error."""
    if dtype == "f32":
        err = max_abs_over_rms(y, ref)
        assert err <= TOL_F32, f"{what}: fp32 max-abs/RMS {err:.3e} > {TOL_F32}"
    elif dtype == "bf16":
        err = bf16_excess_over_rms(y, ref)
        assert err <= TOL_BF16, f"{what}: bf16 excess/RMS {err:.3e} > {TOL_BF16}"
    elif dtype == "f32_from_bf16":
        err = max_abs_over_rms(y, ref)
        assert err <= TOL_BF16, f"{what}: max-abs/RMS {err:.3e} > {TOL_BF16}"
    else:
        raise ValueError(dtype)
    return err
