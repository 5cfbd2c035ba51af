"""Rounding of fp64 results to the storage dtype -- oracle, test infrastructure.

The attention interface is dtype preserving: a bf16 input yields a bf16
output.  The oracle therefore rounds each fp64 result once, directly to the
storage type, with round-to-nearest, ties-to-even (no intermediate fp32 step,
which could round twice).

bf16 keeps 8 significant bits (7 stored), the exponent range of fp32, and
subnormals down to 2**-133.
"""
import numpy as np

_BF16_MIN_EXP = -133     # quantum of bf16 subnormals (2**-126 * 2**-7)
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x) -> np.ndarray:
    """fp64 -> nearest bf16 value (ties to even), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)                       # xf = m * 2**e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, _BF16_MIN_EXP)      # 8 significant bits
    y = np.ldexp(np.rint(np.ldexp(xf, -q)), q)    # np.rint: ties to even
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, xf), y)
    out[fin] = y
    out[~fin] = x[~fin]
    return out


def round_f32(x) -> np.ndarray:
    """fp64 -> nearest fp32 value (IEEE cast, ties to even), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


def bf16_bits_of(x) -> np.ndarray:
    """uint16 bit pattern of fp64 values that are exactly bf16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64),
                          equal_nan=True):
        raise ValueError("not representable in bf16")
    u = f.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("not representable in bf16")
    return (u >> np.uint32(16)).astype(np.uint16)
