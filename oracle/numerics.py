"""Exact widening of bfloat16/float32 inputs and correctly rounded output casts.

Readings (the pages name no dtypes):
* bfloat16 is the IEEE-754 binary32 format truncated to its upper 16 bits
  (1 sign, 8 exponent, 7 fraction bits); widening to float64 is exact.
* Output rounding is round-to-nearest, ties-to-even, applied ONCE from the
  float64 result (no intermediate float32 step, so no double rounding).
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> exact float64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bits, round to nearest even, from the definition.

    A bfloat16 number has 8 significant bits; in the binade [2^(e-1), 2^e) its
    spacing is 2^(e-8), and below the smallest normal 2^-126 the spacing stays
    2^-133 (subnormals).  Rounding is therefore rint(|x| / q) * q with q that
    spacing (``rint`` rounds half to even; the scaling by a power of two is
    exact).  Results of magnitude >= 2^128 overflow to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                     # ax = m * 2^e, m in [0.5, 1)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(ax / q) * q
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)          # exact: r has <= 8 significant bits
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(r >= 2.0 ** 128, np.uint16(0x7F80), bits)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def cast_out(x64: np.ndarray, out_dtype: str) -> np.ndarray:
    """Round a float64 result to the output dtype ("bf16" -> uint16 bits, "f32")."""
    if out_dtype == "bf16":
        return f64_to_bf16_bits(x64)
    if out_dtype == "f32":
        return np.asarray(x64, np.float64).astype(np.float32)
    raise ValueError(out_dtype)


def out_to_f64(y: np.ndarray, out_dtype: str) -> np.ndarray:
    """Widen an output array (bf16 bits or float32) to float64."""
    if out_dtype == "bf16":
        return bf16_to_f64(y)
    return np.asarray(y, np.float32).astype(np.float64)
