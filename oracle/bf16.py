"""bf16 <-> fp32 conversions of the oracle (test infrastructure only).

bf16 values are held as their 16-bit patterns in ``numpy.uint16`` arrays and
never pass through a library bf16 type, so every bit (NaN payloads included)
is under the oracle's control.

* Widening bf16 -> fp32 is exact: the 16 bits become the top half of the
  fp32 pattern (bf16 is fp32 with the low 16 mantissa bits dropped).
* Narrowing fp32 -> bf16 is IEEE 754 round-to-nearest, ties-to-even, applied
  to the 16 discarded mantissa bits.  Overflow rounds to +-inf by itself
  (the carry runs into the exponent).  A NaN keeps its sign and top payload
  bits and gets the quiet bit (0x0040) set, so it can never round to inf.
  Subnormals are rounded like any other value (no flush to zero).

Purlin's pages fix no precision for the reduction; the fp32 accumulator and
the single final rounding are the readings this build takes.
"""
import numpy as np

__all__ = ["widen_bf16", "round_bf16", "bf16_to_f32_scalar", "f32_to_bf16_scalar"]


def widen_bf16(bits):
    """bf16 patterns (uint16 array) -> float32 array, exactly."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(values):
    """float32 array -> bf16 patterns (uint16 array), round to nearest even."""
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    # The kept part is u >> 16.  Adding 0x7FFF rounds any discarded half
    # above 0x8000 up; the extra +1 when the kept part is odd turns the exact
    # tie 0x8000 into a round-up only towards an even result.  The uint32 sum
    # can wrap only for patterns above 0xFFFF8000, all of which are NaNs and
    # are replaced below.
    rounded = (u >> 16) & np.uint32(1)
    rounded += u
    rounded += np.uint32(0x7FFF)
    rounded >>= 16
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if is_nan.any():
        rounded[is_nan] = (u[is_nan] >> 16) | np.uint32(0x0040)
    return rounded.astype(np.uint16)


def bf16_to_f32_scalar(b):
    """One bf16 pattern (int) -> Python float, via the same exact widening."""
    return float(widen_bf16(np.array([b], dtype=np.uint16))[0])


def f32_to_bf16_scalar(x):
    """One float (rounded to fp32 first) -> bf16 pattern (int)."""
    return int(round_bf16(np.array([x], dtype=np.float32))[0])
