"""Per-element brute force of the collective definition (tiny inputs only).

A second, independent route to the same result as ``oracle.collective``,
used to pin it (test infrastructure only):

* every element position of every buffer is tagged with (partition name,
  element index inside the partition), straight from the naming table of
  Purlin's Figure 4 caption and abstract;
* an output element takes every input element with the same tag, scanning
  source ranks in ascending order, and applies the op;
* arithmetic is exact rational arithmetic (``fractions.Fraction``) rounded
  to the target binary format after every add (fp32: 24-bit significand)
  and once at the end (bf16: 8-bit significand), with round to nearest,
  ties to even, gradual underflow and overflow to infinity.  No numpy float
  arithmetic and no bit trick is shared with the fast path.

Only finite values are supported here; NaN / inf handling is pinned by the
bf16 tests instead.
"""
import struct
from fractions import Fraction
import math

__all__ = ["collective_brute", "round_binary", "f32_bits_to_float", "float_to_f32_bits"]

_EMIN, _EMAX = -126, 127          # shared by fp32 and bf16


def round_binary(x, p, emin=_EMIN, emax=_EMAX):
    """Round the exact rational x to p significant bits (RNE); returns a float."""
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = abs(Fraction(x))
    # exponent e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                       # subnormals share the minimum exponent
    ulp = Fraction(2) ** (e - p + 1)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    value = n * ulp
    if value >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * float(value)


def f32_bits_to_float(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) & 0xFFFFFFFF))[0]


def float_to_f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def _bf16_bits_to_float(bits):
    return f32_bits_to_float((int(bits) & 0xFFFF) << 16)


def _float_to_bf16_bits(x):
    # x is already representable in bf16, so the low half of its fp32 pattern is 0
    b = float_to_f32_bits(x)
    assert b & 0xFFFF == 0
    return b >> 16


def _fp32_add(a, b):
    """IEEE fp32 a + b (round to nearest even) for finite fp32 values a, b."""
    s = Fraction(a) + Fraction(b)
    if s == 0:
        # exact zero sum: -0 only when both operands are -0
        if math.copysign(1.0, a) < 0 and math.copysign(1.0, b) < 0:
            return -0.0
        return 0.0
    return round_binary(s, 24)


def _element_tags(naming, rank, P, counts, displs_side, length):
    """For each position of one buffer: (name, index in partition) or None."""
    if naming == "whole":
        names = [()]
    elif naming == "by_rank":
        names = [(rank,)]
    elif naming == "by_index":
        names = [(q,) for q in range(P)]
    elif naming == "by_rank_index":
        names = [(rank, q) for q in range(P)]
    elif naming == "by_index_rank":
        names = [(q, rank) for q in range(P)]
    else:
        raise ValueError(naming)

    def number(name):
        return 0 if not name else (name[0] if len(name) == 1 else name[0] * P + name[1])

    tags = [None] * length
    cursor = 0
    for name in names:
        n = counts[number(name)]
        start = cursor if displs_side is None else displs_side[number(name)]
        for e in range(n):
            pos = start + e
            if tags[pos] is not None:
                raise ValueError("overlapping partitions")
            tags[pos] = (name, e)
        cursor += n
    return tags


def collective_brute(in_naming, out_naming, op, dtype, P, counts, displs, inputs, outputs):
    """Same contract as oracle.collective; returns lists of Python ints (bit patterns)."""
    counts = [int(c) for c in counts]
    if displs is None:
        in_d = out_d = None
    else:
        k = len(counts)
        in_d, out_d = [int(v) for v in displs[:k]], [int(v) for v in displs[k:]]
    to_float = _bf16_bits_to_float if dtype == "bf16" else f32_bits_to_float

    in_tags = [_element_tags(in_naming, i, P, counts, in_d, len(inputs[i])) for i in range(P)]
    result = []
    for j in range(P):
        out = [int(v) for v in outputs[j]]
        tags = _element_tags(out_naming, j, P, counts, out_d, len(out))
        for pos, tag in enumerate(tags):
            if tag is None:
                continue
            vals = []
            for i in range(P):                         # ascending source rank
                for p2, t2 in enumerate(in_tags[i]):
                    if t2 == tag:
                        vals.append(int(inputs[i][p2]))
            if op == "copy":
                if len(vals) != 1:
                    raise ValueError("copy needs exactly one source")
                out[pos] = vals[0]
            else:
                if not vals:
                    raise ValueError("sum needs a source")
                acc = to_float(vals[0])
                for v in vals[1:]:
                    acc = _fp32_add(acc, to_float(v))
                if dtype == "bf16":
                    out[pos] = _float_to_bf16_bits(round_binary(Fraction(acc), 8))
                else:
                    out[pos] = float_to_f32_bits(acc)
        result.append(out)
    return result
