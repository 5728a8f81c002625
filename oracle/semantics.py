"""The oracle of Purlin's collective semantics (test infrastructure only).

Purlin specifies a collective by two layout namings, one for the inputs and
one for the outputs, and an operation, copy or reduction (Purlin, abstract).  The layouts
determine the result and leave the data movement open (Purlin, Figure 4
caption), so
this module computes exactly that definition and models none of the
orchestration (SNAC) or the datapath (Atom).

Definition (Purlin, abstract and Figure 4; the readings are listed below):

  Every rank r holds one input buffer and one output buffer.  A naming splits
  a rank's buffer into partitions q and gives each partition a name:

    whole          1 partition,  name ()
    by_rank        1 partition,  name (r,)
    by_index       P partitions, name (q,)
    by_rank_index  P partitions, name (r, q)
    by_index_rank  P partitions, name (q, r)

  Output partition (j, s) receives ``op`` applied to every input partition
  (i, q) whose name equals its own, taken in ascending source rank i.
  ``copy`` needs exactly one such input partition, ``sum`` at least one.

  With these namings (Figure 4 caption; composed AllReduce in Figure 6):
    AllReduce      whole         -> whole          sum
    ReduceScatter  by_index      -> by_rank        sum   (y_k = sum_i x_i[k])
    AllGather      by_rank       -> by_index       copy  (out_j[k] = y_k)
    AllToAll       by_rank_index -> by_index_rank  copy  (out_j[i] = x_i[j])

Counts and displacements are indexed by *name*: ``counts[n]`` is the element
count of every partition named n (names (a, b) are numbered a*P + b), so
matched partitions always have equal sizes.  ``displs`` is None (partitions
packed in index order) or the flat list ``in_displs + out_displs``, each with
one element offset per name, in the buffer of the rank that holds that name.
Non-uniform counts give the variable-length (V) collectives (Purlin, Table 2
and Figure 16 caption).

Arithmetic of ``sum`` (readings, not fixed by the pages):
  * inputs are widened exactly to fp32 (bf16 via ``oracle.bf16``),
  * the fold is left to right in ascending source rank:
        acc = x_0;  acc = fl32(acc + x_1);  ...;  acc = fl32(acc + x_{P-1}),
    each add an IEEE fp32 round-to-nearest-even add, subnormals kept,
  * one final rounding to the output dtype (identity for fp32, round to
    nearest even for bf16).
``copy`` moves the stored bit patterns unchanged.  Output elements outside
every named partition keep their prior contents.

Parity pinning: see the oracle tests (brute-force enumeration, library
identities, invariants, closed forms, error bounds, the Figure 4 fixture).
"""
import numpy as np

from .bf16 import widen_bf16, round_bf16

__all__ = [
    "NAMINGS", "OPS", "DTYPES", "ELEM_BYTES", "COLLECTIVES",
    "name_count", "partitions", "collective", "OracleError",
]

NAMINGS = ("whole", "by_rank", "by_index", "by_rank_index", "by_index_rank")
OPS = ("copy", "sum")
DTYPES = ("f32", "bf16")
ELEM_BYTES = {"f32": 4, "bf16": 2}
STORAGE = {"f32": np.uint32, "bf16": np.uint16}   # bit patterns

# The seven collectives as (input naming, output naming, op).
COLLECTIVES = {
    "allreduce": ("whole", "whole", "sum"),
    "reducescatter": ("by_index", "by_rank", "sum"),
    "allgather": ("by_rank", "by_index", "copy"),
    "alltoall": ("by_rank_index", "by_index_rank", "copy"),
}


class OracleError(ValueError):
    """The arguments do not define a collective."""


def name_count(naming, P):
    """How many distinct names a naming uses over P ranks."""
    if naming == "whole":
        return 1
    if naming in ("by_rank", "by_index"):
        return P
    if naming in ("by_rank_index", "by_index_rank"):
        return P * P
    raise OracleError("unknown naming %r" % (naming,))


def _name_number(name, P):
    """Position of a name in the counts / displs arrays."""
    if len(name) == 0:
        return 0
    if len(name) == 1:
        return name[0]
    return name[0] * P + name[1]


def partitions(naming, rank, P, counts, displs_side=None):
    """List (name, element offset, element count) for each partition of rank's buffer.

    ``displs_side`` is None (packed) or one side's displacements, by name.
    """
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
        raise OracleError("unknown naming %r" % (naming,))
    parts = []
    packed = 0
    for name in names:
        n = int(counts[_name_number(name, P)])
        if displs_side is None:
            off = packed
        else:
            off = int(displs_side[_name_number(name, P)])
        parts.append((name, off, n))
        packed += n
    return parts


def _check_bounds(parts, buf_len, what):
    spans = []
    for name, off, n in parts:
        if off < 0 or n < 0 or off + n > buf_len:
            raise OracleError("%s partition %r [%d, %d) outside a buffer of %d"
                              % (what, name, off, off + n, buf_len))
        if n:
            spans.append((off, off + n))
    return spans


def collective(in_naming, out_naming, op, dtype, P, counts, displs, inputs, outputs):
    """Apply the collective; return new output arrays (inputs are not modified).

    inputs, outputs: sequences of P one-dimensional arrays holding bit patterns
    (uint32 for f32, uint16 for bf16); float32 arrays are accepted for f32 and
    are reinterpreted, not converted.
    """
    if op not in OPS:
        raise OracleError("unknown op %r" % (op,))
    if dtype not in DTYPES:
        raise OracleError("unknown dtype %r" % (dtype,))
    if not (1 <= P):
        raise OracleError("P must be positive")
    if len(inputs) != P or len(outputs) != P:
        raise OracleError("need P input and P output buffers")
    n_names = name_count(in_naming, P)
    if name_count(out_naming, P) != n_names:
        raise OracleError("input and output namings use different name sets")
    counts = [int(c) for c in counts]
    if len(counts) != n_names or min(counts) < 0:
        raise OracleError("counts must hold %d non-negative entries" % n_names)
    if displs is None:
        in_d = out_d = None
    else:
        displs = [int(d) for d in displs]
        if len(displs) != 2 * n_names:
            raise OracleError("displs must hold %d entries" % (2 * n_names))
        in_d, out_d = displs[:n_names], displs[n_names:]

    store = STORAGE[dtype]
    ins = [np.ascontiguousarray(x).view(store) for x in inputs]
    outs = [np.array(np.ascontiguousarray(y).view(store), copy=True) for y in outputs]

    in_parts = [partitions(in_naming, i, P, counts, in_d) for i in range(P)]
    for i in range(P):
        _check_bounds(in_parts[i], ins[i].size, "input")

    # name -> [(source rank, element offset, count)] in ascending source rank
    sources = {}
    for i in range(P):
        for name, off, n in in_parts[i]:
            sources.setdefault(name, []).append((i, off, n))

    for j in range(P):
        out_parts = partitions(out_naming, j, P, counts, out_d)
        spans = sorted(_check_bounds(out_parts, outs[j].size, "output"))
        for a, b in zip(spans, spans[1:]):
            if b[0] < a[1]:
                raise OracleError("output partitions of rank %d overlap" % j)
        for name, off, n in out_parts:
            matches = sources.get(name, [])
            if op == "copy":
                if len(matches) != 1:
                    raise OracleError("copy into %r of rank %d has %d sources"
                                      % (name, j, len(matches)))
                i, soff, _ = matches[0]
                outs[j][off:off + n] = ins[i][soff:soff + n]
            else:
                if len(matches) < 1:
                    raise OracleError("sum into %r of rank %d has no source" % (name, j))
                outs[j][off:off + n] = _reduce(dtype, [ins[i][s:s + n] for i, s, _ in matches])
    return outs


def _widen(dtype, bits):
    if dtype == "bf16":
        return widen_bf16(bits)
    return np.ascontiguousarray(bits).view(np.float32)


def _reduce(dtype, terms):
    """Left fold in the given (ascending rank) order, fp32 accumulator, one rounding."""
    acc = _widen(dtype, terms[0]).copy()
    for t in terms[1:]:
        # float32 + float32 in numpy is one IEEE fp32 add per element.
        acc = acc + _widen(dtype, t)
    assert acc.dtype == np.float32
    if dtype == "bf16":
        return round_bf16(acc)
    return acc.view(np.uint32)
