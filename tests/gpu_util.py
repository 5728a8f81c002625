"""Helpers shared by the GPU tests: move numpy bit patterns to and from the
device, run one collective through the C ABI, compare with the oracle."""
import numpy as np

import oracle

STORE = {"f32": np.uint32, "bf16": np.uint16}
ESZ = {"f32": 4, "bf16": 2}


def torch_dtype(dtype):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


def to_device(bits, dtype, shift=0, pad=0):
    """Upload bit patterns into a fresh tensor whose data starts `shift`
    elements into its allocation (so its address can be misaligned)."""
    import torch
    n = bits.size
    base = torch.empty(shift + n + pad, dtype=torch_dtype(dtype), device="cuda")
    view = base[shift:shift + n]
    if n:
        if dtype == "f32":
            host = torch.from_numpy(np.ascontiguousarray(bits).view(np.float32))
        else:
            host = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
        view.copy_(host)
    return base, view


def to_host(t, dtype):
    import torch
    if dtype == "f32":
        return t.detach().cpu().view(torch.int32).numpy().view(np.uint32).copy()
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy()


def bf16_ulp_distance(a, b):
    """Distance in representable bf16 steps between patterns (NaN == NaN -> 0)."""
    def ordered(x):
        x = x.astype(np.int64)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + (x & 0x7FFF))
    d = np.abs(ordered(a) - ordered(b))
    nan_a = (a & 0x7FFF) > 0x7F80
    nan_b = (b & 0x7FFF) > 0x7F80
    d = np.where(nan_a & nan_b, 0, d)
    d = np.where(nan_a ^ nan_b, 1 << 20, d)
    return d


def compare(name, got, want, dtype, op):
    """Copies and fp32 sums bit for bit; bf16 sums within 1 bf16 ulp."""
    if op == "sum" and dtype == "bf16":
        d = bf16_ulp_distance(got, want)
        assert d.max(initial=0) <= 1, "%s: %d elements beyond 1 ulp" % (name, int((d > 1).sum()))
        return int((d != 0).sum())
    diff = got != want
    if op == "sum":
        # IEEE 754 leaves the payload of a NaN result open: any NaN matches any NaN
        nan = lambda x: (x & 0x7FFFFFFF) > 0x7F800000
        diff &= ~(nan(got) & nan(want))
    mism = np.nonzero(diff)[0]
    assert mism.size == 0, "%s: %d mismatches, first at %d (got %x want %x)" % (
        name, mism.size, mism[0], int(got[mism[0]]), int(want[mism[0]]))
    return 0


def run_collective(purlin, in_naming, out_naming, op, dtype, P, counts, displs, ins, outs,
                   shifts=None, out_shifts=None):
    """Run on the GPU; returns the P output arrays (bit patterns)."""
    shifts = shifts or [0] * P
    out_shifts = out_shifts or [0] * P
    keep = []
    din, dout = [], []
    for r in range(P):
        b, v = to_device(ins[r], dtype, shifts[r])
        keep.append(b)
        din.append(v if ins[r].size else None)
        b, v = to_device(outs[r], dtype, out_shifts[r])
        keep.append(b)
        dout.append(v if outs[r].size else None)
    purlin.collective([x if x is not None else 0 for x in din],
                      [x if x is not None else 0 for x in dout],
                      in_naming, out_naming, op, counts, displs, dtype=dtype)
    purlin.check()
    return [to_host(v, dtype) if v is not None else np.zeros(0, STORE[dtype]) for v in dout]


def oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, displs=None, shifts=None,
                   out_shifts=None):
    in_n, out_n, op = oracle.COLLECTIVES[name]
    want = oracle.collective(in_n, out_n, op, dtype, P, counts, displs, ins, outs)
    got = run_collective(purlin, in_n, out_n, op, dtype, P, counts, displs, ins, outs,
                         shifts, out_shifts)
    inexact = 0
    for j in range(P):
        inexact += compare("%s rank %d" % (name, j), got[j], want[j], dtype, op)
    # The contract allows 1 bf16 step; the kernel folds in the oracle's order
    # and precision, so every element is expected to be exact.
    assert inexact == 0, "%s: %d bf16 sums one step off the oracle" % (name, inexact)
    return inexact
