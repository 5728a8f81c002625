"""The C ABI on the CPU: exported symbols, argument checks, plan derivation.

No GPU is needed: the library is loaded, and only calls that return before
any HIP call are made (plan_describe, policy, invalid arguments).
"""
import os
import re

import numpy as np
import pytest

import oracle
import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "purlin.h")


@pytest.fixture(scope="module")
def purlin():
    from reduce_atom_02_amd import purlin as p
    return p


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"PURLIN_API\s+[\w\s\*]*?\b(purlin_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(purlin):
    import ctypes
    declared = header_functions()
    assert len(declared) == 14, declared
    lib = ctypes.CDLL(purlin.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(purlin.exported_symbols()) == declared


def test_only_the_abi_is_exported(purlin):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", purlin.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    funcs = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert funcs == header_functions()


A_IN, A_OUT = 0x7f0000000000, 0x7f8000000000


def bufs(P, base, stride=1 << 30):
    return [base + r * stride for r in range(P)]


def expected_segments(name, P, counts, displs=None):
    """(src, dst, src_off, dst_off, len) from the oracle's naming rule."""
    in_n, out_n, op = oracle.COLLECTIVES[name]
    n = len(counts)
    in_d = out_d = None
    if displs is not None:
        in_d, out_d = displs[:n], displs[n:]
    srcs = {}
    for i in range(P):
        for nm, off, c in oracle.partitions(in_n, i, P, counts, in_d):
            srcs.setdefault(nm, []).append((i, off))
    segs = []
    for j in range(P):
        for nm, off, c in oracle.partitions(out_n, j, P, counts, out_d):
            for i, soff in srcs[nm]:
                segs.append((i, j, soff, off, c))
    return sorted(segs)


@pytest.mark.parametrize("variant", ["uniform", "v", "gapped"])
@pytest.mark.parametrize("name", list(oracle.COLLECTIVES))
@pytest.mark.parametrize("P", [1, 2, 3, 8])
def test_plan_matches_oracle_naming(purlin, P, name, variant):
    rng = np.random.default_rng([P, len(name), len(variant)])
    nparts = P * P if name == "alltoall" else P
    sizes = [5] * nparts if variant == "uniform" else [int(v) for v in rng.integers(0, 9, nparts)]
    counts = pins.counts_for(name, P, sizes)
    displs = pins.gapped_displs(name, P, counts, rng) if variant == "gapped" else None
    in_n, out_n, op = oracle.COLLECTIVES[name]
    got = purlin.plan_describe(in_n, out_n, op, "bf16", counts, bufs(P, A_IN), bufs(P, A_OUT),
                               displs)
    assert sorted(got) == expected_segments(name, P, counts, displs)


def test_plan_describe_from_many_threads(purlin):
    """Eight host threads plan 32 different collectives at once, 100 rounds
    each (the library's plan cache is shared and evicts under them): every
    plan matches the oracle's naming rule."""
    import threading
    rng = np.random.default_rng(97)
    cases = []
    for k in range(32):
        name = list(oracle.COLLECTIVES)[k % len(oracle.COLLECTIVES)]
        P = int(rng.integers(2, 9))
        nparts = P * P if name == "alltoall" else P
        counts = pins.counts_for(name, P, [int(v) for v in rng.integers(0, 9, nparts)])
        displs = pins.gapped_displs(name, P, counts, rng) if k % 3 == 0 else None
        cases.append((name, P, counts, displs, expected_segments(name, P, counts, displs)))
    errors = []
    start = threading.Barrier(8)

    def work(t):
        try:
            start.wait()
            for rnd in range(100):
                name, P, counts, displs, want = cases[(t * 5 + rnd) % len(cases)]
                in_n, out_n, op = oracle.COLLECTIVES[name]
                got = purlin.plan_describe(in_n, out_n, op, "bf16", counts, bufs(P, A_IN),
                                           bufs(P, A_OUT), displs)
                if sorted(got) != want:
                    errors.append((t, rnd, name, P))
        except Exception as e:  # reported below, with the thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors[:5]


def st(purlin, in_n, out_n, op, dtype, counts, P=8, ins=None, outs=None, displs=None):
    return purlin.plan_status(in_n, out_n, op, dtype, counts,
                              ins if ins is not None else bufs(P, A_IN),
                              outs if outs is not None else bufs(P, A_OUT), displs, P=P)


def test_valid_collectives_plan_ok(purlin):
    for name, (i, o, op) in oracle.COLLECTIVES.items():
        counts = [64] if name == "allreduce" else [8] * (64 if name == "alltoall" else 8)
        for dt in ("f32", "bf16"):
            assert st(purlin, i, o, op, dt, counts) == "OK", name


def test_invalid_arguments(purlin):
    ok = bufs(8, A_IN)
    assert st(purlin, "by_index", "by_rank", "sum", "bf16", [4] * 8, P=0, ins=ok[:0], outs=ok[:0]) == "INVALID_ARG"
    assert st(purlin, "by_index", "by_rank", "sum", "bf16", [4] * 9, P=9,
              ins=bufs(9, A_IN), outs=bufs(9, A_OUT)) == "INVALID_ARG"
    assert st(purlin, "by_index", "by_rank", "sum", "bf16", [4, -1] + [4] * 6) == "INVALID_ARG"
    # a buffer that holds elements must not be NULL
    ins = bufs(8, A_IN)
    ins[3] = 0
    assert st(purlin, "by_index", "by_rank", "sum", "bf16", [4] * 8, ins=ins) == "INVALID_ARG"
    # ... but one that holds nothing may be
    outs = bufs(8, A_OUT)
    outs[2] = 0
    counts = [4, 4, 0, 4, 4, 4, 4, 4]
    assert st(purlin, "by_index", "by_rank", "sum", "bf16", counts, outs=outs) == "OK"
    # misaligned for the element size
    ins = bufs(8, A_IN)
    ins[1] += 2
    assert st(purlin, "by_index", "by_rank", "sum", "f32", [4] * 8, ins=ins) == "INVALID_ARG"
    assert st(purlin, "by_index", "by_rank", "sum", "bf16", [4] * 8, ins=ins) == "OK"
    # input overlapping an output
    outs = bufs(8, A_OUT)
    outs[5] = A_IN + 6
    assert st(purlin, "by_index", "by_rank", "sum", "bf16", [4] * 8, outs=outs) == "INVALID_ARG"
    # two ranks' outputs overlapping
    outs = bufs(8, A_OUT)
    outs[1] = outs[0] + 2
    assert st(purlin, "by_rank", "by_index", "copy", "bf16", [4] * 8, outs=outs) == "INVALID_ARG"
    # output partitions of one rank overlapping through displs
    displs = [0] * 8 + [0, 4, 8, 12, 16, 20, 24, 26]
    assert st(purlin, "by_rank", "by_index", "copy", "bf16", [4] * 8, displs=displs) == "INVALID_ARG"
    # negative displacement
    displs = [0] * 8 + [0, 4, 8, 12, 16, 20, 24, -28]
    assert st(purlin, "by_rank", "by_index", "copy", "bf16", [4] * 8, displs=displs) == "INVALID_ARG"
    # bad enum values
    assert st(purlin, "by_index", "by_rank", 7, "bf16", [4] * 8) == "INVALID_ARG"
    assert st(purlin, "by_index", "by_rank", "sum", 9, [4] * 8) == "INVALID_ARG"


def test_unsupported_triples(purlin):
    assert st(purlin, "whole", "whole", "copy", "bf16", [16]) == "UNSUPPORTED"        # 8 sources
    assert st(purlin, "whole", "by_rank", "sum", "bf16", [16]) == "UNSUPPORTED"       # name sets differ
    assert st(purlin, "by_rank", "by_index", "sum", "bf16", [4] * 8) == "OK"          # one-term sums
    assert st(purlin, "by_index", "by_rank", "copy", "bf16", [4] * 8) == "UNSUPPORTED"
    assert st(purlin, "by_rank_index", "by_rank_index", "copy", "bf16", [2] * 64) == "OK"
    assert st(purlin, "by_index", "by_index", "sum", "bf16", [4] * 8) == "OK"
    # at P = 1 every naming has one name, but names of different lengths
    # never match: () is not (0), and (0) is not (0, 0)
    for i_, o_ in (("whole", "by_rank"), ("by_index", "whole"), ("by_rank", "by_rank_index"),
                   ("by_index_rank", "by_index")):
        for op in ("copy", "sum"):
            assert st(purlin, i_, o_, op, "bf16", [4], P=1) == "UNSUPPORTED", (i_, o_, op)
    assert st(purlin, "by_rank", "by_index", "copy", "bf16", [4], P=1) == "OK"


def test_null_layouts(purlin):
    import ctypes
    lib = purlin._lib
    c = (ctypes.c_int64 * 1)(4)
    assert lib.purlin_collective(None, None, 0, 0, 1, c, None, None) == 1
    n = ctypes.c_int64(0)
    assert lib.purlin_plan_describe(None, None, 0, 0, 1, c, None, None, ctypes.byref(n)) == 1


def test_policy_roundtrip_and_validation(purlin):
    purlin.set_policy(chunk_bytes=8192, depth=3, wgs_per_rank=4, zero_staging="staged",
                      sync=False, watchdog_ns=10 ** 7)
    p = purlin.get_policy()
    assert (p["chunk_bytes"], p["depth"], p["wgs_per_rank"], p["zero_staging"], p["sync"],
            p["watchdog_ns"]) == (8192, 3, 4, 2, 2, 10 ** 7)
    with pytest.raises(purlin.PurlinError):
        purlin.set_policy(chunk_bytes=1000)            # not a multiple of 4096
    with pytest.raises(purlin.PurlinError):
        purlin.set_policy(depth=9)
    purlin.set_policy(reset=True)
    assert purlin.get_policy()["chunk_bytes"] == 0


def test_strerror(purlin):
    assert purlin._lib.purlin_strerror(5) == b"device wait timed out"
    assert purlin._lib.purlin_strerror(6) == b"protocol check failed"
    assert purlin._lib.purlin_strerror(42) == b"unknown status"


def test_moe_argument_checks(purlin):
    """MoE dispatch / combine reject bad arguments before any HIP call."""
    import ctypes
    lib = purlin._lib
    P = 2
    V = ctypes.c_void_p * P
    x = V(A_IN, A_IN + (1 << 30))
    y = V(A_OUT, A_OUT + (1 << 30))
    idx = V(0x10000, 0x20000)
    w = V(0x30000, 0x40000)
    I64 = ctypes.c_int64

    def disp(counts, x_rows, row_bytes=64, P_=P, idx_=idx, y_=y):
        return lib.purlin_moe_dispatch(x, y_, P_, row_bytes, idx_, (I64 * len(counts))(*counts),
                                       (I64 * len(x_rows))(*x_rows), 0, None)

    def comb(counts, x_rows, row_bytes=64, w_=w, out=x):
        return lib.purlin_moe_combine(y, out, P, row_bytes, idx, w_, (I64 * len(counts))(*counts),
                                      (I64 * len(x_rows))(*x_rows), None)

    assert disp([1, 1, 1, 1], [4, 4], P_=0) == 1
    assert disp([1, 1, 1, 1], [4, 4], P_=9) == 1
    assert disp([1, -1, 1, 1], [4, 4]) == 1                 # negative count
    assert disp([1, 1, 1, 1], [4, -4]) == 1                 # negative row count
    assert disp([1, 1, 1, 1], [4, 4], row_bytes=63) == 1    # odd row
    assert disp([1, 1, 1, 1], [4, 4], row_bytes=0) == 1
    assert disp([1, 1, 1, 1], [4, 4], row_bytes=(1 << 30) + 2) == 1   # a row above 1 GiB
    assert disp([1, 1, 1, 1], [4, 0]) == 1                  # entries for a rank with no rows
    assert disp([1, 1, 1, 1], [4, 4], idx_=V(0x10000, 0)) == 1   # NULL index array with entries
    assert disp([1, 1, 1, 1], [4, 4], y_=V(A_OUT, A_OUT + 64)) == 1  # outputs overlap
    assert disp([1, 1, 1, 1], [4, 4], y_=V(A_IN + 64, A_OUT)) == 1   # output inside an input
    assert comb([1, 1, 1, 1], [4, 4], row_bytes=24) == 1    # combine rows: 16-byte multiples
    assert comb([1, 1, 1, 1], [4, 4], w_=V(0x30000, 0)) == 1     # NULL weights with entries
    assert comb([1, 1, 1, 1], [4, 4], out=V(A_IN + 8, A_IN + (1 << 30))) == 1  # misaligned


def test_ulysses_argument_checks(purlin):
    """The Ulysses exchange rejects bad arguments before any HIP call."""
    import ctypes
    lib = purlin._lib
    P = 2
    V = ctypes.c_void_p * P
    I64 = ctypes.c_int64
    ins = V(A_IN, A_IN + (1 << 30))
    outs = V(A_OUT, A_OUT + (1 << 30))

    def uly(seq, heads=4, head_bytes=256, to_sequence=0, P_=P, in_=ins, out_=outs):
        return lib.purlin_ulysses(in_, out_, P_, (I64 * len(seq))(*seq), heads, head_bytes,
                                  to_sequence, None)

    assert uly([4, 4], P_=0) == 1
    assert uly([4, 4], P_=9) == 1
    assert uly([4, 4], heads=3) == 1                 # heads not a multiple of P
    assert uly([4, 4], heads=0) == 1
    assert uly([4, 4], head_bytes=255) == 1          # odd head size
    assert uly([4, 4], head_bytes=0) == 1
    assert uly([4, -1]) == 1                         # negative token count
    assert uly([4, 4], to_sequence=2) == 1
    assert uly([4, 4], in_=V(A_IN, 0)) == 1          # NULL buffer that holds tokens
    assert uly([4, 4], in_=V(A_IN + 1, A_IN + (1 << 30))) == 1          # odd address
    assert uly([4, 4], out_=V(A_IN + 512, A_OUT)) == 1                  # output inside an input
    assert uly([4, 4], to_sequence=1, out_=V(A_OUT, A_IN)) == 1         # and the other way
    assert uly([4, 4], out_=V(A_OUT, A_OUT + 1024)) == 1                # outputs overlap
    assert uly([1 << 41, 4]) == 1                                       # too many tokens
    assert uly([0, 0], in_=V(0, 0), out_=V(0, 0)) == 0                  # nothing to move


def test_binding_structs_match_the_header(purlin, tmp_path):
    """The binding's ctypes structures have the size and field offsets of
    the header's structs (compiled with the host compiler), so that no call
    writes past a structure the binding passes."""
    import ctypes
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no host compiler")
    here = os.path.dirname(os.path.abspath(__file__))
    inc = os.path.join(here, "..", "include")
    structs = {"purlin_launch_info": purlin.LaunchInfo, "purlin_policy": purlin.Policy,
               "purlin_layout": purlin.Layout, "purlin_segment": purlin.Segment}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "purlin.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append('  printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in py._fields_:
            lines.append('  printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I", "/opt/rocm/include",
                    "-o", str(exe), str(src)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True,
                               text=True).stdout.splitlines():
        a, b, v = line.split()
        got[(a, b)] = int(v)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_stream_pattern_argument_checks(purlin):
    """The ceiling pattern rejects bad arguments before any HIP call; a
    zero-byte pattern with valid arguments is a no-op."""
    import ctypes
    lib = purlin._lib
    V = ctypes.c_void_p * 8
    srcs = V(*[A_IN + r * (1 << 30) for r in range(8)])
    dsts = V(*[A_OUT + r * (1 << 30) for r in range(8)])

    def pat(n_src=1, n_dst=1, nbytes=0, grid=0, tile=0, unroll=0, access=3):
        return lib.purlin_stream_pattern(srcs, n_src, dsts, n_dst, nbytes, grid, tile, unroll,
                                         access, None)

    assert pat(n_src=0, n_dst=0) == 1                # nothing read or written
    assert pat(n_src=2) == 1                         # 0, 1 or 8 streams only
    assert pat(nbytes=24) == 1                       # not a multiple of 16
    assert pat(grid=65537) == 1
    assert pat(tile=24) == 1
    assert pat(tile=1 << 32) == 1                    # a tile spans less than 4 GiB
    assert pat(unroll=3) == 1
    assert pat(access=8) == 1                        # bits 0-2 only
    assert pat(access=-1) == 1
    for access in range(8):                          # every store and load mode
        assert pat(access=access) == 0


@pytest.mark.parametrize("P", [5, 6, 7, 8])
def test_job_bound_after_the_broadcast_split(purlin, P):
    """A sum of P partitions broadcast to every rank (by_index -> by_index)
    derives P * P pieces; outputs off each other's 16-byte phase would split
    each into P single-destination jobs, past the 64 a launch plan holds:
    refused as UNSUPPORTED before any HIP call (describe and collective)."""
    counts = [40] * P
    outs = [A_OUT + r * (1 << 30) + 2 * r for r in range(P)]   # phases 0, 2, 4, ... bytes
    assert st(purlin, "by_index", "by_index", "sum", "bf16", counts, P=P,
              ins=bufs(P, A_IN), outs=outs) == "UNSUPPORTED"
    with pytest.raises(purlin.PurlinError) as e:
        purlin.collective(bufs(P, A_IN), outs, "by_index", "by_index", "sum", counts, dtype="bf16",
                          stream=0)
    assert e.value.status == "UNSUPPORTED"
    # congruent outputs keep the broadcast jobs: within the bound
    assert st(purlin, "by_index", "by_index", "sum", "bf16", counts, P=P,
              ins=bufs(P, A_IN), outs=bufs(P, A_OUT)) == "OK"
    # the same split of a single sum (AllReduce) stays at P * P jobs
    assert st(purlin, "whole", "whole", "sum", "bf16", [40 * P], P=P, ins=bufs(P, A_IN),
              outs=outs) == "OK"


def test_binding_rejects_tensors_it_would_misread(purlin):
    """The Python binding checks tensors before the C call: CPU tensors, a
    dtype mismatch, non-contiguous views and buffers shorter than their
    partitions raise ValueError (no GPU work is started)."""
    import torch
    P = 8
    x = [torch.zeros(8, dtype=torch.bfloat16) for _ in range(P)]
    y = [torch.zeros(64, dtype=torch.bfloat16) for _ in range(P)]
    with pytest.raises(ValueError, match="not on the current GPU"):
        purlin.all_gather(x, y)
    # the extents each rank's buffer must reach
    assert purlin.extents("by_rank", P, [8] * P) == [8] * P
    assert purlin.extents("by_index", P, [8] * P) == [64] * P
    assert purlin.extents("by_index", 2, [3, 0], [10, 40]) == [13, 13]
    assert purlin.extents("by_rank_index", 2, [1, 2, 3, 4]) == [3, 7]
    assert purlin.extents("by_index_rank", 2, [1, 2, 3, 4]) == [4, 6]
    assert purlin.extents("whole", 3, [5], [2]) == [7, 7, 7]
    # tensor checks, device check skipped (no GPU here)
    need = [64] * P
    purlin.check_tensors(y, need, "bf16", "copy", "output")
    short = list(y)
    short[3] = torch.zeros(63, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="output 3 holds 63 elements"):
        purlin.check_tensors(short, need, "bf16", "copy", "output")
    mixed = list(y)
    mixed[5] = torch.zeros(64, dtype=torch.float16)
    with pytest.raises(ValueError, match="dtype"):
        purlin.check_tensors(mixed, need, "bf16", "copy", "output")
    with pytest.raises(ValueError, match="dtype"):
        purlin.check_tensors([torch.zeros(64, dtype=torch.float16)] * P, need, "bf16", "sum", "input")
    with pytest.raises(ValueError, match="dtype"):
        purlin.check_tensors(y, [16] * P, "f32", "copy", "input")
    strided = list(y)
    strided[0] = torch.zeros(128, dtype=torch.bfloat16)[::2]
    with pytest.raises(ValueError, match="not contiguous"):
        purlin.check_tensors(strided, need, "bf16", "copy", "output")
    # raw addresses and None pass unchecked
    purlin.check_tensors([A_IN, None] + y[2:], need, "bf16", "copy", "output")
    # a counts array of the wrong length never reaches the library
    with pytest.raises(ValueError, match="counts"):
        purlin.collective(bufs(P, A_IN), bufs(P, A_OUT), "by_rank", "by_index", "copy", [8] * 7,
                          dtype="bf16")
    with pytest.raises(ValueError, match="displs"):
        purlin.collective(bufs(P, A_IN), bufs(P, A_OUT), "by_rank", "by_index", "copy", [8] * 8,
                          [0] * 8, dtype="bf16")
