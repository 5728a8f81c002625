"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer,
fuzzed against the oracle's naming rule (CPU only).

tests/planner_fuzz/fuzz_main.cpp drives the planner's own source (built here
with g++ and both sanitizers, aborting on the first report) over seeded
random specifications: every pair of namings, both ops and dtypes, P from 1
to 8, counts with zeros and occasional invalid values, packed or random
displacements, and output buffers at random 16-byte phases for the launch
split.  Checked for every case: no sanitizer report; a derivation that
succeeds lists exactly the (source, destination, offsets, length) segments
the oracle's naming rule gives; a refusal is one the rules explain (an
invalid count or displacement -> INVALID_ARG; name sets that differ, a copy
output without exactly one source, a sum whose sources are not every rank at
one offset -> UNSUPPORTED); the launch split stays within 64 jobs or is
refused.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = [os.path.join(HERE, "planner_fuzz", "fuzz_main.cpp"),
       os.path.join(os.path.dirname(HERE), "reduce_atom_02_amd", "csrc", "planner.cpp")]
NAMINGS = ["whole", "by_rank", "by_index", "by_rank_index", "by_index_rank"]
OK, INVALID, UNSUPPORTED = 0, 1, 2


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path_factory.mktemp("pfuzz") / "pfuzz")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-o", exe] + SRC, check=True, capture_output=True, text=True)
    return exe


def expected(in_n, out_n, op, P, counts, displs):
    """Status and segments by the oracle's naming rule and the planner's
    documented limits (a sum: one source, or every rank at one offset)."""
    nn, nn_out = oracle.name_count(in_n, P), oracle.name_count(out_n, P)
    if any(c < 0 or c > (1 << 40) for c in counts):
        return INVALID, None
    if displs is not None and any(d < 0 or d > (1 << 40) for d in displs[:2 * min(nn, nn_out)]):
        return INVALID, None
    if nn != nn_out:
        return UNSUPPORTED, None
    in_d = displs[:nn] if displs is not None else None
    out_d = displs[nn:] if displs is not None else None
    srcs = {}
    for i in range(P):
        for name, off, c in oracle.partitions(in_n, i, P, counts, in_d):
            srcs.setdefault(name, []).append((i, off))
    segs = []
    for j in range(P):
        for name, off, c in oracle.partitions(out_n, j, P, counts, out_d):
            m = srcs.get(name, [])
            if op == "copy" and len(m) != 1:
                return UNSUPPORTED, None
            if op == "sum" and not m:
                return UNSUPPORTED, None
            for i, soff in m:
                segs.append((i, j, soff, off, c))
            if c and len(m) > 1 and (len(m) != P or any(s[1] != m[0][1] for s in m)):
                return UNSUPPORTED, None
    return OK, sorted(segs)


def make_case(rng):
    in_n = NAMINGS[int(rng.integers(0, 5))]
    # half the cases use a matching pair of the seven collectives' shapes
    out_n = NAMINGS[int(rng.integers(0, 5))] if rng.random() < 0.5 else {
        "whole": "whole", "by_index": "by_rank", "by_rank": "by_index",
        "by_rank_index": "by_index_rank", "by_index_rank": "by_rank_index"}[in_n]
    op = "sum" if rng.random() < 0.5 else "copy"
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    P = int(rng.integers(1, 9))
    nn = oracle.name_count(in_n, P)
    counts = [int(v) for v in rng.integers(0, 50, nn)]
    if rng.random() < 0.3:
        counts[int(rng.integers(0, nn))] = 0
    if rng.random() < 0.05:
        counts[int(rng.integers(0, nn))] = -int(rng.integers(1, 5))
    displs = None
    if rng.random() < 0.4:
        nd = 2 * min(nn, oracle.name_count(out_n, P))
        displs = [int(v) for v in rng.integers(0, 4000, nd)]
        if rng.random() < 0.05:
            displs[int(rng.integers(0, nd))] = -1
    esz = 2 if dtype == "bf16" else 4
    outs = [0x7f0000000000 + r * (1 << 32) + esz * int(rng.integers(0, 16 // esz)) for r in range(P)]
    return in_n, out_n, op, dtype, P, counts, displs, outs


def test_planner_fuzz_under_sanitizers(driver):
    # PURLIN_FUZZ_SEED / PURLIN_FUZZ_CASES: another seed and more cases for a
    # longer search (defaults: the committed 3000)
    rng = np.random.default_rng(20261203 + int(os.environ.get("PURLIN_FUZZ_SEED", "0")))
    cases = [make_case(rng) for _ in range(int(os.environ.get("PURLIN_FUZZ_CASES", "3000")))]
    # the seven collectives at P = 8 with misaligned outputs, and the case that
    # overflows the launch plan (by_index -> by_index sum, outputs off phase)
    for name, (i_, o_, op_) in oracle.COLLECTIVES.items():
        nn = oracle.name_count(i_, 8)
        cases.append((i_, o_, op_, "bf16", 8, [7] * nn, None,
                      [0x7f0000000000 + r * (1 << 32) + 2 * r for r in range(8)]))
    cases.append(("by_index", "by_index", "sum", "bf16", 8, [40] * 8, None,
                  [0x7f0000000000 + r * (1 << 32) + 2 * r for r in range(8)]))
    lines = []
    for in_n, out_n, op, dtype, P, counts, displs, outs in cases:
        d = displs or []
        lines.append(" ".join(str(v) for v in (
            [NAMINGS.index(in_n), NAMINGS.index(out_n), 1 if op == "sum" else 0,
             1 if dtype == "bf16" else 0, P, len(counts)] + counts + [len(d)] + d + [len(outs)] + outs)))
    res = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"), timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]
    blocks = res.stdout.split("end\n")[:-1]
    assert len(blocks) == len(cases)
    n_ok = n_split_refused = 0
    for case, block in zip(cases, blocks):
        in_n, out_n, op, dtype, P, counts, displs, outs = case
        rows = block.strip().splitlines()
        status = int(rows[0].split()[1])
        want_status, want_segs = expected(in_n, out_n, op, P, counts, displs)
        assert status == want_status, (case, status, want_status)
        if status != OK:
            continue
        n_ok += 1
        segs = sorted(tuple(int(x) for x in r.split()[1:]) for r in rows if r.startswith("seg "))
        assert segs == want_segs, case
        js, njobs = [int(x) for x in next(r for r in rows if r.startswith("jobs ")).split()[1:]]
        assert js in (OK, UNSUPPORTED)
        if js == OK:
            assert njobs <= 64, case
        else:
            n_split_refused += 1
    assert n_ok > 500
    assert n_split_refused >= 1          # the overflowing case is refused, not written past the plan
