"""Checks that pin the oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix.  They are run by
``test_oracle_pins.py`` and, against deliberately broken copies of the
oracle, by ``test_oracle_mutations.py``.
"""
import math
import os
from fractions import Fraction

import numpy as np

import oracle
from oracle import collective, collective_brute, COLLECTIVES

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

STORE = {"f32": np.uint32, "bf16": np.uint16}


def _rand_bits(rng, n, dtype):
    x = rng.standard_normal(n).astype(np.float32)
    if dtype == "f32":
        return x.view(np.uint32)
    return oracle.round_bf16(x)


def layout_sizes(name, P, counts, displs):
    """(input length, output length) per rank that hold every partition."""
    n = len(counts)
    in_n, out_n, op = COLLECTIVES[name]
    in_d = out_d = None
    if displs is not None:
        in_d, out_d = displs[:n], displs[n:]
    ins, outs = [], []
    for r in range(P):
        a = oracle.partitions(in_n, r, P, counts, in_d)
        b = oracle.partitions(out_n, r, P, counts, out_d)
        ins.append(max([o + c for _, o, c in a] + [0]))
        outs.append(max([o + c for _, o, c in b] + [0]))
    return ins, outs


def make_case(name, P, counts, dtype, rng, displs=None, sentinel=0xABCD):
    in_len, out_len = layout_sizes(name, P, counts, displs)
    ins = [_rand_bits(rng, in_len[r], dtype) for r in range(P)]
    outs = [np.full(out_len[r], sentinel, dtype=STORE[dtype]) for r in range(P)]
    return ins, outs


def run(name, P, counts, dtype, ins, outs, displs=None):
    in_n, out_n, op = COLLECTIVES[name]
    return collective(in_n, out_n, op, dtype, P, counts, displs, ins, outs)


def counts_for(name, P, sizes):
    """sizes: list of P per-partition sizes (or P*P for alltoall)."""
    if name == "allreduce":
        return [sum(sizes)]
    return list(sizes)


def gapped_displs(name, P, counts, rng):
    """Non-packed displacements with random gaps, indexed by name."""
    in_n, out_n, _ = COLLECTIVES[name]
    n = len(counts)
    side = []
    for naming in (in_n, out_n):
        d = [0] * n
        for r in range(P):
            parts = oracle.partitions(naming, r, P, counts, None)
            cursor = int(rng.integers(0, 3))
            order = list(range(len(parts)))
            rng.shuffle(order)                      # partitions need not be in index order
            for q in order:
                nm, _, c = parts[q]
                num = 0 if not nm else (nm[0] if len(nm) == 1 else nm[0] * P + nm[1])
                d[num] = cursor
                cursor += c + int(rng.integers(0, 3))
        side.append(d)
    # by_index (and whole) partitions share one offset across ranks: the
    # last rank's choice wins, and the packed widths above keep it disjoint
    # only if every rank agrees; rebuild those sides rank-independently.
    for s, naming in enumerate((in_n, out_n)):
        if naming in ("whole", "by_index"):
            cursor = 0
            d = [0] * n
            for num in rng.permutation(n):
                d[int(num)] = cursor
                cursor += counts[int(num)] + int(rng.integers(0, 3))
            side[s] = d
    return side[0] + side[1]


def pin_brute_force(seed=1, Ps=(1, 2, 3, 4, 8)):
    """Oracle == per-element brute force (exact rational arithmetic), bitwise."""
    rng = np.random.default_rng(seed)
    for P in Ps:
        for name in COLLECTIVES:
            for dtype in ("f32", "bf16"):
                for variant in ("uniform", "v", "gapped"):
                    nparts = P * P if name == "alltoall" else P
                    hi = 2 if (name == "alltoall" and P == 8) else 4
                    if variant == "uniform":
                        sizes = [2] * nparts
                    else:
                        sizes = [int(v) for v in rng.integers(0, hi, nparts)]
                    counts = counts_for(name, P, sizes)
                    displs = gapped_displs(name, P, counts, rng) if variant == "gapped" else None
                    ins, outs = make_case(name, P, counts, dtype, rng, displs)
                    got = run(name, P, counts, dtype, ins, outs, displs)
                    in_n, out_n, op = COLLECTIVES[name]
                    want = collective_brute(in_n, out_n, op, dtype, P, counts, displs, ins, outs)
                    for j in range(P):
                        assert [int(v) for v in got[j]] == want[j], (P, name, dtype, variant, j)


def pin_allgather_concat(seed=2):
    """AllGather output of every rank == numpy.concatenate of the inputs."""
    rng = np.random.default_rng(seed)
    for P in (2, 5, 8):
        for sizes in ([7] * P, [int(v) for v in rng.integers(0, 9, P)]):
            ins = [_rand_bits(rng, sizes[r], "bf16") for r in range(P)]
            outs = [np.zeros(sum(sizes), np.uint16) for _ in range(P)]
            got = run("allgather", P, sizes, "bf16", ins, outs)
            ref = np.concatenate(ins)
            for j in range(P):
                assert np.array_equal(got[j], ref), (P, j)


def pin_alltoall_swapaxes(seed=3):
    """Equal-partition AllToAll == numpy.swapaxes of a [src, dst, n] block array."""
    rng = np.random.default_rng(seed)
    for P, n in ((2, 3), (4, 1), (8, 5)):
        blocks = _rand_bits(rng, P * P * n, "f32").reshape(P, P, n)
        ins = [blocks[i].reshape(-1).copy() for i in range(P)]
        outs = [np.zeros(P * n, np.uint32) for _ in range(P)]
        got = run("alltoall", P, [n] * (P * P), "f32", ins, outs)
        ref = np.swapaxes(blocks, 0, 1)
        for j in range(P):
            assert np.array_equal(got[j], ref[j].reshape(-1)), (P, j)


def pin_alltoall_involution(seed=4):
    """AllToAll(V) followed by AllToAll(V) with the transposed counts is the identity."""
    rng = np.random.default_rng(seed)
    for P in (1, 3, 8):
        counts = [int(v) for v in rng.integers(0, 6, P * P)]
        t_counts = [counts[j * P + i] for i in range(P) for j in range(P)]
        ins, outs = make_case("alltoall", P, counts, "bf16", rng)
        mid = run("alltoall", P, counts, "bf16", ins, outs)
        back_outs = [np.zeros_like(x) for x in ins]
        back = run("alltoall", P, t_counts, "bf16", mid, back_outs)
        for i in range(P):
            assert np.array_equal(back[i], ins[i]), (P, i)


def pin_allreduce_composition(seed=5):
    """AllReduce == AllGather(ReduceScatter(x)) bitwise (Figure 6 composition)."""
    rng = np.random.default_rng(seed)
    for dtype in ("f32", "bf16"):
        for P in (1, 3, 8):
            sizes = [int(v) for v in rng.integers(0, 7, P)]
            N = sum(sizes)
            ins = [_rand_bits(rng, N, dtype) for _ in range(P)]
            ar = run("allreduce", P, [N], dtype, ins, [np.zeros(N, STORE[dtype]) for _ in range(P)])
            ys = run("reducescatter", P, sizes, dtype, ins,
                     [np.zeros(sizes[k], STORE[dtype]) for k in range(P)])
            ag = run("allgather", P, sizes, dtype, ys, [np.zeros(N, STORE[dtype]) for _ in range(P)])
            for j in range(P):
                assert np.array_equal(ar[j], ag[j]), (dtype, P, j)


def pin_integer_sums(seed=6):
    """Integer-valued inputs: every fp32 partial sum is exact, so the result is the int sum."""
    rng = np.random.default_rng(seed)
    for P in (2, 8):
        n = 37
        ints = [rng.integers(-(1 << 20), 1 << 20, n * P) for _ in range(P)]
        ins = [v.astype(np.float32).view(np.uint32) for v in ints]
        exact = sum(v.astype(np.int64) for v in ints)
        ar = run("allreduce", P, [n * P], "f32", ins, [np.zeros(n * P, np.uint32) for _ in range(P)])
        for j in range(P):
            assert np.array_equal(ar[j].view(np.float32).astype(np.int64), exact)
        rs = run("reducescatter", P, [n] * P, "f32", ins, [np.zeros(n, np.uint32) for _ in range(P)])
        for k in range(P):
            assert np.array_equal(rs[k].view(np.float32).astype(np.int64), exact[k * n:(k + 1) * n])
        # bf16: inputs are small integers (exact in bf16); the fp32 sum is exact
        # and the single bf16 rounding is torch's CPU conversion of that sum.
        import torch
        small = [rng.integers(-256, 257, n * P) for _ in range(P)]
        ins16 = [torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
                 .numpy().view(np.uint16) for v in small]
        tot = sum(v.astype(np.int64) for v in small).astype(np.float32)
        ref = torch.from_numpy(tot).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        ar16 = run("allreduce", P, [n * P], "bf16", ins16, [np.zeros(n * P, np.uint16) for _ in range(P)])
        for j in range(P):
            assert np.array_equal(ar16[j], ref)


def pin_error_bound(seed=7):
    """Recursive fp32 summation error <= gamma_{P-1} * sum|x_i| (Higham), vs math.fsum."""
    rng = np.random.default_rng(seed)
    P, n = 8, 2000
    u = 2.0 ** -24
    gamma = (P - 1) * u / (1 - (P - 1) * u)
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(P)]
    got = run("allreduce", P, [n], "f32", [x.view(np.uint32) for x in xs],
              [np.zeros(n, np.uint32) for _ in range(P)])[0].view(np.float32)
    for e in range(n):
        terms = [float(x[e]) for x in xs]
        exact = math.fsum(terms)
        bound = gamma * math.fsum(abs(t) for t in terms)
        assert abs(float(got[e]) - exact) <= bound, e
    # bf16 output adds at most half a bf16 ulp of the fp32 result
    xs16 = [oracle.round_bf16(x) for x in xs]
    got16 = run("allreduce", P, [n], "bf16", xs16, [np.zeros(n, np.uint16) for _ in range(P)])[0]
    w = [oracle.widen_bf16(x) for x in xs16]
    res = oracle.widen_bf16(got16)
    for e in range(n):
        terms = [float(x[e]) for x in w]
        exact = math.fsum(terms)
        s = abs(exact) if exact else 1e-30
        half_ulp = 2.0 ** (math.floor(math.log2(s)) - 8) if exact else 0.0
        bound = gamma * math.fsum(abs(t) for t in terms) * (1 + 2.0 ** -8) + half_ulp * 1.0001
        assert abs(float(res[e]) - exact) <= bound, e


def load_fig4():
    rows = []
    with open(os.path.join(GOLDEN, "fig4_three_ranks.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            name, rank, rest = line.split(None, 2)
            cells = []
            for cell in rest.split("|"):
                terms = [tuple(int(x) for x in t.strip().split(".")) for t in cell.split("+")]
                cells.append(terms)
            rows.append((name, int(rank), cells))
    return rows


def pin_fig4(m=2):
    """The three-rank layouts of Figure 4 (and Figure 6's AllReduce), from the fixture."""
    P = 3
    rows = load_fig4()
    assert len(rows) == 12
    for name in COLLECTIVES:
        # one m-element block per input partition, values 100*i + 10*q + e
        if name in ("allgather", "allreduce"):
            n_in_parts = 1
        else:
            n_in_parts = P
        ins_val = [[[100 * i + 10 * q + e for e in range(m)] for q in range(n_in_parts)]
                   for i in range(P)]
        ins = [np.array(sum(ins_val[i], []), np.float32).view(np.uint32) for i in range(P)]
        if name == "allreduce":
            counts = [m]
        elif name == "alltoall":
            counts = [m] * (P * P)
        else:
            counts = [m] * P
        out_len = {"allreduce": m, "reducescatter": m, "allgather": P * m, "alltoall": P * m}[name]
        got = run(name, P, counts, "f32", ins, [np.zeros(out_len, np.uint32) for _ in range(P)])
        for cname, j, cells in rows:
            if cname != name:
                continue
            want = []
            for terms in cells:
                want.extend(sum(ins_val[i][q][e] for i, q in terms) for e in range(m))
            assert got[j].view(np.float32).tolist() == [float(v) for v in want], (name, j)


def pin_p1_identity(seed=8):
    """P = 1: every collective is the identity (a one-term sum rounds to itself)."""
    rng = np.random.default_rng(seed)
    for name in COLLECTIVES:
        for dtype in ("f32", "bf16"):
            n = 11
            x = _rand_bits(rng, n, dtype)
            got = run(name, 1, [n], dtype, [x], [np.zeros(n, STORE[dtype])])
            assert np.array_equal(got[0], x), (name, dtype)


def pin_untouched(seed=9):
    """Output elements outside every named partition keep their prior contents."""
    rng = np.random.default_rng(seed)
    for name in COLLECTIVES:
        P = 4
        nparts = P * P if name == "alltoall" else P
        counts = counts_for(name, P, [int(v) for v in rng.integers(0, 4, nparts)])
        displs = gapped_displs(name, P, counts, rng)
        ins, outs = make_case(name, P, counts, "bf16", rng, displs, sentinel=0x7E57)
        outs = [np.concatenate([o, np.full(3, 0x7E57, np.uint16)]) for o in outs]
        got = run(name, P, counts, "bf16", ins, outs, displs)
        in_n, out_n, _ = COLLECTIVES[name]
        n = len(counts)
        for j in range(P):
            covered = np.zeros(got[j].size, bool)
            for _, off, c in oracle.partitions(out_n, j, P, counts, displs[n:]):
                covered[off:off + c] = True
            assert np.all(got[j][~covered] == 0x7E57), (name, j)


def pin_subnormals():
    """fp32 subnormals are added exactly, never flushed."""
    tiny = np.float32(2.0 ** -149)
    P = 8
    ins = [np.array([tiny * (i + 1), -tiny, tiny * 3], np.float32).view(np.uint32) for i in range(P)]
    got = run("allreduce", P, [3], "f32", ins, [np.zeros(3, np.uint32) for _ in range(P)])[0]
    want = np.array([tiny * 36, -tiny * 8, tiny * 24], np.float32)
    assert np.array_equal(got.view(np.float32), want)
    assert got.view(np.float32)[0] != 0


def pin_rne_values():
    """bf16 rounding on values whose correct rounding is known by hand."""
    one = 1.0
    cases = [
        (one, 0x3F80),
        (one + 2.0 ** -8, 0x3F80),                  # tie -> even (down)
        (one + 3 * 2.0 ** -8, 0x3F82),              # tie -> even (up)
        (one + 2.0 ** -8 + 2.0 ** -20, 0x3F81),     # above the tie -> up
        (-(one + 2.0 ** -8), 0xBF80),
        (float(np.finfo(np.float32).max), 0x7F80),  # max fp32 -> +inf
        (3.3895313892515355e38, 0x7F7F),            # max bf16 stays
        (float(np.float32(2.0 ** -149)), 0x0000),   # smallest subnormal -> +0
        (float(np.float32(2.0 ** -133)), 0x0001),   # smallest bf16 subnormal stays
        (float("inf"), 0x7F80),
        (float("-inf"), 0xFF80),
    ]
    for x, want in cases:
        assert oracle.round_bf16(np.array([x], np.float32))[0] == want, (x, hex(want))
    nan = np.array([0x7F800001, 0xFFC12345, 0x7FFFFFFF], np.uint32).view(np.float32)
    assert oracle.round_bf16(nan).tolist() == [0x7FC0, 0xFFC1, 0x7FFF]


ALL_PINS = [pin_brute_force, pin_allgather_concat, pin_alltoall_swapaxes,
            pin_alltoall_involution, pin_allreduce_composition, pin_integer_sums,
            pin_error_bound, pin_fig4, pin_p1_identity, pin_untouched, pin_subnormals,
            pin_rne_values]
