"""Pins of the MoE dispatch / combine oracle (oracle/moe.py), each checked
against something other than the oracle's own code:

* dispatch, brute force on tagged rows: every output row decodes to the
  (source rank, token) the routing puts at that position, found by walking
  the routing table entry by entry;
* dispatch with every row in order is the AllToAllV oracle (pinned on its
  own) over the same bytes;
* combine(dispatch(x)) with unit weights, small integer rows and the
  deduplicated routing is n(t) * x[t] exactly, n(t) = ranks token t goes to;
* combine against an exact-rational brute force that rounds each product
  and each add to fp32 and the result to bf16 (oracle/brute.round_binary);
* a cancellation that fp32 rounding in ascending rank order decides;
* a token routed nowhere comes back +0; a token twice in one group is
  rejected; an index outside its rank's rows is rejected;
* five planted mistakes (sources in the wrong order, fp64 accumulator,
  descending ranks, weights ignored, truncation) each fail some pin.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from oracle import moe
from oracle.brute import round_binary


def routing(P, x_rows, rng, dedup=True, fanout=3):
    """Random routing: each token goes to up to `fanout` distinct ranks."""
    idx, counts = [], []
    for i in range(P):
        dest = [rng.choice(P, size=int(rng.integers(0, fanout + 1)), replace=False)
                for _ in range(x_rows[i])]
        groups = [[t for t in range(x_rows[i]) if j in dest[t]] for j in range(P)]
        if not dedup:
            groups = [g + g[:1] for g in groups]
        idx.append(np.array([t for g in groups for t in g], dtype=np.int32))
        counts.extend(len(g) for g in groups)
    return idx, counts


def test_dispatch_brute_force_on_tagged_rows(dispatch=moe.dispatch):
    P, H = 4, 3
    rng = np.random.default_rng(1)
    x_rows = [5, 0, 7, 3]
    # row t of rank i holds (i, t, 0x7E57)
    x = [np.array([[i, t, 0x7E57] for t in range(x_rows[i])], dtype=np.uint16).reshape(-1, H)
         for i in range(P)]
    idx, counts = routing(P, x_rows, rng)
    y = dispatch(x, idx, counts, P)
    for j in range(P):
        want = []
        for i in range(P):
            start = sum(counts[i * P + q] for q in range(j))
            for k in range(counts[i * P + j]):
                want.append((i, int(idx[i][start + k])))
        assert len(y[j]) == len(want)
        for row, (i, t) in zip(y[j], want):
            assert tuple(int(v) for v in row) == (i, t, 0x7E57)


def test_dispatch_in_order_is_alltoallv(dispatch=moe.dispatch):
    P, H = 3, 4
    rng = np.random.default_rng(2)
    counts = [int(v) for v in rng.integers(0, 5, P * P)]
    x_rows = [sum(counts[i * P:(i + 1) * P]) for i in range(P)]
    x = [rng.integers(0, 1 << 16, (x_rows[i], H)).astype(np.uint16) for i in range(P)]
    idx = [np.arange(x_rows[i], dtype=np.int32) for i in range(P)]
    y = dispatch(x, idx, counts, P)
    elems = [c * H for c in counts]
    outs = [np.zeros(sum(elems[q * P + j] for q in range(P)), np.uint16) for j in range(P)]
    want = oracle.collective("by_rank_index", "by_index_rank", "copy", "bf16", P, elems, None,
                             [a.reshape(-1) for a in x], outs)
    for j in range(P):
        assert np.array_equal(y[j].reshape(-1), want[j])


def test_combine_of_dispatch_counts_the_ranks(dispatch=moe.dispatch, combine=moe.combine):
    P, H = 4, 5
    rng = np.random.default_rng(3)
    x_rows = [6, 4, 0, 9]
    idx, counts = routing(P, x_rows, rng)
    vals = [rng.integers(-4, 5, (x_rows[i], H)).astype(np.float32) for i in range(P)]
    x = [oracle.round_bf16(v) for v in vals]
    y = dispatch(x, idx, counts, P)
    w = [np.ones(len(a), np.float32) for a in idx]
    out = combine(y, idx, w, counts, x_rows, P)
    for i in range(P):
        n = np.bincount(np.asarray(idx[i], dtype=np.int64), minlength=x_rows[i])
        assert np.array_equal(oracle.widen_bf16(out[i]), vals[i] * n[:, None])


def _combine_exact(y, idx, w, counts, x_rows, P):
    """Per element, exact rationals, each op rounded to fp32, result to bf16."""
    out = []
    for i in range(P):
        H = y[0].shape[1]
        res = np.zeros((x_rows[i], H), np.float32)
        for t in range(x_rows[i]):
            for h in range(H):
                acc = Fraction(0)
                for j in range(P):
                    start = sum(counts[i * P + q] for q in range(j))
                    pos = sum(counts[q * P + j] for q in range(i))
                    for k in range(counts[i * P + j]):
                        if int(idx[i][start + k]) != t:
                            continue
                        yv = Fraction(float(oracle.widen_bf16(y[j][pos + k:pos + k + 1, h])[0]))
                        prod = Fraction(round_binary(Fraction(float(w[i][start + k])) * yv, 24))
                        acc = Fraction(round_binary(acc + prod, 24))
                res[t, h] = round_binary(acc, 8)
        out.append(oracle.round_bf16(res))
    return out


def test_combine_against_exact_rounding(combine=moe.combine):
    P, H = 3, 4
    rng = np.random.default_rng(4)
    x_rows = [4, 6, 5]
    idx, counts = routing(P, x_rows, rng)
    ysz = [sum(counts[q * P + j] for q in range(P)) for j in range(P)]
    y = [oracle.round_bf16(rng.standard_normal((ysz[j], H)).astype(np.float32)) for j in range(P)]
    w = [rng.random(len(a)).astype(np.float32) for a in idx]
    got = combine(y, idx, w, counts, x_rows, P)
    want = _combine_exact(y, idx, w, counts, x_rows, P)
    for i in range(P):
        assert np.array_equal(got[i], want[i])


def test_combine_cancellation_shows_fp32_order(combine=moe.combine):
    """Token 0 of rank 0 comes back from ranks 0, 1, 2 as 2^24, 1, -2^24
    (weights 1): in fp32, ascending rank, 2^24 + 1 rounds to 2^24 and the
    sum is 0; an fp64 accumulator or the descending order would give 1."""
    P, H = 3, 1
    x_rows = [1, 0, 0]
    idx = [np.array([0, 0, 0], np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32)]
    counts = [1, 1, 1, 0, 0, 0, 0, 0, 0]
    vals = [np.float32(2.0 ** 24), np.float32(1.0), np.float32(-2.0 ** 24)]
    y = [oracle.round_bf16(np.array([[v]], np.float32)) for v in vals]
    w = [np.ones(3, np.float32), np.zeros(0, np.float32), np.zeros(0, np.float32)]
    out = combine(y, idx, w, counts, x_rows, P)
    assert out[0].tolist() == [[0]]
    assert np.array_equal(out[0], _combine_exact(y, idx, w, counts, x_rows, P)[0])


def test_unrouted_token_is_positive_zero_and_duplicates_are_rejected():
    P, H = 2, 2
    x_rows = [3, 1]
    idx = [np.array([0, 2], np.int32), np.array([0], np.int32)]
    counts = [1, 1, 1, 0]             # rank 0: token 0 -> rank 0, token 2 -> rank 1
    y = [np.full((2, H), 0x3F80, np.uint16), np.full((1, H), 0x4000, np.uint16)]
    w = [np.array([1, 1], np.float32), np.array([1], np.float32)]
    out = moe.combine(y, idx, w, counts, x_rows, P)
    assert out[0][1].tolist() == [0, 0]            # token 1 of rank 0: routed nowhere, +0
    assert out[0][2].tolist() == [0x4000, 0x4000]  # from rank 1's group
    dup = [np.array([1, 1], np.int32), np.array([0], np.int32)]
    with pytest.raises(oracle.OracleError):
        moe.combine(y, dup, w, [2, 0, 1, 0], x_rows, P)
    with pytest.raises(oracle.OracleError):
        moe.dispatch([np.zeros((3, H), np.uint16), np.zeros((1, H), np.uint16)],
                     [np.array([0, 3], np.int32), np.array([0], np.int32)], counts, P)


def test_moe_routing_of_the_workload():
    """The generator's routing feeds the oracle: dedup groups are ascending
    and distinct, and the weights line up with them."""
    rows = workloads.moe_rows(0, tokens=64, experts=32)
    wts = workloads.moe_weights(0, tokens=64, experts=32)
    for r, w in zip(rows, wts):
        assert np.all(np.diff(r) > 0) and len(r) == len(w)
        assert np.all((w > 0) & (w <= 1))


# ---- the pins catch plausible mistakes -------------------------------------

def _dispatch_sources_descending(x, idx, counts, P):
    y = moe.dispatch(x, idx, counts, P)
    out = []
    for j in range(P):
        sizes = [counts[i * P + j] for i in range(P)]
        parts = np.split(y[j], np.cumsum(sizes)[:-1])
        out.append(np.concatenate(parts[::-1]))
    return out


def _combine_variant(how):
    def combine(y, idx, w, counts, x_rows, P):
        out = []
        for i in range(P):
            off = moe.group_offsets(counts, P, i)
            acc = np.zeros((x_rows[i], y[0].shape[1]), np.float64 if how == "fp64" else np.float32)
            order = range(P - 1, -1, -1) if how == "descending" else range(P)
            for j in order:
                toks = np.asarray(idx[i][off[j]:off[j + 1]], dtype=np.int64)
                pos = sum(int(counts[q * P + j]) for q in range(i))
                rows = oracle.widen_bf16(y[j][pos:pos + len(toks)]).astype(acc.dtype)
                wts = np.asarray(w[i][off[j]:off[j + 1]], dtype=acc.dtype)[:, None]
                if how == "no_weights":
                    wts = np.ones_like(wts)
                acc[toks] = acc[toks] + wts * rows
            if how == "truncate":
                out.append((acc.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
            else:
                out.append(oracle.round_bf16(acc.astype(np.float32)))
        return out
    return combine


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_fail_some_pin():
    assert _fails(lambda: test_dispatch_brute_force_on_tagged_rows(_dispatch_sources_descending))
    for how in ("fp64", "descending", "no_weights", "truncate"):
        comb = _combine_variant(how)
        assert (_fails(lambda: test_combine_against_exact_rounding(comb))
                or _fails(lambda: test_combine_cancellation_shows_fp32_order(comb))
                or _fails(lambda: test_combine_of_dispatch_counts_the_ranks(combine=comb))), how
