"""Seeded random collectives on the GPU against the oracle (needs a GPU).

Each case draws a naming pair (one of the four collective shapes, or any
pair with as many names on both sides), the operation and element type, P
from 1 to 8, counts with empty and ragged partitions, packed or gapped
displacements, buffers at random element offsets, zero staging or staged
(random chunk and ring depth), the handshake on or off, and at times one
datapath switch away from its default.  A case the library refuses as
UNSUPPORTED (a plan it does not derive) or the oracle rejects is counted and
skipped; every other one must match the oracle: copies and fp32 sums bit
for bit, bf16 sums exactly (the fold follows the oracle's order).
"""
import os

import numpy as np
import pytest

import oracle
import pins
from gpu_util import compare, run_collective, STORE

pytestmark = pytest.mark.gpu

# PURLIN_FUZZ_SEED: another seed set for a longer search (0 = the committed
# cases; any other value shifts both tests' seeds)
SEED = int(os.environ.get("PURLIN_FUZZ_SEED", "0"))

NAMINGS = ["whole", "by_rank", "by_index", "by_rank_index", "by_index_rank"]
SWITCHES = [("PURLIN_SHIFT_STORES", "0"), ("PURLIN_SHIFT_STORES", "2"), ("PURLIN_UNALIGNED_LOADS", "1"),
            ("PURLIN_BCAST_PLAIN", "0"), ("PURLIN_NT_ANY_PHASE", "0"), ("PURLIN_UNROLL", "1"),
            ("PURLIN_MID_CHUNKS", "0"), ("PURLIN_NT", "0"), ("PURLIN_DEVICE_STORES", "1")]


@pytest.fixture(scope="module")
def purlin():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from reduce_atom_02_amd import purlin as p
    return p


def _gapped(in_n, out_n, P, counts, rng):
    """Displacements with random gaps between partitions (names in a random
    order); a naming whose names every rank holds (whole, by_index) gets one
    offset per name, shared by all ranks."""
    n = len(counts)
    side = []
    for naming in (in_n, out_n):
        d = [0] * n
        if naming in ("whole", "by_index"):
            cursor = 0
            for num in rng.permutation(n):
                d[int(num)] = cursor
                cursor += counts[int(num)] + int(rng.integers(0, 5))
        else:
            for r in range(P):
                parts = oracle.partitions(naming, r, P, counts, None)
                cursor = int(rng.integers(0, 5))
                for q in rng.permutation(len(parts)):
                    nm, _, c = parts[int(q)]
                    num = nm[0] if len(nm) == 1 else nm[0] * P + nm[1]
                    d[num] = cursor
                    cursor += c + int(rng.integers(0, 5))
        side.append(d)
    return side[0] + side[1]


def _draw(rng, scales=(40, 700, 3000, 20000)):
    if rng.random() < 0.6:
        in_n, out_n, op = oracle.COLLECTIVES[list(oracle.COLLECTIVES)[int(rng.integers(0, 4))]]
    else:
        in_n, out_n = NAMINGS[int(rng.integers(0, 5))], NAMINGS[int(rng.integers(0, 5))]
        op = "sum" if rng.random() < 0.5 else "copy"
    P = int(rng.integers(1, 9))
    nn = oracle.name_count(in_n, P)
    if oracle.name_count(out_n, P) != nn:
        return None
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    scale = int(rng.choice(list(scales)))
    counts = [int(v) for v in rng.integers(0, scale + 1, nn)]
    for _ in range(int(rng.integers(0, 3))):
        counts[int(rng.integers(0, nn))] = 0
    displs = _gapped(in_n, out_n, P, counts, rng) if rng.random() < 0.35 else None
    return in_n, out_n, op, dtype, P, counts, displs


def test_random_collectives_match_oracle(purlin, monkeypatch):
    rng = np.random.default_rng(20261204 + SEED)
    ran = skipped = 0
    for case in range(260):
        spec = _draw(rng)
        if spec is None:
            skipped += 1
            continue
        in_n, out_n, op, dtype, P, counts, displs = spec
        n = len(counts)
        in_d, out_d = (displs[:n], displs[n:]) if displs is not None else (None, None)
        in_len = [max([o + c for _, o, c in oracle.partitions(in_n, r, P, counts, in_d)] + [0])
                  for r in range(P)]
        out_len = [max([o + c for _, o, c in oracle.partitions(out_n, r, P, counts, out_d)] + [0])
                   for r in range(P)]
        ins = [pins._rand_bits(rng, in_len[r], dtype) for r in range(P)]
        outs = [np.full(out_len[r], 0x3C5A, dtype=STORE[dtype]) for r in range(P)]
        try:
            want = oracle.collective(in_n, out_n, op, dtype, P, counts, displs, ins, outs)
        except oracle.OracleError:
            skipped += 1
            continue
        staged = rng.random() < 0.3
        policy = dict(zero_staging="staged" if staged else "zs",
                      sync=bool(rng.random() < 0.3))
        if staged:
            policy.update(chunk_bytes=int(rng.choice([4096, 8192, 16384])),
                          depth=int(rng.integers(1, 5)))
        switch = SWITCHES[int(rng.integers(0, len(SWITCHES)))] if rng.random() < 0.4 else None
        shifts = [int(v) for v in rng.integers(0, 8, P)]
        out_shifts = [int(v) for v in rng.integers(0, 8, P)]
        print("case fuzz", case, in_n, out_n, op, dtype, P, sum(counts), displs is not None,
              policy, switch, flush=True)
        purlin.set_policy(**policy)
        if switch:
            monkeypatch.setenv(*switch)
        try:
            got = run_collective(purlin, in_n, out_n, op, dtype, P, counts, displs, ins, outs,
                                 shifts, out_shifts)
        except purlin.PurlinError as e:
            assert e.status == "UNSUPPORTED", (case, e.status)
            skipped += 1
            continue
        finally:
            if switch:
                monkeypatch.delenv(switch[0])
            purlin.set_policy(reset=True)
        for j in range(P):
            inexact = compare("fuzz case %d rank %d" % (case, j), got[j], want[j], dtype, op)
            assert inexact == 0, (case, j)
        ran += 1
    print("fuzz: %d cases ran, %d skipped" % (ran, skipped), flush=True)
    assert ran >= 120


def test_random_large_collectives_match_oracle(purlin, monkeypatch):
    """Fewer, larger cases (partitions up to 300 000 elements), with explicit
    chunks of 16 and 64 KiB among the policies, so that wavefronts take
    several rows of a tile and workgroups several tiles in every tile form
    (carried rows, misaligned loads and stores, device-scope stores)."""
    rng = np.random.default_rng(20261205 + SEED)
    ran = skipped = 0
    for case in range(48):
        spec = _draw(rng, scales=(60000, 150000, 300000))
        if spec is None:
            skipped += 1
            continue
        in_n, out_n, op, dtype, P, counts, displs = spec
        n = len(counts)
        in_d, out_d = (displs[:n], displs[n:]) if displs is not None else (None, None)
        in_len = [max([o + c for _, o, c in oracle.partitions(in_n, r, P, counts, in_d)] + [0])
                  for r in range(P)]
        out_len = [max([o + c for _, o, c in oracle.partitions(out_n, r, P, counts, out_d)] + [0])
                   for r in range(P)]
        ins = [pins._rand_bits(rng, in_len[r], dtype) for r in range(P)]
        outs = [np.full(out_len[r], 0x3C5A, dtype=STORE[dtype]) for r in range(P)]
        try:
            want = oracle.collective(in_n, out_n, op, dtype, P, counts, displs, ins, outs)
        except oracle.OracleError:
            skipped += 1
            continue
        policy = dict(zero_staging="staged" if rng.random() < 0.2 else "zs",
                      chunk_bytes=int(rng.choice([0, 16384, 65536])))
        switch = SWITCHES[int(rng.integers(0, len(SWITCHES)))] if rng.random() < 0.5 else None
        shifts = [int(v) for v in rng.integers(0, 8, P)]
        out_shifts = [int(v) for v in rng.integers(0, 8, P)]
        print("case fuzz-large", case, in_n, out_n, op, dtype, P, sum(counts), displs is not None,
              policy, switch, flush=True)
        purlin.set_policy(**policy)
        if switch:
            monkeypatch.setenv(*switch)
        try:
            got = run_collective(purlin, in_n, out_n, op, dtype, P, counts, displs, ins, outs,
                                 shifts, out_shifts)
        except purlin.PurlinError as e:
            assert e.status == "UNSUPPORTED", (case, e.status)
            skipped += 1
            continue
        finally:
            if switch:
                monkeypatch.delenv(switch[0])
            purlin.set_policy(reset=True)
        for j in range(P):
            inexact = compare("fuzz-large case %d rank %d" % (case, j), got[j], want[j], dtype, op)
            assert inexact == 0, (case, j)
        ran += 1
    print("fuzz-large: %d cases ran, %d skipped" % (ran, skipped), flush=True)
    assert ran >= 20

