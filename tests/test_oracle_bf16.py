"""Exhaustive check of the oracle's bf16 conversions (CPU only).

Round to nearest even over all 2**32 fp32 patterns is compared with torch's
CPU float32 -> bfloat16 conversion, a library routine independent of the
GPU path.  torch returns one canonical NaN, so NaNs are only checked to stay
NaNs with the sign kept and the quiet bit set (the oracle's documented NaN
rule is pinned by hand in pins.pin_rne_values).
"""
import multiprocessing as mp
import os

import numpy as np
import pytest

CHUNK = 1 << 24


def _check_chunk(c):
    import torch
    from oracle.bf16 import round_bf16
    torch.set_num_threads(1)
    u = np.arange(c * CHUNK, (c + 1) * CHUNK, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    mine = round_bf16(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    bad = int(np.count_nonzero((mine != ref) & ~nan))
    m = mine[nan]
    bad_nan = int(np.count_nonzero(((m & 0x7FC0) != 0x7FC0) | ((m >> 15) != (u[nan] >> 31))))
    return bad, bad_nan


def test_round_bf16_exhaustive():
    n_chunks = (1 << 32) // CHUNK
    workers = min(8, os.cpu_count() or 1)
    with mp.get_context("spawn").Pool(workers) as pool:
        res = pool.map(_check_chunk, range(n_chunks))
    assert sum(r[0] for r in res) == 0
    assert sum(r[1] for r in res) == 0


def test_widen_bf16_all_patterns():
    import torch
    from oracle.bf16 import widen_bf16
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = widen_bf16(b).view(np.uint32)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy().view(np.uint32)
    nan = ((b & 0x7FFF) > 0x7F80)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.all(np.isnan(mine[nan].view(np.float32)))
