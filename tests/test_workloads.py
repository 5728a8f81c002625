"""Seeded input generators: reproducibility pins and count invariants (CPU only)."""
import numpy as np
import pytest

import workloads as w


def test_zipf_permutation_pin():
    assert w.zipf_perm(8) == [2, 5, 0, 4, 3, 1, 7, 6]


def test_zipf_counts_pin_1mib():
    c = w.zipf_counts((1 << 20) // 2, 8)
    assert c == [67189, 61613, 77080, 63033, 64816, 70683, 59437, 60437]
    # byte sizes are not multiples of 16: the partitions really are unaligned
    assert [x * 2 % 16 for x in c] == [10, 10, 0, 2, 0, 6, 10, 10]


@pytest.mark.parametrize("log2_bytes", range(20, 31))
def test_zipf_counts_sum_to_total(log2_bytes):
    total = (1 << log2_bytes) // 2
    c = w.zipf_counts(total, 8)
    assert sum(c) == total and min(c) > 0
    share = np.array(c) / total
    # exponent 1/8 over 8 ranks: shares between 8^-1/8 / H and 1 / H
    H = sum((k + 1) ** -0.125 for k in range(8))
    assert abs(share.max() - 1 / H) < 1e-6 and abs(share.min() - 8 ** -0.125 / H) < 1e-6


def test_moe_counts_pin_rank0():
    rows = w.moe_rows(0)
    assert [len(r) for r in rows] == [2661, 2744, 2705, 2717, 2709, 2748, 2631, 2749]
    for r in rows:
        assert np.all(np.diff(r) > 0)          # ascending token order, no repeats


def test_moe_counts_total_per_expert_variant():
    rows = w.moe_rows(3, dedup=False)
    assert sum(len(r) for r in rows) == 4096 * 8   # one row per (token, expert)


def test_host_values_reproducible_and_blocked():
    a = w.host_values(w.BLOCK + 5, "normal", "f32", 2, 3)
    b = w.host_values(w.BLOCK + 5, "normal", "f32", 2, 3)
    assert np.array_equal(a, b)
    # the second block is generated from its own seed, independently
    tail = w.block_rng(0, 2, 3, 1).standard_normal(5, dtype=np.float32)
    assert np.array_equal(a[w.BLOCK:], tail)
    u = w.host_values(4096, "uniform", "f32", 0, 0)
    assert u.min() >= -1.0 and u.max() < 1.0


def test_host_values_bf16_is_bit_patterns():
    x = w.host_values(1000, "normal", "bf16", 1, 0)
    assert x.dtype == np.uint16
    f = w.host_values(1000, "normal", "f32", 1, 0)
    # bf16 samples are within half a bf16 ulp of the float32 samples
    wide = (x.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(wide - f) <= np.abs(f) * 2.0 ** -8 + 1e-38)
