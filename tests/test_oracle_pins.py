"""The oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_invalid_specs_rejected():
    x = [np.zeros(4, np.uint32) for _ in range(2)]
    with pytest.raises(oracle.OracleError):      # copy with two sources
        oracle.collective("whole", "whole", "copy", "f32", 2, [4], None, x, x)
    with pytest.raises(oracle.OracleError):      # name sets differ
        oracle.collective("whole", "by_rank", "sum", "f32", 2, [4], None, x, x)
    with pytest.raises(oracle.OracleError):      # partition outside the buffer
        oracle.collective("by_index", "by_rank", "sum", "f32", 2, [3, 3], None, x, x)
    with pytest.raises(oracle.OracleError):      # overlapping output partitions
        oracle.collective("by_rank", "by_index", "copy", "f32", 2, [2, 2], [0, 0, 0, 1], x, x)


def test_zero_counts_write_nothing():
    P = 3
    ins = [np.arange(4, dtype=np.uint16) + 10 * i for i in range(P)]
    outs = [np.full(4, 7, np.uint16) for _ in range(P)]
    got = oracle.collective("by_index", "by_rank", "sum", "bf16", P, [0, 0, 0], None, ins, outs)
    for j in range(P):
        assert np.all(got[j] == 7)
