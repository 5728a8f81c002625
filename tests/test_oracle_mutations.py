"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Every mutation below is a plausible slip (a dropped term, a wrong order, a
transposed name, an offset off by one, a truncating rounding, a wider
accumulator); it is planted into the oracle module with monkeypatch and the
pins must notice.  This checks the pins, not the GPU path.
"""
import numpy as np
import pytest

import oracle.semantics as oc
import pins

_orig_partitions = oc.partitions
_orig_reduce = oc._reduce
_orig_round = oc.round_bf16


def _reversed_order(dtype, terms):
    return _orig_reduce(dtype, terms[::-1])


def _dropped_last(dtype, terms):
    return _orig_reduce(dtype, terms[:-1] if len(terms) > 1 else terms)


def _f64_accumulate(dtype, terms):
    acc = oc._widen(dtype, terms[0]).astype(np.float64)
    for t in terms[1:]:
        acc = acc + oc._widen(dtype, t)
    acc = acc.astype(np.float32)
    return oc.round_bf16(acc) if dtype == "bf16" else acc.view(np.uint32)


def _transposed_names(naming, rank, P, counts, displs_side=None):
    if naming == "by_index_rank":
        naming = "by_rank_index"
    return _orig_partitions(naming, rank, P, counts, displs_side)


def _packed_off_by_one(naming, rank, P, counts, displs_side=None):
    parts = _orig_partitions(naming, rank, P, counts, displs_side)
    if displs_side is None:
        parts = [(nm, off + (1 if k else 0), n) for k, (nm, off, n) in enumerate(parts)]
    return parts


def _truncate(values):
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


def _tie_away(values):
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint64 if False else np.uint32)
    return ((u.astype(np.uint64) + 0x8000) >> 16).astype(np.uint16)


def _widen_shift15(dtype, bits):
    if dtype == "bf16":
        return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32)
    return np.ascontiguousarray(bits).view(np.float32)


MUTATIONS = {
    "reduce_reversed_order": ("_reduce", _reversed_order),
    "reduce_dropped_term": ("_reduce", _dropped_last),
    "reduce_f64_accumulator": ("_reduce", _f64_accumulate),
    "names_transposed": ("partitions", _transposed_names),
    "packed_offset_off_by_one": ("partitions", _packed_off_by_one),
    "bf16_truncation": ("round_bf16", _truncate),
    "bf16_ties_away": ("round_bf16", _tie_away),
    "widen_wrong_shift": ("_widen", _widen_shift15),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(monkeypatch, name):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oc, attr, fn)
    failed = []
    for pin in pins.ALL_PINS:
        if pin is pins.pin_rne_values:
            continue        # calls oracle.round_bf16 directly, not through the module
        try:
            pin()
        except (AssertionError, ValueError, IndexError) as e:
            failed.append(pin.__name__)
    assert failed, "mutation %s went unnoticed by every pin" % name
