"""Pins of the Ulysses AllToAll oracle (oracle/ulysses.py), each checked
against something other than the oracle's own code:

* brute force on tagged elements: every element of the head layout decodes
  to the (rank, token, head, channel) that the definition puts there, found
  by walking the global token order element by element;
* one token per rank reduces it to the AllToAll of the collective oracle
  (pinned on its own): rank i's slice for head group j is its index-j piece;
* the head layout of all ranks is the global [S, H, D] tensor viewed as
  [S, P, H/P, D] with the rank axis moved first (numpy transpose);
* to_sequence undoes to_heads, on random bits, ragged shard lengths and
  empty shards;
* three planted mistakes (head groups shifted, ranks reversed, channel and
  head axes swapped) each fail some pin.
"""
import numpy as np
import pytest

import oracle
from oracle import ulysses


def _rand(rng, P, seq, H, D):
    return [rng.integers(0, 1 << 16, (seq[i], H, D)).astype(np.uint16) for i in range(P)]


def test_brute_force_on_tagged_elements(to_heads=ulysses.to_heads):
    P, H, D = 3, 6, 2
    seq = [2, 0, 3]
    # element (s, h, d) of rank i holds the tag ((i * 8 + s) * 8 + h) * 4 + d
    a = [np.array([[[((i * 8 + s) * 8 + h) * 4 + d for d in range(D)] for h in range(H)]
                   for s in range(seq[i])], dtype=np.uint16).reshape(seq[i], H, D)
         for i in range(P)]
    b = to_heads(a, P, seq, H, D)
    g = H // P
    for j in range(P):
        want = []
        for i in range(P):                       # tokens in global order: rank, then token
            for s in range(seq[i]):
                for hh in range(g):
                    for d in range(D):
                        want.append(((i * 8 + s) * 8 + (j * g + hh)) * 4 + d)
        assert b[j].shape == (sum(seq), g, D)
        assert b[j].reshape(-1).tolist() == want


@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_one_token_per_rank_is_alltoall(P, to_heads=ulysses.to_heads):
    H, D = 2 * P, 3
    rng = np.random.default_rng([7, P])
    a = _rand(rng, P, [1] * P, H, D)
    g = H // P
    elems = [g * D] * (P * P)
    outs = [np.zeros(P * g * D, np.uint16) for _ in range(P)]
    want = oracle.collective("by_rank_index", "by_index_rank", "copy", "bf16", P, elems, None,
                             [x.reshape(-1) for x in a], outs)
    got = to_heads(a, P, [1] * P, H, D)
    for j in range(P):
        assert np.array_equal(got[j].reshape(-1), want[j])


def test_head_layout_is_a_transpose_of_the_global_tensor(to_heads=ulysses.to_heads):
    P, H, D = 4, 8, 5
    seq = [3, 1, 4, 2]
    rng = np.random.default_rng(11)
    a = _rand(rng, P, seq, H, D)
    S = sum(seq)
    glob = np.concatenate(a, axis=0).reshape(S, P, H // P, D).transpose(1, 0, 2, 3)
    got = to_heads(a, P, seq, H, D)
    for j in range(P):
        assert np.array_equal(got[j], glob[j])


@pytest.mark.parametrize("seq", [[5, 0, 3, 1, 7, 0, 2, 4], [0] * 8, [9] * 8])
def test_to_sequence_undoes_to_heads(seq, to_sequence=ulysses.to_sequence):
    P, H, D = 8, 16, 3
    rng = np.random.default_rng([13, sum(seq)])
    a = _rand(rng, P, seq, H, D)
    b = ulysses.to_heads(a, P, seq, H, D)
    back = to_sequence(b, P, seq, H, D)
    for i in range(P):
        assert np.array_equal(back[i], a[i])


def test_arguments_are_checked():
    with pytest.raises(oracle.OracleError):
        ulysses.to_heads([np.zeros((1, 3, 1), np.uint16)] * 2, 2, [1, 1], 3, 1)   # H % P
    with pytest.raises(oracle.OracleError):
        ulysses.to_heads([np.zeros((1, 2, 1), np.uint16)] * 2, 2, [1], 2, 1)      # seq per rank


# ---- the pins catch plausible mistakes -------------------------------------

def _heads_shifted(a, P, seq, H, D):
    b = ulysses.to_heads(a, P, seq, H, D)
    return b[1:] + b[:1]


def _ranks_reversed(a, P, seq, H, D):
    return ulysses.to_heads(a[::-1], P, seq[::-1], H, D)


def _axes_swapped(a, P, seq, H, D):
    g = H // P
    b = ulysses.to_heads(a, P, seq, H, D)
    return [np.ascontiguousarray(x.transpose(0, 2, 1)).reshape(-1, g, D) for x in b]


def _fails(fn):
    try:
        fn()
    except (AssertionError, ValueError):
        return True
    return False


@pytest.mark.parametrize("bad", [_heads_shifted, _ranks_reversed, _axes_swapped])
def test_planted_mistakes_fail_some_pin(bad):
    assert (_fails(lambda: test_brute_force_on_tagged_elements(bad))
            or _fails(lambda: test_head_layout_is_a_transpose_of_the_global_tensor(bad)))
