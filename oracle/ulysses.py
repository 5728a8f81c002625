"""Ulysses AllToAll over strided sequence / head layouts.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Purlin names Ulysses sequence parallelism, whose AllToAll moves data from a
sequence-sharded to a head-sharded layout and back, among the call sites of its
collectives (Table 2 of "Purlin: Separating Orchestration from the Datapath
of Collectives"; the diffusion workload).  The send side is strided: rank
i's shard of head group j is every (H/P)-th slice of its rows.

Data (elements held as uint16 / uint32 bit patterns, moved as bits):
  sequence layout:  a[i]  [seq[i], H, D]        rank i's tokens, all heads
  head layout:      b[j]  [sum(seq), H/P, D]    every token, head group j
                          (tokens of rank 0 first, then rank 1, ...)
to_heads:     b[j][off_i + s, :, :] = a[i][s, j*H/P:(j+1)*H/P, :]
to_sequence:  the inverse, a[i][s, j*H/P:(j+1)*H/P, :] = b[j][off_i + s, :, :]
with off_i = seq[0] + ... + seq[i-1].  H must be a multiple of P.
"""
import numpy as np

from .semantics import OracleError


def _check(P, seq, heads):
    if P < 1 or len(seq) != P or heads % P or any(s < 0 for s in seq):
        raise OracleError("need P shard lengths and heads divisible by P")


def to_heads(a, P, seq, heads, dim):
    """Sequence-sharded [seq[i], H, D] -> head-sharded [sum(seq), H/P, D]."""
    _check(P, seq, heads)
    g = heads // P
    b = []
    for j in range(P):
        parts = [np.asarray(a[i]).reshape(seq[i], heads, dim)[:, j * g:(j + 1) * g, :]
                 for i in range(P)]
        b.append(np.ascontiguousarray(np.concatenate(parts, axis=0)))
    return b


def to_sequence(b, P, seq, heads, dim):
    """Head-sharded [sum(seq), H/P, D] -> sequence-sharded [seq[i], H, D]."""
    _check(P, seq, heads)
    g = heads // P
    off = np.concatenate([[0], np.cumsum(seq)]).astype(np.int64)
    a = []
    for i in range(P):
        parts = [np.asarray(b[j]).reshape(-1, g, dim)[off[i]:off[i + 1]] for j in range(P)]
        a.append(np.ascontiguousarray(np.concatenate(parts, axis=1)))
    return a
