"""MoE dispatch and combine with the token permutation folded in.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Purlin names expert-parallel MoE dispatch and combine among the inference
call sites of its AllToAll (Table 2 of "Purlin: Separating Orchestration
from the Datapath of Collectives").  Here the AllToAllV reads its send rows
by token index instead of from a send buffer the caller has permuted first,
and combine is the reverse AllToAllV with a weighted sum per token.

Data, per rank i (P ranks, rows of H bf16 elements held as uint16 bits):
  x[i]     [x_rows[i], H]  the rank's token rows
  idx[i]   row indices into x[i], grouped by destination rank: the counts
           rows_ij = counts[i * P + j] of group j follow group j - 1
  w[i]     float32 weights, one per entry of idx[i] (combine only)

dispatch:  y[j] = for i = 0 .. P-1: x[i][idx[i][off_ij + k]], k < rows_ij,
           where off_ij = sum of rows_ij' over j' < j.
combine:   out[i][t] = RNE_bf16 of the fp32 left fold, from +0.0, over the
           entries (j, k) of idx[i] with idx[i][off_ij + k] == t, in
           ascending j then k, of  float32(w) * float32(y[j][pos_ij + k])
           (each product rounded to fp32 before the add; no fused
           multiply-add), where pos_ij = sum of rows_i'j over i' < i.
           A token routed nowhere gets +0.  A token appearing twice in one
           group (i, j) is rejected: combine takes one row per (token,
           destination rank), the deduplicated routing.
"""
import numpy as np

from .bf16 import round_bf16, widen_bf16
from .semantics import OracleError


def group_offsets(counts, P, i):
    """Start of each destination group j in idx[i], and the total."""
    off = [0] * (P + 1)
    for j in range(P):
        c = int(counts[i * P + j])
        if c < 0:
            raise OracleError("negative row count")
        off[j + 1] = off[j] + c
    return off


def _check(x_rows, idx, counts, P):
    if len(counts) != P * P or len(idx) != P or len(x_rows) != P:
        raise OracleError("need P index arrays, P row counts and P*P group counts")
    for i in range(P):
        off = group_offsets(counts, P, i)
        if len(idx[i]) != off[P]:
            raise OracleError("idx[%d] holds %d entries, counts say %d" % (i, len(idx[i]), off[P]))
        if off[P] and (np.min(idx[i]) < 0 or np.max(idx[i]) >= x_rows[i]):
            raise OracleError("idx[%d] points outside x[%d]" % (i, i))


def dispatch(x, idx, counts, P):
    """Rows gathered by index and exchanged; returns the P arrays y[j]."""
    _check([len(a) for a in x], idx, counts, P)
    H = x[0].shape[1] if x else 0
    y = []
    for j in range(P):
        parts = []
        for i in range(P):
            off = group_offsets(counts, P, i)
            parts.append(x[i][np.asarray(idx[i][off[j]:off[j + 1]], dtype=np.int64)])
        y.append(np.concatenate(parts) if parts else np.zeros((0, H), np.uint16))
    return y


def combine(y, idx, w, counts, x_rows, P):
    """The reverse exchange with a weighted fp32 fold per token; returns out[i]."""
    _check(x_rows, idx, counts, P)
    H = y[0].shape[1] if y else 0
    out = []
    for i in range(P):
        off = group_offsets(counts, P, i)
        acc = np.zeros((x_rows[i], H), np.float32)
        for j in range(P):
            toks = np.asarray(idx[i][off[j]:off[j + 1]], dtype=np.int64)
            if len(np.unique(toks)) != len(toks):
                raise OracleError("token twice in group (%d, %d): combine needs one row per "
                                  "(token, destination rank)" % (i, j))
            pos = sum(int(counts[q * P + j]) for q in range(i))
            rows = widen_bf16(y[j][pos:pos + len(toks)])
            wts = np.asarray(w[i][off[j]:off[j + 1]], dtype=np.float32)[:, None]
            # tokens are distinct inside the group, so this is one add per token
            acc[toks] = acc[toks] + wts * rows
        out.append(round_bf16(acc))
    return out
