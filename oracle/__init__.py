"""Plain CPU oracle of Purlin's collectives.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) imports, links or calls this package; only the tests, the
smoke check and the benchmark's CPU-baseline leg do.  It shares no code with
the GPU path: it is numpy and plain Python, written from the definitions in
"Purlin: Separating Orchestration from the Datapath of Collectives"
(arXiv 2609.36954): the abstract (a collective is given by two layout
namings, inputs and outputs, and an operation, copy or reduction), Figure 4 (ReduceScatter,
AllGather and AllToAll layouts), Figure 6 (AllReduce composed of both) and
Table 2 / Figure 16 (variable-length variants), and ``moe.py``: MoE dispatch
and combine with the token permutation folded in (Table 2's expert-parallel
call sites), and ``ulysses.py``: the sequence-parallel AllToAll between
sequence-sharded and head-sharded layouts (Table 2's Ulysses call site).

Every function is pinned by the oracle tests; the readings it takes where the
pages are silent are documented in ``semantics.py``.
"""
from .bf16 import widen_bf16, round_bf16
from .semantics import (NAMINGS, OPS, DTYPES, ELEM_BYTES, COLLECTIVES,
                         name_count, partitions, collective, OracleError)
from .brute import collective_brute
from . import moe, ulysses

__all__ = [
    "widen_bf16", "round_bf16", "NAMINGS", "OPS", "DTYPES", "ELEM_BYTES",
    "COLLECTIVES", "name_count", "partitions", "collective", "OracleError",
    "collective_brute", "moe", "ulysses",
]
