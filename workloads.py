"""Seeded synthetic inputs for the collectives (shared by tests and the benchmark).

This module only draws numbers and partition sizes; it holds none of the
collective arithmetic, and it imports neither the oracle nor the GPU
library.  Recipes (all seeded, all synthetic):

* values: per (config id c, rank r, block b) a numpy Generator seeded with
  ``SeedSequence([seed, c, r, b])``, blocks of 2**22 elements, so host memory
  stays bounded and any block can be regenerated alone;
  - ``uniform``: ``2*U - 1`` with U a float32 in [0, 1), so values lie in
    [-1, 1) and are exact in fp32;
  - ``normal``: ``standard_normal`` in float32; bf16 inputs are those float32
    samples converted by torch's CPU bf16 conversion (a library routine).
* large device-resident inputs (bandwidth sweeps) are drawn on the GPU by
  torch's seeded generator (``device_values``); tests read back the elements
  they check.
* Zipf partition sizes (Purlin, Figure 16 caption: Zipf, s = 0.125): partition k weighs ``(pi(k)+1) ** -s`` for a seeded permutation
  pi of the P ranks; counts are the floors of T * w_k / sum(w), the remainder
  going one element each to the largest fractional parts (ties: lower k).
  Sizes are in elements with no alignment.
* MoE dispatch counts (Purlin, Table 2: expert parallelism uses AllToAll(V)
  to dispatch tokens): per source rank, float32 N(0,1) router logits
  [tokens x experts]; a token's top-k experts are the k largest logits (the
  top-k of the softmax is the top-k of the logits), ties to the lower expert;
  expert e lives on rank e // (experts / P); one row per (token, destination
  rank), deduplicated, rows grouped by destination in ascending token order.
* Ulysses exchanges (Purlin, Table 2 and Figure 12(c): Qwen-Image with
  Ulysses sequence parallelism on eight GPUs): the attention of a 1024x1024
  image, 64x64 = 4096 image tokens (8x latent downsampling, 2x2 patches)
  plus 256 text tokens (a stated choice: the pages give no prompt length),
  split evenly over the ranks, 24 heads of 128 bf16 (the model's published
  attention shape, not given on the pages), query / key / value fused;
  values are uniform random bit patterns (the exchange copies bytes).  The
  bandwidth case keeps that head shape at about 64 MiB per rank.
"""
import numpy as np

__all__ = [
    "BLOCK", "block_rng", "host_values", "device_values", "zipf_perm",
    "zipf_counts", "moe_rows", "moe_counts", "uniform_counts",
]

BLOCK = 1 << 22


def block_rng(seed, cfg, rank, block):
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, rank, block]))


def host_values(n, dist, dtype, cfg, rank, seed=0):
    """n values for one rank: float32 array (dtype 'f32') or bf16 bit patterns (uint16)."""
    out = np.empty(n, dtype=np.float32)
    for b, start in enumerate(range(0, n, BLOCK)):
        m = min(BLOCK, n - start)
        rng = block_rng(seed, cfg, rank, b)
        if dist == "uniform":
            out[start:start + m] = 2.0 * rng.random(m, dtype=np.float32) - 1.0
        elif dist == "normal":
            out[start:start + m] = rng.standard_normal(m, dtype=np.float32)
        elif dist == "int":
            # small integers: every fp32 sum of a few of them is exact
            out[start:start + m] = rng.integers(-1024, 1024, m).astype(np.float32)
        else:
            raise ValueError(dist)
    if dtype == "f32":
        return out
    if dtype == "bf16":
        import torch
        return torch.from_numpy(out).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def device_values(n, dist, dtype, cfg, rank, device, seed=0):
    """n values for one rank drawn on ``device`` by torch's seeded generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + cfg * 10007 + rank * 101 + 7) & 0x7FFFFFFFFFFFFFFF)
    if dist == "uniform":
        x = torch.rand(n, generator=g, device=device, dtype=torch.float32) * 2 - 1
    elif dist == "normal":
        x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    else:
        raise ValueError(dist)
    return x if dtype == "f32" else x.to(torch.bfloat16)


def uniform_counts(total, P):
    """Equal partitions of ``total`` elements (total must divide by P)."""
    if total % P:
        raise ValueError("total %d does not split into %d equal partitions" % (total, P))
    return [total // P] * P


def zipf_perm(P, seed=0):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 4, 0x5A1F]))
    return [int(v) for v in rng.permutation(P)]


def zipf_counts(total, P, s=0.125, seed=0):
    """Zipf(s) partition of ``total`` elements over P partitions (sums to total)."""
    perm = zipf_perm(P, seed)
    w = np.array([(perm[k] + 1) ** (-s) for k in range(P)], dtype=np.float64)
    share = total * w / w.sum()
    counts = np.floor(share).astype(np.int64)
    rest = int(total - counts.sum())
    frac = share - counts
    order = sorted(range(P), key=lambda k: (-frac[k], k))
    for k in order[:rest]:
        counts[k] += 1
    return [int(c) for c in counts]


def moe_rows(rank, seed=0, tokens=4096, experts=256, topk=8, P=8, dedup=True):
    """Token ids sent from ``rank`` to each destination rank (list of P int arrays)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 5, rank, 1]))
    logits = rng.standard_normal((tokens, experts), dtype=np.float32)
    top = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    dest = top // (experts // P)
    rows = []
    for j in range(P):
        hits = (dest == j)
        if dedup:
            rows.append(np.nonzero(hits.any(axis=1))[0])
        else:
            rows.append(np.repeat(np.arange(tokens), hits.sum(axis=1)))
    return rows


def moe_weights(rank, seed=0, tokens=4096, experts=256, topk=8, P=8):
    """Combine weights aligned with ``moe_rows(rank)`` (deduplicated routing):
    for each (token, destination rank) the sum of the token's softmax gate
    values (over its top-k logits, float32) of the experts on that rank."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 5, rank, 1]))
    logits = rng.standard_normal((tokens, experts), dtype=np.float32)
    top = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    sel = np.take_along_axis(logits, top, axis=1)
    g = np.exp(sel - sel.max(axis=1, keepdims=True)).astype(np.float32)
    g = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    dest = top // (experts // P)
    out = []
    for j in range(P):
        per_tok = np.where(dest == j, g, np.float32(0)).sum(axis=1, dtype=np.float32)
        out.append(per_tok[(dest == j).any(axis=1)].astype(np.float32))
    return out


def moe_counts(P=8, hidden=7168, seed=0, **kw):
    """P x P element counts (row-major, [src * P + dst]) of the MoE dispatch."""
    counts = []
    for i in range(P):
        rows = moe_rows(i, seed=seed, P=P, **kw)
        counts.extend(int(len(r)) * hidden for r in rows)
    return counts


# Ulysses exchange shapes (see the module docstring).
ULYSSES_QWEN_IMAGE_1024 = {"P": 8, "seq": [(4096 + 256) // 8] * 8, "heads": 24, "head_dim": 128,
                           "n_pack": 3}
ULYSSES_64MIB = {"P": 8, "seq": [10922] * 8, "heads": 24, "head_dim": 128, "n_pack": 1}
