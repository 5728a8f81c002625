"""Ulysses AllToAll on the GPU against the oracle (needs a GPU).

Both directions, bit for bit (a byte copy), on random bit patterns:
P in {1, 2, 3, 4, 8}; head sizes whose rows move in 16-, 8-, 4- and 2-byte
units; ragged and empty shards; buffers shifted off their allocation's
alignment; pairs of many tiles with a ragged last tile; the fused query /
key / value layout [tokens, 3, heads, head]; the Qwen-Image 1024x1024
attention shape (4096 image + 256 text tokens, 24 heads of 128 bf16) and
one 64 MiB per rank exchange in the launch configuration the benchmark
times, both against the oracle at full size.
"""
import numpy as np
import pytest

import workloads
from gpu_util import to_device, to_host
from oracle import ulysses

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def purlin():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from reduce_atom_02_amd import purlin as p
    return p


def run(purlin, P, seq, H, D, rng, shift=0, n_pack=1, direction="both"):
    """Exchange random uint16 data [seq[i] * n_pack, H, D] both ways and
    compare each way with the oracle."""
    import torch
    rows = [s * n_pack for s in seq]
    S = sum(rows)
    g = H // P
    a = [rng.integers(0, 1 << 16, (rows[i], H, D)).astype(np.uint16) for i in range(P)]
    want_b = ulysses.to_heads(a, P, rows, H, D)
    bases, views = [], []
    for i in range(P):
        base, view = to_device(a[i].reshape(-1), "bf16", shift=shift, pad=8)
        bases.append(base)
        views.append(view)
    outs = [to_device(np.full(S * g * D, 0x5A5A, np.uint16), "bf16", shift=shift, pad=8)
            for _ in range(P)]
    head = [v for _, v in outs]
    purlin.ulysses(views, head, H, seq=rows, head_bytes=2 * D)
    purlin.check()
    for j in range(P):
        assert np.array_equal(to_host(head[j], "bf16"), want_b[j].reshape(-1)), ("to_heads", j)
    if direction == "to_heads":
        return
    back = [to_device(np.full(rows[i] * H * D, 0x7E7E, np.uint16), "bf16", shift=shift, pad=8)[1]
            for i in range(P)]
    purlin.ulysses(head, back, H, seq=rows, head_bytes=2 * D, to_sequence=True)
    purlin.check()
    want_a = ulysses.to_sequence(want_b, P, rows, H, D)
    for i in range(P):
        got = to_host(back[i], "bf16")
        assert np.array_equal(got, want_a[i].reshape(-1)), ("to_sequence", i)
        assert np.array_equal(got, a[i].reshape(-1)), ("round trip", i)
    torch.cuda.synchronize()


# head sizes (bf16 elements) whose rows move in 16-, 8-, 4- and 2-byte units
@pytest.mark.parametrize("D", [128, 8, 4, 6, 2, 13])
@pytest.mark.parametrize("P", [1, 2, 3, 8])
def test_ulysses_matches_oracle(purlin, P, D):
    print("case ulysses", P, D, flush=True)
    rng = np.random.default_rng([43, P, D])
    seq = [int(v) for v in rng.integers(0, 50, P)]
    seq[0] = max(1, seq[0])
    run(purlin, P, seq, 3 * P, D, rng)
    assert purlin.last_launch()["unit"] == {128: 16, 8: 16, 4: 8, 6: 4, 2: 4, 13: 2}[D]


@pytest.mark.parametrize("shift", [1, 4])
def test_ulysses_shifted_buffers(purlin, shift):
    """Buffers 2 or 8 bytes past 16-byte alignment: narrower units, same result."""
    rng = np.random.default_rng([47, shift])
    run(purlin, 4, [33, 0, 61, 7], 8, 128, rng, shift=shift)
    assert purlin.last_launch()["unit"] == (2 if shift == 1 else 8)


def test_ulysses_with_handshake(purlin):
    """Both directions with the full entry / exit handshake."""
    rng = np.random.default_rng(49)
    purlin.set_policy(sync=True)
    try:
        run(purlin, 8, [40, 0, 33, 51, 7, 29, 45, 12], 24, 128, rng)
        assert purlin.last_launch()["sync"] == 1
    finally:
        purlin.set_policy(reset=True)


def test_ulysses_many_tiles_ragged(purlin):
    """Pairs of about 230 KB: several 32 KiB tiles each, ragged last tiles,
    ranks of different lengths and one empty rank."""
    print("case ulysses many tiles", flush=True)
    rng = np.random.default_rng(53)
    run(purlin, 8, [300, 289, 0, 313, 301, 77, 299, 302], 24, 128, rng)
    assert purlin.last_launch()["tiles"] > 64


def test_ulysses_all_empty(purlin):
    rng = np.random.default_rng(59)
    run(purlin, 4, [0, 0, 0, 0], 8, 64, rng)


def test_ulysses_fused_qkv(purlin):
    """[tokens, 3, heads, head] exchanges as 3 * tokens rows of one call."""
    rng = np.random.default_rng(61)
    run(purlin, 8, [40, 41, 39, 40, 44, 36, 40, 40], 16, 64, rng, n_pack=3)


def test_ulysses_qwen_image_1024(purlin):
    """The 1024x1024 attention shape: (4096 + 256) tokens over 8 ranks, 24
    heads of 128 bf16, query / key / value fused; checked in full."""
    print("case ulysses qwen-image 1024", flush=True)
    cfg = workloads.ULYSSES_QWEN_IMAGE_1024
    rng = np.random.default_rng(67)
    run(purlin, cfg["P"], cfg["seq"], cfg["heads"], cfg["head_dim"], rng, n_pack=cfg["n_pack"])


def test_ulysses_64mib_per_rank(purlin):
    """The measured size: 64 MiB per rank each way, the benchmark's launch
    configuration (default policy), checked in full against the oracle."""
    print("case ulysses 64 MiB per rank", flush=True)
    cfg = workloads.ULYSSES_64MIB
    rng = np.random.default_rng(71)
    run(purlin, cfg["P"], cfg["seq"], cfg["heads"], cfg["head_dim"], rng, direction="to_heads")
