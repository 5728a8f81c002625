"""Copy collectives on the DMA copy engines against the oracle (needs a GPU).

With the policy's engine set to "copy", AllGather(V) and AllToAll(V) run as
stream-ordered transfers on the copy engines (no kernel): bit-exact with the
oracle for uniform, variable and gapped partitions at any element offset,
P in {1, 3, 8}, and in stream order with kernels before and after.  Sums
keep running on the shader kernels under the same policy.
"""
import numpy as np
import pytest

import oracle
import pins
from gpu_util import oracle_and_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def purlin():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from reduce_atom_02_amd import purlin as p
    return p


@pytest.fixture(autouse=True)
def _policy(purlin):
    purlin.set_policy(reset=True)
    yield
    purlin.set_policy(reset=True)


def _case(name, P, dtype, variant, rng, scale):
    nparts = P * P if name == "alltoall" else P
    if variant == "uniform":
        sizes = [scale] * nparts
    else:
        sizes = [int(v) for v in rng.integers(0, 2 * scale + 1, nparts)]
        sizes[int(rng.integers(0, nparts))] = 0
    counts = pins.counts_for(name, P, sizes)
    displs = pins.gapped_displs(name, P, counts, rng) if variant == "gapped" else None
    ins, outs = pins.make_case(name, P, counts, dtype, rng, displs, sentinel=0x6C6C)
    return counts, displs, ins, outs


@pytest.mark.parametrize("variant", ["uniform", "v", "gapped"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", ["allgather", "alltoall"])
@pytest.mark.parametrize("P", [1, 3, 8])
def test_copy_engine_matches_oracle(purlin, P, name, dtype, variant):
    print("case copy-engine", P, name, dtype, variant, flush=True)
    rng = np.random.default_rng([81, P, len(name), len(dtype), len(variant)])
    counts, displs, ins, outs = _case(name, P, dtype, variant, rng, 5000 if name != "alltoall" else 900)
    esz = 4 if dtype == "f32" else 2
    shifts = [int(v) for v in rng.integers(0, 16 // esz, P)]
    out_shifts = [int(v) for v in rng.integers(0, 16 // esz, P)]
    purlin.set_policy(engine="copy")
    oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, displs, shifts, out_shifts)
    info = purlin.last_launch()
    nonempty = sum(1 for c in counts if c) if name == "alltoall" else P * sum(1 for c in counts if c)
    if nonempty:          # (a call with nothing to move launches nothing and reports nothing)
        assert info["grid"] == 0 and info["engine_copies"] == nonempty, info


def test_sums_stay_on_the_shader_kernels(purlin):
    P = 8
    rng = np.random.default_rng(83)
    counts, displs, ins, outs = _case("reducescatter", P, "bf16", "v", rng, 4000)
    purlin.set_policy(engine="copy")
    oracle_and_gpu(purlin, "reducescatter", P, counts, "bf16", ins, outs, displs)
    info = purlin.last_launch()
    assert info["grid"] > 0 and info["engine_copies"] == 0, info


def test_copy_engine_in_stream_order_with_kernels(purlin):
    """A shader AllReduce writes the buffer the copy-engine AllGather reads,
    and a shader ReduceScatter reads what the AllGather wrote, all enqueued
    back to back on one stream: the copies see the kernel's results and the
    next kernel sees the copies'."""
    import torch
    P = 8
    n = 1 << 18
    rng = np.random.default_rng(85)
    xs = [torch.from_numpy(rng.standard_normal(P * n).astype(np.float32)).cuda() for _ in range(P)]
    ar = [torch.empty(P * n, device="cuda") for _ in range(P)]
    ag = [torch.empty(P * P * n, device="cuda") for _ in range(P)]
    rs = [torch.empty(P * n, device="cuda") for _ in range(P)]
    purlin.set_policy(engine="copy")
    for rep in range(3):
        purlin.all_reduce(xs, ar)                                     # shader kernel
        purlin.all_gather(ar, ag)                                     # copy engines
        purlin.reduce_scatter(ag, rs)                                 # shader kernel
        purlin.check()
        for r in range(P):
            xs[r].mul_(-0.5)
    torch.cuda.synchronize()
    # the last round's inputs: before the scaling by -0.5 (exact)
    host = [x.cpu().numpy() * np.float32(-2.0) for x in xs]
    acc = host[0].copy()
    for r in range(1, P):
        acc = acc + host[r]
    for r in range(P):
        assert np.array_equal(ar[r].cpu().numpy(), acc)
        assert np.array_equal(ag[r].cpu().numpy(), np.tile(acc, P))
        # reduce-scatter of P identical gathered copies, in rank order
        s = acc.copy()
        for _ in range(P - 1):
            s = s + acc
        assert np.array_equal(rs[r].cpu().numpy(), s)
