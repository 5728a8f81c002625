"""The staged SNAC protocol with its checks compiled in (needs a GPU).

libpurlin_debug.so is the library built with PURLIN_DEBUG_PROTOCOL: every
staged consumer checks that the flag it waited for holds exactly the value
it waited for and that the slot's header and canary are the ones its
producer wrote for that chunk, and every producer that its credits are
exactly the round's; a failed check makes purlin_check return
PURLIN_ERR_PROTOCOL.  Here staged collectives of every shape, depth 1 to 8,
several launches in a row, on two streams and under graph replay, must pass
every check and match the oracle.  (Planted protocol mistakes are caught by
the CPU model of the protocol, tests/test_snac_model.py.)
"""
import importlib.util
import os

import numpy as np
import pytest

import oracle
import pins
from gpu_util import oracle_and_gpu

pytestmark = pytest.mark.gpu

NAMES = ["allreduce", "reducescatter", "allgather", "alltoall"]


@pytest.fixture(scope="module")
def dbg():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from reduce_atom_02_amd import purlin as p
    path = os.path.join(os.path.dirname(p.LIB_PATH), "libpurlin_debug.so")
    assert os.path.exists(path), "libpurlin_debug.so is not built (python -m reduce_atom_02_amd.build --debug)"
    spec = importlib.util.spec_from_file_location("purlin_debug", p.__file__)
    mod = importlib.util.module_from_spec(spec)
    os.environ["PURLIN_LIBRARY"] = path
    try:
        spec.loader.exec_module(mod)
    finally:
        del os.environ["PURLIN_LIBRARY"]
    assert mod.LIB_PATH == path
    yield mod
    mod.set_policy(reset=True)


@pytest.mark.parametrize("depth", [1, 2, 8])
@pytest.mark.parametrize("name", NAMES)
def test_staged_protocol_checks_pass(dbg, name, depth):
    P = 8
    print("case protocol", name, depth, flush=True)
    rng = np.random.default_rng([91, NAMES.index(name), depth])
    nparts = P * P if name == "alltoall" else P
    for rep in range(3):
        sizes = [int(v) | 1 for v in rng.integers(3000, 30000 if name != "alltoall" else 6000, nparts)]
        counts = pins.counts_for(name, P, sizes)
        ins, outs = pins.make_case(name, P, counts, "bf16", rng, None, sentinel=0x3A3A)
        dbg.set_policy(zero_staging="staged", chunk_bytes=4096 * (1 + rep), depth=depth,
                       wgs_per_rank=2)
        # raises PurlinError PROTOCOL if any check failed
        oracle_and_gpu(dbg, name, P, counts, "bf16", ins, outs, None, [(rep + r) % 8 for r in range(P)],
                       [rep % 8] * P)


def test_protocol_checks_on_two_streams_and_graph_replay(dbg):
    import torch
    P = 8
    rng = np.random.default_rng(93)
    counts = pins.counts_for("reducescatter", P, [40001] * P)
    ins, outs = pins.make_case("reducescatter", P, counts, "f32", rng)
    from gpu_util import to_device, to_host
    din = [to_device(x, "f32")[1] for x in ins]
    dout = [[to_device(y, "f32")[1] for y in outs] for _ in range(2)]
    dbg.set_policy(zero_staging="staged", chunk_bytes=8192, depth=2)
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    for k in range(2):
        dbg.collective(din, dout[k], "by_index", "by_rank", "sum", counts, stream=s[k])
    for k in range(2):
        dbg.check(s[k])
    want = oracle.collective("by_index", "by_rank", "sum", "f32", P, counts, None, ins, outs)
    for k in range(2):
        for j in range(P):
            assert np.array_equal(to_host(dout[k][j], "f32"), want[j])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s[0]):
        dbg.collective(din, dout[0], "by_index", "by_rank", "sum", counts)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        dbg.check(s[0])
    for j in range(P):
        assert np.array_equal(to_host(dout[0][j], "f32"), want[j])
    del g
