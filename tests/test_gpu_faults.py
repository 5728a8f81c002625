"""Failure handling on the GPU, forced from the host (needs a GPU).

The test policy flag `test_withhold` makes the stager of staging ring 0 skip
one ready notify, and the watchdog is cut to 20 ms: the owner waiting for
that chunk gives up, flags the launch as aborted, every other wait of the
launch gives up too, and every wavefront exits.  The kernel ends normally;
purlin_check reports TIMEOUT, and the next collective is correct again.
"""
import numpy as np
import pytest

import pins
from gpu_util import oracle_and_gpu, run_collective

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


@pytest.mark.parametrize("withhold", [1, 3])
@pytest.mark.parametrize("name", ["reducescatter", "alltoall", "allreduce"])
def test_withheld_notify_times_out_and_recovers(purlin, name, withhold):
    P = 8
    print("case fault", name, withhold, flush=True)
    rng = np.random.default_rng([31, len(name), withhold])
    nparts = P * P if name == "alltoall" else P
    sizes = [6000] * nparts                          # 3 chunks of 4 KiB per job
    counts = pins.counts_for(name, P, sizes)
    ins, outs = pins.make_case(name, P, counts, "bf16", rng)
    in_n, out_n, op = {"reducescatter": ("by_index", "by_rank", "sum"),
                       "alltoall": ("by_rank_index", "by_index_rank", "copy"),
                       "allreduce": ("whole", "whole", "sum")}[name]
    # one lane per job, so lane 0 of ring 0 owns all three chunks
    purlin.set_policy(chunk_bytes=4096, depth=2, zero_staging="staged", wgs_per_rank=1,
                      watchdog_ns=20_000_000, test_withhold=withhold)
    with pytest.raises(purlin.PurlinError) as err:
        run_collective(purlin, in_n, out_n, op, "bf16", P, counts, None, ins, outs)
    assert err.value.status == "TIMEOUT"
    purlin.check()                                   # the status word was cleared
    # the library recovers: staged and ZS calls are correct afterwards
    purlin.set_policy(chunk_bytes=4096, depth=2, zero_staging="staged")
    oracle_and_gpu(purlin, name, P, counts, "bf16", ins, outs)
    purlin.set_policy(zero_staging="zs")
    oracle_and_gpu(purlin, name, P, counts, "bf16", ins, outs)


def test_short_watchdog_does_not_fire_on_a_healthy_run(purlin):
    P = 8
    rng = np.random.default_rng(33)
    counts = pins.counts_for("reducescatter", P, [20000] * P)
    ins, outs = pins.make_case("reducescatter", P, counts, "f32", rng)
    purlin.set_policy(chunk_bytes=4096, depth=4, zero_staging="staged", watchdog_ns=50_000_000)
    for _ in range(3):
        oracle_and_gpu(purlin, "reducescatter", P, counts, "f32", ins, outs)
    purlin.set_policy(zero_staging="zs", watchdog_ns=50_000_000, sync=True)
    for _ in range(3):
        oracle_and_gpu(purlin, "reducescatter", P, counts, "f32", ins, outs)
