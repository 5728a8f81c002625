"""Parity of the HIP path with the oracle, through the C ABI (needs a GPU).

Element by element on seeded inputs at sizes the oracle finishes in seconds
that still span several chunks and a ragged tail; copies and fp32 sums must
match bit for bit, bf16 sums within 1 bf16 ulp (the kernel folds in the
oracle's order, so the distance is expected to be 0 and is reported).
"""
import numpy as np
import pytest

import oracle
import pins
import workloads
from gpu_util import oracle_and_gpu, run_collective, compare, STORE

pytestmark = pytest.mark.gpu

NAMES = ["allreduce", "reducescatter", "allgather", "alltoall"]


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
        sizes[int(rng.integers(0, nparts))] = 0           # an empty partition
    counts = pins.counts_for(name, P, sizes)
    displs = pins.gapped_displs(name, P, counts, rng) if variant == "gapped" else None
    ins, outs = pins.make_case(name, P, counts, dtype, rng, displs, sentinel=0x5A5A)
    return counts, displs, ins, outs


@pytest.mark.parametrize("chunk", [4096, 0])
@pytest.mark.parametrize("variant", ["uniform", "v", "gapped"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("P", [1, 2, 3, 8])
def test_zs_matches_oracle(purlin, P, name, dtype, variant, chunk):
    print("case zs", P, name, dtype, variant, chunk, flush=True)
    rng = np.random.default_rng([P, NAMES.index(name), len(dtype), len(variant), chunk])
    scale = 3000 if name != "alltoall" else 700
    counts, displs, ins, outs = _case(name, P, dtype, variant, rng, scale)
    purlin.set_policy(chunk_bytes=chunk, zero_staging="zs")
    oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, displs)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", NAMES)
def test_unaligned_buffers(purlin, name, dtype):
    """Buffer bases at every element offset: sources realign in registers."""
    P = 8
    rng = np.random.default_rng([7, NAMES.index(name), len(dtype)])
    counts, displs, ins, outs = _case(name, P, dtype, "v", rng, 2500)
    esz = 4 if dtype == "f32" else 2
    shifts = [int(v) for v in rng.integers(0, 16 // esz, P)]
    # broadcast destinations must share their alignment for the one-pass
    # write; give them different ones too, which splits the broadcast
    out_shifts = [int(v) for v in rng.integers(0, 16 // esz, P)]
    purlin.set_policy(chunk_bytes=4096, zero_staging="zs")
    oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, displs, shifts, out_shifts)
    out_same = [3 % (16 // esz)] * P
    oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, displs, shifts, out_same)


@pytest.mark.parametrize("depth", [1, 2, 3, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", NAMES)
def test_staged_matches_oracle(purlin, name, dtype, depth):
    P = 8
    print("case staged", name, dtype, depth, flush=True)
    rng = np.random.default_rng([11, NAMES.index(name), len(dtype), depth])
    counts, displs, ins, outs = _case(name, P, dtype, "v", rng, 9000 if name != "alltoall" else 2000)
    purlin.set_policy(chunk_bytes=4096, depth=depth, zero_staging="staged", wgs_per_rank=2)
    oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, displs)
    info = purlin.last_launch()
    assert info["zero_staging"] == 0 and info["depth"] == depth


@pytest.mark.parametrize("P", [1, 3, 8])
@pytest.mark.parametrize("name", NAMES)
def test_staged_unaligned_and_gapped(purlin, name, P):
    rng = np.random.default_rng([13, NAMES.index(name), P])
    counts, displs, ins, outs = _case(name, P, "bf16", "gapped", rng, 3000)
    shifts = [int(v) for v in rng.integers(0, 8, P)]
    purlin.set_policy(chunk_bytes=4096, depth=2, zero_staging="staged")
    oracle_and_gpu(purlin, name, P, counts, "bf16", ins, outs, displs, shifts, [5] * P)


@pytest.mark.parametrize("sync", [True, False])
def test_repeated_calls_and_sync_modes(purlin, sync):
    """Many launches in a row (epochs advance, flags are never reset)."""
    P = 8
    purlin.set_policy(sync=sync, zero_staging="zs")
    rng = np.random.default_rng(21)
    for it in range(12):
        name = NAMES[it % 4]
        counts, displs, ins, outs = _case(name, P, "bf16", "v", rng, 500)
        oracle_and_gpu(purlin, name, P, counts, "bf16", ins, outs, displs)
    assert purlin.last_launch()["sync"] == (1 if sync else 0)


@pytest.mark.parametrize("variant", ["zs", "staged"])
@pytest.mark.parametrize("name", NAMES)
def test_handshake_on_every_shape(purlin, name, variant):
    """The full per-rank entry / exit handshake (policy sync) on every
    collective shape, uniform and variable, in both variants, three calls in
    a row (each launch waits for the previous one's exit counts)."""
    print("case handshake", name, variant, flush=True)
    P = 8
    rng = np.random.default_rng([23, NAMES.index(name), len(variant)])
    purlin.set_policy(sync=True, zero_staging=variant)
    for rep, kind in enumerate(("uniform", "v", "gapped")):
        counts, displs, ins, outs = _case(name, P, "bf16", kind, rng, 700)
        oracle_and_gpu(purlin, name, P, counts, "bf16", ins, outs, displs)
        info = purlin.last_launch()
        assert info["sync"] == 1 and info["zero_staging"] == (1 if variant == "zs" else 0), info


def test_zero_counts_launch_nothing(purlin):
    P = 8
    ins = [np.zeros(4, np.uint16) for _ in range(P)]
    outs = [np.full(4, 0x1234, np.uint16) for _ in range(P)]
    got = run_collective(purlin, "by_index", "by_rank", "sum", "bf16", P, [0] * P, None, ins, outs)
    for j in range(P):
        assert np.all(got[j] == 0x1234)


def test_special_values_sum(purlin):
    """inf, -inf, NaN, subnormals and overflow follow the oracle's rules."""
    P = 8
    f = np.float32
    vals = np.array([np.inf, -np.inf, np.nan, 2.0 ** -149, 3e38, -0.0, 1.0, 2.0 ** -130],
                    dtype=f)
    ins = [np.roll(vals, r).astype(f).view(np.uint32) for r in range(P)]
    ins[3] = np.array([1.0, 2.0, 3e38, -0.0, 3e38, -0.0, 2.0 ** -149, 5.0], f).view(np.uint32)
    outs = [np.zeros(8, np.uint32) for _ in range(P)]
    oracle_and_gpu(purlin, "allreduce", P, [8], "f32", ins, outs)
    ins16 = [oracle.round_bf16(x.view(np.float32)) for x in ins]
    outs16 = [np.zeros(8, np.uint16) for _ in range(P)]
    oracle_and_gpu(purlin, "allreduce", P, [8], "bf16", ins16, outs16)


def test_other_derivable_specs(purlin):
    """Namings outside the seven collectives run when the rule derives a plan."""
    P = 4
    rng = np.random.default_rng(5)
    # by_index -> by_index sum: AllReduce of P named partitions
    counts = [1000, 0, 37, 2048]
    ins = [oracle.round_bf16(rng.standard_normal(sum(counts)).astype(np.float32)) for _ in range(P)]
    outs = [np.zeros(sum(counts), np.uint16) for _ in range(P)]
    want = oracle.collective("by_index", "by_index", "sum", "bf16", P, counts, None, ins, outs)
    got = run_collective(purlin, "by_index", "by_index", "sum", "bf16", P, counts, None, ins, outs)
    for j in range(P):
        compare("by_index sum %d" % j, got[j], want[j], "bf16", "sum")
    # by_rank -> by_rank copy: every rank copies its own buffer
    counts = [5, 6000, 0, 77]
    ins = [rng.integers(0, 65535, counts[r]).astype(np.uint16) for r in range(P)]
    outs = [np.zeros(counts[r], np.uint16) for r in range(P)]
    want = oracle.collective("by_rank", "by_rank", "copy", "bf16", P, counts, None, ins, outs)
    got = run_collective(purlin, "by_rank", "by_rank", "copy", "bf16", P, counts, None, ins, outs)
    for j in range(P):
        compare("by_rank copy %d" % j, got[j], want[j], "bf16", "copy")


@pytest.mark.parametrize("chunk", [4096, 65536, 1 << 20])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", NAMES)
def test_large_unaligned_tiles(purlin, name, dtype, chunk):
    """Partitions of ~100k elements at odd offsets: realigned rows, many passes per tile."""
    P = 8
    print("case large-unaligned", name, dtype, chunk, flush=True)
    rng = np.random.default_rng([17, NAMES.index(name), len(dtype), chunk])
    nparts = P * P if name == "alltoall" else P
    hi = 60000 if name == "alltoall" else 150000
    sizes = [int(v) | 1 for v in rng.integers(hi // 3, hi, nparts)]   # odd sizes
    counts = pins.counts_for(name, P, sizes)
    ins, outs = pins.make_case(name, P, counts, dtype, rng, None, sentinel=0x3C3C)
    esz = 4 if dtype == "f32" else 2
    shifts = [int(v) for v in rng.integers(0, 16 // esz, P)]
    out_shift = [int(rng.integers(0, 16 // esz))] * P
    for unroll in ("0", "1", "2"):
        import os
        os.environ["PURLIN_UNROLL"] = unroll
        try:
            purlin.set_policy(chunk_bytes=chunk, zero_staging="zs")
            oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, None, shifts, out_shift)
        finally:
            os.environ.pop("PURLIN_UNROLL", None)
    purlin.set_policy(chunk_bytes=chunk, zero_staging="staged", depth=2)
    oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, None, shifts, out_shift)


@pytest.mark.parametrize("body", ["shifted_stores", "rows"])
@pytest.mark.parametrize("chunk", [4096, 65536, 0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reduce_one_destination_shifted_sources(purlin, dtype, chunk, body, monkeypatch):
    """ReduceScatter whose sources all share one shift off the destination's
    16-byte phase (as with variable-length partitions), in both tile forms:
    source-aligned units with misaligned stores (the default for sums) and
    the realigning row body that follows the sources' lines (folded before
    the shift); tiles whose unit counts sit on and around the passes."""
    P = 8
    print("case reduce-shifted", dtype, chunk, body, flush=True)
    monkeypatch.setenv("PURLIN_SHIFT_STORES", "1" if body == "shifted_stores" else "0")
    esz = 4 if dtype == "f32" else 2
    per = 16 // esz
    rng = np.random.default_rng([23, esz, chunk])
    units = [1, 7, 8, 9, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025, 3000]
    sizes = [u * per + int(rng.integers(0, per)) for u in units[:P]]
    sizes2 = [u * per + int(rng.integers(0, per)) for u in units[P:]] + [5, 40000]
    for sz in (sizes, sizes2):
        counts = pins.counts_for("reducescatter", P, sz)
        ins, outs = pins.make_case("reducescatter", P, counts, dtype, rng, None, sentinel=0x3C3C)
        for shift in range(1, per):
            purlin.set_policy(chunk_bytes=chunk, zero_staging="zs")
            oracle_and_gpu(purlin, "reducescatter", P, counts, dtype, ins, outs, None,
                           [shift] * P, [0] * P)


@pytest.mark.parametrize("unroll", ["0", "1", "2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", NAMES)
def test_rows_at_pass_boundaries(purlin, name, dtype, unroll):
    """Misaligned partitions whose unit counts sit on and around the row
    body's passes (512 units for sums, 1024 / 2048 / 4096 for copies at
    unroll 0 / 1 / 2), at every source phase; one chunk per job so a tile
    is a whole partition."""
    import os
    P = 8
    print("case rows-pass", name, dtype, unroll, flush=True)
    esz = 4 if dtype == "f32" else 2
    per = 16 // esz
    rng = np.random.default_rng([29, NAMES.index(name), esz, int(unroll)])
    kpass = 512 if name in ("allreduce", "reducescatter") else 1024 << int(unroll)
    units = [kpass - 1, kpass, kpass + 1, 2 * kpass - 1, 2 * kpass + 1, 63, 64, 65]
    nparts = P * P if name == "alltoall" else P
    sizes = [units[k % len(units)] * per + int(rng.integers(0, per)) for k in range(nparts)]
    counts = pins.counts_for(name, P, sizes)
    ins, outs = pins.make_case(name, P, counts, dtype, rng, None, sentinel=0x7E7E)
    os.environ["PURLIN_UNROLL"] = unroll
    try:
        purlin.set_policy(chunk_bytes=1 << 20, zero_staging="zs")
        for shift in (1, per // 2, per - 1):
            in_shifts = [(shift + r) % per for r in range(P)] if name == "allreduce" else [shift] * P
            oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, None, in_shifts, [0] * P)
    finally:
        os.environ.pop("PURLIN_UNROLL", None)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", ["reducescatter", "alltoall"])
def test_wide_element_pass_at_its_size_limit(purlin, name, dtype, monkeypatch):
    """Small misaligned single-destination tiles in the latency regime (4 KiB
    chunks, under 512 KiB of jobs) take one wide element pass instead of a
    row body when they hold at most 4224 bytes: partitions on both sides of
    that limit and of one-element-per-thread, at every source phase."""
    P = 8
    print("case wide-pass", name, dtype, flush=True)
    esz = 4 if dtype == "f32" else 2
    per = 16 // esz
    rng = np.random.default_rng([31, esz, len(name)])
    lim = 4224 // esz
    elems = [lim - 1, lim, lim + 1, 4096 // esz, 4096 // esz + 1, 512 // esz, 512 // esz + 1,
             lim - per]
    nparts = P * P if name == "alltoall" else P
    sizes = [elems[k % len(elems)] for k in range(nparts)]
    counts = pins.counts_for(name, P, sizes)
    ins, outs = pins.make_case(name, P, counts, dtype, rng, None, sentinel=0x6B6B)
    purlin.set_policy(zero_staging="zs")
    # sums whose sources share one phase take source-aligned units by
    # default; the wide pass is their form without that
    for shifted in (("1", "0") if name == "reducescatter" else ("0",)):
        monkeypatch.setenv("PURLIN_SHIFT_STORES", shifted)
        for shift in range(1, per):
            oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, None, [shift] * P, [0] * P)
            info = purlin.last_launch()
            assert info["chunk_bytes"] == 4096, info


@pytest.mark.parametrize("name", ["alltoall", "allgather", "reducescatter"])
def test_staged_small_misaligned_chunks_repeated(purlin, name):
    """Staged chunks of 4 KiB at shifted offsets, several launches in a row:
    a stager's head and tail element passes run on wavefronts 2 and 3, and
    its ready notify must not overtake their stores (every wavefront drains
    before the release), or the owner reads a stale line."""
    P = 8
    print("case staged-small-repeated", name, flush=True)
    rng = np.random.default_rng([37, len(name)])
    nparts = P * P if name == "alltoall" else P
    hi = 30000 if name == "alltoall" else 90000
    sizes = [int(v) | 1 for v in rng.integers(hi // 3, hi, nparts)]
    counts = pins.counts_for(name, P, sizes)
    ins, outs = pins.make_case(name, P, counts, "bf16", rng, None, sentinel=0x2D2D)
    purlin.set_policy(chunk_bytes=4096, zero_staging="staged", depth=2)
    for rep in range(4):
        shifts = [(rep + 3 * r) % 8 for r in range(P)]
        oracle_and_gpu(purlin, name, P, counts, "bf16", ins, outs, None, shifts, [rep % 8] * P)


@pytest.mark.parametrize("name,dstores", [("allgather", None), ("allgather", "0"),
                                          ("alltoall", None)])
def test_store_builds_at_the_broadcast_switch(purlin, name, dstores, monkeypatch):
    """Copy broadcasts of 16 MiB of jobs or more on the row body store at
    device scope (the build with plain stores when that is switched off),
    single-destination copies nontemporally: element-by-element parity just
    above the switch (AllGatherV-like odd sizes), and the build the launch
    reports."""
    if dstores is not None:
        monkeypatch.setenv("PURLIN_DEVICE_STORES", dstores)
    P = 8
    print("case store-build", name, flush=True)
    rng = np.random.default_rng([41, len(name)])
    nparts = P * P if name == "alltoall" else P
    # about 16.5 MiB of bf16 jobs per launch, odd partition sizes
    per = (33 << 20) // 4 // nparts
    sizes = [per + 2 * k + 1 for k in range(nparts)]
    counts = pins.counts_for(name, P, sizes)
    ins, outs = pins.make_case(name, P, counts, "bf16", rng, None, sentinel=0x4E4E)
    purlin.set_policy(zero_staging="zs")
    oracle_and_gpu(purlin, name, P, counts, "bf16", ins, outs, None, [3] * P, [0] * P)
    info = purlin.last_launch()
    if name == "allgather":
        assert sum(sizes) * 2 >= 16 << 20 and info["rows"] == 1, info
        if dstores == "0":
            assert info["plain_stores"] == 1 and info["device_stores"] == 0, info
        else:
            assert info["plain_stores"] == 0 and info["device_stores"] == 1, info
    else:
        assert info["plain_stores"] == 0 and info["device_stores"] == 0, info


def test_overlap_checks_survive_the_pointer_cache(purlin):
    """The per-call overlap check is skipped only for the same plan and buffers."""
    import torch
    P = 8
    ins = [torch.zeros(64, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    outs = [torch.zeros(64 * P, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    purlin.all_gather([x[:8] for x in ins], [y[:64] for y in outs], [8] * P)
    purlin.check()
    # same buffers, another plan whose output partitions overlap
    displs = [0] * P + [0, 8, 16, 24, 32, 40, 48, 50]
    with pytest.raises(purlin.PurlinError) as e:
        purlin.collective([x[:8] for x in ins], [y[:64] for y in outs], "by_rank", "by_index",
                          "copy", [8] * P, displs)
    assert e.value.status == "INVALID_ARG"
    # same plan as the valid call, but an input inside an output
    with pytest.raises(purlin.PurlinError) as e:
        purlin.all_gather([outs[r][60:68] for r in range(P)], [y[:64] for y in outs], [8] * P)
    assert e.value.status == "INVALID_ARG"
    purlin.all_gather([x[:8] for x in ins], [y[:64] for y in outs], [8] * P)
    purlin.check()


@pytest.mark.parametrize("name", ["allgather", "alltoall", "reducescatter"])
def test_tile_forms_at_the_mid_size_broadcast_window(purlin, name):
    """Odd partition sizes around 40 MiB of jobs: copy broadcasts take
    destination-aligned units with misaligned loads (from 32 MiB of jobs),
    point-to-point copies the row body, reductions source-aligned units
    shifted across carried rows (from 32 MiB of jobs); element-by-element
    parity and the form each launch reports."""
    P = 8
    print("case tile-forms", name, flush=True)
    rng = np.random.default_rng([43, len(name)])
    nparts = P * P if name == "alltoall" else P
    per = (40 << 20) // 2 // nparts
    sizes = [per + 2 * k + 1 for k in range(nparts)]
    counts = pins.counts_for(name, P, sizes)
    ins, outs = pins.make_case(name, P, counts, "bf16", rng, None, sentinel=0x5E5E)
    purlin.set_policy(zero_staging="zs")
    oracle_and_gpu(purlin, name, P, counts, "bf16", ins, outs, None, [3] * P, [0] * P)
    info = purlin.last_launch()
    assert info["rows"] == 1, info
    assert info["unaligned_loads"] == (1 if name == "allgather" else 0), info
    assert info["shift_stores"] == (2 if name == "reducescatter" else 0), info


@pytest.mark.parametrize("chunk", [16384, 65536])
@pytest.mark.parametrize("name,dtype", [("reducescatter", "bf16"), ("reducescatter", "f32"),
                                        ("allreduce", "bf16")])
def test_carried_rows_span_several_rows_per_wavefront(purlin, name, dtype, chunk, monkeypatch):
    """Sums whose sources share a 16-byte phase off their destinations'
    (every input shifted by 3 elements, outputs aligned) on the carried-row
    body, with chunks of 16 and 64 KiB, so that each wavefront carries 4-16
    rows within a tile and workgroups take several tiles; variable
    partitions; the oracle element by element (AllReduce: eight
    destinations per unit)."""
    monkeypatch.setenv("PURLIN_SHIFT_STORES", "2")
    P = 8
    print("case carried-rows", name, dtype, chunk, flush=True)
    rng = np.random.default_rng([53, len(name), chunk, len(dtype)])
    counts, displs, ins, outs = _case(name, P, dtype, "v", rng, 90000)
    purlin.set_policy(chunk_bytes=chunk, zero_staging="zs")
    oracle_and_gpu(purlin, name, P, counts, dtype, ins, outs, displs, [3] * P, [0] * P)
    assert purlin.last_launch()["shift_stores"] == 2


# every datapath switch the header lists, away from its default
SWITCHES = [{"PURLIN_SHIFT_STORES": "0"}, {"PURLIN_SHIFT_STORES": "1"}, {"PURLIN_SHIFT_STORES": "2"},
            {"PURLIN_UNALIGNED_LOADS": "1"}, {"PURLIN_UNALIGNED_LOADS": "0"},
            {"PURLIN_BCAST_PLAIN": "0"}, {"PURLIN_NT": "0"}, {"PURLIN_NT_ANY_PHASE": "0"},
            {"PURLIN_UNROLL": "1"}, {"PURLIN_UNROLL": "2"}, {"PURLIN_LDS": "1"},
            {"PURLIN_MID_CHUNKS": "0"}, {"PURLIN_OWNER_TEAM": "1"}, {"PURLIN_OWNER_TEAM": "3"},
            {"PURLIN_DEVICE_STORES": "1"}, {"PURLIN_DEVICE_STORES": "0"}]


@pytest.mark.parametrize("switch", SWITCHES, ids=lambda d: ",".join("%s=%s" % kv for kv in d.items()))
def test_datapath_switches_match_oracle(purlin, switch, monkeypatch):
    """Each datapath switch only chooses between forms that give the same
    result: every collective shape, uniform and variable, misaligned, in
    zero staging (and staged for the owner-team switch), at sizes that span
    several tiles, matches the oracle with the switch set."""
    for k, v in switch.items():
        monkeypatch.setenv(k, v)
    P = 8
    staged = "PURLIN_OWNER_TEAM" in switch
    rng = np.random.default_rng([97, len(str(switch))])
    for name in NAMES:
        for kind in ("uniform", "v"):
            print("case switch", switch, name, kind, flush=True)
            counts, displs, ins, outs = _case(name, P, "bf16", kind, rng,
                                              30000 if name != "alltoall" else 6000)
            shifts = [int(v) for v in rng.integers(0, 8, P)] if kind == "v" else None
            purlin.set_policy(zero_staging="staged" if staged else "zs",
                              chunk_bytes=16384 if staged else 0)
            oracle_and_gpu(purlin, name, P, counts, "bf16", ins, outs, displs, shifts)
