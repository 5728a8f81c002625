"""MoE dispatch / combine on the GPU against the oracle (needs a GPU).

Random routings with P in {1, 3, 8}, rows of aligned and unaligned sizes,
empty groups and ranks; the deduplicated top-8-of-256 routing of the MoE
configuration at its full size (4096 tokens x 7168 per rank); device-side
argument errors; repeated calls (the combine's inverse table carries the
launch epoch and is never cleared).  Dispatch is a byte copy (bit-exact);
combine folds in the oracle's order and precision and must match it bit for
bit (the tolerance of the sums, 1 bf16 step, is not needed).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import compare
from oracle import moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def purlin():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from reduce_atom_02_amd import purlin as p
    return p


def dev_rows(a, shift_elems=0):
    """uint16 rows -> a device bf16 view [rows, H] starting shift_elems into its allocation."""
    import torch
    flat = torch.zeros(a.size + shift_elems + 8, dtype=torch.int16, device="cuda")
    view = flat[shift_elems:shift_elems + a.size]
    view.copy_(torch.from_numpy(a.reshape(-1).view(np.int16)).cuda())
    return view.view(torch.bfloat16).view(a.shape)


def host_rows(t):
    return t.contiguous().view(-1).view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16) \
        .reshape(t.shape)


def routing(P, x_rows, rng, fanout):
    idx, counts = [], []
    for i in range(P):
        dest = [rng.choice(P, size=int(rng.integers(0, min(P, fanout) + 1)), replace=False)
                for _ in range(x_rows[i])]
        groups = [[t for t in range(x_rows[i]) if j in dest[t]] for j in range(P)]
        idx.append(np.array([t for g in groups for t in g], dtype=np.int32))
        counts.extend(len(g) for g in groups)
    return idx, counts


def run_case(purlin, P, H, x_rows, rng, fanout=3, shift=0):
    import torch
    idx, counts = routing(P, x_rows, rng, fanout)
    x = [rng.integers(0, 1 << 16, (x_rows[i], H)).astype(np.uint16) for i in range(P)]
    # finite values for the combine (NaN payloads stay a copy-only matter)
    xv = [oracle.round_bf16(rng.standard_normal((x_rows[i], H)).astype(np.float32)) for i in range(P)]
    y_rows = [sum(counts[i * P + j] for i in range(P)) for j in range(P)]
    w = [rng.random(len(a)).astype(np.float32) for a in idx]
    d_idx = [torch.from_numpy(a).cuda() for a in idx]
    d_w = [torch.from_numpy(a).cuda() for a in w]
    # dispatch of random bits, bit for bit
    dx = [dev_rows(x[i], shift) for i in range(P)]
    dy = [dev_rows(np.zeros((y_rows[j], H), np.uint16), shift) for j in range(P)]
    want = moe.dispatch(x, idx, counts, P)
    for unique in (False, True):
        for t in dy:
            t.view(torch.int16).fill_(0x5A5A)
        purlin.moe_dispatch(dx, dy, d_idx, counts, x_rows, H * 2, unique=unique)
        purlin.check()
        for j in range(P):
            assert np.array_equal(host_rows(dy[j]), want[j]), ("dispatch", unique, j)
    if (H * 2) % 16 or shift:
        return
    # combine of the dispatched finite rows
    dxv = [dev_rows(xv[i]) for i in range(P)]
    purlin.moe_dispatch(dxv, dy, d_idx, counts, x_rows, H * 2, unique=True)
    out = [dev_rows(np.full((x_rows[i], H), 0x7E7E, np.uint16)) for i in range(P)]
    purlin.moe_combine(dy, out, d_idx, d_w, counts, x_rows, H * 2)
    purlin.check()
    yv = moe.dispatch(xv, idx, counts, P)
    want_c = moe.combine(yv, idx, w, counts, x_rows, P)
    for i in range(P):
        inexact = compare("combine rank %d" % i, host_rows(out[i]).reshape(-1),
                          want_c[i].reshape(-1), "bf16", "sum")
        assert inexact == 0, "combine rank %d: %d elements off by one step" % (i, inexact)


@pytest.mark.parametrize("H", [8, 13, 448, 7168])
@pytest.mark.parametrize("P", [1, 3, 8])
def test_moe_matches_oracle(purlin, P, H):
    print("case moe", P, H, flush=True)
    rng = np.random.default_rng([31, P, H])
    x_rows = [int(v) for v in rng.integers(0, 40, P)]
    x_rows[0] = max(1, x_rows[0])
    run_case(purlin, P, H, x_rows, rng)


@pytest.mark.parametrize("shift", [1, 3])
def test_moe_dispatch_unaligned_rows(purlin, shift):
    rng = np.random.default_rng([37, shift])
    run_case(purlin, 8, 7168, [30, 17, 0, 25, 9, 33, 12, 28], rng, fanout=4, shift=shift)


def test_moe_repeated_calls_new_routing(purlin):
    """The inverse table is never cleared: a second routing must not see the first."""
    for seed in range(3):
        rng = np.random.default_rng([41, seed])
        run_case(purlin, 8, 448, [int(v) for v in rng.integers(1, 60, 8)], rng, fanout=2 + seed)


def test_moe_with_handshake(purlin):
    """Dispatch (both forms) and combine with the full entry / exit handshake."""
    purlin.set_policy(sync=True)
    try:
        for seed in range(2):
            rng = np.random.default_rng([45, seed])
            run_case(purlin, 8, 448, [int(v) for v in rng.integers(1, 50, 8)], rng, fanout=3)
        assert purlin.last_launch()["sync"] == 1
    finally:
        purlin.set_policy(reset=True)


def test_moe_device_side_errors(purlin):
    import torch
    P, H = 2, 8
    x_rows = [4, 4]
    counts = [1, 1, 1, 1]
    dx = [dev_rows(np.zeros((4, H), np.uint16)) for _ in range(P)]
    dy = [dev_rows(np.zeros((2, H), np.uint16)) for _ in range(P)]
    bad = [torch.tensor([0, 4], dtype=torch.int32, device="cuda"),
           torch.tensor([1, 2], dtype=torch.int32, device="cuda")]
    purlin.moe_dispatch(dx, dy, bad, counts, x_rows, H * 2)
    with pytest.raises(purlin.PurlinError) as e:
        purlin.check()
    assert e.value.status == "INVALID_ARG"
    purlin.check()                                   # the status word was cleared
    dup = [torch.tensor([1, 1], dtype=torch.int32, device="cuda"),
           torch.tensor([0, 3], dtype=torch.int32, device="cuda")]
    # a repeat is fine for the row-by-row dispatch, reported for the unique one
    purlin.moe_dispatch(dx, [dev_rows(np.zeros((3, H), np.uint16)), dev_rows(np.zeros((1, H), np.uint16))],
                        dup, [2, 0, 1, 1], x_rows, H * 2, unique=False)
    purlin.check()
    purlin.moe_dispatch(dx, [dev_rows(np.zeros((3, H), np.uint16)), dev_rows(np.zeros((1, H), np.uint16))],
                        dup, [2, 0, 1, 1], x_rows, H * 2, unique=True)
    with pytest.raises(purlin.PurlinError) as e:
        purlin.check()
    assert e.value.status == "INVALID_ARG"
    purlin.check()
    w = [torch.ones(2, device="cuda"), torch.ones(2, device="cuda")]
    out = [dev_rows(np.zeros((4, H), np.uint16)) for _ in range(P)]
    purlin.moe_combine(dy, out, dup, w, [2, 0, 1, 1], x_rows, H * 2)
    with pytest.raises(purlin.PurlinError) as e:
        purlin.check()
    assert e.value.status == "INVALID_ARG"
    purlin.check()


def test_moe_full_configuration(purlin):
    """4096 tokens x 7168 bf16 per rank, top-8 of 256 experts, deduplicated
    routing: dispatch compared on the device row by row with torch indexing;
    combine on 64 sampled tokens per rank against the oracle."""
    import torch
    P, H, tokens = 8, 7168, 4096
    dev = torch.device("cuda", 0)
    rows = [workloads.moe_rows(i) for i in range(P)]
    wts = [workloads.moe_weights(i) for i in range(P)]
    counts = [len(rows[i][j]) for i in range(P) for j in range(P)]
    idx = [torch.from_numpy(np.concatenate(rows[i]).astype(np.int32)).to(dev) for i in range(P)]
    w = [torch.from_numpy(np.concatenate(wts[i]).astype(np.float32)).to(dev) for i in range(P)]
    x = [workloads.device_values(tokens * H, "normal", "bf16", 5, i, dev).view(tokens, H)
         for i in range(P)]
    y_rows = [sum(counts[i * P + j] for i in range(P)) for j in range(P)]
    y = [torch.empty(y_rows[j], H, dtype=torch.bfloat16, device=dev) for j in range(P)]
    for unique in (False, True):
        for t in y:
            t.zero_()
        purlin.moe_dispatch(x, y, idx, counts, unique=unique)
        purlin.check()
        for j in range(P):
            want = torch.cat([x[i][torch.as_tensor(rows[i][j], device=dev)] for i in range(P)])
            assert torch.equal(y[j], want), (unique, j)
    out = [torch.empty(tokens, H, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    purlin.moe_combine(y, out, idx, w, counts)
    purlin.check()
    rng = np.random.default_rng(5)
    for i in range(P):
        sample = np.sort(rng.choice(tokens, 64, replace=False))
        # the oracle on the sampled tokens: their entries only, same order
        sub_idx, sub_w, sub_counts, sub_y = [], [], [], [[] for _ in range(P)]
        remap = {int(t): q for q, t in enumerate(sample)}
        for j in range(P):
            sel = np.nonzero(np.isin(rows[i][j], sample))[0]
            pos = sum(counts[q * P + j] for q in range(i))
            sub_idx.extend(remap[int(t)] for t in rows[i][j][sel])
            sub_w.extend(wts[i][j][sel])
            sub_counts.append(len(sel))
            sub_y[j] = host_rows(y[j][torch.as_tensor(pos + sel, device=dev)])
        full_counts = [0] * (P * P)
        for j in range(P):
            full_counts[j] = sub_counts[j]
        got = host_rows(out[i][torch.as_tensor(sample, device=dev)])
        want = moe.combine([np.asarray(a, np.uint16).reshape(-1, H) for a in sub_y],
                           [np.asarray(sub_idx, np.int32)] + [np.zeros(0, np.int32)] * (P - 1),
                           [np.asarray(sub_w, np.float32)] + [np.zeros(0, np.float32)] * (P - 1),
                           full_counts, [len(sample)] + [0] * (P - 1), P)[0]
        inexact = compare("combine full rank %d" % i, got.reshape(-1), want.reshape(-1), "bf16", "sum")
        assert inexact == 0, (i, inexact)
