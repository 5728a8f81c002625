"""The boundary's stream contract on the GPU: HIP graph capture and replay,
calls interleaved on two streams, the staged kernel beside another stream's
work, and the refusals (needs a GPU).

Every result is compared with the oracle, element by element (copies and
fp32 sums bit for bit, bf16 sums exactly: the kernel folds in the oracle's
order).  Graph replays run with the program's own eager work (new inputs,
output resets) and synchronizations between them, and every replay is
checked; nothing the library enqueues inside a capture is a memset.
"""
import numpy as np
import pytest

import oracle
import pins
from gpu_util import compare, to_device, to_host
from oracle import moe

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


class Case:
    """One collective on persistent device buffers whose inputs can be
    redrawn in place."""

    def __init__(self, name, P, dtype, sizes, rng, shifts=None, out_shift=0):
        self.name, self.P, self.dtype = name, P, dtype
        self.counts = pins.counts_for(name, P, sizes)
        self.ins, self.outs = pins.make_case(name, P, self.counts, dtype, rng, None, 0x5A5A)
        shifts = shifts or [0] * P
        self.keep, self.din, self.dout = [], [], []
        for r in range(P):
            b, v = to_device(self.ins[r], dtype, shifts[r])
            self.keep.append(b)
            self.din.append(v)
            b, v = to_device(self.outs[r], dtype, out_shift)
            self.keep.append(b)
            self.dout.append(v)

    def redraw(self, rng):
        """New input values (same shapes), outputs back to the sentinel:
        eager copies on the current stream."""
        import torch
        ins, outs = pins.make_case(self.name, self.P, self.counts, self.dtype, rng, None, 0x5A5A)
        self.ins, self.outs = ins, outs
        for r in range(self.P):
            _, v = to_device(ins[r], self.dtype)
            self.din[r].copy_(v)
            _, v = to_device(outs[r], self.dtype)
            self.dout[r].copy_(v)
        torch.cuda.synchronize()

    def call(self, purlin, stream=None):
        in_n, out_n, op = oracle.COLLECTIVES[self.name]
        purlin.collective(self.din, self.dout, in_n, out_n, op, self.counts, stream=stream)

    def verify(self, what):
        in_n, out_n, op = oracle.COLLECTIVES[self.name]
        want = oracle.collective(in_n, out_n, op, self.dtype, self.P, self.counts, None,
                                 self.ins, self.outs)
        for j in range(self.P):
            inexact = compare("%s %s rank %d" % (what, self.name, j), to_host(self.dout[j], self.dtype),
                              want[j], self.dtype, op)
            assert inexact == 0, "%s %s rank %d: %d elements not exact" % (what, self.name, j, inexact)


def _sizes(name, P, rng, scale):
    nparts = P * P if name == "alltoall" else P
    return [int(v) | 1 for v in rng.integers(scale // 2, scale, nparts)]


@pytest.mark.parametrize("variant", ["zs", "staged", "zs_sync"])
@pytest.mark.parametrize("name", ["allreduce", "reducescatter", "allgather", "alltoall"])
def test_graph_replay_matches_oracle(purlin, name, variant):
    """A call captured into a HIP graph and replayed four times with new
    inputs each time: every replay matches the oracle (the staged kernel's
    flags and the handshake take a fresh epoch from device memory)."""
    import torch
    P = 8
    print("case graph", name, variant, flush=True)
    rng = np.random.default_rng([51, len(name), len(variant)])
    c = Case(name, P, "bf16", _sizes(name, P, rng, 20000 if name != "alltoall" else 4000), rng,
             shifts=[r % 8 for r in range(P)])
    if variant == "staged":
        purlin.set_policy(zero_staging="staged", chunk_bytes=16384, depth=2)
    elif variant == "zs_sync":
        purlin.set_policy(zero_staging="zs", sync=True)
    else:
        purlin.set_policy(zero_staging="zs")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c.call(purlin)                       # sets up the stream's workspace
        purlin.check(s)
    c.verify("eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        c.call(purlin)
    for rep in range(4):
        c.redraw(rng)
        g.replay()
        torch.cuda.synchronize()
        purlin.check(s)
        c.verify("replay %d" % rep)
    # eager calls on the same stream after the replays see a fresh epoch too
    c.redraw(rng)
    with torch.cuda.stream(s):
        c.call(purlin)
        purlin.check(s)
    c.verify("eager after replays")
    del g


def _routing(P, x_rows, rng, fanout):
    idx, counts = [], []
    for i in range(P):
        dest = [rng.choice(P, size=int(rng.integers(0, min(P, fanout) + 1)), replace=False)
                for _ in range(x_rows[i])]
        groups = [[t for t in range(x_rows[i]) if j in dest[t]] for j in range(P)]
        idx.append(np.array([t for g in groups for t in g], dtype=np.int32))
        counts.extend(len(g) for g in groups)
    return idx, counts


def _dev_rows(a):
    import torch
    return torch.from_numpy(a.reshape(-1).view(np.int16)).cuda().view(torch.bfloat16).view(a.shape)


def _host_rows(t):
    import torch
    return t.contiguous().view(-1).view(torch.int16).cpu().numpy().view(np.uint16).reshape(t.shape)


def test_graph_replay_moe_new_routing(purlin):
    """MoE dispatch (one row per token and rank) and combine captured in one
    graph, replayed with new token rows, weights and routing each time (the
    same group sizes, other tokens in them): the inverse table's entries of
    an earlier replay carry an older epoch and are ignored."""
    import torch
    P, H = 8, 448
    rng = np.random.default_rng(53)
    x_rows = [int(v) for v in rng.integers(20, 60, P)]
    idx, counts = _routing(P, x_rows, rng, 3)
    y_rows = [sum(counts[i * P + j] for i in range(P)) for j in range(P)]
    xv = [oracle.round_bf16(rng.standard_normal((x_rows[i], H)).astype(np.float32)) for i in range(P)]
    w = [rng.random(len(a)).astype(np.float32) for a in idx]
    dx = [_dev_rows(a) for a in xv]
    dy = [torch.zeros(y_rows[j], H, dtype=torch.bfloat16, device="cuda") for j in range(P)]
    dout = [torch.zeros(x_rows[i], H, dtype=torch.bfloat16, device="cuda") for i in range(P)]
    d_idx = [torch.from_numpy(a).cuda() for a in idx]
    d_w = [torch.from_numpy(a).cuda() for a in w]

    def step():
        purlin.moe_dispatch(dx, dy, d_idx, counts, x_rows, H * 2, unique=True)
        purlin.moe_combine(dy, dout, d_idx, d_w, counts, x_rows, H * 2)

    def verify(what):
        want_y = moe.dispatch(xv, idx, counts, P)
        for j in range(P):
            assert np.array_equal(_host_rows(dy[j]), want_y[j]), (what, "dispatch", j)
        want = moe.combine(want_y, idx, w, counts, x_rows, P)
        for i in range(P):
            inexact = compare("%s combine %d" % (what, i), _host_rows(dout[i]).reshape(-1),
                              want[i].reshape(-1), "bf16", "sum")
            assert inexact == 0, (what, i, inexact)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
        purlin.check(s)
    verify("eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(4):
        # new routing with the same group sizes: relabel every rank's tokens
        for i in range(P):
            perm = rng.permutation(x_rows[i]).astype(np.int32)
            idx[i] = perm[idx[i]]
            d_idx[i].copy_(torch.from_numpy(idx[i]))
            w[i] = rng.random(len(idx[i])).astype(np.float32)
            d_w[i].copy_(torch.from_numpy(w[i]))
            xv[i] = oracle.round_bf16(rng.standard_normal((x_rows[i], H)).astype(np.float32))
            dx[i].copy_(_dev_rows(xv[i]))
        for t in dy + dout:
            t.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        purlin.check(s)
        verify("replay %d" % rep)
    del g


def test_capture_needing_new_workspace_is_refused(purlin):
    """A staged call captured on a stream that has no workspace yet cannot
    allocate during capture: it is refused (UNSUPPORTED) and enqueues
    nothing; a zero-staging call needs no workspace and captures."""
    import torch
    P = 8
    rng = np.random.default_rng(57)
    c = Case("reducescatter", P, "f32", [3000] * P, rng)
    # torch hands out streams from a pool, so the capture stream may have
    # served earlier calls: drop every stream's workspace first
    purlin.release()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    statuses = []
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        purlin.set_policy(zero_staging="staged", chunk_bytes=16384)
        try:
            c.call(purlin)
            statuses.append("OK")
        except purlin.PurlinError as e:
            statuses.append(e.status)
        purlin.set_policy(zero_staging="zs")
        c.call(purlin)
    assert statuses == ["UNSUPPORTED"]
    c.redraw(rng)
    g.replay()
    torch.cuda.synchronize()
    c.verify("zs replay on a fresh stream")
    del g


def test_two_streams_interleaved(purlin):
    """Calls enqueued alternately on two streams without synchronizing in
    between (staged and zero-staging, with and without the handshake, MoE on
    both): each stream has its own workspace, so neither waits for the
    other's flags, and every result matches the oracle."""
    import torch
    P = 8
    rng = np.random.default_rng(59)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    plan = [("reducescatter", "staged", sa), ("alltoall", "zs", sb), ("allgather", "zs_sync", sa),
            ("allreduce", "staged", sb), ("alltoall", "staged", sa), ("reducescatter", "zs_sync", sb),
            ("allreduce", "zs", sa), ("allgather", "staged", sb)]
    cases = []
    for k, (name, variant, _) in enumerate(plan):
        scale = 24000 if name != "alltoall" else 5000
        cases.append(Case(name, P, "bf16" if k % 2 else "f32", _sizes(name, P, rng, scale), rng,
                          shifts=[(k + r) % 4 for r in range(P)]))
    torch.cuda.synchronize()
    for rnd in range(2):
        for (name, variant, stream), c in zip(plan, cases):
            if variant == "staged":
                purlin.set_policy(zero_staging="staged", chunk_bytes=16384, depth=2)
            else:
                purlin.set_policy(zero_staging="zs", sync=variant == "zs_sync")
            c.call(purlin, stream=stream)
        purlin.check(sa)
        purlin.check(sb)
        for (name, variant, stream), c in zip(plan, cases):
            c.verify("round %d %s" % (rnd, variant))
        for c in cases:
            c.redraw(rng)


@pytest.mark.parametrize("variant", ["zs", "staged", "zs_sync"])
def test_host_threads_on_their_own_streams(purlin, variant):
    """Four host threads, each enqueueing six collectives on a stream of its
    own with no synchronization in between: the library serializes its host
    bookkeeping, every stream has its own workspace, every result matches the
    oracle, and each thread's purlin_last_launch describes its own calls."""
    import threading
    import torch
    P = 8
    print("case host threads", variant, flush=True)
    rng = np.random.default_rng([61, len(variant)])
    names = ["reducescatter", "alltoall", "allgather", "allreduce"]
    work_of = []
    for t in range(4):
        cases = []
        for k in range(6):
            name = names[(t + k) % 4]
            scale = 20000 if name != "alltoall" else 4000
            cases.append(Case(name, P, "bf16" if (t + k) % 2 else "f32",
                              _sizes(name, P, rng, scale), rng))
        work_of.append(cases)
    torch.cuda.synchronize()
    if variant == "staged":
        purlin.set_policy(zero_staging="staged", chunk_bytes=16384, depth=2)
    else:
        purlin.set_policy(zero_staging="zs", sync=variant == "zs_sync")
    streams = [torch.cuda.Stream() for _ in range(4)]
    seen = [[] for _ in range(4)]
    errors = []
    start = threading.Barrier(4)

    def work(t):
        try:
            start.wait()
            for c in work_of[t]:
                c.call(purlin, stream=streams[t])
                seen[t].append(purlin.last_launch()["bytes_min"])
        except Exception as e:  # reported below, with the thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for s_ in streams:
        purlin.check(s_)
    for t in range(4):
        for k, c in enumerate(work_of[t]):
            c.verify("thread %d call %d" % (t, k))
    # each thread saw its own launches: the same calls again, one thread
    for t in range(4):
        for k, c in enumerate(work_of[t]):
            c.call(purlin)
            assert purlin.last_launch()["bytes_min"] == seen[t][k], (t, k)
    purlin.check()


def test_two_streams_moe(purlin):
    """MoE dispatch and combine on two streams at once: one inverse table
    per stream."""
    import torch
    P, H = 8, 448
    rng = np.random.default_rng(61)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for s in streams:
        x_rows = [int(v) for v in rng.integers(20, 60, P)]
        idx, counts = _routing(P, x_rows, rng, 4)
        y_rows = [sum(counts[i * P + j] for i in range(P)) for j in range(P)]
        xv = [oracle.round_bf16(rng.standard_normal((x_rows[i], H)).astype(np.float32))
              for i in range(P)]
        w = [rng.random(len(a)).astype(np.float32) for a in idx]
        runs.append(dict(s=s, x_rows=x_rows, idx=idx, counts=counts, xv=xv, w=w,
                         dx=[_dev_rows(a) for a in xv],
                         dy=[torch.zeros(y_rows[j], H, dtype=torch.bfloat16, device="cuda")
                             for j in range(P)],
                         dout=[torch.zeros(x_rows[i], H, dtype=torch.bfloat16, device="cuda")
                               for i in range(P)],
                         d_idx=[torch.from_numpy(a).cuda() for a in idx],
                         d_w=[torch.from_numpy(a).cuda() for a in w]))
    torch.cuda.synchronize()
    for r in runs:
        purlin.moe_dispatch(r["dx"], r["dy"], r["d_idx"], r["counts"], r["x_rows"], H * 2,
                            unique=True, stream=r["s"])
    for r in runs:
        purlin.moe_combine(r["dy"], r["dout"], r["d_idx"], r["d_w"], r["counts"], r["x_rows"],
                           H * 2, stream=r["s"])
    for r in runs:
        purlin.check(r["s"])
    for k, r in enumerate(runs):
        want_y = moe.dispatch(r["xv"], r["idx"], r["counts"], P)
        for j in range(P):
            assert np.array_equal(_host_rows(r["dy"][j]), want_y[j]), ("dispatch", k, j)
        want = moe.combine(want_y, r["idx"], r["w"], r["counts"], r["x_rows"], P)
        for i in range(P):
            inexact = compare("combine %d %d" % (k, i), _host_rows(r["dout"][i]).reshape(-1),
                              want[i].reshape(-1), "bf16", "sum")
            assert inexact == 0


@pytest.mark.parametrize("variant", ["staged", "zs_sync"])
def test_beside_a_busy_kernel_on_another_stream(purlin, variant):
    """Another stream keeps the device busy (elementwise passes over 512 MiB)
    while a collective whose workgroups wait for each other runs: it is
    delayed, not blocked, and matches the oracle."""
    import torch
    P = 8
    print("case busy", variant, flush=True)
    rng = np.random.default_rng([63, len(variant)])
    c = Case("allreduce", P, "bf16", [1 << 20], rng)
    busy = torch.ones(1 << 27, dtype=torch.float32, device="cuda")
    sb = torch.cuda.Stream()
    sa = torch.cuda.Stream()
    if variant == "staged":
        purlin.set_policy(zero_staging="staged", depth=2)
    else:
        purlin.set_policy(zero_staging="zs", sync=True)
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(sb):
            for _ in range(8):
                busy.mul_(1.0000001)
        c.call(purlin, stream=sa)
        purlin.check(sa)
        torch.cuda.synchronize()
        c.verify("beside busy %d" % rep)
        c.redraw(rng)
    del busy


def test_job_bound_is_refused_on_the_gpu(purlin):
    """A plan that would exceed the launch plan's 64 jobs (a sum of P
    partitions broadcast to ranks whose outputs sit at different 16-byte
    phases) is refused before any launch; the outputs stay untouched."""
    import torch
    P = 8
    counts = [40] * P
    ins = [torch.zeros(320, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    base = [torch.full((336,), 3.0, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    outs = [base[r][r:r + 320] for r in range(P)]
    with pytest.raises(purlin.PurlinError) as e:
        purlin.collective(ins, outs, "by_index", "by_index", "sum", counts)
    assert e.value.status == "UNSUPPORTED"
    torch.cuda.synchronize()
    for b in base:
        assert bool((b == 3.0).all())
