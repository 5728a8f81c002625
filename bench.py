"""Benchmark of the collective hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--size BYTES] [--variant zs|staged]

One step runs the seven collectives once each -- AllReduce, ReduceScatter,
AllGather, AllToAll and the Zipf(s = 0.125) variable-length ReduceScatterV,
AllGatherV, AllToAllV -- over P = 8 ranks emulated as 8 buffer sets in one
GPU's HBM, bf16, at T bytes per rank (default 1 GiB, the top of the pages'
1 MiB - 1 GiB bandwidth sweep).  T is the per-rank size of the partitioned
side (AllReduce buffer, ReduceScatter input, AllGather output, AllToAll
input; for the V variants the total of the Zipf partition).  Inputs are
N(0,1) values drawn on the device from a seed and are resident in HBM
before the timed region starts.

Printed: one JSON line with the aggregate algorithm bandwidth
(sum of T over the calls / elapsed time), the fraction of the HBM peak
(8 TB/s) that the compulsory traffic B_min (every input byte read once,
every output byte written once) reaches, per-collective kernel times from
HIP events, the roofline of the dominant kernel, and the oracle's
throughput on the host cores on a bounded sample.
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "algorithm GB/s + fraction of HBM peak; p50 latency, 1 KiB–1 GiB, P=8"
HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
P = 8
ESZ = 2                    # bf16

# name -> (in naming, out naming, op)
SPECS = {
    "allreduce": ("whole", "whole", "sum"),
    "reducescatter": ("by_index", "by_rank", "sum"),
    "allgather": ("by_rank", "by_index", "copy"),
    "alltoall": ("by_rank_index", "by_index_rank", "copy"),
    "reducescatterv": ("by_index", "by_rank", "sum"),
    "allgatherv": ("by_rank", "by_index", "copy"),
    "alltoallv": ("by_rank_index", "by_index_rank", "copy"),
}


def collective_shapes(T):
    """Per collective: counts (elements), input and output elements per rank,
    compulsory bytes B_min and the algorithm size T (bytes)."""
    import workloads
    n = T // ESZ
    z = workloads.zipf_counts(n, P)
    shapes = {}
    shapes["allreduce"] = dict(counts=[n], ins=[n] * P, outs=[n] * P)
    shapes["reducescatter"] = dict(counts=[n // P] * P, ins=[n] * P, outs=[n // P] * P)
    shapes["allgather"] = dict(counts=[n // P] * P, ins=[n // P] * P, outs=[n] * P)
    shapes["alltoall"] = dict(counts=[n // P] * (P * P), ins=[n] * P, outs=[n] * P)
    shapes["reducescatterv"] = dict(counts=z, ins=[n] * P, outs=list(z))
    shapes["allgatherv"] = dict(counts=z, ins=list(z), outs=[n] * P)
    shapes["alltoallv"] = dict(counts=[z[j] for _ in range(P) for j in range(P)], ins=[n] * P,
                               outs=[P * z[j] for j in range(P)])
    for name, s in shapes.items():
        s["bmin"] = ESZ * (sum(s["ins"]) + sum(s["outs"]))
        s["T"] = T
    return shapes


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "zs_kernels_seven_collectives_1GiB_hbm_counters.txt")


def kernel_source_hash():
    """Hash of the HIP and host sources with comments and whitespace removed:
    counters taken from other code do not apply (a comment edit changes no
    kernel)."""
    import re
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "reduce_atom_02_amd", "csrc", "*"))):
        with open(f, "r", encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(os.path.basename(f).encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, T, names, variant):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by a known-size copy), or
    None when that summary was taken on other sources or another workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            line = next(l for l in f if l.startswith("traffic_json: "))
        rec = json.loads(line[len("traffic_json: "):])
    except (OSError, StopIteration, ValueError):
        return None
    if (rec.get("source_hash") != kernel_source_hash() or rec.get("T") != T
            or rec.get("names") != list(names) or variant != "zs"):
        return None
    k = rec["kernels"].get(kernel)
    return None if k is None else int(k["traffic_per_launch"])


def kernel_of(name, rows, one, plain=False, device=False):
    """The kernel a collective's launch ran, named as in the rocprofv3
    summaries: the operation, whether it was the build with the realigning
    row bodies (some source off its destinations' 16-byte phase) or the
    aligned-only one, whether it was the build for single-destination jobs
    ("one") or the general one ("general"), and ",plain" for the build with
    plain body stores (large copy broadcasts), ",device" for the one with
    device-scope stores (broadcasts in their windows)."""
    op = "SumBf16" if SPECS[name][2] == "sum" else "CopyOp"
    store = ",device" if device else ",plain" if plain else ""
    return "zs_kernel<%s,%s,%s%s>" % (op, "rows" if rows else "aligned",
                                      "one" if one else "general", store)


def cpu_baseline(T_sample, names, reps=5):
    """The oracle, as it stands, on the host cores: seven collectives at
    T_sample bytes per rank, same seeds, the p50 of `reps` calls each;
    generation is not timed."""
    import numpy as np
    import oracle
    import workloads
    shapes = collective_shapes(T_sample)
    n = T_sample // ESZ
    ins = [workloads.host_values(n, "normal", "bf16", 3, r) for r in range(P)]
    total_T, total_t, spent = 0, 0.0, 0.0
    for name in names:
        s = shapes[name]
        in_n, out_n, op = SPECS[name]
        xs = [ins[r][:s["ins"][r]] for r in range(P)]
        ts = []
        for _ in range(reps):
            ys = [np.zeros(s["outs"][r], np.uint16) for r in range(P)]
            t0 = time.perf_counter()
            oracle.collective(in_n, out_n, op, "bf16", P, s["counts"], None, xs, ys)
            ts.append(time.perf_counter() - t0)
        ts.sort()
        total_t += ts[len(ts) // 2]
        spent += sum(ts)
        total_T += s["T"]
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": round(total_T / total_t / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "the same seven collectives, bf16, P=8, at %d MiB per rank instead of "
                      "the timed size; the p50 of %d calls each (sum of T over the sum of the "
                      "p50s); numpy oracle single-threaded; %.1f s of oracle time; host: %d "
                      "CPUs, %d in this process's affinity, %s"
                      % (T_sample >> 20, reps, spent, os.cpu_count() or 0,
                         len(os.sched_getaffinity(0)), model)}


# The collectives' bare access patterns: label, sources, destinations,
# bytes per stream as a multiple of T, the collectives the pattern bounds.
# 1->1 over P*T is AllToAll's pattern and footprint, 1->8 of T AllGather's,
# 8->1 ReduceScatter's, 8->8 AllReduce's; read-only and write-only streams
# bound every mix of the two.
PATTERNS = [
    ("1->1", 1, 1, P, ("alltoall", "alltoallv")),
    ("1->8", 1, 8, 1, ("allgather", "allgatherv")),
    ("8->1", 8, 1, 1, ("reducescatter", "reducescatterv")),
    ("8->8", 8, 8, 1, ("allreduce",)),
    ("read-only x8", 8, 0, 1, ()),
    ("write-only x8", 0, 8, 1, ()),
]
# (nontemporal loads, store mode) -> label; "device": stores written through
# the L2 (device scope), the form the broadcasts take in their windows
ACCESS = {(True, "nt"): "nt/nt", (True, "plain"): "nt/plain", (False, "nt"): "plain/nt",
          (False, "plain"): "plain/plain", (True, "device"): "nt/device",
          (False, "device"): "plain/device"}


def ceilings(purlin, T, reps, dev, full=False, path=None):
    """HBM ceiling of each collective's access pattern (purlin_stream_pattern:
    n read streams, m write streams, no planning or flags), the best over a
    sweep of nontemporal or plain loads x nontemporal, plain or device-scope
    stores x tile (4 KiB - 1 MiB) x grid x unroll (full=True: 6 x 5 x 4
    grids x 3 unrolls; else 6 x 3 x 2 x 1), p50 of `reps` cold calls per point (a 1 GiB
    fill between calls, outside the events).  Also hipMemcpyAsync device to
    device (torch's copy_) over P*T bytes, as a context figure.  Every point
    goes to `path` (JSONL) when given."""
    import torch
    big_src = torch.ones(P * T // 4, dtype=torch.float32, device=dev)
    big_dst = torch.empty(P * T // 4, dtype=torch.float32, device=dev)
    srcs = [big_src[r * (T // 4):(r + 1) * (T // 4)] for r in range(P)]
    dsts = [big_dst[r * (T // 4):(r + 1) * (T // 4)] for r in range(P)]
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def p50_of(fn):
        fn()
        ev = []
        for _ in range(reps):
            flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        return ts[len(ts) // 2]

    tiles = ((4 << 10, 16 << 10, 64 << 10, 256 << 10, 1 << 20) if full
             else (4 << 10, 16 << 10, 256 << 10))
    grids = (256, 512, 1024, 2048) if full else (512, 1024)
    out = {}
    f = open(path, "w") if path else None
    for label, nr, nw, mult, bounds in PATTERNS:
        nbytes = mult * T
        if nr <= 1 and nw <= 1:
            s_, d_ = ([big_src] if nr else []), ([big_dst] if nw else [])
        else:
            s_, d_ = srcs[:nr], dsts[:nw]
        unrolls = ((2, 4, 8) if nr < 8 else (2, 4)) if full else (4,)
        best = None
        for (ntl, smode) in ACCESS:
            if nr == 0 and not ntl or nw == 0 and smode != "nt":
                continue                       # the unused side: one setting
            for tile in tiles:
                for g in grids:
                    for u in unrolls:
                        t = p50_of(lambda: purlin.stream_pattern(
                            s_, d_, nbytes, grid=g, tile_bytes=tile, unroll=u, nt_loads=ntl,
                            nt_stores=smode == "nt", device_stores=smode == "device",
                            stream=stream))
                        frac = (nr + nw) * nbytes / t / HBM_PEAK
                        point = {"pattern": label, "access": ACCESS[(ntl, smode)], "tile": tile,
                                 "grid": g, "unroll": u, "p50_us": round(t * 1e6, 1),
                                 "hbm_frac": round(frac, 4), "bytes": (nr + nw) * nbytes}
                        if f:
                            f.write(json.dumps(point) + "\n")
                            f.flush()
                        if best is None or frac > best["hbm_frac"]:
                            best = dict(point, hbm_frac=round(frac, 4))
        out[label] = {"hbm_frac": best["hbm_frac"], "access": best["access"],
                      "tile": best["tile"], "grid": best["grid"], "unroll": best["unroll"],
                      "bounds": list(bounds)}
        print("ceiling %s done" % label, flush=True)
    t = p50_of(lambda: big_dst.copy_(big_src))
    out["hipMemcpyAsync D2D"] = {"hbm_frac": round(2 * P * T / t / HBM_PEAK, 4)}
    if f:
        f.close()
    del srcs, dsts, big_src, big_dst, flush
    torch.cuda.empty_cache()
    return out


def latency_block(purlin, dev, ins):
    """Device p50 latency of each collective at 1 KiB, 64 KiB and 512 KiB
    per rank (warm, 200 timed calls queued behind a spin kernel so that the
    events bracket GPU work only) and at 1 MiB (cold: a 1 GiB fill between
    calls, 50 calls), the fp32 AllReduce of 1 MiB per rank (values 2U - 1)
    and the TP8 AllReduce of [t x 7168] bf16 activations for t = 1, 64, 256
    (warm, queued), and the empty-kernel floor timed the same way.  Inputs
    are prefixes of the bench's resident buffers; 20 warm-up calls per
    point; P = 8, zero staging, default policy."""
    import torch
    import workloads
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    outs = [torch.empty(256 * 7168, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    empty = torch.empty(1, device=dev)

    def timed(fn, reps, cold):
        for _ in range(20):
            fn()
        ev = []
        for k in range(reps):
            if not cold and k % 200 == 0:
                torch.cuda.synchronize()
                torch.cuda._sleep(20_000_000)     # ~10 ms: covers 200 enqueues
            if cold:
                flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        return round(ts[len(ts) // 2] * 1e6, 2)

    res = {"empty_kernel_p50_us": timed(lambda: empty.add_(0), 200, False), "collectives": {}}
    for T in (1 << 10, 64 << 10, 512 << 10, 1 << 20):
        shapes = collective_shapes(T)
        row = {}
        for name, s in shapes.items():
            in_n, out_n, op = SPECS[name]
            xi = [ins[r][:s["ins"][r]] for r in range(P)]
            yo = [outs[r][:s["outs"][r]] for r in range(P)]
            row[name] = timed(lambda: purlin.collective(xi, yo, in_n, out_n, op, s["counts"],
                                                        stream=stream), 50 if T >= 1 << 20 else 200,
                              T >= 1 << 20)
        res["collectives"]["%d_KiB" % (T >> 10)] = row
    purlin.check(stream)
    n = 262144
    xf = [workloads.device_values(n, "uniform", "f32", 0, r, dev) for r in range(P)]
    yf = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(P)]
    res["allreduce_f32_1MiB_warm_p50_us"] = timed(
        lambda: purlin.collective(xf, yf, "whole", "whole", "sum", [n], stream=stream), 200, False)
    res["allreduce_f32_1MiB_cold_p50_us"] = timed(
        lambda: purlin.collective(xf, yf, "whole", "whole", "sum", [n], stream=stream), 50, True)
    for t in (1, 64, 256):
        m = t * 7168
        xi = [ins[r][:m] for r in range(P)]
        yo = [outs[r][:m] for r in range(P)]
        res["tp8_allreduce_bf16_%dx7168_p50_us" % t] = timed(
            lambda: purlin.collective(xi, yo, "whole", "whole", "sum", [m], stream=stream), 200,
            False)
    purlin.check(stream)
    del flush, outs, xf, yf
    return res


def placement_spread(purlin, T, names, steps, dev, first):
    """The step on two more sets of freshly allocated rank buffers (held at
    the same time as the first, so every set has its own physical pages):
    `steps` timed steps per set after one warm-up step.  Returns the B_min
    fraction of the whole step and of each collective per set, the first
    set's (`first`, from the timed run) included, with min / median / max."""
    import torch
    import workloads
    shapes = collective_shapes(T)
    stream = torch.cuda.current_stream()
    sets = [first]
    keep = []
    for k in range(2):
        n = T // ESZ
        ins = [workloads.device_values(n, "normal", "bf16", 3, r, dev) for r in range(P)]
        out_len = max(max(s["outs"]) for s in shapes.values())
        outs = [torch.empty(out_len, dtype=torch.bfloat16, device=dev) for _ in range(P)]
        keep.append((ins, outs))
        per = {}
        total_b, total_t = 0, 0.0
        for name in names:
            s = shapes[name]
            in_n, out_n, op = SPECS[name]
            xi = [ins[r][:s["ins"][r]] for r in range(P)]
            yo = [outs[r][:s["outs"][r]] for r in range(P)]
            purlin.collective(xi, yo, in_n, out_n, op, s["counts"], stream=stream)
            ev = []
            for _ in range(steps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                purlin.collective(xi, yo, in_n, out_n, op, s["counts"], stream=stream)
                e1.record(stream)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
            p50 = ts[len(ts) // 2]
            per[name] = round(s["bmin"] / p50 / HBM_PEAK, 4)
            total_b += s["bmin"]
            total_t += p50
        purlin.check(stream)
        sets.append({"hbm_frac": round(total_b / total_t / HBM_PEAK, 4), "collectives": per})
    del keep
    torch.cuda.empty_cache()

    def spread(vals):
        v = sorted(vals)
        return {"min": v[0], "median": v[len(v) // 2], "max": v[-1]}

    return {"sets": len(sets), "steps_per_set": steps,
            "step_hbm_frac": spread([x["hbm_frac"] for x in sets]),
            "collectives": {n_: spread([x["collectives"][n_] for x in sets]) for n_ in names},
            "per_set": sets}


def calibrate_copy(purlin, T, steps, warmup, dev):
    import torch
    src = torch.empty(T // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        purlin.stream_copy(dst, src, T, stream=stream)
    ev = []
    torch.cuda.synchronize()
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        purlin.stream_copy(dst, src, T, stream=stream)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
    p50 = ts[len(ts) // 2]
    print(json.dumps({"calibration": "stream_copy_kernel", "bytes_read": T, "bytes_written": T,
                      "launches": steps + warmup, "p50_us": round(p50 * 1e6, 2),
                      "GBps_read_plus_write": round(2 * T / p50 / 1e9, 1),
                      "hbm_frac": round(2 * T / p50 / HBM_PEAK, 4)}), flush=True)


def sweep(purlin, T_max, variant, path, dev):
    """p50 per-call latency from HIP events, T = 1 KiB .. T_max per rank.

    Every point: 20 warm-up calls first.
    Latency regime (T <= 512 KiB), warm caches, 1000 timed calls, three figures:
      p50_us       device latency: a spin kernel is queued before each batch
                   of 200 calls, so every timed launch is already enqueued
                   when the GPU reaches it and the events bracket only GPU
                   work (back to back);
      submit_p50_us  the same call timed with events from an idle GPU, so
                   host-side argument marshalling (Python, ctypes) and the
                   launch are in it;
      host_p50_us  call to completion on the host: perf_counter around the
                   call and a stream synchronize.
    Bandwidth regime (T >= 1 MiB): a 1 GiB fill runs between calls, outside
    the events, so inputs come from HBM, not the 256 MiB Infinity Cache;
    100 timed calls up to 64 MiB, 20 above.  The empty-kernel floor is
    measured the same three ways."""
    import torch
    import workloads
    purlin.set_policy(zero_staging=variant)
    stream = torch.cuda.current_stream()
    n_max = T_max // ESZ
    ins = [workloads.device_values(n_max, "normal", "bf16", 3, r, dev) for r in range(P)]
    shapes_max = collective_shapes(T_max)
    out_len = max(max(s["outs"]) for s in shapes_max.values())
    outs = [torch.empty(out_len, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    empty = torch.empty(1, device=dev)

    def timed(fn, reps, cold, queued=False):
        ev = []
        for k in range(reps):
            if queued and k % 200 == 0:
                torch.cuda.synchronize()
                torch.cuda._sleep(20_000_000)      # ~10 ms at 2.4 GHz: covers 200 enqueues
            if cold:
                flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        return ts[len(ts) // 10], ts[len(ts) // 2], ts[(9 * len(ts)) // 10]

    def host_p50(fn, reps):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            stream.synchronize()
            ts.append(time.perf_counter() - t0)
        ts.sort()
        return ts[len(ts) // 2]

    def empty_kernel():
        empty.add_(0)

    floor = timed(empty_kernel, 1000, False, queued=True)[1]
    floor_submit = timed(empty_kernel, 1000, False)[1]
    floor_host = host_p50(empty_kernel, 1000)
    rows = []
    with open(path, "w") as f:
        for lg in range(10, T_max.bit_length()):
            T = 1 << lg
            shapes = collective_shapes(T)
            cold = T >= (1 << 20)
            reps = 1000 if not cold else (100 if T <= (64 << 20) else 20)
            for name, s in shapes.items():
                in_n, out_n, op = SPECS[name]
                xi = [ins[r][:s["ins"][r]] for r in range(P)]
                yo = [outs[r][:s["outs"][r]] for r in range(P)]

                def fn():
                    purlin.collective(xi, yo, in_n, out_n, op, s["counts"], stream=stream)

                for _ in range(20):
                    fn()
                submit = host = None
                if cold:
                    p10, p50, p90 = timed(fn, reps, cold)
                else:
                    p10, p50, p90 = timed(fn, 1000, cold, queued=True)
                    submit = round(timed(fn, 1000, cold)[1] * 1e6, 2)
                    host = round(host_p50(fn, 1000) * 1e6, 2)
                purlin.check(stream)
                info = purlin.last_launch()
                row = {"collective": name, "variant": variant, "dtype": "bf16", "P": P,
                       "T_bytes": T, "cold": cold, "reps": reps,
                       "p10_us": round(p10 * 1e6, 2), "p50_us": round(p50 * 1e6, 2),
                       "p90_us": round(p90 * 1e6, 2), "algbw_GBps": round(T / p50 / 1e9, 2),
                       "hbm_frac": round(s["bmin"] / p50 / HBM_PEAK, 4), "bmin": s["bmin"],
                       "submit_p50_us": submit, "host_p50_us": host,
                       "grid": info["grid"], "chunk_bytes": info["chunk_bytes"],
                       "empty_kernel_p50_us": round(floor * 1e6, 2),
                       "empty_kernel_submit_p50_us": round(floor_submit * 1e6, 2),
                       "empty_kernel_host_p50_us": round(floor_host * 1e6, 2)}
                f.write(json.dumps(row) + "\n")
                f.flush()
                rows.append(row)
            print("T=%d KiB done" % (T >> 10), flush=True)
    return rows


def policy_sweep(purlin, sizes, names, path, dev, reps=30):
    """Grid and chunk of the zero-staging kernel swept where the launch
    dominates less and less (T = 1 MiB .. 32 MiB per rank by default): for
    each collective and T, workgroups per rank in {auto, 16, 32, 64, 128,
    256} x chunk in {auto, 4, 8, 16, 32, 64 KiB}, the p50 of `reps` cold
    calls (a 1 GiB fill between calls, outside the events); below 1 MiB per
    rank, the latency sweep's device latency instead (warm, 200 calls queued
    behind a spin kernel).  One JSONL row per point, with the grid and chunk
    the launch took."""
    import torch
    import workloads
    stream = torch.cuda.current_stream()
    Tmax = max(sizes)
    n = Tmax // ESZ
    ins = [workloads.device_values(n, "normal", "bf16", 3, r, dev) for r in range(P)]
    shapes_max = collective_shapes(Tmax)
    outs = [torch.empty(max(max(shapes_max[nm]["outs"]) for nm in names), dtype=torch.bfloat16,
                        device=dev) for _ in range(P)]
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    rows = []
    with open(path, "w") as f:
        for T in sizes:
            shapes = collective_shapes(T)
            for name in names:
                s = shapes[name]
                in_n, out_n, op = SPECS[name]
                xi = [ins[r][:s["ins"][r]] for r in range(P)]
                yo = [outs[r][:s["outs"][r]] for r in range(P)]
                for g in (0, 16, 32, 64, 128, 256):
                    for c in (0, 4 << 10, 8 << 10, 16 << 10, 32 << 10, 64 << 10):
                        purlin.set_policy(zero_staging="zs", wgs_per_rank=g, chunk_bytes=c)
                        purlin.collective(xi, yo, in_n, out_n, op, s["counts"], stream=stream)
                        info = purlin.last_launch()
                        ev = []
                        cold = T >= (1 << 20)
                        n_calls = reps if cold else 200
                        if not cold:
                            torch.cuda.synchronize()
                            torch.cuda._sleep(20_000_000)   # the calls queue up behind it
                        for _ in range(n_calls):
                            if cold:
                                flush.fill_(1.0)
                            e0 = torch.cuda.Event(enable_timing=True)
                            e1 = torch.cuda.Event(enable_timing=True)
                            e0.record(stream)
                            purlin.collective(xi, yo, in_n, out_n, op, s["counts"], stream=stream)
                            e1.record(stream)
                            ev.append((e0, e1))
                        torch.cuda.synchronize()
                        purlin.check(stream)
                        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
                        p50 = ts[len(ts) // 2]
                        row = {"collective": name, "T_bytes": T, "wgs_per_rank_policy": g,
                               "chunk_policy": c, "grid": info["grid"],
                               "chunk_bytes": info["chunk_bytes"], "p50_us": round(p50 * 1e6, 2),
                               "hbm_frac": round(s["bmin"] / p50 / HBM_PEAK, 4)}
                        f.write(json.dumps(row) + "\n")
                        f.flush()
                        rows.append(row)
            print("T=%d KiB done" % (T >> 10), flush=True)
    purlin.set_policy(reset=True)
    return rows


def config_bench(purlin, path, dev):
    """The AllReduce workloads the latency sweep does not cover, timed like
    its latency regime (20 warm-up calls, 1000 timed calls; device p50
    queued behind a spin kernel, p50 from an idle GPU, host call to
    completion): the fp32 AllReduce of 262144 elements (1 MiB) per rank,
    values 2U - 1, and the tensor-parallel AllReduce of bf16 activations
    [t x 7168] for t in 1, 4, 16, 64, 256 (N(0,1)); both also cold (a 1 GiB
    fill between calls, 100 calls).  P = 8, zero staging."""
    import torch
    import workloads
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def timed(fn, reps, cold=False, queued=False):
        ev = []
        for k in range(reps):
            if queued and k % 200 == 0:
                torch.cuda.synchronize()
                torch.cuda._sleep(20_000_000)
            if cold:
                flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        return ts[len(ts) // 10], ts[len(ts) // 2], ts[(9 * len(ts)) // 10]

    def host_p50(fn, reps):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            stream.synchronize()
            ts.append(time.perf_counter() - t0)
        ts.sort()
        return ts[len(ts) // 2]

    cases = [("allreduce_f32_1MiB", "f32", 262144, "uniform", 0)]
    cases += [("tp8_allreduce_bf16_%dx7168" % t, "bf16", t * 7168, "normal", 5) for t in
              (1, 4, 16, 64, 256)]
    rows = []
    purlin.set_policy(reset=True)
    with open(path, "w") as f:
        for label, dtype, n, dist, cfg in cases:
            esz = 4 if dtype == "f32" else 2
            tdt = torch.float32 if dtype == "f32" else torch.bfloat16
            ins = [workloads.device_values(n, dist, dtype, cfg, r, dev) for r in range(P)]
            outs = [torch.empty(n, dtype=tdt, device=dev) for _ in range(P)]

            def fn():
                purlin.collective(ins, outs, "whole", "whole", "sum", [n], stream=stream)

            for _ in range(20):
                fn()
            purlin.check(stream)
            p10, p50, p90 = timed(fn, 1000, queued=True)
            submit = timed(fn, 1000)[1]
            host = host_p50(fn, 1000)
            cold = timed(fn, 100, cold=True)[1]
            purlin.check(stream)
            info = purlin.last_launch()
            bmin = 2 * P * n * esz
            row = {"case": label, "dtype": dtype, "P": P, "bytes_per_rank": n * esz,
                   "p10_us": round(p10 * 1e6, 2), "p50_us": round(p50 * 1e6, 2),
                   "p90_us": round(p90 * 1e6, 2), "submit_p50_us": round(submit * 1e6, 2),
                   "host_p50_us": round(host * 1e6, 2), "cold_p50_us": round(cold * 1e6, 2),
                   "algbw_GBps": round(n * esz / p50 / 1e9, 2),
                   "hbm_frac_warm": round(bmin / p50 / HBM_PEAK, 4),
                   "hbm_frac_cold": round(bmin / cold / HBM_PEAK, 4), "bmin": bmin,
                   "grid": info["grid"], "chunk_bytes": info["chunk_bytes"]}
            f.write(json.dumps(row) + "\n")
            f.flush()
            rows.append(row)
            print("%s done" % label, flush=True)
            del ins, outs
    return rows


def moe_bench(purlin, steps, warmup, dev):
    """MoE dispatch and combine at the configuration of the pages' expert-
    parallel call sites: 4096 tokens x 7168 bf16 per rank, top-8 of 256
    experts on P = 8 ranks, one row per (token, destination rank).  Timed
    with HIP events, p50 over `steps` calls: the by-token dispatch (each
    token row read once), the row-by-row dispatch, the unfused path (torch
    index_select into a send buffer, then the AllToAllV) as context, and
    combine.  B_min: dispatch reads every routed token row once and writes
    every sent row; combine reads every sent row and writes every token row."""
    import numpy as np
    import torch
    import workloads
    H, tokens = 7168, 4096
    rb = H * 2
    rows = [workloads.moe_rows(i) for i in range(P)]
    wts = [workloads.moe_weights(i) for i in range(P)]
    counts = [len(rows[i][j]) for i in range(P) for j in range(P)]
    idx = [torch.from_numpy(np.concatenate(rows[i]).astype(np.int32)).to(dev) for i in range(P)]
    w = [torch.from_numpy(np.concatenate(wts[i]).astype(np.float32)).to(dev) for i in range(P)]
    x = [workloads.device_values(tokens * H, "normal", "bf16", 5, i, dev).view(tokens, H)
         for i in range(P)]
    y_rows = [sum(counts[i * P + j] for i in range(P)) for j in range(P)]
    y = [torch.empty(y_rows[j], H, dtype=torch.bfloat16, device=dev) for j in range(P)]
    out = [torch.empty(tokens, H, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    send = [torch.empty(sum(counts[i * P:(i + 1) * P]), H, dtype=torch.bfloat16, device=dev)
            for i in range(P)]
    sent = sum(counts)
    routed = sum(len(np.unique(np.concatenate(rows[i]))) for i in range(P))
    stream = torch.cuda.current_stream()
    a2a_counts = [c * H for c in counts]

    def unfused():
        for i in range(P):
            torch.index_select(x[i], 0, idx[i], out=send[i])
        purlin.all_to_all([s_.view(-1) for s_ in send], [t.view(-1) for t in y], a2a_counts,
                          stream=stream)

    cases = {
        "dispatch_by_token": (lambda: purlin.moe_dispatch(x, y, idx, counts, unique=True, stream=stream),
                              (routed + sent) * rb),
        "dispatch_by_row": (lambda: purlin.moe_dispatch(x, y, idx, counts, unique=False, stream=stream),
                            2 * sent * rb),
        "unfused_index_select_then_alltoallv": (unfused, (routed + sent) * rb),
        "combine": (lambda: purlin.moe_combine(y, out, idx, w, counts, stream=stream),
                    (sent + P * tokens) * rb),
    }
    res = {}
    for name, (fn, bmin) in cases.items():
        for _ in range(warmup):
            fn()
        purlin.check(stream)
        ev = []
        for _ in range(steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        purlin.check(stream)
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        p50 = ts[len(ts) // 2]
        res[name] = {"p50_us": round(p50 * 1e6, 1), "bmin_bytes": bmin,
                     "hbm_frac": round(bmin / p50 / HBM_PEAK, 4)}
        if name != "unfused_index_select_then_alltoallv":
            res[name]["grid"] = purlin.last_launch()["grid"]
    return {"moe": res, "config": {"P": P, "tokens_per_rank": tokens, "hidden": H,
                                   "dtype": "bf16", "experts": 256, "topk": 8,
                                   "rows_sent": sent, "token_rows_routed": routed},
            "steps": steps, "data": "synthetic"}


def ulysses_bench(purlin, steps, warmup, dev):
    """The Ulysses exchange (the pages' diffusion workload: Qwen-Image with
    Ulysses sequence parallelism) at the 1024x1024 attention shape, query /
    key / value fused into one call to the head layout and the attention
    output back to the sequence layout, and at about 64 MiB per rank each
    way.  Timed with HIP events, p50 over `steps` back-to-back calls (inputs
    stay hot in the caches between calls, as they would after the producing
    projection).  Context: the unfused path, a torch transpose into a packed
    send buffer, then the contiguous AllToAll.  B_min: every byte read once
    and written once."""
    import torch
    import workloads
    stream = torch.cuda.current_stream()
    res = {}

    def timed(fn):
        for _ in range(warmup):
            fn()
        purlin.check(stream)
        ev = []
        for _ in range(steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        purlin.check(stream)
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        return ts[len(ts) // 2]

    for label, cfg in (("qwen_image_1024", workloads.ULYSSES_QWEN_IMAGE_1024),
                       ("64MiB_per_rank", workloads.ULYSSES_64MIB)):
        H, D = cfg["heads"], cfg["head_dim"]
        g = H // P
        for direction, n_pack in (("to_heads", cfg["n_pack"]), ("to_sequence", 1)):
            rows = [s_ * n_pack for s_ in cfg["seq"]]
            S = sum(rows)
            seq_bufs = [workloads.device_values(rows[i] * H * D, "normal", "bf16", 7, i, dev)
                        for i in range(P)]
            head_bufs = [torch.empty(S * g * D, dtype=torch.bfloat16, device=dev) for _ in range(P)]
            to_seq = direction == "to_sequence"
            if to_seq:
                purlin.ulysses(seq_bufs, head_bufs, H, seq=rows, head_bytes=2 * D, stream=stream)
                ins, outs = head_bufs, seq_bufs
            else:
                ins, outs = seq_bufs, head_bufs
            nbytes = sum(rows) * H * D * 2
            t = timed(lambda: purlin.ulysses(ins, outs, H, seq=rows, head_bytes=2 * D,
                                             to_sequence=to_seq, stream=stream))
            info = purlin.last_launch()
            entry = {"p50_us": round(t * 1e6, 2), "bytes_each_way": nbytes,
                     "hbm_frac": round(2 * nbytes / t / HBM_PEAK, 4), "grid": info["grid"],
                     "chunk_bytes": info["chunk_bytes"], "unit": info["unit"],
                     "tokens_per_rank": rows[0], "heads": H, "head_dim": D}
            if not to_seq:
                # unfused: pack each rank's rows by destination, then the plain AllToAll
                send = [torch.empty(rows[i] * H * D, dtype=torch.bfloat16, device=dev)
                        for i in range(P)]
                counts = [rows[i] * g * D for i in range(P) for _ in range(P)]

                def unfused():
                    for i in range(P):
                        send[i].view(P, rows[i], g, D).copy_(
                            seq_bufs[i].view(rows[i], P, g, D).transpose(0, 1))
                    purlin.all_to_all(send, head_bufs, counts, stream=stream)
                tu = timed(unfused)
                entry["unfused_pack_then_alltoall_p50_us"] = round(tu * 1e6, 2)
                del send
            res["%s_%s" % (label, direction)] = entry
            del seq_bufs, head_bufs, ins, outs
            torch.cuda.empty_cache()
    return {"ulysses": res, "P": P, "steps": steps, "dtype": "bf16", "data": "synthetic"}


def engine_bench(purlin, T, steps, dev):
    """The copy collectives on the DMA copy engines (no kernel) against the
    shader kernels, at T bytes per rank: p50 of `steps` calls each (a 1 GiB
    fill between calls, outside the events, so inputs come from HBM), and
    what a compute-bound kernel on another stream keeps of its throughput
    beside each: a bf16 GEMM [8192 x 8192] x [8192 x 8192] (hipBLASLt through
    torch), timed alone and while the collective runs back to back on its
    own stream for longer than the GEMMs; the collective's throughput beside
    the GEMM is reported too."""
    import torch
    import workloads
    names = ["allgather", "alltoall", "allgatherv", "alltoallv"]
    shapes = collective_shapes(T)
    n = T // ESZ
    ins = [workloads.device_values(n, "normal", "bf16", 3, r, dev) for r in range(P)]
    out_len = max(max(shapes[nm]["outs"]) for nm in names)
    outs = [torch.empty(out_len, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    sx, sc = torch.cuda.Stream(), torch.cuda.Stream()

    def call(name, stream):
        s = shapes[name]
        in_n, out_n, op = SPECS[name]
        purlin.collective([ins[r][:s["ins"][r]] for r in range(P)],
                          [outs[r][:s["outs"][r]] for r in range(P)],
                          in_n, out_n, op, s["counts"], stream=stream)

    def p50(fn, stream, reps):
        fn()
        ev = []
        for _ in range(reps):
            with torch.cuda.stream(stream):
                flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        return ts[len(ts) // 2]

    res = {}
    for name in names:
        row = {}
        for engine in ("shader", "copy"):
            purlin.set_policy(engine=engine)
            t = p50(lambda: call(name, sx), sx, steps)
            info = purlin.last_launch()
            row[engine] = {"p50_us": round(t * 1e6, 1), "algbw_GBps": round(T / t / 1e9, 1),
                           "hbm_frac": round(shapes[name]["bmin"] / t / HBM_PEAK, 4),
                           "kernel_grid": info["grid"], "engine_copies": info["engine_copies"]}
        res[name] = row
        print("%s done" % name, flush=True)
    purlin.set_policy(reset=True)

    # a compute-bound kernel beside the collective
    m = 8192
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    a = torch.randn(m, m, dtype=torch.bfloat16, device=dev, generator=g)
    b = torch.randn(m, m, dtype=torch.bfloat16, device=dev, generator=g)
    c = torch.empty(m, m, dtype=torch.bfloat16, device=dev)
    n_gemm = 40
    flops = 2.0 * m * m * m * n_gemm

    def gemms():
        with torch.cuda.stream(sc):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(sc)
            for _ in range(n_gemm):
                torch.matmul(a, b, out=c)
            e1.record(sc)
        return e0, e1

    torch.cuda.synchronize()
    gemms()
    torch.cuda.synchronize()
    e0, e1 = gemms()
    torch.cuda.synchronize()
    t_alone = e0.elapsed_time(e1) * 1e-3
    beside = {"gemm_alone_TFLOPs": round(flops / t_alone / 1e12, 1), "gemm": "bf16 %dx%dx%d x%d"
              % (m, m, m, n_gemm)}
    name = "alltoall"
    for engine in ("shader", "copy"):
        purlin.set_policy(engine=engine)
        t_one = res[name][engine]["p50_us"] * 1e-6
        reps = max(4, int(1.5 * t_alone / t_one) + 1)
        torch.cuda.synchronize()
        x0 = torch.cuda.Event(enable_timing=True)
        x1 = torch.cuda.Event(enable_timing=True)
        x0.record(sx)
        for _ in range(reps):
            call(name, sx)
        x1.record(sx)
        g0, g1 = gemms()
        torch.cuda.synchronize()
        purlin.check(sx)
        t_g = g0.elapsed_time(g1) * 1e-3
        t_x = x0.elapsed_time(x1) * 1e-3 / reps
        beside[engine] = {"gemm_TFLOPs_beside": round(flops / t_g / 1e12, 1),
                          "gemm_kept_frac": round(t_alone / t_g, 3),
                          "alltoall_calls": reps,
                          "alltoall_algbw_GBps_beside_gemm": round(T / t_x / 1e9, 1)}
    purlin.set_policy(reset=True)
    return {"engines": res, "beside_gemm": beside, "T_bytes_per_rank": T, "P": P,
            "dtype": "bf16", "steps": steps, "data": "synthetic"}


def pipeline_sweep(purlin, T, names, path, dev):
    """Staged SNAC pipeline against zero staging, in the shape of the pages'
    pipelining figure (a 256 MiB one-sided transfer; pipeline depth 1-8;
    eight or sixteen workgroups): for each name in `names` at T bytes per
    rank -- a collective, or "onesided", rank 0's T bytes to rank 1 --
    every depth D in 1..8, staging chunk C in 16 KiB .. 1 MiB and
    workgroups per job (lanes: 8-256 for the one-sided transfer, 1-32 for a
    collective) and the staged default policy, the p50 over 10 cold calls (a 1 GiB fill between calls,
    outside the events), and the zero-staging kernel at its default policy
    and at several grid sizes.  B_min
    fraction as everywhere: compulsory bytes / (p50 x 8 TB/s); staging's
    extra passes show up as lost fraction."""
    import torch
    import workloads
    stream = torch.cuda.current_stream()
    shapes = collective_shapes(T)
    n = T // ESZ
    ins = [workloads.device_values(n, "normal", "bf16", 3, r, dev) for r in range(P)]
    out_len = max(max(shapes[nm]["outs"]) if nm in shapes else n for nm in names)
    outs = [torch.empty(out_len, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def p50(fn, reps=10):
        fn()
        ev = []
        for _ in range(reps):
            flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        purlin.check(stream)
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        return ts[len(ts) // 2]

    rows = []
    with open(path, "w") as f:
        for name in names:
            if name == "onesided":
                # the pages' two-GPU transfer: rank 0's T bytes to rank 1, as
                # an AllToAllV over two ranks with one non-empty partition
                s = {"counts": [0, n, 0, 0], "bmin": 2 * T}
                in_n, out_n, op = SPECS["alltoall"]
                xi, yo = ins[:2], outs[:2]
                wgs = (0, 2, 4, 8, 16, 64)
                lanes = (8, 16, 64, 128, 256)
            else:
                s = shapes[name]
                in_n, out_n, op = SPECS[name]
                xi = [ins[r][:s["ins"][r]] for r in range(P)]
                yo = [outs[r][:s["outs"][r]] for r in range(P)]
                wgs = (0, 32, 64, 128, 256)
                lanes = (1, 2, 4, 8, 16, 32)

            def fn():
                purlin.collective(xi, yo, in_n, out_n, op, s["counts"], stream=stream)

            points = [("zs", 0, 0, g) for g in wgs] + [("staged", 0, 0, 0)]
            points += [("staged", d, c, l) for l in lanes
                       for c in (16 << 10, 32 << 10, 64 << 10, 256 << 10, 1 << 20)
                       for d in range(1, 9)]
            for variant, d, c, g in points:
                purlin.set_policy(zero_staging=variant, depth=d, chunk_bytes=c, wgs_per_rank=g)
                t = p50(fn)
                info = purlin.last_launch()
                row = {"collective": name, "variant": variant, "T_bytes": T, "depth": info["depth"],
                       "chunk_bytes": info["chunk_bytes"], "wgs_per_rank_policy": g,
                       "grid": info["grid"], "p50_us": round(t * 1e6, 1),
                       "algbw_GBps": round(T / t / 1e9, 2),
                       "hbm_frac": round(s["bmin"] / t / HBM_PEAK, 4)}
                f.write(json.dumps(row) + "\n")
                f.flush()
                rows.append(row)
            print("%s done" % name, flush=True)
    purlin.set_policy(reset=True)
    return rows


def paired_bench(purlin, sizes, names, env_b, reps, dev, alloc=0):
    """Two settings of the library compared on the same buffers: the
    defaults (A) and the environment overrides `env_b` (B, e.g.
    {"PURLIN_SHIFT_STORES": "0"}), each collective at each T bytes per rank,
    `reps` calls per setting alternated call by call (A B, then B A, so
    neither always runs first), a 1 GiB fill between calls outside the
    events; below 1 MiB per rank warm instead, at least 200 calls each,
    queued behind a spin kernel (device latency).  The buffers are allocated
    for max(sizes, alloc) bytes per rank and every call uses their prefix
    (results depend on where the buffers sit, so `alloc` reproduces another
    run's placement).  One JSON line per (collective, T) with both p50s and
    the speed ratio A/B of B over A."""
    import torch
    import workloads
    stream = torch.cuda.current_stream()
    Tmax = max(max(sizes), alloc)
    shapes_max = collective_shapes(Tmax)
    n = Tmax // ESZ
    ins = [workloads.device_values(n, "normal", "bf16", 3, r, dev) for r in range(P)]
    out_len = max(max(shapes_max[nm]["outs"]) for nm in names)
    outs = [torch.empty(out_len, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    saved = {k: os.environ.get(k) for k in env_b}

    def setting(b):
        for k, v in env_b.items():
            if b:
                os.environ[k] = v
            elif saved[k] is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = saved[k]

    rows = []
    try:
        for T in sizes:
            shapes = collective_shapes(T)
            for name in names:
                s = shapes[name]
                in_n, out_n, op = SPECS[name]
                xi = [ins[r][:s["ins"][r]] for r in range(P)]
                yo = [outs[r][:s["outs"][r]] for r in range(P)]
                ev = [[], []]
                info = [None, None]
                for b in (0, 1):
                    setting(b)
                    purlin.collective(xi, yo, in_n, out_n, op, s["counts"], stream=stream)
                    info[b] = purlin.last_launch()
                cold = T >= (1 << 20)
                n_calls = reps if cold else max(reps, 200)
                for it in range(n_calls):
                    if not cold and it % 100 == 0:
                        # below 1 MiB: warm, the calls queued behind a spin
                        # kernel (device latency, as in the latency sweep)
                        torch.cuda.synchronize()
                        torch.cuda._sleep(20_000_000)
                    for b in ((0, 1) if it % 2 == 0 else (1, 0)):
                        setting(b)
                        if cold:
                            flush.fill_(1.0)
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        purlin.collective(xi, yo, in_n, out_n, op, s["counts"], stream=stream)
                        e1.record(stream)
                        ev[b].append((e0, e1))
                torch.cuda.synchronize()
                purlin.check(stream)
                p50 = []
                for b in (0, 1):
                    ts = sorted(a.elapsed_time(c) * 1e-3 for a, c in ev[b])
                    p50.append(ts[len(ts) // 2])
                row = {"collective": name, "T_bytes": T, "reps": reps, "b_env": env_b,
                       "a_p50_us": round(p50[0] * 1e6, 2), "b_p50_us": round(p50[1] * 1e6, 2),
                       "a_hbm_frac": round(s["bmin"] / p50[0] / HBM_PEAK, 4),
                       "b_hbm_frac": round(s["bmin"] / p50[1] / HBM_PEAK, 4),
                       "speed_b_over_a": round(p50[0] / p50[1], 4),
                       "a_grid": info[0]["grid"], "b_grid": info[1]["grid"]}
                print(json.dumps(row), flush=True)
                rows.append(row)
    finally:
        setting(0)
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--size", type=int, default=1 << 30, help="T, bytes per rank")
    ap.add_argument("--variant", choices=["zs", "staged"], default="zs")
    ap.add_argument("--only", default="", help="comma-separated subset of collectives")
    ap.add_argument("--cpu-sample", type=int, default=64 << 20,
                    help="T of the oracle sample, bytes per rank (0 skips it)")
    ap.add_argument("--sweep", default="",
                    help="write p50 latency / algorithm bandwidth of every collective over "
                         "T = 1 KiB .. --size to this JSONL file instead of the step benchmark")
    ap.add_argument("--ceilings", default="",
                    help="sweep the bare read/write patterns of the collectives (1->1, 1->8, "
                         "8->1, 8->8, read-only, write-only; loads / stores nontemporal or "
                         "plain x tile x grid x unroll) at --size bytes, cold, every point to "
                         "this JSONL file")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the pattern ceilings, the latency block and the placement "
                         "spread after the timed steps")
    ap.add_argument("--engines", action="store_true",
                    help="time the copy collectives on the DMA copy engines against the shader "
                         "kernels at --size bytes per rank, and a bf16 GEMM beside each")
    ap.add_argument("--moe", action="store_true",
                    help="time MoE dispatch / combine at 4096 x 7168 bf16 per rank, top-8 of 256")
    ap.add_argument("--ulysses", action="store_true",
                    help="time the Ulysses sequence <-> head exchange (Qwen-Image 1024x1024 "
                         "attention shape and ~64 MiB per rank)")
    ap.add_argument("--pipeline", default="",
                    help="write the staged pipeline sweep (depth 1-8 x chunk x workgroups per "
                         "job, against zero staging) of --only (default alltoall) at --size "
                         "bytes per rank to this JSONL file")
    ap.add_argument("--configs", default="",
                    help="write p50 latency of the fp32 AllReduce at 1 MiB per rank and the TP8 "
                         "AllReduce of [t x 7168] bf16 activations to this JSONL file")
    ap.add_argument("--paired", default="",
                    help="compare the defaults with environment overrides KEY=VALUE[,KEY=VALUE] "
                         "on the same buffers, calls alternated, for --only (default all) at "
                         "each of --sizes (default --size) bytes per rank, --steps calls each")
    ap.add_argument("--sizes", default="",
                    help="comma-separated T values for --paired and --policy-sweep")
    ap.add_argument("--alloc", type=int, default=0,
                    help="--paired: allocate the buffers for this many bytes per rank (at least "
                         "the largest of --sizes)")
    ap.add_argument("--policy-sweep", default="",
                    help="sweep workgroups per rank x chunk of the zero-staging kernel for --only "
                         "(default all) at --sizes (default 1-32 MiB) bytes per rank, cold p50, "
                         "every point to this JSONL file")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time only the plain 128-bit streaming copy of --size bytes "
                         "(HBM counter calibration and copy ceiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the P ranks are emulated in one GPU's HBM and no "
              "multi-GPU path exists in this build (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") != "1":
        print("bench.py runs as a single process", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from reduce_atom_02_amd import purlin

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    T = args.size
    if args.calibrate_copy:
        calibrate_copy(purlin, T, args.steps, args.warmup, dev)
        return
    if args.engines:
        print(json.dumps(engine_bench(purlin, T, args.steps, dev)), flush=True)
        return
    if args.moe:
        print(json.dumps(moe_bench(purlin, args.steps, args.warmup, dev)), flush=True)
        return
    if args.ulysses:
        print(json.dumps(ulysses_bench(purlin, args.steps, args.warmup, dev)), flush=True)
        return
    if args.configs:
        config_bench(purlin, args.configs, dev)
        return
    if args.policy_sweep:
        sizes = ([int(v) for v in args.sizes.split(",")] if args.sizes
                 else [1 << k for k in range(20, 26)])
        names = [n for n in SPECS if not args.only or n in args.only.split(",")]
        policy_sweep(purlin, sizes, names, args.policy_sweep, dev)
        return
    if args.paired:
        env_b = dict(kv.split("=", 1) for kv in args.paired.split(","))
        sizes = [int(v) for v in args.sizes.split(",")] if args.sizes else [T]
        names = [n for n in SPECS if not args.only or n in args.only.split(",")]
        paired_bench(purlin, sizes, names, env_b, args.steps, dev, args.alloc)
        return
    if args.pipeline:
        names = args.only.split(",") if args.only else ["alltoall"]
        pipeline_sweep(purlin, T, names, args.pipeline, dev)
        return
    if args.sweep:
        sweep(purlin, T, args.variant, args.sweep, dev)
        return
    if args.ceilings:
        print(json.dumps({"ceilings_hbm_frac": ceilings(purlin, T, args.steps, dev, full=True,
                                                        path=args.ceilings),
                          "T_bytes_per_stream": T, "cold": True}), flush=True)
        return
    names = [n for n in SPECS if not args.only or n in args.only.split(",")]
    shapes = collective_shapes(T)
    purlin.set_policy(zero_staging=args.variant)

    # one input set (N(0,1) bf16, drawn on the device) and one output set,
    # shared by the collectives; each uses the prefix it needs
    n = T // ESZ
    ins = [workloads.device_values(n, "normal", "bf16", 3, r, dev) for r in range(P)]
    out_len = max(max(s["outs"]) for s in shapes.values())
    outs = [torch.empty(out_len, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def call(name):
        s = shapes[name]
        in_n, out_n, op = SPECS[name]
        purlin.collective([ins[r][:s["ins"][r]] for r in range(P)],
                          [outs[r][:s["outs"][r]] for r in range(P)],
                          in_n, out_n, op, s["counts"], stream=stream)

    for _ in range(args.warmup):
        for name in names:
            call(name)
    purlin.check(stream)
    launch = {}
    for name in names:
        call(name)
        launch[name] = purlin.last_launch()
        assert launch[name]["bytes_min"] == shapes[name]["bmin"], name
    purlin.check(stream)

    events = {name: [] for name in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for name in names:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(name)
            e1.record(stream)
            events[name].append((e0, e1))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    purlin.check(stream)

    per = {}
    kern = {}
    for name in names:
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in events[name])
        mean = sum(ts) / len(ts)
        p50 = ts[len(ts) // 2]
        s = shapes[name]
        per[name] = {"p50_us": round(p50 * 1e6, 2), "mean_us": round(mean * 1e6, 2),
                     "p10_us": round(ts[len(ts) // 10] * 1e6, 2),
                     "p90_us": round(ts[min(len(ts) - 1, (9 * len(ts)) // 10)] * 1e6, 2),
                     "algbw_GBps": round(s["T"] / p50 / 1e9, 1),
                     "hbm_frac": round(s["bmin"] / p50 / HBM_PEAK, 4),
                     "bmin_bytes": s["bmin"], "grid": launch[name]["grid"],
                     "chunk_bytes": launch[name]["chunk_bytes"]}
        kname = kernel_of(name, launch[name]["rows"], launch[name]["one"],
                          launch[name]["plain_stores"], launch[name]["device_stores"])
        # HBM bytes per launch from the committed counter summary (when it was
        # taken on these sources and this workload): dram_frac is the rate HBM
        # sustained on the bytes actually moved
        tr = measured_traffic(kname, T, names, args.variant)
        if tr is not None:
            per[name]["traffic_bytes"] = tr
            per[name]["dram_frac"] = round(tr / p50 / HBM_PEAK, 4)
            # fewer bytes reached HBM than the collective must move: caches
            # (L2, the Infinity Cache) served part of it
            per[name]["cache_assisted"] = tr < 0.99 * s["bmin"]
        k = kern.setdefault(kname, {"bytes": 0, "time": 0.0, "launches": 0})
        k["bytes"] += s["bmin"] * len(ts)
        k["time"] += sum(ts)
        k["launches"] += len(ts)

    dom_name, dom = max(kern.items(), key=lambda kv: kv[1]["time"])
    achieved = dom["bytes"] / dom["time"] / 1e9
    total_T = sum(shapes[n_]["T"] for n_ in names) * args.steps
    total_bmin = sum(shapes[n_]["bmin"] for n_ in names) * args.steps
    value = total_T / elapsed / 1e9
    cpu = cpu_baseline(min(args.cpu_sample, T), names) if args.cpu_sample else None
    # after the timed region: the latency half of the metric (device p50 at
    # small sizes), the step on two more allocation sets, and what HBM
    # sustains for each collective's bare access pattern at this size
    latency = placement = pattern = None
    if not args.no_ceilings:
        latency = latency_block(purlin, dev, ins)
        first = {"hbm_frac": round(sum(shapes[n_]["bmin"] for n_ in names) /
                                   sum(per[n_]["p50_us"] * 1e-6 for n_ in names) / HBM_PEAK, 4),
                 "collectives": {n_: per[n_]["hbm_frac"] for n_ in names}}
        placement = placement_spread(purlin, T, names, 5, dev, first)
    del ins, outs
    torch.cuda.empty_cache()
    if not args.no_ceilings:
        pattern = ceilings(purlin, T, 3, dev)
        for label, c in pattern.items():
            for n_ in c.get("bounds", ()):
                if n_ in per:
                    per[n_]["frac_of_pattern_ceiling"] = round(per[n_]["hbm_frac"] / c["hbm_frac"], 4)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "seven collectives (%s), P=8 virtual ranks in one HBM, bf16, "
                               "T=%d MiB per rank, Zipf s=0.125 for the V variants, %s"
                               % (",".join(names), T >> 20,
                                  "zero staging" if args.variant == "zs" else "staged SNAC"),
                   "P": P, "T_bytes_per_rank": T, "variant": args.variant},
        "hbm_frac": round(total_bmin / elapsed / HBM_PEAK, 4),
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved * 1e9 / HBM_PEAK, 4),
                     "traffic": measured_traffic(dom_name, T, names, args.variant),
                     "launches": dom["launches"],
                     "avg_launch_us": round(dom["time"] / dom["launches"] * 1e6, 2),
                     "bytes_per_launch": dom["bytes"] // dom["launches"]},
        "cpu_baseline": cpu,
        "latency_p50_us": latency,
        "placement": placement,
        "pattern_ceilings": pattern,
        "collectives": per,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
