"""Python binding of libpurlin: argument marshalling only.

Every step of a collective runs in the HIP library; this module turns
Python values (torch tensors or raw device addresses) into the C ABI's
arguments and status codes into exceptions.  The library is loaded at import
time and the import fails when it has not been built (``python -m
reduce_atom_02_amd.build``): there is no other implementation to fall back to.

Names follow include/purlin.h: namings ``whole``, ``by_rank``, ``by_index``,
``by_rank_index``, ``by_index_rank``; ops ``copy`` and ``sum``; dtypes
``f32`` and ``bf16``.
"""
import ctypes
import itertools
import os

__all__ = [
    "LIB_PATH", "NAMINGS", "OPS", "DTYPES", "STATUS", "PurlinError", "collective",
    "all_reduce", "reduce_scatter", "all_gather", "all_to_all", "check",
    "collective_noalloc", "set_policy", "get_policy", "plan_describe", "last_launch",
    "stream_copy", "stream_pattern",
    "moe_dispatch", "moe_combine", "ulysses", "release", "exported_symbols",
    "name_count", "extents", "check_tensors",
]

# PURLIN_LIBRARY names another build of the library to load (the tests load
# libpurlin_debug.so, the build with the protocol checks, this way).
LIB_PATH = os.environ.get("PURLIN_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpurlin.so")

NAMINGS = {"whole": 0, "by_rank": 1, "by_index": 2, "by_rank_index": 3, "by_index_rank": 4}
OPS = {"copy": 0, "sum": 1}
DTYPES = {"f32": 0, "bf16": 1}
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "NO_MEMORY", 4: "HIP", 5: "TIMEOUT",
          6: "PROTOCOL"}
STAGING = {"auto": 0, "zs": 1, "staged": 2}
ENGINES = {"auto": 0, "shader": 1, "copy": 2}

COLLECTIVES = {
    "allreduce": ("whole", "whole", "sum"),
    "reducescatter": ("by_index", "by_rank", "sum"),
    "allgather": ("by_rank", "by_index", "copy"),
    "alltoall": ("by_rank_index", "by_index_rank", "copy"),
}


class PurlinError(RuntimeError):
    def __init__(self, status, what):
        self.status = STATUS.get(status, str(status))
        super().__init__("%s: %s (%s)" % (what, self.status, _lib.purlin_strerror(status).decode()))


class Layout(ctypes.Structure):
    _fields_ = [("naming", ctypes.c_int), ("bufs", ctypes.POINTER(ctypes.c_void_p))]


class Policy(ctypes.Structure):
    _fields_ = [("chunk_bytes", ctypes.c_int64), ("depth", ctypes.c_int32),
                ("wgs_per_rank", ctypes.c_int32), ("zero_staging", ctypes.c_int32),
                ("sync", ctypes.c_int32), ("watchdog_ns", ctypes.c_int64),
                ("test_withhold", ctypes.c_int32), ("engine", ctypes.c_int32)]


class Segment(ctypes.Structure):
    _fields_ = [("src_rank", ctypes.c_int32), ("dst_rank", ctypes.c_int32),
                ("src_off", ctypes.c_int64), ("dst_off", ctypes.c_int64),
                ("len", ctypes.c_int64)]


class LaunchInfo(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("zero_staging", ctypes.c_int32), ("depth", ctypes.c_int32),
                ("chunk_bytes", ctypes.c_int64), ("tiles", ctypes.c_int64),
                ("bytes_min", ctypes.c_int64), ("njobs", ctypes.c_int32),
                ("sync", ctypes.c_int32), ("rows", ctypes.c_int32), ("unit", ctypes.c_int32),
                ("one", ctypes.c_int32), ("plain_stores", ctypes.c_int32),
                ("engine_copies", ctypes.c_int32), ("shift_stores", ctypes.c_int32),
                ("unaligned_loads", ctypes.c_int32), ("device_stores", ctypes.c_int32),
                ("unroll", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libpurlin.so is not built (%s); run: python -m reduce_atom_02_amd.build"
                          % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P_LAYOUT = ctypes.POINTER(Layout)
    P_I64 = ctypes.POINTER(ctypes.c_int64)
    lib.purlin_collective.argtypes = [P_LAYOUT, P_LAYOUT, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      P_I64, P_I64, ctypes.c_void_p]
    lib.purlin_collective.restype = ctypes.c_int
    lib.purlin_collective_noalloc.argtypes = lib.purlin_collective.argtypes
    lib.purlin_collective_noalloc.restype = ctypes.c_int
    lib.purlin_check.argtypes = [ctypes.c_void_p]
    lib.purlin_check.restype = ctypes.c_int
    lib.purlin_set_policy.argtypes = [ctypes.POINTER(Policy)]
    lib.purlin_set_policy.restype = ctypes.c_int
    lib.purlin_get_policy.argtypes = [ctypes.POINTER(Policy)]
    lib.purlin_get_policy.restype = ctypes.c_int
    lib.purlin_plan_describe.argtypes = [P_LAYOUT, P_LAYOUT, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, P_I64, P_I64, ctypes.POINTER(Segment),
                                         P_I64]
    lib.purlin_plan_describe.restype = ctypes.c_int
    lib.purlin_last_launch.argtypes = [ctypes.POINTER(LaunchInfo)]
    lib.purlin_last_launch.restype = ctypes.c_int
    lib.purlin_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p]
    lib.purlin_stream_copy.restype = ctypes.c_int
    lib.purlin_stream_pattern.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                          ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    P_VP = ctypes.POINTER(ctypes.c_void_p)
    lib.purlin_moe_dispatch.argtypes = [P_VP, P_VP, ctypes.c_int, ctypes.c_int64, P_VP, P_I64,
                                        P_I64, ctypes.c_int, ctypes.c_void_p]
    lib.purlin_moe_dispatch.restype = ctypes.c_int
    lib.purlin_moe_combine.argtypes = [P_VP, P_VP, ctypes.c_int, ctypes.c_int64, P_VP, P_VP,
                                       P_I64, P_I64, ctypes.c_void_p]
    lib.purlin_moe_combine.restype = ctypes.c_int
    lib.purlin_ulysses.argtypes = [P_VP, P_VP, ctypes.c_int, P_I64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p]
    lib.purlin_ulysses.restype = ctypes.c_int
    lib.purlin_stream_pattern.restype = ctypes.c_int
    lib.purlin_strerror.argtypes = [ctypes.c_int]
    lib.purlin_strerror.restype = ctypes.c_char_p
    lib.purlin_release.argtypes = []
    lib.purlin_release.restype = None
    return lib


_lib = _load()


def exported_symbols():
    """Names of the C ABI functions the loaded library resolves."""
    names = ["purlin_collective", "purlin_collective_noalloc", "purlin_check", "purlin_set_policy", "purlin_get_policy",
             "purlin_plan_describe", "purlin_last_launch", "purlin_stream_copy",
             "purlin_stream_pattern", "purlin_moe_dispatch", "purlin_moe_combine",
             "purlin_ulysses", "purlin_strerror", "purlin_release"]
    return [n for n in names if hasattr(_lib, n)]


def _raise(status, what):
    if status != 0:
        raise PurlinError(status, what)


def _ptr(x):
    if x is None or isinstance(x, int):
        return x
    return x.data_ptr()          # torch tensor


def _dtype_of(bufs, dtype):
    """The element type: `dtype`, else that of the first tensor in `bufs`
    (every buffer is taken to hold it)."""
    if dtype is not None:
        return dtype
    for b in bufs:
        if b is not None and not isinstance(b, int):
            name = str(b.dtype)
            if name == "torch.float32":
                return "f32"
            if name == "torch.bfloat16":
                return "bf16"
            raise ValueError("unsupported tensor dtype %s" % name)
    raise ValueError("dtype must be given for raw pointers")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# Marshalled arguments of recent calls, keyed by value: building ctypes
# arrays costs microseconds per call, and loops repeat the same buffers and
# counts.  The library only reads them.  Bounded; cleared when full.
_CACHE = {}
_CACHE_MAX = 512


def _cached(key, make):
    v = _CACHE.get(key)
    if v is None:
        if len(_CACHE) >= _CACHE_MAX:
            _CACHE.clear()
        v = _CACHE[key] = make()
    return v


def _layout(naming, bufs, ptrs=None):
    if ptrs is None:
        ptrs = tuple(map(_ptr, bufs))

    def make():
        arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
        return Layout(NAMINGS[naming], arr), arr

    return _cached(("layout", naming, ptrs), make)


def _i64(values):
    if values is None:
        return None
    vals = tuple(values)             # ints of any integer type hash by value
    return _cached(("i64", vals),
                   lambda: (ctypes.c_int64 * max(1, len(vals)))(*map(int, vals)))


_TORCH_DTYPES = {"torch.float32": "f32", "torch.bfloat16": "bf16"}
_ESZ = {"f32": 4, "bf16": 2}


def name_count(naming, P):
    """Names of a naming at P ranks (the length of its counts array)."""
    return 1 if naming == "whole" else (P if naming in ("by_rank", "by_index") else P * P)


def extents(naming, P, counts, displs_side=None):
    """Elements each rank's buffer must hold under `naming`: the end of its
    last non-empty partition (counts and displacements indexed by name, as
    in include/purlin.h; displs_side None means packed in index order)."""
    ext = []
    for r in range(P):
        if naming == "whole":
            names = (0,)
        elif naming == "by_rank":
            names = (r,)
        elif naming == "by_index":
            names = range(P)
        elif naming == "by_rank_index":
            names = [r * P + q for q in range(P)]
        else:
            names = [q * P + r for q in range(P)]
        end = packed = 0
        for nm in names:
            c = int(counts[nm])
            off = int(displs_side[nm]) if displs_side is not None else packed
            packed += c
            if c > 0:
                end = max(end, off + c)
        ext.append(end)
    return ext


def check_tensors(bufs, need, dt, op, what, device=None):
    """Reject, before any GPU work, a tensor the library would misread:
    not on the GPU `device` (None skips that check), not contiguous, of
    another element type than the others or than `dt`, or smaller than the
    `need` elements its rank's partitions reach.  Raw addresses (ints) and
    None pass unchecked.  Raises ValueError."""
    tdtype = None
    for r, t in enumerate(bufs):
        if t is None or isinstance(t, int):
            continue
        if device is not None and (not t.is_cuda or t.get_device() != device):
            raise ValueError("%s %d is not on the current GPU (device %s)" % (what, r, t.device))
        if not t.is_contiguous():
            raise ValueError("%s %d is not contiguous" % (what, r))
        if tdtype is None:
            tdtype = t.dtype
        elif t.dtype != tdtype:
            raise ValueError("%s %d has dtype %s, another buffer %s" % (what, r, t.dtype, tdtype))
        if t.element_size() != _ESZ[dt] or (op == "sum" and _TORCH_DTYPES.get(str(t.dtype)) != dt):
            raise ValueError("%s %d has dtype %s, the collective %s" % (what, r, t.dtype, dt))
        if t.numel() < need[r]:
            raise ValueError("%s %d holds %d elements, its partitions reach %d"
                             % (what, r, t.numel(), need[r]))


_CHECKED = {}


def _validate(ins, outs, pin, pout, in_naming, out_naming, op, dt, counts, displs):
    """The binding's checks of one call (cached by buffers and plan); pin and
    pout are the buffers' addresses."""
    P = len(ins)
    key = (in_naming, out_naming, op, dt, P, tuple(counts),
           None if displs is None else tuple(displs), pin, pout,
           tuple(None if t is None or isinstance(t, int) else (t.numel(), t.dtype)
                 for t in itertools.chain(ins, outs)))
    if key in _CHECKED:
        return
    nn = name_count(in_naming, P)
    if len(counts) != nn:
        raise ValueError("%s at P=%d takes %d counts, got %d" % (in_naming, P, nn, len(counts)))
    if displs is not None and len(displs) != 2 * nn:
        raise ValueError("displs takes %d entries, got %d" % (2 * nn, len(displs)))
    if name_count(out_naming, P) == nn:
        import torch
        dev = torch.cuda.current_device() if torch.cuda.is_available() else -1
        din = None if displs is None else displs[:nn]
        dout = None if displs is None else displs[nn:]
        check_tensors(ins, extents(in_naming, P, counts, din), dt, op, "input", dev)
        check_tensors(outs, extents(out_naming, P, counts, dout), dt, op, "output", dev)
    if len(_CHECKED) >= _CACHE_MAX:
        _CHECKED.clear()
    _CHECKED[key] = True


def collective(ins, outs, in_naming, out_naming, op, counts, displs=None, dtype=None,
               stream=None, noalloc=False):
    """Enqueue one collective on ``stream`` (torch's current stream by default).

    ins, outs: P torch tensors or device addresses, one per rank.
    counts: one element count per name (see include/purlin.h).
    displs: None (packed) or input offsets then output offsets, by name.
    noalloc: run purlin_collective_noalloc (the library's fixed scratch
    array instead of the stream's workspace; nothing is allocated).
    Tensors are checked before the call (on the current GPU, contiguous, one
    element type, large enough for their partitions): ValueError otherwise.
    """
    P = len(ins)
    if len(outs) != P:
        raise ValueError("need as many output buffers as input buffers")
    dt = _dtype_of(itertools.chain(ins, outs), dtype)
    pin = tuple(map(_ptr, ins))
    pout = tuple(map(_ptr, outs))
    _validate(ins, outs, pin, pout, in_naming, out_naming, op, dt, counts, displs)
    lin, keep_in = _layout(in_naming, ins, pin)
    lout, keep_out = _layout(out_naming, outs, pout)
    c = _i64(counts)
    d = _i64(displs)
    fn = _lib.purlin_collective_noalloc if noalloc else _lib.purlin_collective
    status = fn(ctypes.byref(lin), ctypes.byref(lout), OPS[op], DTYPES[dt], P, c, d,
                ctypes.c_void_p(_stream(stream)))
    _raise(status, "purlin_collective_noalloc" if noalloc else "purlin_collective")


def collective_noalloc(ins, outs, in_naming, out_naming, op, counts, displs=None, dtype=None,
                       stream=None):
    """collective() through purlin_collective_noalloc (see include/purlin.h)."""
    collective(ins, outs, in_naming, out_naming, op, counts, displs, dtype, stream, noalloc=True)


def _numel(t):
    return t if isinstance(t, int) else t.numel()


def all_reduce(ins, outs, count=None, **kw):
    n = count if count is not None else _numel(ins[0])
    collective(ins, outs, "whole", "whole", "sum", [n], **kw)


def reduce_scatter(ins, outs, counts=None, **kw):
    if counts is None:
        counts = [_numel(o) for o in outs]
    collective(ins, outs, "by_index", "by_rank", "sum", counts, **kw)


def all_gather(ins, outs, counts=None, **kw):
    if counts is None:
        counts = [_numel(i) for i in ins]
    collective(ins, outs, "by_rank", "by_index", "copy", counts, **kw)


def all_to_all(ins, outs, counts=None, **kw):
    """counts: P*P (row-major [src * P + dst]), or P (every source sends c_j to rank j)."""
    P = len(ins)
    if counts is None:
        n = _numel(ins[0])
        if n % P:
            raise ValueError("equal partitions need a size divisible by P")
        counts = [n // P] * (P * P)
    elif len(counts) == P:
        counts = [counts[j] for _ in range(P) for j in range(P)]
    collective(ins, outs, "by_rank_index", "by_index_rank", "copy", counts, **kw)


def check(stream=None):
    """Synchronize the stream; raise PurlinError on a device-side timeout."""
    _raise(_lib.purlin_check(ctypes.c_void_p(_stream(stream))), "purlin_check")


def set_policy(chunk_bytes=0, depth=0, wgs_per_rank=0, zero_staging="auto", sync=None,
               watchdog_ns=0, test_withhold=0, engine="auto", reset=False):
    """engine: "auto" / "shader" (the Atom kernels) or "copy" (copy collectives
    on the DMA copy engines, no kernel)."""
    if reset:
        _raise(_lib.purlin_set_policy(None), "purlin_set_policy")
        return
    p = Policy(chunk_bytes, depth, wgs_per_rank, STAGING[zero_staging],
               0 if sync is None else (1 if sync else 2), watchdog_ns, test_withhold,
               ENGINES[engine])
    _raise(_lib.purlin_set_policy(ctypes.byref(p)), "purlin_set_policy")


def get_policy():
    p = Policy()
    _raise(_lib.purlin_get_policy(ctypes.byref(p)), "purlin_get_policy")
    return {f: getattr(p, f) for f, _ in Policy._fields_}


def plan_describe(in_naming, out_naming, op, dtype, counts, in_bufs, out_bufs, displs=None):
    """Segments (src_rank, dst_rank, src_off, dst_off, len) of a plan; runs no HIP call."""
    P = len(in_bufs)
    lin, keep_in = _layout(in_naming, in_bufs)
    lout, keep_out = _layout(out_naming, out_bufs)
    c = _i64(counts)
    d = _i64(displs)
    n = ctypes.c_int64(0)
    _raise(_lib.purlin_plan_describe(ctypes.byref(lin), ctypes.byref(lout), OPS[op], DTYPES[dtype],
                                     P, c, d, None, ctypes.byref(n)), "purlin_plan_describe")
    segs = (Segment * max(1, n.value))()
    _raise(_lib.purlin_plan_describe(ctypes.byref(lin), ctypes.byref(lout), OPS[op], DTYPES[dtype],
                                     P, c, d, segs, ctypes.byref(n)), "purlin_plan_describe")
    return [(s.src_rank, s.dst_rank, s.src_off, s.dst_off, s.len) for s in segs[:n.value]]


def plan_status(in_naming, out_naming, op, dtype, counts, in_bufs, out_bufs, displs=None, P=None):
    """Status name of planning a collective (no HIP call); 'OK' when it is valid."""
    P = len(in_bufs) if P is None else P
    lin, keep_in = _layout(in_naming, in_bufs)
    lout, keep_out = _layout(out_naming, out_bufs)
    n = ctypes.c_int64(0)
    s = _lib.purlin_plan_describe(ctypes.byref(lin), ctypes.byref(lout),
                                  OPS.get(op, op) if isinstance(op, str) else op,
                                  DTYPES.get(dtype, dtype) if isinstance(dtype, str) else dtype,
                                  P, _i64(counts), _i64(displs), None, ctypes.byref(n))
    return STATUS[s]


def last_launch():
    info = LaunchInfo()
    _raise(_lib.purlin_last_launch(ctypes.byref(info)), "purlin_last_launch")
    return {f: getattr(info, f) for f, _ in LaunchInfo._fields_}


def stream_copy(dst, src, nbytes, stream=None):
    """The plain 128-bit streaming copy (calibration / ceiling kernel)."""
    _raise(_lib.purlin_stream_copy(ctypes.c_void_p(_ptr(dst)), ctypes.c_void_p(_ptr(src)),
                                   int(nbytes), ctypes.c_void_p(_stream(stream))),
           "purlin_stream_copy")


def stream_pattern(srcs, dsts, nbytes, grid=0, tile_bytes=0, unroll=0, nt_loads=True,
                   nt_stores=True, stream=None, device_stores=False):
    """Bare read/write pattern of a collective (ceiling measurement): srcs
    and dsts hold 0, 1 or 8 buffers each; grid 0 is four workgroups per CU,
    tile_bytes 0 is 16 KiB, unroll 0 is 4 units per lane; device_stores
    writes through the L2 (nt_stores is then ignored)."""
    sa = (ctypes.c_void_p * max(1, len(srcs)))(*[_ptr(x) for x in srcs])
    da = (ctypes.c_void_p * max(1, len(dsts)))(*[_ptr(x) for x in dsts])
    access = (1 if nt_loads else 0) | (2 if nt_stores else 0) | (4 if device_stores else 0)
    _raise(_lib.purlin_stream_pattern(sa, len(srcs), da, len(dsts), int(nbytes), int(grid),
                                      int(tile_bytes), int(unroll), access,
                                      ctypes.c_void_p(_stream(stream))), "purlin_stream_pattern")


def _ptrs(bufs):
    vals = tuple(map(_ptr, bufs))
    return _cached(("ptrs", vals), lambda: (ctypes.c_void_p * max(1, len(vals)))(*vals))


def moe_dispatch(x, y, idx, counts, x_rows=None, row_bytes=None, unique=False, stream=None):
    """MoE dispatch: y[j] = for i ascending, x[i] rows idx[i][group j] (see
    include/purlin.h).  x, y: P tensors (or addresses) of rows; idx: P int32
    device tensors grouped by destination; counts: P*P rows [i*P + j];
    unique: one row per (token, destination rank), each token row read once."""
    P = len(x)
    if row_bytes is None:
        row_bytes = x[0].shape[-1] * x[0].element_size()
    if x_rows is None:
        x_rows = [xi.shape[0] for xi in x]
    _raise(_lib.purlin_moe_dispatch(_ptrs(x), _ptrs(y), P, int(row_bytes), _ptrs(idx),
                                    _i64(counts), _i64(x_rows), 1 if unique else 0,
                                    ctypes.c_void_p(_stream(stream))),
           "purlin_moe_dispatch")


def moe_combine(y, out, idx, w, counts, x_rows=None, row_bytes=None, stream=None):
    """MoE combine: out[i][t] = bf16 of the fp32 fold, ascending (rank,
    entry), of w * y rows routed back to token t (see include/purlin.h)."""
    P = len(out)
    if row_bytes is None:
        row_bytes = out[0].shape[-1] * out[0].element_size()
    if x_rows is None:
        x_rows = [o.shape[0] for o in out]
    _raise(_lib.purlin_moe_combine(_ptrs(y), _ptrs(out), P, int(row_bytes), _ptrs(idx), _ptrs(w),
                                   _i64(counts), _i64(x_rows), ctypes.c_void_p(_stream(stream))),
           "purlin_moe_combine")


def ulysses(ins, outs, heads, seq=None, head_bytes=None, to_sequence=False, stream=None):
    """Ulysses AllToAll (see include/purlin.h): sequence layout [seq[i], heads,
    head] on rank i <-> head layout [S, heads / P, head] on rank j.  ins, outs:
    P tensors (or addresses); seq and head_bytes default to what the
    sequence-layout tensors hold (their bytes / (heads * head_bytes) tokens,
    their last dimension times the element size)."""
    P = len(ins)
    sq = outs if to_sequence else ins
    if head_bytes is None:
        head_bytes = sq[0].shape[-1] * sq[0].element_size()
    if seq is None:
        seq = [t.numel() * t.element_size() // (int(heads) * int(head_bytes)) for t in sq]
    _raise(_lib.purlin_ulysses(_ptrs(ins), _ptrs(outs), P, _i64(seq), int(heads), int(head_bytes),
                               1 if to_sequence else 0, ctypes.c_void_p(_stream(stream))),
           "purlin_ulysses")


def release():
    _lib.purlin_release()
