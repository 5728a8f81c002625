"""Build libpurlin.so (HIP for gfx950) in place, next to this file.

    python -m reduce_atom_02_amd.build            # libpurlin.so
    python -m reduce_atom_02_amd.build --debug    # libpurlin_debug.so (protocol checks)

Every source under csrc/ is compiled by hipcc into one shared library with
no dependency other than the HIP runtime.  Packed fp32 instructions are
disabled for the device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpurlin.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["kernels.hip", "noalloc.hip", "planner.cpp", "purlin.cpp"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


DEBUG_LIB = os.path.join(HERE, "libpurlin_debug.so")


def build(verbose=False, extra=(), debug=False):
    """Build libpurlin.so, or with debug=True libpurlin_debug.so: the same
    library with the staged protocol's checks compiled in
    (PURLIN_DEBUG_PROTOCOL: exact flag and credit values, slot headers and
    canaries, reported by purlin_check as PURLIN_ERR_PROTOCOL)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    lib = DEBUG_LIB if debug else LIB
    if debug:
        extra = list(extra) + ["-DPURLIN_DEBUG_PROTOCOL"]
    tmp = lib + ".tmp"
    cmd = [HIPCC] + FLAGS + list(extra) + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed (%d)" % res.returncode)
    if verbose and res.stderr.strip():
        # the host pass does not know the packed-fp32 target feature: harmless
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, lib)
    return lib


def build_all(verbose=False):
    """Both libraries, compiled concurrently (two hipcc processes)."""
    import threading
    out, errs = {}, []

    def one(debug):
        try:
            out[debug] = build(verbose=verbose, debug=debug)
        except Exception as e:  # re-raised below, from the calling thread
            errs.append(e)

    threads = [threading.Thread(target=one, args=(d,)) for d in (False, True)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    if errs:
        raise errs[0]
    return out[False], out[True]


if __name__ == "__main__":
    print(build(verbose=True, debug="--debug" in sys.argv))
