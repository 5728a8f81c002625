"""Host-side logic of bench.py (no GPU): the compulsory-byte formulas, the
workload shapes, the rule that decides whether committed HBM counters still
apply, and the refusal of more than one GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

P = bench.P


@pytest.mark.parametrize("T", [1 << 20, 3 << 20, 1 << 30])
def test_bmin_formulas(T):
    """Every input byte read once and every output byte written once: AllReduce
    2PS, ReduceScatter(V) and AllGather(V) (P+1)T, AllToAll(V) 2PT."""
    s = bench.collective_shapes(T)
    assert s["allreduce"]["bmin"] == 2 * P * T
    for name in ("reducescatter", "allgather", "reducescatterv", "allgatherv"):
        assert s[name]["bmin"] == (P + 1) * T, name
    for name in ("alltoall", "alltoallv"):
        assert s[name]["bmin"] == 2 * P * T, name


def test_shapes_are_consistent_with_counts():
    T = 1 << 20
    n = T // bench.ESZ
    s = bench.collective_shapes(T)
    z = s["reducescatterv"]["counts"]
    assert sum(z) == n and len(z) == P
    assert s["allgatherv"]["outs"] == [n] * P and s["allgatherv"]["ins"] == z
    a2av = s["alltoallv"]["counts"]
    assert len(a2av) == P * P and sum(a2av[:P]) == n      # every input is T
    assert s["alltoallv"]["outs"] == [P * z[j] for j in range(P)]
    assert sum(s["alltoall"]["counts"]) == P * n


def _copy_sources(dst):
    shutil.copytree(os.path.join(ROOT, "reduce_atom_02_amd", "csrc"),
                    os.path.join(dst, "reduce_atom_02_amd", "csrc"))


def test_counter_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    _copy_sources(str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    f = os.path.join(str(tmp_path), "reduce_atom_02_amd", "csrc", "atom.hpp")
    with open(f) as fh:
        text = fh.read()
    with open(f, "w") as fh:
        fh.write("// a new comment line\n/* and a block\n   comment */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash() == h0
    with open(f, "w") as fh:
        fh.write(text.replace("constexpr int kWideElems = 9;", "constexpr int kWideElems = 8;"))
    assert bench.kernel_source_hash() != h0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
