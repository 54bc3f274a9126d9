"""The K/V ring schedule of the 16-bit forward (csrc/ring.hpp), which the
kernel executes: the compile-time hazard checker accepts the tables and
rejects each mutation that would let a wave read a stage beside a copy into it
(the barrier after the prologue's scores, the waits, the per-step barriers, a
copy into the stage being read).  Host-only: g++ compiles the checker."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_ring_schedule_mutations(tmp_path):
    exe = tmp_path / "ring_mutations"
    src = os.path.join(ROOT, "tests", "ring_mutations.cpp")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", src, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    got = dict(line.split() for line in r.stdout.strip().splitlines())
    assert got.pop("tables") == "1"
    assert got.pop("tables_spread") == "1"
    assert got.pop("step_copies_v_after_math") == "1"
    assert got, "no mutation cases ran"
    assert all(v == "0" for v in got.values()), got
    assert r.returncode == 0, r.stdout
