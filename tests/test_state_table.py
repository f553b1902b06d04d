"""The scratch state table on the host (no GPU): build tests/state_table_check.cpp
against prefix_scan_amd/csrc/scratch_state.hpp with g++ and run it.  It checks
that no call, eager or replayed from a HIP graph, ever reads state it cannot
trust (including a captured scan followed by a captured one-bit radix sort,
replayed twice), and that the same check catches a table that is not told
about capture."""
import os
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_state_table_scenarios():
    src = os.path.join(ROOT, "tests", "state_table_check.cpp")
    inc = os.path.join(ROOT, "prefix_scan_amd", "csrc")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "state_table_check")
        subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", inc, "-o", exe, src],
                       check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr + r.stdout
    assert "all scenarios ok" in r.stdout
