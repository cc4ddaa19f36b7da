"""The late decode workgroups' ticket rule (``csrc/tickets.h``), checked on the
host: the header is compiled with g++ into a small program that applies the
hardware's wrapping increment for every claimer count up to 300 and counter
start values from 0 to past the limit (and near 2^32), and checks that every
late place is taken exactly once."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_260_amd", "csrc")


def test_ticket_places_permutation_from_any_start(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "ticket_places"
    subprocess.run([gxx, "-std=c++17", "-O1", f"-I{CSRC}", os.path.join(ROOT, "tests", "ticket_places.cpp"),
                    "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok ")
    _, cases, raw_fail = res.stdout.split()
    assert int(cases) > 300 * 10
    # the unclamped ticket misses a place in every one of those cases
    assert int(raw_fail) == 300
