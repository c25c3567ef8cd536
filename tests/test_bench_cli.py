"""The benchmark's command-line contract, on the CPU: a request for more than one GPU exits
with status 2 and says why (the library measures one GPU), and every named workload is of a
kind the benchmark knows how to run."""
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_workload_recipes_are_known_kinds(name):
    assert workloads.WORKLOADS[name]["kind"] in ("gdn", "varlen", "bigdn", "bigdn_merged",
                                                 "summary", "cam", "dhu", "cam_bwd", "bigdn_bwd",
                                                 "bigdn_block_bwd", "cam_branch_bwd")
