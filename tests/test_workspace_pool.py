"""The workspace registry never frees a buffer it has handed out: a graph
captured before a growth keeps a valid address.  Host-only: the registry
(csrc/workspace_pool.hpp) is free of HIP and is built here with g++ against
a fake allocator."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_workspace_pool_retires_instead_of_freeing(tmp_path):
    exe = str(tmp_path / "pool_check")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-Wall", "-o", exe,
                           os.path.join(ROOT, "tests", "workspace_pool_check.cpp"), "-lpthread"])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "workspace pool ok" in r.stdout
