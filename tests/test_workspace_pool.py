"""The workspace registry never frees a buffer it has handed out: a graph
captured before a growth keeps a valid address.  It also stays consistent
when several host threads ask for workspaces at once.  Host-only: the
registry (csrc/workspace_pool.hpp) is free of HIP and is built here with g++
against a fake allocator, once plainly and once with ThreadSanitizer."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "workspace_pool_check.cpp")


def _build_and_run(tmp_path, name, extra):
    exe = str(tmp_path / name)
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-Wall", *extra, "-o", exe, SRC, "-lpthread"])
    return subprocess.run([exe], capture_output=True, text=True, timeout=120)


def test_workspace_pool_retires_instead_of_freeing(tmp_path):
    r = _build_and_run(tmp_path, "pool_check", [])
    assert r.returncode == 0, r.stderr
    assert "workspace pool ok" in r.stdout


def test_workspace_pool_has_no_data_race(tmp_path):
    probe = subprocess.run(["g++", "-fsanitize=thread", "-x", "c++", "-", "-o", str(tmp_path / "t")],
                           input="int main(){return 0;}", capture_output=True, text=True)
    if probe.returncode != 0 or subprocess.run([str(tmp_path / "t")], capture_output=True).returncode != 0:
        pytest.skip("ThreadSanitizer is not usable with this g++")
    r = _build_and_run(tmp_path, "pool_check_tsan", ["-fsanitize=thread", "-g"])
    assert r.returncode == 0, r.stderr[-2000:]
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr[-2000:]
    assert "workspace pool ok" in r.stdout
