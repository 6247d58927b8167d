"""Host logic of the paged cache (long_context_attention_22_amd/csrc/pager.h), no GPU.

tests/pager_host_test.cpp drives the page bookkeeping against a simulated address space: a model
of what contiguous caches would hold is checked row by row after every reserve, fork and close
(fixed cases: forks inside a page, on a page boundary and of a full sequence, pool exhaustion, a
backend failure part way with rollback; then random sequences of operations), together with the
reference counts and the free list.  Built with g++ and the host sanitizers.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_pager_bookkeeping(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    exe = tmp_path / "pager_host_test"
    cmd = [gxx, "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "long_context_attention_22_amd", "csrc"),
           os.path.join(ROOT, "tests", "pager_host_test.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "pager host test: ok" in r.stdout
