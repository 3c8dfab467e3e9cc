"""Host check of the paged-cache addressing (csrc/paged.h) that the paged
decode and reuse-prefill kernels use: tests/paged_rows_check.cpp, built with
the host C++ compiler, drives the same header over random caches, block
tables with out-of-range entries, ragged last blocks, list padding, every KV
head and both [nb,Hkv,bs,d] and [nb,bs,Hkv,d] layouts, and asserts every row
address stays inside the cache."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_paged_row_addresses_stay_in_the_cache(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "paged_rows_check"
    subprocess.run([cxx, "-O1", "-std=c++17", "-Wall", os.path.join(HERE, "paged_rows_check.cpp"), "-o",
                    str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
