"""Host check of the key-split planner's index arithmetic (no GPU): a C++
program includes the planner header, decodes every plan the way the attention
kernel does and checks coverage, segment bounds, scratch slots, counter indices
and piece counts over many launch shapes (tests/c/split_plan_check.cpp)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_split_plan_decode(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no C++ compiler")
    exe = tmp_path / "split_plan_check"
    src = os.path.join(HERE, "c", "split_plan_check.cpp")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-Werror", "-o", str(exe), src], check=True)
    r = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout
    assert r.stdout.startswith("ok"), r.stdout
