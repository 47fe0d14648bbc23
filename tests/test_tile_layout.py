"""Host check of the staged query-tile layout (no GPU): a C++ program includes
the layout header, plans layouts for many launch shapes, decodes every tile
the way the attention kernel does and checks that the tiles cover every query
row exactly once (tests/c/tile_layout_check.cpp)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_staged_layout_decode(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no C++ compiler")
    exe = tmp_path / "tile_layout_check"
    src = os.path.join(HERE, "c", "tile_layout_check.cpp")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-Werror", "-o", str(exe), src], check=True)
    r = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout
    assert r.stdout.startswith("ok"), r.stdout
