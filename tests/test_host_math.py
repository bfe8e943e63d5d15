"""Host-side arithmetic of the library compiled with g++ (no GPU): the
multiply-shift division that maps GEMM output rows/columns to addresses, and
the K/V ring placement built on it."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_host(tmp_path, name):
    exe = tmp_path / name
    cmd = ["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROOT, "transformer_xl_relative_attn_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", name + ".cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")


def test_axis_division_exact(tmp_path):
    _run_host(tmp_path, "axis_check")


def test_ring_placement(tmp_path):
    _run_host(tmp_path, "ring_map_check")
