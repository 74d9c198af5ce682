"""Host-only checks of the HIP kernels' index logic (compiled with hipcc, run
on the CPU; no GPU is touched): LDS block layouts and the exact division used
to decode problems and row maps."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sub_quadratic_factorized_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


def build_and_run(src, tmp_path):
    exe = tmp_path / (os.path.splitext(os.path.basename(src))[0])
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC, "-I",
           os.path.join(ROOT, "include"), os.path.join(HOST, src), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    return r.returncode, r.stdout + r.stderr


def test_lds_layouts(tmp_path):
    rc, out = build_and_run("lds_layout_check.cpp", tmp_path)
    assert rc == 0 and out.strip().endswith("OK"), out


def test_index_maps(tmp_path):
    rc, out = build_and_run("index_check.cpp", tmp_path)
    assert rc == 0 and out.strip().endswith("OK"), out
