"""Build the SQuad-Attention HIP library in-tree for gfx950.

    python -m sub_quadratic_factorized_amd.build

compiles every source under csrc/ with hipcc and links
sub_quadratic_factorized_amd/libsquad_attn.so.  hipcc cross-compiles, so this
works on a machine without a GPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libsquad_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["squad_abi.hip", "squad_pass_bf16.hip", "squad_pass_f32.hip", "squad_bwd_bf16.hip", "squad_bwd_f32.hip"]

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand) and shutil.which(cand) is None:
        raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")
    return cand


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile all sources and link the shared library; returns its path."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="squad_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
            if len(procs) >= jobs:
                _drain(procs, verbose)
        _drain(procs, verbose)
        out_tmp = LIB_PATH + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}")
        os.replace(out_tmp, LIB_PATH)
        return LIB_PATH
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _drain(procs, verbose):
    while procs:
        src, p = procs.pop(0)
        out, _ = p.communicate()
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out, flush=True)


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
