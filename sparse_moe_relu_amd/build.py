"""Build libdeco_moe.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m sparse_moe_relu_amd.build   (or call build_library()).
Cross-compiles without a GPU.  Each .hip source becomes an object; the
objects are linked into sparse_moe_relu_amd/libdeco_moe.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdeco_moe.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["host.hip", "pack.hip", "decode.hip", "prefill.hip", "backward.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-variable", "-Wno-unused-function",
    # packed-fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str, build_dir: str, extra: list) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip():
        print(f"[build] {src}:\n{errs}", file=sys.stderr)
    return obj


def build_library(verbose: bool = True, out: str = LIB, defines: list | None = None) -> str:
    """Compile every source and link `out`.  `defines` (NAME=VALUE strings)
    override the kernels' compile-time launch parameters."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    extra = [f"-D{d}" for d in (defines or [])]
    build_dir = BUILD_DIR if out == LIB else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    shutil.rmtree(build_dir, ignore_errors=True)
    if verbose:
        print(f"[build] wrote {out}")
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    a = ap.parse_args()
    build_library(out=a.out, defines=a.defines)
