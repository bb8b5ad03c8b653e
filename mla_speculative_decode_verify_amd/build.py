"""Build libmla_verify.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m mla_speculative_decode_verify_amd.build [--jobs N]
Every HIP translation unit is compiled with the packed-fp32 target feature
disabled; the host layer is plain C++ compiled by the same driver.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla_verify.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "split_bf16.hip", "split_fp8.hip", "combine.hip", "append.hip", "topk.hip", "absorb.hip"]
# Per-source extra compiler flags.
EXTRA_FLAGS = {}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def compile_one(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = ([hipcc()] + common_flags() + EXTRA_FLAGS.get(src, []) + [f"-D{d}" for d in defines] +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 4, verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile and link the library; `defines` (NAME=VALUE) and `out` serve tuning builds."""
    build_dir = BUILD if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda src: compile_one(src, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    args = ap.parse_args()
    build(args.jobs, verbose=True, out=os.path.abspath(args.out), defines=args.defines)
    sys.exit(0)
