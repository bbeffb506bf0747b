"""Builds libzipccl.so in-tree with hipcc for gfx950.

    python -m lossless_bf16_exponent_codec_amd.build [--save-temps DIR]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzipccl.so")
SOURCES = [os.path.join(CSRC, "zipccl_kernels.hip"), os.path.join(CSRC, "zipccl_host.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def command(out: str = LIB, save_temps: str | None = None) -> list:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed FP32 instructions stay off: the codec needs none and some of their
           # forms are not trusted on this hardware
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           "-I", INCLUDE, "-I", CSRC, "-o", out]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd += ["-save-temps=obj"]
    cmd += ["-x", "hip"] + SOURCES
    return cmd


def build(out: str = LIB, save_temps: str | None = None, verbose: bool = False) -> str:
    cmd = command(out, save_temps)
    if save_temps:
        cmd[cmd.index("-o") + 1] = os.path.abspath(out)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=save_temps or None)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("--out", default=LIB)
    args = ap.parse_args(argv)
    build(args.out, args.save_temps, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
