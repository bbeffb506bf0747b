"""Builds libzipccl.so in-tree with hipcc for gfx950, and libzcprobe.so, the benchmark's
streaming probes (plain memory-moving kernels, no part of the codec).

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
PROBE_LIB = os.path.join(PKG, "libzcprobe.so")
PROBE_SOURCES = [os.path.join(CSRC, "stream_probe.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def command(out: str = LIB, save_temps: str | None = None, sources=None) -> list:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed FP32 instructions stay off: the codec needs none and some of their
           # forms are not trusted on this hardware
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           "-I", INCLUDE, "-I", CSRC, "-o", out]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd += ["-save-temps=obj"]
    cmd += ["-x", "hip"] + (SOURCES if sources is None else sources)
    return cmd


def build(out: str = LIB, save_temps: str | None = None, verbose: bool = False) -> str:
    cmd = command(out, save_temps)
    if save_temps:
        cmd[cmd.index("-o") + 1] = os.path.abspath(out)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=save_temps or None)
    return out


def build_probe(out: str = PROBE_LIB, verbose: bool = False) -> str:
    """The benchmark's streaming probes (libzcprobe.so)."""
    cmd = command(out, sources=PROBE_SOURCES)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("--out", default=LIB)
    ap.add_argument("--no-probe", action="store_true", help="build libzipccl.so only")
    args = ap.parse_args(argv)
    build(args.out, args.save_temps, verbose=True)
    if not args.no_probe:
        build_probe(verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
