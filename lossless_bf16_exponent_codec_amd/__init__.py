"""Lossless BF16 exponent codec (ZipCCL's data-parallel hot path) for AMD MI355X.

The product is libzipccl.so (C ABI in include/zipccl.h, HIP kernels for gfx950);
`lossless_bf16_exponent_codec_amd.zipccl` is its ctypes binding.  `workloads` holds the
seeded synthetic inputs.  Importing the package itself loads nothing native.
"""

__all__ = ["zipccl", "workloads", "build"]
