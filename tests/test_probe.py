"""The benchmark's streaming probes (libzcprobe.so): the library loads and exports its two
calls, the byte counts the benchmark divides by, argument checks on the host (no GPU
needed), and on the GPU that the copy, decode-accumulate-like and mix probes move the bytes
they claim."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "lossless_bf16_exponent_codec_amd", "libzcprobe.so")
COPY, READ, WRITE, MIX, ACC = 0, 1, 2, 3, 4
MiB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(PATH), "libzcprobe.so is built by python -m lossless_bf16_exponent_codec_amd.build"
    L = ctypes.CDLL(PATH)
    L.zcprobe_launch.restype = ctypes.c_int
    L.zcprobe_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    L.zcprobe_moved_bytes.restype = ctypes.c_uint64
    L.zcprobe_moved_bytes.argtypes = [ctypes.c_int, ctypes.c_uint64]
    return L


def test_moved_bytes(lib):
    G = 1 << 30
    assert lib.zcprobe_moved_bytes(COPY, G) == 2 * G
    assert lib.zcprobe_moved_bytes(READ, G) == G
    assert lib.zcprobe_moved_bytes(WRITE, G) == G
    assert lib.zcprobe_moved_bytes(MIX, G) == G // 2 + (G // 2) * 12 // 16   # half read, 12/16 of it written
    T = (G // (7 * 704 + 1024)) // 8 * 8                                      # tiles of 512 values
    assert lib.zcprobe_moved_bytes(ACC, G) == T * (7 * 704 + 2 * 1024)        # 7 peers' A + planes, local, out
    assert lib.zcprobe_moved_bytes(5, G) == 0


def test_bad_arguments_launch_nothing(lib):
    bad = 1   # hipErrorInvalidValue
    p = 1 << 20   # an aligned host-side stand-in: every call below is refused before any launch
    assert lib.zcprobe_launch(7, p, p, MiB, None) == bad          # no such probe
    assert lib.zcprobe_launch(COPY, p, p, MiB + 16, None) == bad  # not a multiple of 2^20
    assert lib.zcprobe_launch(COPY, p, p, 0, None) == bad
    assert lib.zcprobe_launch(COPY, p + 16, p, MiB, None) == bad  # not 256-byte aligned
    assert lib.zcprobe_launch(COPY, None, p, MiB, None) == bad    # nothing to read
    assert lib.zcprobe_launch(WRITE, p, None, MiB, None) == bad   # nothing to write


@pytest.mark.gpu
def test_copy_accumulate_and_mix_probes_move_their_bytes(lib):
    import torch
    n = 4 * MiB
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert lib.zcprobe_launch(COPY, src.data_ptr(), dst.data_ptr(), n, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    # the decode-accumulate-like probe: per tile, the xor of 7 peers' A words and plane
    # dwords goes into the first word of each lane's 16 local bytes
    dst.zero_()
    assert lib.zcprobe_launch(ACC, src.data_ptr(), dst.data_ptr(), n, s) == 0
    torch.cuda.synchronize()
    T = (n // (7 * 704 + 1024)) // 8 * 8
    h = src.cpu().numpy()
    lane = np.arange(64)
    c, q = lane & 31, lane & 3
    pdw = np.where(q < 3, 2 * (8 * q + (c >> 2)) + (lane >> 5), 0)
    acc = np.zeros((T, 64), np.uint32)
    for p in range(7):
        base = h[p * 704 * T:(p + 1) * 704 * T]
        A = base[:512 * T].view(np.uint32).reshape(T, 64, 2)
        planes = base[512 * T:].view(np.uint32).reshape(T, 48)
        acc ^= A[:, :, 0] ^ A[:, :, 1] ^ planes[:, pdw]
    local = h[7 * 704 * T:7 * 704 * T + 1024 * T].view(np.uint32).reshape(T, 64, 4).copy()
    local[:, :, 0] ^= acc
    got = dst.cpu().numpy()
    assert np.array_equal(got[:1024 * T].view(np.uint32).reshape(T, 64, 4), local)
    assert not got[1024 * T:].any()
    # the compress-like mix: per 16-byte lane of src's first half, its first 8 bytes to
    # dst's first section and the xor of its last two words to the second
    dst.zero_()
    assert lib.zcprobe_launch(MIX, src.data_ptr(), dst.data_ptr(), n, s) == 0
    torch.cuda.synchronize()
    lanes = src.cpu().numpy()[:n // 2].view(np.uint32).reshape(-1, 4)
    m = lanes.shape[0]
    got = dst.cpu().numpy()
    assert np.array_equal(got[:8 * m].view(np.uint32).reshape(-1, 2), lanes[:, :2])
    assert np.array_equal(got[8 * m:12 * m].view(np.uint32), lanes[:, 2] ^ lanes[:, 3])
    assert not got[12 * m:].any()
