"""The no-allocation compress (zipccl_compress_noalloc, workspace in the library's static
device array) against zipccl_compress with a caller workspace, byte for byte, through the
C ABI: two calls in a row, the second smaller, with and without a status word."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from lossless_bf16_exponent_codec_amd import workloads as W

pytestmark = pytest.mark.gpu

POISON = 0xAA


@pytest.fixture(scope="module")
def Z():
    from lossless_bf16_exponent_codec_amd import zipccl
    return zipccl


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def outputs(Z, segs):
    sizes = [s.size for s in segs]
    static = torch.full((sum(Z.static_size(n) for n in sizes),), POISON, dtype=torch.uint8, device="cuda")
    esc = torch.full((max(sum(sizes), 1),), POISON, dtype=torch.uint8, device="cuda")
    n_esc = torch.full((len(segs) + 1,), -1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    return static, esc, n_esc, status


def run_both(Z, segs, plans, with_status):
    tens = [dev(s) for s in segs]
    st_a, esc_a, ne_a, status_a = outputs(Z, segs)
    ws = torch.zeros(Z.workspace_size(sum(s.size for s in segs), len(segs)), dtype=torch.uint8, device="cuda")
    Z.compress(list(zip(tens, plans)), st_a, esc_a, ws, ne_a, status_a)
    st_b, esc_b, ne_b, status_b = outputs(Z, segs)
    Z.compress_noalloc(list(zip(tens, plans)), st_b, esc_b, ne_b, status_b if with_status else None)
    torch.cuda.synchronize()
    assert int(status_a.item()) == 0 and int(status_b.item()) == 0
    assert torch.equal(ne_a, ne_b)
    total = int(ne_a[-1].item())
    assert torch.equal(st_a, st_b)
    assert torch.equal(esc_a[:total], esc_b[:total])
    # and the oracle agrees
    st_o, esc_o, ne_o, _ = O.compress_batch(segs, [np.array(p.exponents, np.uint8) for p in plans])
    assert np.array_equal(st_b.cpu().numpy(), st_o)
    assert np.array_equal(esc_b.cpu().numpy()[:total], esc_o)


@pytest.mark.parametrize("with_status", [True, False])
def test_noalloc_matches_workspace_compress_twice(Z, with_status):
    # first call: 3 segments, 5.2 M values; second: 2 segments, 0.3 M values, so the
    # static array still holds the first call's ready words and staged escapes
    big = [W.gaussian_bf16(1 << 22, 0.02, 71), W.gaussian_bf16(1000003, 1e-3, 72), W.gaussian_bf16(4097, 3.0, 73)]
    small = [W.gaussian_bf16(300001, 0.5, 74), W.gaussian_bf16(513, 1.0, 75)]
    run_both(Z, big, [Z.plan(sigma=s) for s in (0.02, 1e-3, 3.0)], with_status)
    run_both(Z, small, [Z.plan(sigma=s) for s in (0.5, 1.0)], with_status)


def test_noalloc_at_its_maximum_size(Z):
    # exactly ZIPCCL_NOALLOC_MAX_VALUES values in 64 segments (the most units the array holds)
    n = Z.NOALLOC_MAX_VALUES
    sizes = [n // 64 - 7] * 63
    sizes.append(n - sum(sizes))
    segs = [W.gaussian_bf16(m, 1e-2, 80 + k) for k, m in enumerate(sizes)]
    run_both(Z, segs, [Z.plan(sigma=1e-2)] * 64, True)
