"""The reduce-scatter share in the benchmark's launch shapes (up to 16 chunk calls per
compress launch, every chunk in one decode-accumulate launch) with peers of every kind a receiver
can meet: Gaussian shards under their own plan, random bits (uncoded blocks), an
activation-like shard with zeros, outliers and special values, an all-zero shard, a
shard coded under a plan for another scale, and a shard whose blocks alternate between
coded and uncoded.  The decoded sum is compared with the oracle's element by element,
and sampled chunks' compressed bytes with the oracle's byte by byte."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from lossless_bf16_exponent_codec_amd import workloads as W
from tests.test_gpu_parity import dev_bf16, first_diff, host_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    from lossless_bf16_exponent_codec_amd import zipccl
    return zipccl


def mixed_peers(n):
    rng = np.random.default_rng(2024)
    gauss = W.gaussian_bf16(n, 1e-3, 900)
    bits = rng.integers(0, 1 << 16, n, dtype=np.int64).astype(np.uint16)
    act = W.act_8192x7168(rows=-(-n // 7168), seed=901).segments[0][:n]
    zeros = np.zeros(n, np.uint16)
    wrong = W.gaussian_bf16(n, 1e-3, 902)
    g02 = W.gaussian_bf16(n, 0.02, 903)
    alt = W.gaussian_bf16(n, 1e-3, 904)
    blocks = alt.reshape(-1, 4096)
    blocks[1::3] = rng.integers(0, 1 << 16, blocks[1::3].shape, dtype=np.int64).astype(np.uint16)
    peers = [gauss, bits, act, zeros, wrong, g02, alt]
    sigmas = [1e-3, 1e-3, 1.0, 1e-3, 1.0, 0.02, 1e-3]   # wrong: coded under sigma 1
    return peers, sigmas


def test_mixed_peers_in_benchmark_launch_shapes(Z):
    P, chunk, nch = 7, 1 << 21, 12
    n = chunk * nch
    print(f"mixed share P={P} chunks={nch}", flush=True)
    peers_h, sigmas = mixed_peers(n)
    local_h = W.gaussian_bf16(n, 1e-3, 905)
    plans = [Z.plan(sigma=s) for s in sigmas]
    peers = [dev_bf16(x) for x in peers_h]
    local = dev_bf16(local_h)
    S = Z.static_size(chunk)
    static = torch.full((nch * P * S,), 0xAA, dtype=torch.uint8, device="cuda")
    esc = torch.full((nch * P * chunk,), 0xAA, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(Z.workspace_size(16 * P * chunk, 16 * P), dtype=torch.uint8, device="cuda")
    n_esc = torch.full((nch, P + 1), -1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.PreparedCompressChunks([[p[c * chunk:(c + 1) * chunk] for p in peers] for c in range(nch)],
                             [static[c * P * S:(c + 1) * P * S] for c in range(nch)],
                             [esc[c * P * chunk:(c + 1) * P * chunk] for c in range(nch)], ws,
                             n_esc.view(-1), status).run(plans)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    tables = [np.array(p.exponents, np.uint8) for p in plans]
    # chunks at the launch's start, in its middle and at its end, byte for byte
    for c in (0, 7, 11):
        segs = [x[c * chunk:(c + 1) * chunk] for x in peers_h]
        st, e, ne, rc = O.compress_batch(segs, tables)
        got_st = static[c * P * S:(c + 1) * P * S].cpu().numpy()
        assert np.array_equal(got_st, st), f"chunk {c}: " + first_diff(got_st, st)
        assert list(n_esc[c].cpu().numpy()[:P]) == ne
        assert np.array_equal(esc[c * P * chunk:c * P * chunk + sum(ne)].cpu().numpy(), e), f"chunk {c}"
    out = torch.full((n,), -21846, dtype=torch.int16, device="cuda").view(torch.bfloat16)   # 0xAAAA
    Z.PreparedAccumulateChunks([static.data_ptr() + (c * P + p) * S for c in range(nch) for p in range(P)],
                               [esc.data_ptr() + c * P * chunk for c in range(nch) for _ in range(P)],
                               P, chunk, n, local, out, status, esc_bytes=[P * chunk] * (P * nch)).run()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    comp = [O.compress(x, t) for x, t in zip(peers_h, tables)]
    want = O.decompress_accumulate([c[0] for c in comp], [c[1] for c in comp], n, local_h)
    got = host_u16(out)
    assert np.array_equal(got, want), first_diff(got, want)
