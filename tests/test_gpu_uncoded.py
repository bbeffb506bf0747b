"""GPU parity of uncoded blocks (the codec's fallback to no compression, block by block):
blocks whose escapes reach their overflow store exponents in their plane bytes and the
escape buffer.  Compressed bytes, escape bytes and decoded values against the oracle, on
every placement path, in decompress, decode-accumulate, gathered compress and shards."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from lossless_bf16_exponent_codec_amd import workloads as W
from tests.test_gpu_parity import (POISON16, check_against_oracle, dev_bf16, first_diff, gpu_accumulate,
                                   gpu_compress, gpu_compress_gather, gpu_decompress, host_u16, oracle_accumulate)
from tests.test_oracle_pins import coded_exhaustive_input, escape_stream, exhaustive_input

pytestmark = pytest.mark.gpu

TABLE = list(range(122, 129))          # the plan of sigma = 1
OUTSIDE = np.array([0, 5, 100, 121, 129, 140, 255], np.int64)


@pytest.fixture(scope="module")
def Z():
    from lossless_bf16_exponent_codec_amd import zipccl
    return zipccl


def blocks_with_escapes(counts, last=4096, seed=0):
    """Values block by block: block k has counts[k] values outside TABLE (at random
    positions), the rest inside; the last block has `last` values."""
    rng = np.random.default_rng(seed)
    parts = []
    for k, c in enumerate(counts):
        m = last if k == len(counts) - 1 else 4096
        c = min(c, m)
        e = np.asarray(TABLE, np.int64)[rng.integers(0, 7, m)]
        pos = rng.permutation(m)[:c]
        e[pos] = OUTSIDE[rng.integers(0, OUTSIDE.size, c)]
        x = (rng.integers(0, 2, m) << 15) | (e << 7) | rng.integers(0, 128, m)
        parts.append(x.astype(np.uint16))
    return np.concatenate(parts)


MIXES = [
    ([0, 2560, 2559, 4096, 1000, 3000], 4096),   # threshold both ways, full blocks
    ([4096, 4096, 4096], 1000),                  # last block: 1 full tile + 488 (overflow 320 + 296)
    ([2560, 0, 4096], 513),                      # last block 513 values: overflow 320
    ([4096, 0, 4096], 100),                      # last block within 192 values: never uncoded
    ([4096] * 9, 4096),                          # a whole unit and more, all uncoded
]


def mixed_segments(seed):
    return [blocks_with_escapes(c, last, seed + k) for k, (c, last) in enumerate(MIXES)]


def round_trip(Z, segs, plans):
    r = gpu_compress(Z, segs, plans)
    st, esc, ne = check_against_oracle(Z, segs, plans, r)
    outs, status = gpu_decompress(Z, r)
    assert status == 0
    for x, y in zip(segs, outs):
        assert np.array_equal(x, y), first_diff(x, y)
    return ne


def test_oracle_sees_both_modes():
    # the inputs above do hold coded and uncoded blocks, by the brute-force rule
    modes = [u for x in mixed_segments(1) for u in escape_stream(x, TABLE)[1]]
    assert any(modes) and not all(modes)


def test_mixed_blocks_single_launch(Z):
    segs = mixed_segments(1)
    round_trip(Z, segs, [Z.plan(sigma=1.0)] * len(segs))


@pytest.fixture
def two_launches(monkeypatch):
    monkeypatch.setenv("ZIPCCL_SINGLE_LAUNCH", "0")
    yield


@pytest.fixture
def scan_path(monkeypatch):
    monkeypatch.setenv("ZIPCCL_DIRECT_PREFIX_MAX_UNITS", "0")
    yield


def test_mixed_blocks_two_launches(Z, two_launches):
    segs = mixed_segments(2)
    round_trip(Z, segs, [Z.plan(sigma=1.0)] * len(segs))


def test_mixed_blocks_scan_path(Z, scan_path):
    segs = mixed_segments(3)
    round_trip(Z, segs, [Z.plan(sigma=1.0)] * len(segs))


def test_random_bits_do_not_expand(Z):
    # uniformly random BF16 patterns under a Gaussian plan: every full block uncoded, so
    # the compressed size is 2n plus header, offsets and padding
    for n in [4096 * 64, 4096 * 100 + 1234]:
        x = np.random.default_rng(n).integers(0, 1 << 16, n, dtype=np.int64).astype(np.uint16)
        ne = round_trip(Z, [x], [Z.plan(sigma=0.02)])
        assert Z.static_size(n) + ne[0] <= 2 * n + 128 + 128 * (-(-4 * (-(-n // 4096)) // 128)) + 512


@pytest.mark.parametrize("mode", ["uncoded", "coded"])
def test_exhaustive_patterns_both_modes(Z, mode):
    t = Z.plan(sigma=1.0)
    x = exhaustive_input() if mode == "uncoded" else coded_exhaustive_input(np.array(t.exponents, np.uint8))
    round_trip(Z, [x], [t])


@pytest.mark.parametrize("npeers", [3, 7, 16])
def test_accumulate_with_uncoded_peers(Z, npeers):
    # peers whose blocks are coded or uncoded in different places (random-bit peers and
    # mixed peers), so a workgroup meets every combination; the last block is partial
    print(f"accumulate uncoded P={npeers}", flush=True)
    n = 4096 * 9 + 1000
    rng = np.random.default_rng(npeers)
    peers = []
    for p in range(npeers):
        if p % 3 == 0:
            peers.append(rng.integers(0, 1 << 16, n, dtype=np.int64).astype(np.uint16))
        else:
            counts = rng.choice([0, 1000, 2559, 2560, 4096], 10)
            peers.append(blocks_with_escapes(list(counts), 1000, seed=100 * npeers + p))
    local = W.gaussian_bf16(n, 1.0, 7)
    plans = [Z.plan(sigma=1.0)] * npeers
    got, status, _ = gpu_accumulate(Z, peers, plans, local)
    assert status == 0
    want = oracle_accumulate(Z, peers, plans, local)
    assert np.array_equal(got, want), first_diff(got, want)


def test_accumulate_chunks_with_uncoded_peers(Z):
    # the reduce-scatter launch shape: 7 peers, several chunks per launch
    npeers, chunk, n = 7, 16384, 5 * 16384 + 4096
    rng = np.random.default_rng(77)
    peers = [blocks_with_escapes(list(rng.choice([0, 2560, 4096, 1500], -(-n // 4096))), 4096, seed=500 + p)
             for p in range(npeers)]
    local = W.gaussian_bf16(n, 1.0, 8)
    plans = [Z.plan(sigma=1.0)] * npeers
    sin, ein, eb, keep = [], [], [], []
    for c0 in range(0, n, chunk):
        segs = [p[c0:c0 + chunk] for p in peers]
        r = gpu_compress(Z, segs, plans)
        keep.append(r)
        S = Z.static_size(segs[0].size)
        for p in range(npeers):
            sin.append(r["static"].data_ptr() + p * S)
            ein.append(r["esc"].data_ptr())
            eb.append(r["esc"].numel())
    dst = torch.full((n,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.PreparedAccumulateChunks(sin, ein, npeers, chunk, n, dev_bf16(local), dst, status, esc_bytes=eb).run()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = host_u16(dst)
    want = oracle_accumulate(Z, peers, plans, local)
    assert np.array_equal(got, want), first_diff(got, want)


def test_gathered_rows_uncoded(Z):
    # random-bit token rows picked by index: the uncoded rewrite reloads gathered rows
    H, tokens = 1000, 300
    mat = np.random.default_rng(3).integers(0, 1 << 16, tokens * H, dtype=np.int64).astype(np.uint16)
    mat = mat.reshape(tokens, H)
    rng = np.random.default_rng(4)
    rows_list = [rng.permutation(tokens)[:90], np.sort(rng.permutation(tokens)[:41]), np.arange(7)]
    plans = [Z.plan(sigma=1.0)] * 3
    res = gpu_compress_gather(Z, mat, rows_list, plans)
    segs = [mat[idx].reshape(-1) for idx in rows_list]
    check_against_oracle(Z, segs, plans, res)
    outs, status = gpu_decompress(Z, res)
    assert status == 0
    for x, y in zip(segs, outs):
        assert np.array_equal(x, y), first_diff(x, y)


def test_shards_uncoded_escapes_at_first(Z):
    # a receiver of the two-phase all-to-all holds each sender's static part and that
    # segment's escape bytes on their own
    pre = blocks_with_escapes([4096, 100], 4096, seed=9)
    shard = blocks_with_escapes([2560, 0, 4096], 700, seed=10)
    pl = Z.plan(sigma=1.0)
    r = gpu_compress(Z, [pre, shard], [pl, pl])
    ne = r["n_esc"]
    esc_own = r["esc"][int(ne[0]):int(ne[0]) + int(ne[1])].clone()
    out = torch.full((shard.size,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.decompress_shards([r["static"].data_ptr() + Z.static_size(pre.size)], [esc_own], [out], status,
                        flags=Z.SHARDS_ESC_AT_FIRST)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(host_u16(out), shard)
