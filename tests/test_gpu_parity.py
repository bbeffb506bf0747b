"""GPU parity: the HIP path through the C ABI against the CPU oracle, byte for byte.

Compressed static bytes, escape bytes, per-segment escape counts and decoded tensors
must be identical to the oracle's on the same seeded inputs; decode-accumulate is
bit-exact too.  Outputs are pre-filled with 0xAA so that an unwritten byte shows.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from lossless_bf16_exponent_codec_amd import workloads as W

pytestmark = pytest.mark.gpu

POISON = 0xAA
POISON16 = 0xAAAA - 0x10000      # the 0xAAAA pattern as int16


@pytest.fixture(scope="module")
def Z():
    from lossless_bf16_exponent_codec_amd import zipccl
    return zipccl


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_compress(Z, segs, plans, esc_cap=None, workspace=None, poison=True, with_status=True):
    tens = [dev_bf16(s) for s in segs]
    sizes = [s.size for s in segs]
    total_static = sum(Z.static_size(n) for n in sizes)
    static = torch.full((max(total_static, 1),), POISON, dtype=torch.uint8, device="cuda")
    cap = sum(sizes) if esc_cap is None else esc_cap
    esc = torch.full((max(cap, 1),), POISON, dtype=torch.uint8, device="cuda")
    n_esc = torch.full((len(segs) + 1,), -1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if workspace is None:
        workspace = torch.zeros(Z.workspace_size(sum(sizes), len(segs)), dtype=torch.uint8, device="cuda")
    Z.compress(list(zip(tens, plans)), static, esc, workspace, n_esc, status if with_status else None, esc_cap=cap)
    torch.cuda.synchronize()
    ne = n_esc.cpu().numpy()
    return dict(static=static, esc=esc, n_esc=ne, status=int(status.item()), sizes=sizes,
                static_h=static.cpu().numpy()[:total_static], esc_h=esc.cpu().numpy())


def oracle_tables(plans):
    return [np.array(p.exponents, np.uint8) for p in plans]


def check_against_oracle(Z, segs, plans, r):
    st, esc, ne, rc = O.compress_batch(segs, oracle_tables(plans))
    assert r["status"] == 0
    assert list(r["n_esc"][:-1]) == ne
    assert int(r["n_esc"][-1]) == sum(ne)
    assert np.array_equal(r["static_h"], st), first_diff(r["static_h"], st)
    assert np.array_equal(r["esc_h"][:sum(ne)], esc)
    return st, esc, ne


def first_diff(a, b):
    if a.shape != b.shape:
        return f"shape {a.shape} vs {b.shape}"
    d = np.nonzero(a != b)[0]
    return f"{d.size} bytes differ, first at {d[0]}: {a[d[0]]:#x} vs {b[d[0]]:#x}" if d.size else "equal"


def gpu_decompress(Z, r, poison=True):
    outs = [torch.full((n,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            for n in r["sizes"]]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.decompress(r["static"], r["esc"], outs, status)
    torch.cuda.synchronize()
    return [host_u16(o) for o in outs], int(status.item())


def round_trip(Z, segs, plans):
    r = gpu_compress(Z, segs, plans)
    check_against_oracle(Z, segs, plans, r)
    outs, status = gpu_decompress(Z, r)
    assert status == 0
    for x, y in zip(segs, outs):
        assert np.array_equal(x, y), first_diff(x, y)
    return r


# ------------------------------------------------------------------------------------
def test_worked_example(Z):
    x = np.array([0x3F80, 0xBF00, 0x4040, 0x0000, 0x42C8, 0x7FC0, 0x3D00, 0x3C80], np.uint16)
    r = round_trip(Z, [x], [Z.plan(sigma=1.0)])
    assert r["static_h"].size == 1024 and list(r["esc_h"][:4]) == [0x00, 0x85, 0xFF, 0x79]


@pytest.mark.parametrize("n", [0, 1, 7, 8, 63, 64, 511, 512, 513, 4095, 4096, 4097, 16383, 16384, 16385,
                               65536 + 7, 100003])
def test_edge_sizes_random_bits(Z, n):
    rng = np.random.default_rng(1000 + n)
    x = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
    round_trip(Z, [x], [Z.plan(sigma=0.02)])


@pytest.mark.parametrize("n", [1, 513, 4097, 16385, 250001])
def test_edge_sizes_gaussian(Z, n):
    round_trip(Z, [W.gaussian_bf16(n, 0.7, n)], [Z.plan(sigma=0.7)])


def test_exhaustive_patterns(Z):
    all16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = np.concatenate([np.roll(all16, s) for s in range(8)] + [all16[:517]])
    plans = [Z.plan(sigma=1.0), Z.plan(table=[1, 2, 3, 4, 5, 6, 7]), Z.plan(table=[248, 249, 250, 251, 252, 253, 254]),
             Z.plan(table=[3, 77, 120, 128, 129, 200, 254])]
    for p in plans:
        round_trip(Z, [x], [p])
    # all four in one launch
    round_trip(Z, [x, x[:70000], x[5:], x[:1]], plans)


def test_no_escapes_and_all_escapes(Z):
    p = Z.plan(sigma=1.0)
    t = p.exponents
    x = np.array([(e << 7) | (s << 15) | m for e in t for s in (0, 1) for m in (0, 5, 127)] * 3000, np.uint16)
    r = round_trip(Z, [x], [p])
    assert int(r["n_esc"][0]) == 0
    r = round_trip(Z, [x], [Z.plan(table=[1, 2, 3, 4, 5, 6, 7])])
    # every value escapes: the full blocks are uncoded (2560 escape-buffer bytes each),
    # the last (3120 values: 6 full tiles and one of 48) too (6 x 320)
    assert int(r["n_esc"][0]) == 30 * 2560 + 6 * 320


def test_many_segments_one_launch(Z):
    rng = np.random.default_rng(5)
    segs, plans = [], []
    for k in range(64):
        n = int(rng.choice([0, 1, 700, 4096, 16384, 20000, 70001]))
        s = float(10 ** rng.uniform(-4, 1))
        segs.append(W.gaussian_bf16(n, s, 300 + k))
        plans.append(Z.plan(sigma=s))
    round_trip(Z, segs, plans)


@pytest.mark.parametrize("sizes", [[0, 0, 5000], [5000, 0, 0], [4096, 0, 4097], [0] * 63 + [20000],
                                   [20000] + [0] * 63, [1, 0, 0, 1, 0, 16385, 0, 0], [0, 16384, 0, 0, 700]])
def test_empty_segments_around_data(Z, sizes):
    # segments with no units share their first unit with the next one: each workgroup must
    # still find the segment that holds its unit, with empty runs before, between and after
    segs = [W.gaussian_bf16(n, 0.05, 700 + k) if n else np.zeros(0, np.uint16) for k, n in enumerate(sizes)]
    round_trip(Z, segs, [Z.plan(sigma=0.05)] * len(segs))


@pytest.mark.parametrize("seed", range(6))
def test_random_segments_random_tables(Z, seed):
    # random bit patterns (mostly escapes) and random explicit tables, up to 64 segments
    # of random sizes in one launch
    rng = np.random.default_rng(1000 + seed)
    nseg = int(rng.integers(1, 65))
    segs, plans = [], []
    for _ in range(nseg):
        n = int(rng.choice([0, 1, 8, 511, 4097, int(rng.integers(0, 40000))]))
        segs.append(rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16))
        plans.append(Z.plan(table=sorted(int(v) for v in rng.choice(np.arange(1, 255), 7, replace=False))))
    print(f"random segments seed={seed} nseg={nseg} n={sum(x.size for x in segs)}", flush=True)
    round_trip(Z, segs, plans)


def test_determinism_and_workspace_reuse(Z):
    # the workspace needs no initialisation and carries nothing between calls: start
    # from garbage and alternate two different batches through one workspace
    ws = torch.full((Z.workspace_size(1 << 22, 64),), 0xAB, dtype=torch.uint8, device="cuda")
    x1 = [W.gaussian_bf16(1 << 20, 0.02, 1)]
    x2 = [W.gaussian_bf16(n, 1e-3, 7 + n) for n in (1000, 300000, 0, 77777)]
    p1 = [Z.plan(sigma=0.02)]
    p2 = [Z.plan(sigma=1e-3)] * 4
    first = None
    for rep in range(6):
        segs, plans = (x1, p1) if rep % 2 == 0 else (x2, p2)
        r = gpu_compress(Z, segs, plans, workspace=ws)
        check_against_oracle(Z, segs, plans, r)
        if rep == 0:
            first = r["static_h"].copy()
        elif rep % 2 == 0:
            assert np.array_equal(first, r["static_h"])


def test_prepared_calls_match_plain_calls(Z):
    # the marshalled-once call objects give the same bytes as the plain calls
    segs = [W.gaussian_bf16(n, s, 300 + k) for k, (n, s) in enumerate([(70001, 0.02), (0, 1.0), (4096, 3e-3)])]
    sig = [0.02, 1.0, 3e-3]
    r = gpu_compress(Z, segs, list(Z.plan_many(sig)))
    check_against_oracle(Z, segs, list(Z.plan_many(sig)), r)
    tens = [dev_bf16(x) for x in segs]
    static = torch.full_like(r["static"], POISON)
    esc = torch.full_like(r["esc"], POISON)
    n_esc = torch.full((len(segs) + 1,), -1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(Z.workspace_size(sum(x.size for x in segs), len(segs)), dtype=torch.uint8, device="cuda")
    pc = Z.PreparedCompress(tens, static, esc, ws, n_esc, status)
    for _ in range(2):
        pc.run(Z.plan_many(sig))
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and list(n_esc.cpu().numpy()) == list(r["n_esc"])
    assert torch.equal(static, r["static"]) and torch.equal(esc[:int(r["n_esc"][-1])], r["esc"][:int(r["n_esc"][-1])])
    outs = [torch.full((x.size,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16) for x in segs]
    Z.PreparedDecompress(static, esc, outs, status).run()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for x, o in zip(segs, outs):
        assert np.array_equal(x, host_u16(o))
    # accumulate: three 9000-value peers against the plain call
    n = 9000
    peers = [W.gaussian_bf16(n, 0.1, 40 + p) for p in range(3)]
    local = W.gaussian_bf16(n, 0.1, 50)
    plans = [Z.plan(sigma=0.1)] * 3
    want, st_plain, rr = gpu_accumulate(Z, peers, plans, local)
    S = Z.static_size(n)
    dst = torch.full((n,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    base = rr["static"].data_ptr()
    Z.PreparedAccumulate([base + p * S for p in range(3)], [rr["esc"].data_ptr()] * 3, n, dev_bf16(local), dst,
                         status, esc_bytes=[rr["esc"].numel()] * 3).run()
    torch.cuda.synchronize()
    assert st_plain == 0 and int(status.item()) == 0 and np.array_equal(host_u16(dst), want)


def test_all_empty_and_boundary_segments(Z):
    # empty segments first, between blocks and at the end; a segment of exactly 256
    # blocks puts the following ones on a finalize-workgroup boundary
    sizes = [0, 0, 256 * 4096, 0, 5, 0, 4096 * 300 + 17, 0, 0]
    segs = [W.gaussian_bf16(n, 0.05, 70 + k) for k, n in enumerate(sizes)]
    round_trip(Z, segs, [Z.plan(sigma=0.05)] * len(segs))
    r = round_trip(Z, [np.zeros(0, np.uint16)] * 3, [Z.plan(sigma=1.0)] * 3)
    assert r["static_h"].size == 3 * 128 and list(r["n_esc"]) == [0, 0, 0, 0]


def test_escape_overflow_sets_status(Z):
    x = W.gaussian_bf16(50000, 1.0, 5)
    p = Z.plan(table=[1, 2, 3, 4, 5, 6, 7])
    r = gpu_compress(Z, [x], [p], esc_cap=1000)
    assert r["status"] & Z.STATUS_ESC_OVERFLOW
    st, esc, ne, rc = O.compress_batch([x], oracle_tables([p]))
    assert int(r["n_esc"][0]) == ne[0] and np.array_equal(r["static_h"], st)
    assert np.array_equal(r["esc_h"][:1000], esc[:1000])


def test_corrupt_header_is_reported_and_not_decoded(Z):
    x = W.gaussian_bf16(20000, 0.5, 8)
    r = gpu_compress(Z, [x], [Z.plan(sigma=0.5)])
    r["static"][0] ^= 1
    outs, status = gpu_decompress(Z, r)
    assert status & Z.STATUS_CORRUPT
    assert (outs[0] == POISON * 257).all()
    r["static"][0] ^= 1
    # escape buffer too small for the header's escape range
    outs = [torch.zeros(20000, dtype=torch.bfloat16, device="cuda")]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.decompress(r["static"], r["esc"], outs, status, esc_bytes=int(r["n_esc"][0]) - 1)
    torch.cuda.synchronize()
    assert int(status.item()) & Z.STATUS_CORRUPT


# ------------------------------------------------------------------------------------
# decode-accumulate
# ------------------------------------------------------------------------------------
def gpu_accumulate(Z, peer_bits, plans, local_bits, inplace=False):
    n = local_bits.size
    r = gpu_compress(Z, peer_bits, plans)
    S = Z.static_size(n)
    base = r["static"].data_ptr()
    ins = [base + p * S for p in range(len(peer_bits))]
    ebase = r["esc"].data_ptr()
    local = dev_bf16(local_bits)
    dst = local if inplace else torch.full((n,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.decompress_accumulate(ins, [ebase] * len(ins), n, local, dst, status,
                            esc_bytes=[r["esc"].numel()] * len(ins))
    torch.cuda.synchronize()
    return host_u16(dst), int(status.item()), r


def oracle_accumulate(Z, peer_bits, plans, local_bits):
    comp = [O.compress(p, np.array(pl.exponents, np.uint8)) for p, pl in zip(peer_bits, plans)]
    return O.decompress_accumulate([c[0] for c in comp], [c[1] for c in comp], local_bits.size, local_bits)


@pytest.mark.parametrize("n,npeers", [(1, 1), (4097, 7), (16385, 3), (100000, 7), (262144, 16), (70001, 2),
                                     (50000, 4), (33333, 5), (20000, 6), (8192, 8), (9000, 9)])
def test_accumulate_matches_oracle(Z, n, npeers):
    peers = [W.gaussian_bf16(n, 1e-3, 500 + p) for p in range(npeers)]
    local = W.gaussian_bf16(n, 1e-3, 600)
    plans = [Z.plan(sigma=1e-3)] * npeers
    got, status, _ = gpu_accumulate(Z, peers, plans, local)
    assert status == 0
    want = oracle_accumulate(Z, peers, plans, local)
    assert np.array_equal(got, want), first_diff(got, want)


def test_accumulate_in_place(Z):
    n = 50000
    peers = [W.gaussian_bf16(n, 0.3, 20 + p) for p in range(7)]
    local = W.gaussian_bf16(n, 0.3, 30)
    plans = [Z.plan(sigma=0.3)] * 7
    got, status, _ = gpu_accumulate(Z, peers, plans, local, inplace=True)
    assert status == 0 and np.array_equal(got, oracle_accumulate(Z, peers, plans, local))


def test_accumulate_special_values(Z):
    # subnormals (no flush), signed zeros, infinities, NaNs, overflow and exact ties
    rng = np.random.default_rng(9)
    n = 3 * 4096 + 99
    specials = np.array([0x0001, 0x8001, 0x007F, 0x8000, 0x0000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F7F,
                         0xFF7F, 0x3F80, 0x3B80, 0x3F81, 0x0080, 0x8080], np.uint16)
    peers = [specials[rng.integers(0, specials.size, n)] for _ in range(5)]
    local = specials[rng.integers(0, specials.size, n)]
    plans = [Z.plan(sigma=1.0), Z.plan(table=[1, 2, 3, 4, 5, 6, 7]), Z.plan(sigma=1e-38),
             Z.plan(table=[120, 121, 122, 123, 124, 125, 127]), Z.plan(sigma=1e30)]
    got, status, _ = gpu_accumulate(Z, peers, plans, local)
    assert status == 0
    want = oracle_accumulate(Z, peers, plans, local)
    assert np.array_equal(got, want), first_diff(got, want)
    two = np.array([0x0001] * 8, np.uint16)
    got, _, _ = gpu_accumulate(Z, [two], [Z.plan(sigma=1.0)], two)
    assert (got == 0x0002).all()


@pytest.mark.parametrize("npeers,band", [(3, False), (7, False), (2, True), (7, True)])
def test_accumulate_random_bits_and_ties(Z, npeers, band):
    # the one rounding of the fp32 sum, bit for bit: uniformly random BF16 patterns (NaN
    # payloads of both signs, subnormals, infinities: NaN -> 0x7FC0 by the rule), or values
    # from a narrow exponent band, where sums of few terms often fall exactly on a tie
    rng = np.random.default_rng(40 + npeers + 10 * band)
    n = 200000 + 77

    def draw():
        if not band:
            return rng.integers(0, 1 << 16, n, dtype=np.int64).astype(np.uint16)
        e = rng.integers(124, 128, n)
        return ((rng.integers(0, 2, n) << 15) | (e << 7) | rng.integers(0, 128, n)).astype(np.uint16)

    peers = [draw() for _ in range(npeers)]
    local = draw()
    plans = [Z.plan(sigma=1.0)] * npeers
    got, status, _ = gpu_accumulate(Z, peers, plans, local)
    assert status == 0
    want = oracle_accumulate(Z, peers, plans, local)
    assert np.array_equal(got, want), first_diff(got, want)


def test_accumulate_corrupt_peer(Z):
    n = 9000
    peers = [W.gaussian_bf16(n, 0.1, 40 + p) for p in range(3)]
    local = W.gaussian_bf16(n, 0.1, 50)
    plans = [Z.plan(sigma=0.1)] * 3
    r = gpu_compress(Z, peers, plans)
    S = Z.static_size(n)
    r["static"][S + 8] ^= 4      # peer 1 header: n
    dst = torch.full((n,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    base = r["static"].data_ptr()
    Z.decompress_accumulate([base + p * S for p in range(3)], [r["esc"].data_ptr()] * 3, n, dev_bf16(local), dst,
                            status, esc_bytes=[r["esc"].numel()] * 3)
    torch.cuda.synchronize()
    assert int(status.item()) & Z.STATUS_CORRUPT


def accumulate_chunks_setup(Z, npeers, chunk, n, seed):
    peers = [W.gaussian_bf16(n, 1e-3, seed + p) for p in range(npeers)]
    local = W.gaussian_bf16(n, 1e-3, seed + 99)
    plans = [Z.plan(sigma=1e-3)] * npeers
    comps, sin, ein, eb = [], [], [], []
    for c0 in range(0, n, chunk):
        segs = [p[c0:c0 + chunk] for p in peers]
        r = gpu_compress(Z, segs, plans)
        comps.append(r)
        S = Z.static_size(segs[0].size)
        for p in range(npeers):
            sin.append(r["static"].data_ptr() + p * S)
            ein.append(r["esc"].data_ptr())
            eb.append(r["esc"].numel())
    return peers, local, plans, comps, sin, ein, eb


@pytest.mark.parametrize("npeers,chunk,n", [(3, 8192, 5 * 8192 + 1000),   # ragged last chunk
                                             (16, 4096, 17 * 4096 + 1000),  # 16 chunks per launch: two launches
                                             (7, 1 << 20, (1 << 20) + 4096)])
def test_accumulate_chunks_matches_oracle(Z, npeers, chunk, n):
    print(f"accumulate chunks P={npeers} chunk={chunk} n={n}", flush=True)
    peers, local, plans, comps, sin, ein, eb = accumulate_chunks_setup(Z, npeers, chunk, n, 1300)
    dst = torch.full((n,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.PreparedAccumulateChunks(sin, ein, npeers, chunk, n, dev_bf16(local), dst, status, esc_bytes=eb).run()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = host_u16(dst)
    want = oracle_accumulate(Z, peers, plans, local)
    assert np.array_equal(got, want), first_diff(got, want)


def test_accumulate_chunks_corrupt_chunk(Z):
    npeers, chunk, n = 2, 8192, 4 * 8192
    peers, local, plans, comps, sin, ein, eb = accumulate_chunks_setup(Z, npeers, chunk, n, 1400)
    comps[2]["static"][Z.static_size(chunk) + 8] ^= 4   # chunk 2, peer 1: header n
    dst = torch.full((n,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.PreparedAccumulateChunks(sin, ein, npeers, chunk, n, dev_bf16(local), dst, status, esc_bytes=eb).run()
    torch.cuda.synchronize()
    assert int(status.item()) & Z.STATUS_CORRUPT
    got = host_u16(dst)
    want = oracle_accumulate(Z, peers, plans, local)
    want[2 * chunk:3 * chunk] = 0xAAAA
    assert np.array_equal(got, want), first_diff(got, want)


@pytest.mark.parametrize("npeers,chunk,n", [(2, 4096, 40 * 4096 + 100),   # 3 hand-offs of 16 chunks: the ring wraps
                                             (3, 8192, 5 * 8192),          # fewer chunks than one hand-off
                                             (16, 1 << 20, (2 << 20) + 4097)])   # hand-offs of 2, ragged last chunk
def test_pipeline_matches_oracle(Z, npeers, chunk, n):
    print(f"pipeline P={npeers} chunk={chunk} n={n}", flush=True)
    peers = [W.gaussian_bf16(n, 1e-3, 700 + p) for p in range(npeers)]
    local = W.gaussian_bf16(n, 1e-3, 800)
    plans = [Z.plan(sigma=1e-3)] * npeers
    want = oracle_accumulate(Z, peers, plans, local)
    peer_t = [dev_bf16(p) for p in peers]
    local_t = dev_bf16(local)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    pipe = Z.Pipeline(npeers, chunk, sa, sb)
    for _ in range(2):   # the second call reuses the first call's events and slots
        dst = torch.full((n,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        sb.wait_stream(torch.cuda.current_stream())
        pipe.reduce(peer_t, plans, local_t, dst, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        got = host_u16(dst)
        assert np.array_equal(got, want), first_diff(got, want)
    pipe.close()


def test_decompress_shards_gathers_separate_buffers(Z):
    # shards compressed one call each (as every rank of an all-gather would), plus one
    # that is the second segment of a two-segment call, so that its escapes start past
    # the first segment's in its escape buffer; all decoded in one launch into slices of
    # one gathered tensor
    sizes = [4096 * 5 + 17, 0, 1, 70000, 16384 * 3]
    sigmas = [0.02, 1.0, 0.5, 1e-3, 3.0]
    shards = [W.gaussian_bf16(n, s, 900 + k) for k, (n, s) in enumerate(zip(sizes, sigmas))]
    comp = [gpu_compress(Z, [b], [Z.plan(sigma=s)]) for b, s in zip(shards, sigmas)]
    pre, extra = W.gaussian_bf16(5000, 0.1, 951), W.gaussian_bf16(9000, 0.1, 950)
    pl = Z.plan(sigma=0.1)
    r2 = gpu_compress(Z, [pre, extra], [pl, pl])
    assert r2["n_esc"][0] > 0
    static_ins = [c["static"] for c in comp] + [r2["static"].data_ptr() + Z.static_size(pre.size)]
    esc_ins = [c["esc"] for c in comp] + [r2["esc"]]
    ns = sizes + [extra.size]
    offs = [0]   # slices start 16-byte aligned; the gaps between them must stay untouched
    for m in ns[:-1]:
        offs.append((offs[-1] + m + 7) // 8 * 8)
    out = torch.full((offs[-1] + ns[-1],), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dsts = [out[o:o + m] for o, m in zip(offs, ns)]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.decompress_shards(static_ins, esc_ins, dsts, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    want = np.full(out.numel(), 0xAAAA, np.uint16)
    for o, b in zip(offs, shards + [extra]):
        want[o:o + b.size] = b
    got = host_u16(out)
    assert np.array_equal(got, want), first_diff(got, want)
    # a shard with a bad header is reported and left unwritten; the others decode
    comp[3]["static"][8] ^= 4    # n
    out.view(torch.int16).fill_(POISON16)
    status.zero_()
    Z.decompress_shards(static_ins, esc_ins, dsts, status)
    torch.cuda.synchronize()
    assert int(status.item()) & Z.STATUS_CORRUPT
    got = host_u16(out)
    want[offs[3]:offs[3] + ns[3]] = 0xAAAA
    assert np.array_equal(got, want), first_diff(got, want)


def test_two_phase_all_to_all_on_one_gpu(Z):
    # S senders each compress their tokens for D destinations in one gathered launch.
    # Destination r receives, from every sender, that segment's static part (phase 1:
    # fixed size, known from n alone) and its escape bytes (phase 2: esc_offset ..
    # esc_offset + n_esc of the sender's escape buffer), each into a buffer of its own;
    # device-to-device copies stand in for the transfers.  It decodes the S shards in one
    # launch with the escape buffers starting at each shard's first escape.
    S, D, H = 3, 4, 1024
    rng = np.random.default_rng(77)
    mats, routes, comps = [], [], []
    for s in range(S):
        tokens = int(rng.integers(200, 400))
        mat = W.gaussian_bf16(tokens * H, 0.5, 2000 + s).reshape(tokens, H)
        dest = rng.integers(0, D, tokens)
        rows = [np.flatnonzero(dest == d) for d in range(D)]
        mats.append(mat)
        routes.append(rows)
        comps.append(gpu_compress_gather(Z, mat, rows, [Z.plan(sigma=0.5)] * D))
    for r in range(D):
        recv_st, recv_esc, n_escs, dsts, want = [], [], [], [], []
        for s in range(S):
            c = comps[s]
            n = len(routes[s][r]) * H
            off_st = sum(Z.static_size(m) for m in c["sizes"][:r])
            off_esc = int(sum(c["n_esc"][:r]))
            k = int(c["n_esc"][r])
            recv_st.append(c["static"][off_st:off_st + Z.static_size(n)].clone())
            recv_esc.append(c["esc"][off_esc:off_esc + max(k, 1)].clone())
            n_escs.append(k)
            dsts.append(torch.full((n,), POISON16, dtype=torch.int16, device="cuda").view(torch.bfloat16))
            want.append(mats[s][routes[s][r]].reshape(-1))
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        Z.decompress_shards(recv_st, recv_esc, dsts, status, esc_bytes=n_escs, flags=Z.SHARDS_ESC_AT_FIRST)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        for got_t, w in zip(dsts, want):
            got = host_u16(got_t)
            assert np.array_equal(got, w), first_diff(got, w)
        # the same shards without the flag: their headers point past the received bytes
        if r > 0:
            status.zero_()
            Z.decompress_shards(recv_st, recv_esc, dsts, status, esc_bytes=n_escs)
            torch.cuda.synchronize()
            assert int(status.item()) & Z.STATUS_CORRUPT


# ------------------------------------------------------------------------------------
# compress of rows gathered by index (MoE dispatch without a permute copy)
# ------------------------------------------------------------------------------------
def gpu_compress_gather(Z, matrix_bits, rows_list, plans):
    """Compresses matrix rows picked by each int32 index array; returns what
    gpu_compress returns (sizes = values per segment)."""
    H = matrix_bits.shape[1]
    mat = dev_bf16(matrix_bits.reshape(-1)).view(matrix_bits.shape[0], H)
    rows_t = [torch.from_numpy(np.ascontiguousarray(r, np.int32)).cuda() for r in rows_list]
    sizes = [len(r) * H for r in rows_list]
    total_static = sum(Z.static_size(n) for n in sizes)
    static = torch.full((max(total_static, 1),), POISON, dtype=torch.uint8, device="cuda")
    esc = torch.full((max(sum(sizes), 1),), POISON, dtype=torch.uint8, device="cuda")
    n_esc = torch.full((len(sizes) + 1,), -1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(Z.workspace_size(sum(sizes), len(sizes)), dtype=torch.uint8, device="cuda")
    Z.compress_gather(list(zip([mat] * len(rows_t), rows_t, plans)), static, esc, ws, n_esc, status)
    torch.cuda.synchronize()
    return dict(static=static, esc=esc, n_esc=n_esc.cpu().numpy(), status=int(status.item()), sizes=sizes,
                static_h=static.cpu().numpy()[:total_static], esc_h=esc.cpu().numpy())


@pytest.mark.parametrize("tokens,H", [(1200, 7168), (700, 1000), (900, 512)])
def test_compress_gather_matches_oracle(Z, tokens, H):
    # a routed dispatch: tokens go to 8 destinations with Zipf(1.2) counts; bucket 0 keeps
    # the router's (random) order, the others ascending; one bucket also repeats a row
    print(f"gather tokens={tokens} H={H}", flush=True)
    mat = W.gaussian_bf16(tokens * H, 0.5, 70 + H).reshape(tokens, H)
    rng = np.random.default_rng(H)
    perm = rng.permutation(tokens)
    counts = W.zipf_counts(tokens, 8, 1.2)
    rows_list, r = [], 0
    for b, c in enumerate(counts):
        idx = perm[r:r + c]
        rows_list.append(idx if b == 0 else np.sort(idx))
        r += c
    rows_list[3] = np.concatenate([rows_list[3], rows_list[3][:5]])
    rows_list.append(np.zeros(0, np.int64))          # a destination that gets no tokens
    plans = [Z.plan(sigma=0.5)] * 8 + [Z.plan(sigma=1.0)]
    res = gpu_compress_gather(Z, mat, rows_list, plans)
    segs = [mat[idx].reshape(-1) for idx in rows_list]
    check_against_oracle(Z, segs, plans, res)
    outs, status = gpu_decompress(Z, res)
    assert status == 0
    for x, y in zip(segs, outs):
        assert np.array_equal(x, y), first_diff(x, y)


def test_compress_gather_bad_index(Z):
    tokens, H = 64, 1024
    mat = W.gaussian_bf16(tokens * H, 0.5, 77).reshape(tokens, H)
    rows = np.array([5, 63, 64, -1, 7, 2**31 - 1, 0, 9], np.int64)
    res = gpu_compress_gather(Z, mat, [rows], [Z.plan(sigma=0.5)])
    assert res["status"] & Z.STATUS_BAD_INDEX
    used = np.where((rows >= 0) & (rows < tokens), rows, 0)   # row 0 is read in their place
    check_against_oracle(Z, [mat[used].reshape(-1)], [Z.plan(sigma=0.5)], dict(res, status=0))


def test_profile_codec(Z):
    # the switcher's start-up profile: positive rates, and the compressed fraction is the
    # oracle's compressed size over the BF16 bytes, exactly
    n, P = 1 << 21, 7
    x = W.gaussian_bf16(n, 1e-3, 42)
    pl = Z.plan(sigma=1e-3)
    prof = Z.profile_codec(dev_bf16(x), pl, P)
    assert prof.compress_GBps > 50 and prof.accumulate_GBps > 50
    st, esc, k = O.compress(x, np.array(pl.exponents, np.uint8))
    assert abs(prof.compressed_fraction - (st.size + k) / (2 * n)) < 1e-12
    use, tn, tz = Z.rs_choose(prof, Z.LinkT(25.0, 5.0, 1), 8, 1 << 30)
    assert tn > 0 and tz > 0


def test_estimate_plans_64_segments(Z):
    # the most segments one call takes: every part of every segment and every lane of the
    # finishing launch in use, sizes from empty to several parts' worth of sampled tiles
    import math
    rng = np.random.default_rng(77)
    segs, sig = [], []
    for k in range(64):
        n = int(rng.choice([0, 3, 512, 4097, 70000, 300001]))
        s = float(10 ** rng.uniform(-6, 2))
        segs.append(W.gaussian_bf16(n, s, 900 + k) if n else np.zeros(0, np.uint16))
        sig.append(s)
    tens = [dev_bf16(x) for x in segs]
    plans_dev = torch.full((8 * 64,), 0xAA, dtype=torch.uint8, device="cuda")
    est_ws = torch.full((Z.estimate_workspace_size(64),), 0xAA, dtype=torch.uint8, device="cuda")
    Z.estimate_plans(tens, plans_dev, est_ws, stride=3)
    torch.cuda.synchronize()
    raw = plans_dev.cpu().numpy().tobytes()
    for k, x in enumerate(segs):
        got = Z.PlanT.from_buffer_copy(raw[8 * k:8 * k + 8])
        s = O.sample_sigma(x, 3)
        if abs(math.log2(s) - math.floor(math.log2(s)) - 0.7195805543641254) < 1e-9:
            continue                                      # at the switch: either window
        assert list(got.exponents) == [int(v) for v in O.plan_sigma(s)], (k, x.size, s)


@pytest.mark.parametrize("stride", [1, 7, 16])
def test_estimate_plans_and_compress_with_them(Z, stride):
    import math
    nan = np.full(4096, 0x7FC1, np.uint16)
    mixed = W.gaussian_bf16(50000, 0.3, 91)
    mixed[::97] = 0x7F80                                  # +Inf every 97th value
    segs = [W.gaussian_bf16(1 << 22, 0.02, 90), W.gaussian_bf16(70001, 1e-3, 92), np.zeros(0, np.uint16),
            W.gaussian_bf16(5, 1.0, 93), nan, W.gaussian_bf16(100000, 3.0, 94), mixed,
            W.gaussian_bf16(30000, 1e-30, 95)]
    tens = [dev_bf16(x) for x in segs]
    plans_dev = torch.full((8 * len(segs),), 0xAA, dtype=torch.uint8, device="cuda")
    est_ws = torch.full((Z.estimate_workspace_size(len(segs)),), 0xAA, dtype=torch.uint8, device="cuda")
    Z.estimate_plans(tens, plans_dev, est_ws, stride=stride)
    torch.cuda.synchronize()
    raw = plans_dev.cpu().numpy().tobytes()
    # the same plans again, with the first call's partial sums left in the scratch
    again = torch.full_like(plans_dev, 0x55)
    Z.estimate_plans(tens, again, est_ws, stride=stride)
    torch.cuda.synchronize()
    assert again.cpu().numpy().tobytes() == raw
    got = [Z.PlanT.from_buffer_copy(raw[8 * k:8 * k + 8]) for k in range(len(segs))]
    for k, x in enumerate(segs):
        s = O.sample_sigma(x, stride)
        phase = math.log2(s) - math.floor(math.log2(s))
        if abs(phase - 0.7195805543641254) < 1e-9:
            continue                                      # at the switch: either window
        assert list(got[k].exponents) == [int(v) for v in O.plan_sigma(s)], (k, s)
        assert got[k].reserved == 0
    # compress with the device plans == compress with the same plans passed by value
    r_ref = gpu_compress(Z, segs, got)
    check_against_oracle(Z, segs, got, r_ref)
    total_static = sum(Z.static_size(x.size) for x in segs)
    static = torch.full((total_static,), POISON, dtype=torch.uint8, device="cuda")
    esc = torch.full((sum(x.size for x in segs),), POISON, dtype=torch.uint8, device="cuda")
    n_esc = torch.full((len(segs) + 1,), -1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(Z.workspace_size(sum(x.size for x in segs), len(segs)), dtype=torch.uint8, device="cuda")
    Z.compress_device_plans(tens, plans_dev, static, esc, ws, n_esc, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(static.cpu().numpy(), r_ref["static_h"])
    ne = n_esc.cpu().numpy()
    assert np.array_equal(ne, r_ref["n_esc"])
    assert np.array_equal(esc.cpu().numpy()[:ne[-1]], r_ref["esc_h"][:ne[-1]])


# ------------------------------------------------------------------------------------
# the scan-kernel path for escape positions (used above 2^28 values per call), forced
# on small inputs
# ------------------------------------------------------------------------------------
@pytest.fixture
def scan_path(monkeypatch):
    monkeypatch.setenv("ZIPCCL_DIRECT_PREFIX_MAX_UNITS", "0")
    yield


def compress_chunks_vs_oracle(Z, chunks_bits, plans, ws_bytes=None, esc_caps=None, esc_shifts=None):
    # ws_bytes: workspace size (default: twice what the largest chunk needs, so that
    # about two chunks share a launch); esc_caps: per-chunk escape capacities (default:
    # room for every value); esc_shifts: per chunk, how many bytes past a 256-byte boundary
    # its escape buffer starts (the bytes around it must stay unwritten)
    C, S = len(chunks_bits), len(chunks_bits[0])
    tens = [[dev_bf16(b) for b in ch] for ch in chunks_bits]
    sizes = [[b.size for b in ch] for ch in chunks_bits]
    st_sizes = [sum(Z.static_size(n) for n in sz) for sz in sizes]
    statics = [torch.full((max(t, 1),), POISON, dtype=torch.uint8, device="cuda") for t in st_sizes]
    caps = [sum(sz) for sz in sizes] if esc_caps is None else esc_caps
    shifts = [0] * C if esc_shifts is None else esc_shifts
    bufs = [torch.full((shifts[k] + max(caps[k], 1) + 64,), POISON, dtype=torch.uint8, device="cuda") for k in range(C)]
    escs = [bufs[k][shifts[k]:shifts[k] + max(caps[k], 1)] for k in range(C)]
    if ws_bytes is None:
        ws_bytes = 2 * Z.workspace_size(max(sum(sz) for sz in sizes), S)
    ws = torch.full((ws_bytes,), POISON, dtype=torch.uint8, device="cuda")
    n_esc = torch.full((C * (S + 1),), -1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Z.PreparedCompressChunks(tens, statics, escs, ws, n_esc, status, esc_caps=esc_caps).run(plans)
    torch.cuda.synchronize()
    ne = n_esc.cpu().numpy()
    st_all = int(status.item())
    for k in range(C):
        st, esc, ne_o, rc = O.compress_batch(chunks_bits[k], oracle_tables(plans))
        assert list(ne[k * (S + 1):(k + 1) * (S + 1) - 1]) == ne_o, f"chunk {k}"
        assert int(ne[(k + 1) * (S + 1) - 1]) == sum(ne_o), f"chunk {k}"
        sh = statics[k].cpu().numpy()[:st_sizes[k]]
        assert np.array_equal(sh, st), f"chunk {k}: " + first_diff(sh, st)
        m = min(sum(ne_o), caps[k])
        assert np.array_equal(escs[k].cpu().numpy()[:m], esc[:m]), f"chunk {k}"
        bh = bufs[k].cpu().numpy()
        assert (bh[:shifts[k]] == POISON).all() and (bh[shifts[k] + m:] == POISON).all(), f"chunk {k}"
    return st_all


def chunk_sequence():
    # 6 chunks of 3 segments: full, ragged, empty and tiny segments; the last chunk short
    shapes = [[1 << 20, 1 << 20, 1 << 20], [70001, 4096, 1], [0, 5000, 16384 * 3], [1 << 20, 1 << 20, 1 << 20],
              [513, 0, 0], [12345, 8, 100000]]
    sig = [0.02, 1.0, 1e-3]
    return [[W.gaussian_bf16(n, sig[i], 1000 + 10 * k + i) for i, n in enumerate(ch)] for k, ch in enumerate(shapes)]


def test_compress_chunks_matches_per_call_oracle(Z):
    compress_chunks_vs_oracle(Z, chunk_sequence(), [Z.plan(sigma=s) for s in (0.02, 1.0, 1e-3)])


def test_compress_chunks_unaligned_escape_buffers(Z):
    # several calls in one launch, each writing its escapes into a buffer that starts 1, 2
    # or 3 bytes past a dword: few escapes, nearly all (units with more than a record's
    # first 496 bytes), random bits; ragged sizes; one chunk's cap cuts its escapes off
    rng = np.random.default_rng(78)
    shapes = [[70001, 16384, 5000], [1 << 18, 33333, 4097], [1, 100000, 16385], [20000, 0, 65536], [8, 3, 300001]]
    chunks = []
    for k, ch in enumerate(shapes):
        chunks.append([W.gaussian_bf16(ch[0], 0.02, 3000 + 10 * k), W.gaussian_bf16(ch[1], 1.0, 3001 + 10 * k),
                       rng.integers(0, 1 << 16, ch[2], dtype=np.int64).astype(np.uint16)])
    plans = [Z.plan(sigma=0.02), Z.plan(table=[1, 2, 3, 4, 5, 6, 7]), Z.plan(sigma=0.1)]
    totals = [sum(O.compress_batch(ch, oracle_tables(plans))[2]) for ch in chunks]
    caps = [t + 7 for t in totals]
    caps[2] = totals[2] - 1001   # this chunk overflows: only its status bit and its first cap bytes are checked
    status = compress_chunks_vs_oracle(Z, chunks, plans, esc_caps=caps, esc_shifts=[1, 2, 3, 1, 2])
    assert status == Z.STATUS_ESC_OVERFLOW


def test_compress_chunks_scan_path(Z, scan_path):
    compress_chunks_vs_oracle(Z, chunk_sequence()[:3], [Z.plan(sigma=s) for s in (0.02, 1.0, 1e-3)])


def test_scan_path_many_segments(Z, scan_path):
    rng = np.random.default_rng(6)
    segs, plans = [], []
    for k in range(40):
        n = int(rng.choice([0, 1, 700, 4096, 16384, 20000, 70001, 300000]))
        s = float(10 ** rng.uniform(-4, 1))
        segs.append(W.gaussian_bf16(n, s, 900 + k))
        plans.append(Z.plan(sigma=s))
    round_trip(Z, segs, plans)


def test_scan_path_empty_and_overflow(Z, scan_path):
    sizes = [0, 0, 256 * 4096, 0, 5, 0, 4096 * 300 + 17, 0, 0]
    segs = [W.gaussian_bf16(n, 0.05, 70 + k) for k, n in enumerate(sizes)]
    round_trip(Z, segs, [Z.plan(sigma=0.05)] * len(segs))
    round_trip(Z, [np.zeros(0, np.uint16)] * 3, [Z.plan(sigma=1.0)] * 3)
    x = W.gaussian_bf16(50000, 1.0, 5)
    p = Z.plan(table=[1, 2, 3, 4, 5, 6, 7])
    r = gpu_compress(Z, [x], [p], esc_cap=1000)
    assert r["status"] & Z.STATUS_ESC_OVERFLOW
    st, esc, ne, rc = O.compress_batch([x], oracle_tables([p]))
    assert np.array_equal(r["static_h"], st) and np.array_equal(r["esc_h"][:1000], esc[:1000])


# ------------------------------------------------------------------------------------
# one launch (encoders, then placing workgroups that wait for the encoders' ready words)
# against the two-launch path; reused workspaces; graph capture
# ------------------------------------------------------------------------------------
@pytest.fixture
def two_launches(monkeypatch):
    monkeypatch.setenv("ZIPCCL_SINGLE_LAUNCH", "0")
    yield


def mixed_batch(seed, nseg=40):
    rng = np.random.default_rng(seed)
    segs, plans = [], []
    for k in range(nseg):
        n = int(rng.choice([0, 1, 700, 4096, 16384, 20000, 70001, 300000, 1 << 20]))
        s = float(10 ** rng.uniform(-4, 1))
        segs.append(W.gaussian_bf16(n, s, 5000 + 100 * seed + k))
        plans.append(Z_plan(s))
    return segs, plans


def Z_plan(s):
    from lossless_bf16_exponent_codec_amd import zipccl
    return zipccl.plan(sigma=s)


def test_two_launch_path_many_segments(Z, two_launches):
    segs, plans = mixed_batch(1)
    round_trip(Z, segs, plans)


def test_two_launch_path_edges_and_overflow(Z, two_launches):
    for n in (1, 4097, 16385, 250001):
        round_trip(Z, [W.gaussian_bf16(n, 0.02, n)], [Z.plan(sigma=0.02)])
    x = W.gaussian_bf16(50000, 1.0, 5)
    p = Z.plan(table=[1, 2, 3, 4, 5, 6, 7])
    r = gpu_compress(Z, [x], [p], esc_cap=1000)
    assert r["status"] == Z.STATUS_ESC_OVERFLOW
    st, esc, ne, rc = O.compress_batch([x], oracle_tables([p]))
    assert np.array_equal(r["static_h"], st) and np.array_equal(r["esc_h"][:1000], esc[:1000])


def unaligned_escape_batch(Z):
    # units whose escape runs start and end at every offset within a dword: few escapes,
    # nearly all (more than a unit's first 496 staged bytes), random bits, ragged sizes
    rng = np.random.default_rng(77)
    segs, plans = [], []
    for k, n in enumerate([5, 16384, 70001, 4097, 300000, 1, 33333]):
        kind = k % 3
        if kind == 0:
            segs.append(W.gaussian_bf16(n, 0.02, 900 + k))
            plans.append(Z.plan(sigma=0.02))
        elif kind == 1:
            segs.append(W.gaussian_bf16(n, 1.0, 900 + k))
            plans.append(Z.plan(table=[1, 2, 3, 4, 5, 6, 7]))   # nearly every value escapes
        else:
            segs.append(rng.integers(0, 1 << 16, n, dtype=np.int64).astype(np.uint16))
            plans.append(Z.plan(sigma=float(10 ** rng.uniform(-3, 0))))
    return segs, plans


@pytest.mark.parametrize("single", [True, False])
@pytest.mark.parametrize("shift", [1, 2, 3])
def test_escape_buffer_at_unaligned_addresses(Z, monkeypatch, single, shift):
    # the escape buffer starts `shift` bytes past a 256-byte boundary: every escape is the
    # oracle's and no byte outside [0, cap) of the buffer is written, with room for all
    # escapes and with a cap that cuts them off mid-dword
    if not single:
        monkeypatch.setenv("ZIPCCL_SINGLE_LAUNCH", "0")
    segs, plans = unaligned_escape_batch(Z)
    st_o, esc_o, ne_o, _ = O.compress_batch(segs, oracle_tables(plans))
    total = sum(ne_o)
    sizes = [s.size for s in segs]
    tens = [dev_bf16(s) for s in segs]
    for cap in (total + 5, total - 4097):
        static = torch.full((sum(Z.static_size(n) for n in sizes),), POISON, dtype=torch.uint8, device="cuda")
        buf = torch.full((shift + cap + 67,), POISON, dtype=torch.uint8, device="cuda")
        esc = buf[shift:shift + cap]
        assert esc.data_ptr() % 4 == shift
        n_esc = torch.full((len(segs) + 1,), -1, dtype=torch.int64, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        ws = torch.zeros(Z.workspace_size(sum(sizes), len(segs)), dtype=torch.uint8, device="cuda")
        Z.compress(list(zip(tens, plans)), static, esc, ws, n_esc, status, esc_cap=cap)
        torch.cuda.synchronize()
        h = buf.cpu().numpy()
        kept = min(cap, total)
        assert int(status.item()) == (0 if cap >= total else Z.STATUS_ESC_OVERFLOW)
        assert list(n_esc.cpu().numpy()[:-1]) == ne_o
        assert np.array_equal(static.cpu().numpy(), st_o)
        assert np.array_equal(h[shift:shift + kept], esc_o[:kept]), first_diff(h[shift:shift + kept], esc_o[:kept])
        assert (h[:shift] == POISON).all() and (h[shift + kept:] == POISON).all()


def test_single_launch_overflow_status_only(Z):
    # the escape overflow is the only status bit: the placing workgroups never ran out of
    # their bounded wait
    x = W.gaussian_bf16(300000, 1.0, 6)
    p = Z.plan(table=[1, 2, 3, 4, 5, 6, 7])
    r = gpu_compress(Z, [x], [p], esc_cap=5000)
    assert r["status"] == Z.STATUS_ESC_OVERFLOW
    st, esc, ne, rc = O.compress_batch([x], oracle_tables([p]))
    assert np.array_equal(r["static_h"], st) and np.array_equal(r["esc_h"][:5000], esc[:5000])


def test_single_launch_stale_ready_words(Z):
    # one workspace, calls of different sizes in a row: a call with fewer units leaves the
    # later ready words of the call before it, and a call that follows a larger one finds
    # that call's words for every unit.  Each call must wait for its own.  The workspace
    # starts as garbage (0xFF: every ready word claims the largest tag).
    big = 4 << 20
    ws = torch.full((Z.workspace_size(big, 8),), 0xFF, dtype=torch.uint8, device="cuda")
    batches = [([W.gaussian_bf16(big, 0.02, 21)], [Z.plan(sigma=0.02)]),
               ([W.gaussian_bf16(n, 1e-3, 22 + n) for n in (100000, 1 << 20, 0, 7)], [Z.plan(sigma=1e-3)] * 4),
               ([W.gaussian_bf16(big, 0.5, 23)], [Z.plan(sigma=0.5)]),
               ([W.gaussian_bf16(3 << 20, 1.0, 24)], [Z.plan(table=[1, 2, 3, 4, 5, 6, 7])])]   # all escapes
    for rep in range(2):
        for segs, plans in batches:
            print(f"stale ready words rep={rep} sizes={[s.size for s in segs]}", flush=True)
            r = gpu_compress(Z, segs, plans, workspace=ws)
            check_against_oracle(Z, segs, plans, r)


def test_single_and_two_launch_paths_agree(Z, monkeypatch):
    segs, plans = mixed_batch(2, nseg=24)
    r1 = gpu_compress(Z, segs, plans)
    monkeypatch.setenv("ZIPCCL_SINGLE_LAUNCH", "0")
    r2 = gpu_compress(Z, segs, plans)
    assert r1["status"] == r2["status"] == 0
    assert np.array_equal(r1["static_h"], r2["static_h"])
    assert np.array_equal(r1["n_esc"], r2["n_esc"])
    t = int(r1["n_esc"][-1])
    assert np.array_equal(r1["esc_h"][:t], r2["esc_h"][:t])
    check_against_oracle(Z, segs, plans, r1)


def test_compress_in_captured_graph(Z):
    # under graph capture the call takes the two-launch path (no per-call tag is baked
    # into the graph); every replay, with new input between replays, matches the oracle
    n = [300000, 4096, 70001]
    sig = [0.02, 1e-3, 0.5]
    plans = [Z.plan(sigma=s) for s in sig]
    inputs = [dev_bf16(W.gaussian_bf16(k, s, 40 + i)) for i, (k, s) in enumerate(zip(n, sig))]
    total_static = sum(Z.static_size(k) for k in n)
    static = torch.full((total_static,), POISON, dtype=torch.uint8, device="cuda")
    esc = torch.full((sum(n),), POISON, dtype=torch.uint8, device="cuda")
    n_esc = torch.full((len(n) + 1,), -1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(Z.workspace_size(sum(n), len(n)), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        Z.PreparedCompress(inputs, static, esc, ws, n_esc, status).run(plans)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Z.PreparedCompress(inputs, static, esc, ws, n_esc, status).run(plans)
    for rep in range(4):
        segs = [W.gaussian_bf16(k, s, 700 + 10 * rep + i) for i, (k, s) in enumerate(zip(n, sig))]
        for t, x in zip(inputs, segs):
            t.copy_(dev_bf16(x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"graph replay {rep}", flush=True)
        r = dict(status=int(status.item()), n_esc=n_esc.cpu().numpy(), static_h=static.cpu().numpy(),
                 esc_h=esc.cpu().numpy())
        check_against_oracle(Z, segs, plans, r)


# ------------------------------------------------------------------------------------
# chunk sequences whose calls share launches (up to 16 calls and 128 segments per launch)
# ------------------------------------------------------------------------------------
def long_chunk_sequence(nchunks=11, S=3, seed=0):
    # ragged, tiny and empty segments; chunk 4 is all empty (a launch of its own) and
    # chunk 7 has a single tiny segment
    rng = np.random.default_rng(seed)
    sig = [0.02, 1.0, 1e-3][:S]
    out = []
    for k in range(nchunks):
        if k == 4:
            ns = [0] * S
        elif k == 7:
            ns = [0] * (S - 1) + [5]
        else:
            ns = [int(rng.choice([0, 1, 513, 4096, 16385, 70001, 1 << 20])) for _ in range(S)]
        out.append([W.gaussian_bf16(n, sig[i], 3000 + 17 * k + i + 1000 * seed) for i, n in enumerate(ns)])
    return out, [Z_plan(x) for x in sig]


def batch_workspace(Z, chunks):
    return Z.workspace_size(sum(b.size for ch in chunks for b in ch), sum(len(ch) for ch in chunks))


def test_compress_chunks_shared_launches(Z):
    # 40 calls: a launch holds at most 16
    chunks, plans = long_chunk_sequence(nchunks=40)
    print("chunks sharing launches", [[b.size for b in ch] for ch in chunks], flush=True)
    assert compress_chunks_vs_oracle(Z, chunks, plans, ws_bytes=batch_workspace(Z, chunks)) == 0


def test_compress_chunks_shared_launches_many_peers(Z):
    # 7 segments per chunk: 16 chunks (112 segments) per launch, then the last 4
    rng = np.random.default_rng(5)
    chunks = [[W.gaussian_bf16(int(rng.choice([4096, 20000, 65536])), 1e-3, 4000 + 7 * k + i) for i in range(7)]
              for k in range(36)]
    plans = [Z.plan(sigma=1e-3)] * 7
    assert compress_chunks_vs_oracle(Z, chunks, plans, ws_bytes=batch_workspace(Z, chunks)) == 0


def test_compress_chunks_shared_launches_two_launch_path(Z, two_launches):
    chunks, plans = long_chunk_sequence(seed=2)
    assert compress_chunks_vs_oracle(Z, chunks, plans, ws_bytes=batch_workspace(Z, chunks)) == 0


@pytest.mark.parametrize("units", [4096, 4097, 4104, 4105, 4111, 4200])
def test_single_call_around_the_placer_lag(Z, units):
    # a call of `units` encoding workgroups (16384 values each, the last one ragged): the
    # last 512 placing groups follow the last encoder, so the first groups' placers are
    # interleaved with the encoders once the call has more than 4096 units (one group at
    # 4097 to 4104 units, two at 4105)
    n = units * 16384 - 777
    print(f"single call of {units} units", flush=True)
    x = W.gaussian_bf16(n, 0.02, 7000 + units)
    p = Z.plan(sigma=0.02)
    r = gpu_compress(Z, [x], [p])
    check_against_oracle(Z, [x], [p], r)


def test_compress_chunks_interleaved_across_calls(Z):
    # 12 calls of 3 ragged segments (about 9300 units) in one launch: placing groups that
    # span two calls, interleaved with the encoders of later calls
    rng = np.random.default_rng(11)
    chunks = [[W.gaussian_bf16(int((1 << 22) + rng.integers(-50000, 50000)), (0.02, 1.0, 1e-3)[i], 8000 + 3 * k + i)
               for i in range(3)] for k in range(12)]
    plans = [Z.plan(sigma=s) for s in (0.02, 1.0, 1e-3)]
    print("interleaved calls", [[b.size for b in ch] for ch in chunks], flush=True)
    assert compress_chunks_vs_oracle(Z, chunks, plans, ws_bytes=batch_workspace(Z, chunks)) == 0


def test_compress_chunks_interleaved_with_empty_and_tiny_segments(Z):
    # 16 calls in one launch, about 5700 units, whose segments mix multi-million-value
    # stretches with empty, 1-value, 513-value and 16385-value ones, so that interleaved
    # placing groups start, end and span calls at segments that hold a single unit or none
    big = [1 << 22, (1 << 22) + 4097, 3 * (1 << 20) + 1]
    small = [0, 1, 513, 16385, 0]
    chunks = []
    for k in range(16):
        ns = [big[k % 3], small[k % 5], big[(k + 1) % 3] if k % 4 else small[(k + 2) % 5]]
        if k == 9:
            ns = [0, 0, 0]
        chunks.append([W.gaussian_bf16(n, (0.02, 1.0, 1e-3)[i], 8200 + 3 * k + i) for i, n in enumerate(ns)])
    plans = [Z.plan(sigma=s) for s in (0.02, 1.0, 1e-3)]
    print("interleaved calls with small segments", [[b.size for b in ch] for ch in chunks], flush=True)
    assert compress_chunks_vs_oracle(Z, chunks, plans, ws_bytes=batch_workspace(Z, chunks)) == 0


def test_compress_chunks_interleaved_two_launch_path(Z, two_launches):
    # the same launch shape through encode_kernel + place_direct_kernel: each placing
    # group sums only the units of its call (more than 16384 units in the launch)
    rng = np.random.default_rng(12)
    chunks = [[W.gaussian_bf16(int((1 << 24) + rng.integers(-50000, 50000)), 1e-3, 8100 + 3 * k + i)
               for i in range(3)] for k in range(6)]
    plans = [Z.plan(sigma=1e-3)] * 3
    assert compress_chunks_vs_oracle(Z, chunks, plans, ws_bytes=batch_workspace(Z, chunks)) == 0


def test_compress_chunks_overflow_in_one_call(Z):
    # chunk 2 of 5 gets a small escape buffer: the status reports the overflow, its
    # escapes before the cap and every other chunk's bytes are still exact
    chunks = [[W.gaussian_bf16(200000, 1.0, 6100 + 3 * k + i) for i in range(3)] for k in range(5)]
    plans = [Z.plan(table=[120, 121, 122, 123, 124, 125, 126])] * 3   # many escapes
    caps = [600000] * 5
    caps[2] = 5000
    st = compress_chunks_vs_oracle(Z, chunks, plans, ws_bytes=batch_workspace(Z, chunks), esc_caps=caps)
    assert st == Z.STATUS_ESC_OVERFLOW


def test_single_launch_wait_limit_is_reported(Z, monkeypatch):
    # the bounded wait's error path, forced from the host: the placing workgroups wait for
    # a tag no call writes, 4 polls per word; every one gives up, reports
    # ZIPCCL_STATUS_WAIT_LIMIT and writes no header; the next call on the same workspace
    # is exact again
    x = [W.gaussian_bf16(300000, 0.02, 3), W.gaussian_bf16(70001, 1e-3, 4)]
    p = [Z.plan(sigma=0.02), Z.plan(sigma=1e-3)]
    ws = torch.zeros(Z.workspace_size(sum(s.size for s in x), len(x)), dtype=torch.uint8, device="cuda")
    monkeypatch.setenv("ZIPCCL_TEST_WAIT_LIMIT", "1")
    r = gpu_compress(Z, x, p, workspace=ws)
    assert r["status"] & Z.STATUS_WAIT_LIMIT
    assert (r["static_h"][:64] == POISON).all()   # the first segment's header was not written
    monkeypatch.delenv("ZIPCCL_TEST_WAIT_LIMIT")
    r = gpu_compress(Z, x, p, workspace=ws)
    check_against_oracle(Z, x, p, r)


def test_wait_limit_with_interleaved_placers(Z, monkeypatch):
    # the same forced time-out in a launch large enough (4200 units) that the placers of its
    # first groups run among the encoders: every placer gives up within its 4 polls per word,
    # the launch ends, nothing is placed, and the next call is exact again
    x = [W.gaussian_bf16(4200 * 16384 - 5, 0.02, 31)]
    p = [Z.plan(sigma=0.02)]
    print("wait limit, one call of 4200 units", flush=True)
    ws = torch.zeros(Z.workspace_size(x[0].size, 1), dtype=torch.uint8, device="cuda")
    monkeypatch.setenv("ZIPCCL_TEST_WAIT_LIMIT", "1")
    r = gpu_compress(Z, x, p, workspace=ws)
    assert r["status"] & Z.STATUS_WAIT_LIMIT
    assert (r["static_h"][:64] == POISON).all()
    monkeypatch.delenv("ZIPCCL_TEST_WAIT_LIMIT")
    r = gpu_compress(Z, x, p, workspace=ws)
    check_against_oracle(Z, x, p, r)


def test_wait_limit_hook_without_status_word(Z, monkeypatch):
    # without a status word a compress takes the two-launch path, in which no workgroup
    # waits for another: the forced wait limit has nothing to act on, and the output is
    # exact (a time-out could otherwise leave headers unwritten with nobody told)
    x = [W.gaussian_bf16(300000, 0.02, 3), W.gaussian_bf16(70001, 1e-3, 4)]
    p = [Z.plan(sigma=0.02), Z.plan(sigma=1e-3)]
    ws = torch.zeros(Z.workspace_size(sum(s.size for s in x), len(x)), dtype=torch.uint8, device="cuda")
    monkeypatch.setenv("ZIPCCL_TEST_WAIT_LIMIT", "1")
    r = gpu_compress(Z, x, p, workspace=ws, with_status=False)
    check_against_oracle(Z, x, p, r)
    outs, status = gpu_decompress(Z, r)
    assert status == 0
    for a, b in zip(x, outs):
        assert np.array_equal(a, b)
    # with a status word the same hook makes the single launch's placers give up, and
    # the status word says so
    r = gpu_compress(Z, x, p, workspace=ws)
    assert r["status"] & Z.STATUS_WAIT_LIMIT
