"""Property tests on the GPU (hypothesis, derandomized so a run repeats exactly): batches
of segments of random sizes (0 to 10^5 values, tile and block edges drawn often), random
contents (Gaussian at a random scale, random bit patterns, runs of one value, mixtures)
and random tables (the plan for a random sigma, or 7 random exponents) compress to the
oracle's bytes and decode back to the input; decode-accumulate of 1 to 9 such peers
equals the oracle's sum; and every batch compresses to the same bytes twice."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

from tests.test_gpu_parity import (check_against_oracle, first_diff, gpu_accumulate, gpu_compress, gpu_decompress,
                                   oracle_accumulate)

pytestmark = pytest.mark.gpu

EDGES = [0, 1, 7, 8, 63, 64, 191, 192, 193, 511, 512, 513, 4095, 4096, 4097, 8191, 8192, 16383, 16384, 16385,
         2047, 2048, 2049]
SETTINGS = settings(max_examples=100, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


@pytest.fixture(scope="module")
def Z():
    from lossless_bf16_exponent_codec_amd import zipccl
    return zipccl


sizes = st.one_of(st.sampled_from(EDGES), st.integers(0, 100_000))


@st.composite
def segment(draw, n=None):
    n = draw(sizes) if n is None else n
    seed = draw(st.integers(0, 2**32 - 1))
    rng = np.random.default_rng(seed)
    kind = draw(st.sampled_from(["gauss", "bits", "run", "mixed"]))
    if kind == "gauss":
        sigma = 10.0 ** draw(st.floats(-6, 3))
        x = (rng.standard_normal(n) * sigma).astype(np.float32)
        bits = (x.view(np.uint32) >> 16).astype(np.uint16)   # truncated to BF16: every pattern is a value
    elif kind == "bits":
        bits = rng.integers(0, 1 << 16, n, dtype=np.int64).astype(np.uint16)
    elif kind == "run":
        bits = np.full(n, draw(st.integers(0, 0xFFFF)), np.uint16)
    else:
        x = (rng.standard_normal(n) * 0.02).astype(np.float32)
        bits = (x.view(np.uint32) >> 16).astype(np.uint16)
        mask = rng.random(n) < draw(st.floats(0, 1))
        bits[mask] = rng.integers(0, 1 << 16, int(mask.sum()), dtype=np.int64).astype(np.uint16)
    return bits


@st.composite
def plan_spec(draw):
    if draw(st.booleans()):
        return ("sigma", 10.0 ** draw(st.floats(-6, 3)))
    return ("table", sorted(draw(st.lists(st.integers(1, 254), min_size=7, max_size=7, unique=True))))


def make_plan(Z, spec):
    return Z.plan(sigma=spec[1]) if spec[0] == "sigma" else Z.plan(table=spec[1])


@SETTINGS
@given(data=st.data())
def test_batches_match_the_oracle_and_round_trip(Z, data):
    k = data.draw(st.integers(1, 6))
    segs = [data.draw(segment()) for _ in range(k)]
    plans = [make_plan(Z, data.draw(plan_spec())) for _ in range(k)]
    print("batch", [s.size for s in segs], flush=True)
    r = gpu_compress(Z, segs, plans)
    check_against_oracle(Z, segs, plans, r)
    outs, status = gpu_decompress(Z, r)
    assert status == 0
    for x, y in zip(segs, outs):
        assert np.array_equal(x, y), first_diff(x, y)
    again = gpu_compress(Z, segs, plans)   # the same bytes a second time
    assert np.array_equal(again["static_h"], r["static_h"])
    assert np.array_equal(again["esc_h"][:int(r["n_esc"][-1])], r["esc_h"][:int(r["n_esc"][-1])])


@SETTINGS
@given(data=st.data())
def test_accumulate_matches_the_oracle(Z, data):
    n = data.draw(st.one_of(st.sampled_from([e for e in EDGES if e > 0]), st.integers(1, 60_000)))
    npeers = data.draw(st.integers(1, 9))
    peers = [data.draw(segment(n)) for _ in range(npeers)]
    local = data.draw(segment(n))
    plans = [make_plan(Z, data.draw(plan_spec())) for _ in range(npeers)]
    print("accumulate", n, npeers, flush=True)
    got, status, _ = gpu_accumulate(Z, peers, plans, local)
    assert status == 0
    want = oracle_accumulate(Z, peers, plans, local)
    assert np.array_equal(got, want), first_diff(got, want)
