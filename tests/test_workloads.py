"""The seeded input generators: shapes, counts and structure the workloads promise
(no codec arithmetic is involved)."""
import numpy as np

from lossless_bf16_exponent_codec_amd import workloads as W


def test_zipf_counts_sum_and_order():
    c = W.zipf_counts(16384, 8, 1.2)
    assert sum(c) == 16384 and c == sorted(c, reverse=True)
    assert c == [7023, 3057, 1879, 1330, 1018, 818, 680, 579]


def test_routed_moe_rows_partition_the_tokens():
    wl = W.moe_routed_16384x7168(tokens=512, hidden=512)
    rows = wl.extra["rows"]
    assert [len(r) for r in rows] == W.zipf_counts(512, 8, 1.2)
    allr = np.concatenate(rows)
    assert np.array_equal(np.sort(allr), np.arange(512))            # every token exactly once
    assert all(np.all(np.diff(r) > 0) for r in rows)                # ascending within a destination
    assert all(r.dtype == np.int32 for r in rows)
    # the same matrix as the pre-permuted workload, whose buckets are contiguous rows
    flat = W.moe_16384x7168(tokens=512, hidden=512)
    assert np.array_equal(np.concatenate(flat.segments), wl.segments[0])


def test_gaussian_is_seeded_and_bf16():
    a, b = W.gaussian_bf16(1000, 0.5, 7), W.gaussian_bf16(1000, 0.5, 7)
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    assert not np.array_equal(a, W.gaussian_bf16(1000, 0.5, 8))
    f = (a.astype(np.uint32) << 16).view(np.float32)
    assert 0.4 < float(np.std(f)) < 0.6
