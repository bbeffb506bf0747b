"""Host-side checks of the C ABI: the library loads, exports every declared symbol,
and its host-only functions (plan, sizes, argument validation) agree with the oracle.
No compute call touches a GPU here."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zipccl.h")


@pytest.fixture(scope="module")
def Z():
    from lossless_bf16_exponent_codec_amd import zipccl
    return zipccl


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zipccl_[a-z_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    for want in ["zipccl_plan", "zipccl_compress", "zipccl_decompress", "zipccl_decompress_accumulate",
                 "zipccl_compressed_size", "zipccl_static_size", "zipccl_workspace_size",
                 "zipccl_pipeline_create", "zipccl_pipeline_reduce", "zipccl_pipeline_destroy",
                 "zipccl_pipeline_scratch_size", "zipccl_strerror", "zipccl_plan_many",
                 "zipccl_decompress_shards", "zipccl_compress_gather", "zipccl_compress_chunks",
                 "zipccl_decompress_accumulate_chunks", "zipccl_profile_codec", "zipccl_profile_scratch_size",
                 "zipccl_rs_choose", "zipccl_estimate_plans", "zipccl_estimate_workspace_size",
                 "zipccl_compress_device_plans"]:
        assert want in names


def test_library_exports_every_declared_symbol(Z):
    out = subprocess.run(["nm", "-D", "--defined-only", Z.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (zipccl_\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    for f in declared_functions():
        assert hasattr(Z.lib(), f)


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "zipccl.h"\nint main(void){zipccl_plan_t p; (void)p; return 0;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-c",
                    str(src), "-o", str(tmp_path / "t.o")], check=True)


def _phase(s):
    f = math.log2(s)
    return f - math.floor(f)


def test_closed_form_plan_equals_oracle_ranking(Z):
    # the library's closed form against the oracle's ranking of all 254 binade masses
    rng = np.random.default_rng(1)
    sig = 2.0 ** rng.uniform(-140, 140, 20000)
    sig = np.concatenate([sig, [0.02, 1e-3, 0.5, 1.0, 1e-4, 0.1, 1e-45, 1e38, 3e38]])
    checked = 0
    for s in sig:
        s = float(s)
        ph = _phase(s)
        if abs(ph - 0.7195805543641254) < 1e-9:
            continue
        assert Z.plan(sigma=s).exponents == list(O.plan_sigma(s)), s
        checked += 1
    assert checked > 19000


def test_plan_check_values(Z):
    assert Z.plan(sigma=0.02).exponents == list(range(116, 123))
    assert Z.plan(sigma=1e-3).exponents == list(range(112, 119))
    assert Z.plan(sigma=0.5).exponents == list(range(121, 128))
    assert Z.plan(sigma=1.0).exponents == list(range(122, 129))


def test_plan_table_and_errors(Z):
    assert Z.plan(table=[9, 3, 7, 5, 1, 2, 200]).exponents == [1, 2, 3, 5, 7, 9, 200]
    for bad in ([0, 1, 2, 3, 4, 5, 6], [1, 2, 3, 4, 5, 6, 255], [1, 1, 2, 3, 4, 5, 6]):
        with pytest.raises(Z.ZipcclError) as e:
            Z.plan(table=bad)
        assert e.value.status == Z.ERR_INVALID
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(Z.ZipcclError):
            Z.plan(sigma=bad)


def test_plan_many_matches_plan(Z):
    rng = np.random.default_rng(12)
    sig = [float(10 ** x) for x in rng.uniform(-30, 30, 500)] + [1e-300, 1e300, 1.0, 2.0 ** -126]
    many = Z.plan_many(sig)
    for i, s in enumerate(sig):
        assert list(many[i].table) == list(Z.plan(sigma=s).table)
    assert Z.lib().zipccl_plan_many(None, 0, None) == Z.OK
    bad = (ctypes.c_double * 3)(1.0, -1.0, 2.0)
    out = (Z.PlanT * 3)()
    assert Z.lib().zipccl_plan_many(bad, 3, out) == Z.ERR_INVALID
    assert list(out[0].table) == list(Z.plan(sigma=1.0).table)


@pytest.mark.parametrize("n", [0, 1, 7, 8, 511, 512, 513, 4095, 4096, 4097, 16384, 2 ** 22, 2 ** 26 + 3,
                               2 ** 32 - 1])
def test_sizes_match_oracle(Z, n):
    assert Z.static_size(n) == O.static_size(n)
    assert Z.compressed_size(n, 17) == O.static_size(n) + 17
    assert Z.static_size(n) % 128 == 0


def test_workspace_size_is_monotone(Z):
    a = Z.workspace_size(1 << 20, 1)
    assert Z.workspace_size(1 << 21, 1) > a and Z.workspace_size(1 << 20, 4) > a


def test_argument_errors_before_any_launch(Z):
    L = Z.lib()
    p = Z.plan(sigma=1.0)
    seg = (Z.SegmentT * 1)()
    seg[0].src, seg[0].n, seg[0].plan = 0x10000, 100, p
    fake = 0x100000                      # never dereferenced: every case fails validation first
    ws = Z.workspace_size(100, 1)
    assert L.zipccl_compress(seg, 0, fake, 1 << 20, fake, 100, fake, ws, None, None, None) == Z.ERR_INVALID
    assert L.zipccl_compress(seg, 65, fake, 1 << 20, fake, 100, fake, ws, None, None, None) == Z.ERR_INVALID
    assert L.zipccl_compress(seg, 1, fake + 64, 1 << 20, fake, 100, fake, ws, None, None, None) == Z.ERR_ALIGN
    seg[0].src = 0x10002
    assert L.zipccl_compress(seg, 1, fake, 1 << 20, fake, 100, fake, ws, None, None, None) == Z.ERR_ALIGN
    seg[0].src = 0x10000
    assert L.zipccl_compress(seg, 1, fake, 10, fake, 100, fake, ws, None, None, None) == Z.ERR_SIZE
    assert L.zipccl_compress(seg, 1, fake, 1 << 20, fake, 100, fake, 8, None, None, None) == Z.ERR_SIZE
    seg[0].n = 1 << 32
    assert L.zipccl_compress(seg, 1, fake, 1 << 40, fake, 100, fake, 1 << 30, None, None, None) == Z.ERR_SIZE
    seg[0].n = 100
    seg[0].plan.table[3] = seg[0].plan.table[2]
    assert L.zipccl_compress(seg, 1, fake, 1 << 20, fake, 100, fake, ws, None, None, None) == Z.ERR_INVALID
    segs2 = (Z.SegmentT * 2)()
    for e in segs2:
        e.src, e.n, e.plan = 0x10000, 100, Z.plan(sigma=1.0)
    vp_ = ctypes.c_void_p
    so, eo = (vp_ * 2)(fake, fake), (vp_ * 2)(fake, fake)
    sc, ec = (ctypes.c_uint64 * 2)(1 << 20, 1 << 20), (ctypes.c_uint64 * 2)(100, 100)
    cws = 2 * Z.workspace_size(100, 1)
    assert L.zipccl_compress_chunks(segs2, 1, 0, None, None, None, None, None, 0, None, None, None) == Z.OK
    assert L.zipccl_compress_chunks(segs2, 0, 2, so, sc, eo, ec, fake, cws, None, None, None) == Z.ERR_INVALID
    assert L.zipccl_compress_chunks(segs2, 17, 2, so, sc, eo, ec, fake, cws, None, None, None) == Z.ERR_INVALID
    assert L.zipccl_compress_chunks(segs2, 1, -1, so, sc, eo, ec, fake, cws, None, None, None) == Z.ERR_INVALID
    assert L.zipccl_compress_chunks(segs2, 1, 2, so, sc, eo, ec, fake + 16, cws, None, None, None) == Z.ERR_ALIGN
    assert L.zipccl_compress_chunks(segs2, 1, 2, so, sc, eo, ec, fake, 8, None, None, None) == Z.ERR_SIZE
    so[1] = fake + 64                    # the second chunk's static part misaligned: nothing enqueued
    assert L.zipccl_compress_chunks(segs2, 1, 2, so, sc, eo, ec, fake, cws, None, None, None) == Z.ERR_ALIGN
    est = L.zipccl_estimate_plans
    ews = Z.estimate_workspace_size(1)
    assert ews == 256 and Z.estimate_workspace_size(16) == 16 * 256
    assert est(seg, 1, 16, None, fake, ews, None) == Z.ERR_INVALID
    assert est(seg, 1, 16, fake, None, ews, None) == Z.ERR_INVALID
    assert est(seg, 0, 16, fake, fake, ews, None) == Z.ERR_INVALID
    assert est(seg, 1, 0, fake, fake, ews, None) == Z.ERR_INVALID
    assert est(seg, 1, 16, fake + 4, fake, ews, None) == Z.ERR_ALIGN
    assert est(seg, 1, 16, fake, fake + 8, ews, None) == Z.ERR_ALIGN
    assert est(seg, 1, 16, fake, fake, ews - 1, None) == Z.ERR_SIZE
    cdp = L.zipccl_compress_device_plans
    assert cdp(seg, 1, None, fake, 1 << 20, fake, 100, fake, ws, None, None, None) == Z.ERR_INVALID
    assert cdp(seg, 1, fake + 4, fake, 1 << 20, fake, 100, fake, ws, None, None, None) == Z.ERR_ALIGN
    assert cdp(seg, 1, fake, fake, 10, fake, 100, fake, ws, None, None, None) == Z.ERR_SIZE
    g = (Z.GatherSegmentT * 1)()
    g[0].src, g[0].src_rows, g[0].row_len, g[0].rows, g[0].nrows, g[0].plan = 0x10000, 100, 7168, 0x20000, 10, p
    gws = Z.workspace_size(71680, 1)
    assert L.zipccl_compress_gather(g, 0, fake, 1 << 20, fake, 100, fake, gws, None, None, None) == Z.ERR_INVALID
    g[0].row_len = 7170                  # not a multiple of 8
    assert L.zipccl_compress_gather(g, 1, fake, 1 << 20, fake, 100, fake, gws, None, None, None) == Z.ERR_INVALID
    g[0].row_len = 256                   # below 512
    assert L.zipccl_compress_gather(g, 1, fake, 1 << 20, fake, 100, fake, gws, None, None, None) == Z.ERR_INVALID
    g[0].row_len, g[0].rows = 7168, 0x20002
    assert L.zipccl_compress_gather(g, 1, fake, 1 << 20, fake, 100, fake, gws, None, None, None) == Z.ERR_ALIGN
    g[0].rows = None
    assert L.zipccl_compress_gather(g, 1, fake, 1 << 20, fake, 100, fake, gws, None, None, None) == Z.ERR_INVALID
    g[0].rows, g[0].nrows = 0x20000, 1 << 20      # 7168 << 20 values
    assert L.zipccl_compress_gather(g, 1, fake, 1 << 40, fake, 100, fake, 1 << 40, None, None, None) == Z.ERR_SIZE
    g[0].nrows = 10
    assert L.zipccl_compress_gather(g, 1, fake, 10, fake, 100, fake, gws, None, None, None) == Z.ERR_SIZE
    d = (Z.DSegmentT * 1)()
    d[0].dst, d[0].n = 0x10000, 5000
    assert L.zipccl_decompress(fake, 100, fake, 10, d, 1, None, None) == Z.ERR_SIZE
    assert L.zipccl_decompress(fake + 8, 1 << 20, fake, 10, d, 1, None, None) == Z.ERR_ALIGN
    d[0].dst = 0x10001
    assert L.zipccl_decompress(fake, 1 << 20, fake, 10, d, 1, None, None) == Z.ERR_ALIGN
    vp = ctypes.c_void_p
    sp = (vp * 1)(fake)
    ep = (vp * 1)(fake)
    eb = (ctypes.c_uint64 * 1)(10)
    d[0].dst = 0x10000
    assert L.zipccl_decompress_shards(sp, ep, eb, d, 0, 0, None, None) == Z.ERR_INVALID
    assert L.zipccl_decompress_shards(sp, ep, eb, d, 65, 0, None, None) == Z.ERR_INVALID
    assert L.zipccl_decompress_shards(None, ep, eb, d, 1, 0, None, None) == Z.ERR_INVALID
    assert L.zipccl_decompress_shards(sp, (vp * 1)(None), eb, d, 1, 0, None, None) == Z.ERR_INVALID   # 10 escape bytes at NULL
    assert L.zipccl_decompress_shards((vp * 1)(fake + 64), ep, eb, d, 1, 0, None, None) == Z.ERR_ALIGN
    assert L.zipccl_decompress_shards(sp, ep, eb, d, 1, 2, None, None) == Z.ERR_INVALID   # unknown flag
    d[0].dst = 0x10001
    assert L.zipccl_decompress_shards(sp, ep, eb, d, 1, 0, None, None) == Z.ERR_ALIGN
    d[0].dst, d[0].n = 0x10000, 1 << 32
    assert L.zipccl_decompress_shards(sp, ep, eb, d, 1, 1, None, None) == Z.ERR_SIZE
    assert L.zipccl_decompress_accumulate(sp, ep, eb, 0, 10, fake, fake, None, None) == Z.ERR_INVALID
    assert L.zipccl_decompress_accumulate(sp, ep, eb, 17, 10, fake, fake, None, None) == Z.ERR_INVALID
    assert L.zipccl_decompress_accumulate(sp, ep, eb, 1, 1 << 32, fake, fake, None, None) == Z.ERR_SIZE
    assert L.zipccl_decompress_accumulate(sp, ep, eb, 1, 10, fake + 2, fake, None, None) == Z.ERR_ALIGN
    sp2, ep2 = (vp * 2)(fake, fake), (vp * 2)(fake, fake)
    eb2 = (ctypes.c_uint64 * 2)(10, 10)
    acc_chunks = L.zipccl_decompress_accumulate_chunks
    assert acc_chunks(sp2, ep2, eb2, 1, 4096, 0, None, None, None, None) == Z.OK
    assert acc_chunks(sp2, ep2, eb2, 0, 4096, 8192, fake, fake, None, None) == Z.ERR_INVALID
    assert acc_chunks(sp2, ep2, eb2, 1, 4000, 8192, fake, fake, None, None) == Z.ERR_INVALID
    assert acc_chunks(sp2, ep2, eb2, 1, 4096, 1 << 32, fake, fake, None, None) == Z.ERR_SIZE
    assert acc_chunks(sp2, ep2, eb2, 1, 4096, 8192, fake + 2, fake, None, None) == Z.ERR_ALIGN
    sp2[1] = fake + 64                   # the second chunk's static part: nothing is enqueued
    assert acc_chunks(sp2, ep2, eb2, 1, 4096, 8192, fake, fake, None, None) == Z.ERR_ALIGN
    ep2[1] = None
    sp2[1] = fake
    assert acc_chunks(sp2, ep2, eb2, 1, 4096, 8192, fake, fake, None, None) == Z.ERR_INVALID
    h = vp()
    assert L.zipccl_pipeline_create(7, 1000, fake, 1 << 30, None, None, ctypes.byref(h)) == Z.ERR_INVALID
    assert L.zipccl_pipeline_create(7, 4096, fake + 16, 1 << 30, None, None, ctypes.byref(h)) == Z.ERR_ALIGN
    assert L.zipccl_pipeline_create(7, 4096, fake, 16, None, None, ctypes.byref(h)) == Z.ERR_SIZE
    assert L.zipccl_strerror(Z.ERR_CORRUPT) == b"corrupt data or a device status bit set"


def test_rs_switcher_cost_model(Z):
    # a codec of ~2.5 TB/s compressing to 70 %: inside a node (7 xGMI links of ~150 GB/s
    # each) the saved wire time does not pay for the codec; across nodes (one 25 GB/s
    # link) it does.  Small tensors and incompressible data always go native.
    prof = Z.CodecProfileT(2500.0, 3200.0, 0.70)
    xgmi, ib = Z.LinkT(150.0, 5.0, 7), Z.LinkT(25.0, 5.0, 1)
    use, tn, tz = Z.rs_choose(prof, xgmi, 8, 512 << 20)
    assert not use and tz > tn > 0
    use, tn, tz = Z.rs_choose(prof, ib, 8, 512 << 20)
    assert use and tn > tz > 0
    # the times follow the stated model
    shard, m = (512 << 20) / 8, 7
    assert abs(tn - m * (5.0 + shard / 25e3)) < 1e-6 * tn
    assert abs(tz - (m * shard / 2500e3 + m * (5.0 + 0.7 * shard / 25e3) + m * shard / 3200e3)) < 1e-6 * tz
    assert not Z.rs_choose(prof, ib, 8, (1 << 20) - 1)[0]                       # under 1 MiB
    assert not Z.rs_choose(Z.CodecProfileT(2500.0, 3200.0, 1.0), ib, 8, 512 << 20)[0]   # incompressible
    # a slower link never makes the codec less attractive
    prev = None
    for bw in (400.0, 200.0, 100.0, 50.0, 25.0, 12.5):
        use = Z.rs_choose(prof, Z.LinkT(bw, 5.0, 1), 8, 512 << 20)[0]
        assert prev is None or use >= prev
        prev = use
    L = Z.lib()
    assert L.zipccl_rs_choose(None, ctypes.byref(ib), 8, 1 << 30, None, None, None) == Z.ERR_INVALID
    assert L.zipccl_rs_choose(ctypes.byref(prof), None, 8, 1 << 30, None, None, None) == Z.ERR_INVALID
    assert Z.lib().zipccl_rs_choose(ctypes.byref(prof), ctypes.byref(ib), 1, 1 << 30, None, None, None) == Z.ERR_INVALID
    assert Z.lib().zipccl_rs_choose(ctypes.byref(prof), ctypes.byref(Z.LinkT(0.0, 5.0, 1)), 8, 1 << 30, None, None,
                                    None) == Z.ERR_INVALID
    assert Z.lib().zipccl_profile_codec(None, 10, Z.plan(sigma=1.0), 1, None, 0, None, None) == Z.ERR_INVALID


def test_compress_noalloc_rejects_sizes_past_its_static_workspace(Z):
    # checked before anything touches a device: host addresses stand in for the buffers
    buf = np.zeros(64, np.uint64)
    addr = buf.ctypes.data + (-buf.ctypes.data % 256)
    segs = (Z.SegmentT * 2)()
    for k in range(2):
        segs[k].src = addr
        segs[k].plan = Z.plan(sigma=1.0)
    segs[0].n, segs[1].n = Z.NOALLOC_MAX_VALUES, 1              # one value too many
    rc = Z.lib().zipccl_compress_noalloc(segs, 2, addr, 1 << 40, addr, 1 << 40, None, None, None)
    assert rc == Z.ERR_SIZE
    segs[0].n = Z.NOALLOC_MAX_VALUES + 1
    assert Z.lib().zipccl_compress_noalloc(segs, 1, addr, 1 << 40, addr, 1 << 40, None, None, None) == Z.ERR_SIZE
    assert Z.lib().zipccl_compress_noalloc(segs, 0, addr, 1 << 40, addr, 1 << 40, None, None, None) == Z.ERR_INVALID
    assert Z.lib().zipccl_compress_noalloc(segs, 65, addr, 1 << 40, addr, 1 << 40, None, None, None) == Z.ERR_INVALID
