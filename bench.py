#!/usr/bin/env python3
"""Benchmark of the lossless BF16 exponent codec on one MI355X.

One step = the whole hot path over one 64 Mi-value gradient bucket (16 layers of
4 Mi values, each layer with its own sigma-predicted table): plan the 16 tables on the
host, compress all layers in one launch, decompress them in one launch.  Inputs are
resident in HBM before the timed region.  Four input/output buffer sets rotate, and a
set is decompressed two steps after it was compressed, so that neither kernel finds
its input in the 256 MB Infinity Cache (steady state of a pipelined round trip).

Printed (one JSON line on stdout):
  value      BF16 bytes handled per second by the step: (2n compressed + 2n decompressed)
             / step wall time, in GB/s (the harmonic mean of the two codec directions);
  roofline   for the step's dominant operation (compress: compress_single_kernel,
             or decompress: decompress_kernel, whichever takes longer): algorithmic HBM
             bytes per launch (2n BF16 bytes + static part + escapes) / average launch
             time, from HIP events on the launch stream around back-to-back launches over
             the rotating sets, against the 8 TB/s HBM peak; traffic: the HBM bytes per
             launch that rocprofv3's FETCH_SIZE and WRITE_SIZE counters measured
             (profiles/pmc_traffic_bucket_64m.txt; null when that was taken on other
             kernel sources); roofline_other_op for the other operation;
  cpu_baseline  the plain C oracle, single-threaded, on the same bucket;
  per_config the other workloads (1 Mi chunk, activations with escapes and specials,
             MoE dispatch buckets, the same dispatch compressed from the unpermuted
             token matrix by row index (against a permute copy + compress), the
             all-gather receive side decoding 16 separately
             compressed shards in one launch, reduce-scatter share with decode-accumulate
             and the two-stream pipeline), each with GB/s and HBM fraction.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "codec GB/s (bf16 in) compress/decompress, % of HBM peak, compression ratio"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def median(v):
    return statistics.median(v) if v else float("nan")


class Timer:
    """HIP events on the launch stream (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def ms(self):
        self.torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in self.pairs]


def to_dev(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


class BatchCodec:
    """Device buffers for one workload: R rotating sets of inputs and outputs, each with
    its compress and decompress calls marshalled once."""

    def __init__(self, torch, Z, segments, sigmas, sets):
        self.torch, self.Z = torch, Z
        self.sizes = [s.size for s in segments]
        self.n = sum(self.sizes)
        self.sigmas = sigmas
        self.static_bytes = sum(Z.static_size(n) for n in self.sizes)
        self.ws = torch.zeros(Z.workspace_size(self.n, len(self.sizes)), dtype=torch.uint8, device="cuda")
        self.n_esc = torch.zeros(len(self.sizes) + 1, dtype=torch.int64, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.sets = []
        for _ in range(sets):
            ins = [to_dev(torch, s) for s in segments]
            st = dict(
                ins=ins,
                static=torch.empty(self.static_bytes, dtype=torch.uint8, device="cuda"),
                esc=torch.empty(self.n, dtype=torch.uint8, device="cuda"),
                outs=[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in self.sizes])
            st["c"] = Z.PreparedCompress(ins, st["static"], st["esc"], self.ws, self.n_esc, self.status)
            st["d"] = Z.PreparedDecompress(st["static"], st["esc"], st["outs"], self.status)
            self.sets.append(st)

    def plans(self):
        return self.Z.plan_many(self.sigmas)

    def compress(self, k, plans):
        self.sets[k % len(self.sets)]["c"].run(plans)

    def decompress(self, k):
        self.sets[k % len(self.sets)]["d"].run()

    def verify(self):
        """One clean round trip per set, compared on the device with the inputs."""
        plans = self.plans()
        ok = True
        for k in range(len(self.sets)):
            self.compress(k, plans)
            self.decompress(k)
        self.torch.cuda.synchronize()
        ok = int(self.status.item()) == 0
        for s in self.sets:
            for a, b in zip(s["ins"], s["outs"]):
                ok = ok and bool(self.torch.equal(a.view(self.torch.int16), b.view(self.torch.int16)))
        return ok

    def n_esc_total(self):
        return int(self.n_esc[-1].item())


def compress_bytes(n, static_bytes, n_esc):
    return 2 * n + static_bytes + n_esc


LAG = 2   # a set is decompressed two iterations after it was compressed


def run_codec(torch, bc, iters, warmup):
    """Steady-state loop, timed by the host clock between two device synchronisations.
    Iteration i plans the tables on the host, compresses set i % R and decompresses set
    (i - LAG) % R, compressed LAG iterations earlier; in between, other sets' traffic
    (> 2 x 256 MB) has gone through, so neither kernel finds its input in the Infinity
    Cache.  Returns the wall ms per step."""
    R = len(bc.sets)
    assert R > LAG
    plans = bc.plans()
    for i in range(-LAG, 0):
        bc.compress(i % R, plans)
    for i in range(warmup):
        bc.compress(i % R, plans)
        bc.decompress((i - LAG) % R)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, warmup + iters):
        plans = bc.plans()                  # sigma -> tables, on the host
        bc.compress(i % R, plans)
        bc.decompress((i - LAG) % R)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / iters * 1e3


def op_times(torch, bc, rounds, batches=3):
    """Average launch times (ms) of compress and decompress over back-to-back launches on
    the rotating sets: the median over `batches` batches, so that one disturbed batch
    does not set the figure."""
    plans = bc.plans()
    cs, ds = [], []
    for _ in range(batches):
        cs.append(batched_ms(torch, lambda k: bc.compress(k, plans), len(bc.sets), rounds))
        ds.append(batched_ms(torch, bc.decompress, len(bc.sets), rounds))
    return median(cs), median(ds)


def batched_ms(torch, fn, sets, rounds):
    """Average time of one launch of fn(k) over rounds x sets back-to-back launches on
    the rotating sets, from two HIP events on the launch stream around the whole batch
    (the events' own latency is then not counted per launch).  One untimed round comes
    first: the first launch of a kernel also loads it."""
    for k in range(sets):
        fn(k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(rounds):
        for k in range(sets):
            fn(k)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (rounds * sets)


def codec_report(bc, c, d):
    """Per-operation figures from average launch times c, d (ms)."""
    n_esc = bc.n_esc_total()
    moved = compress_bytes(bc.n, bc.static_bytes, n_esc)
    return {
        "elements": bc.n,
        "segments": len(bc.sizes),
        "compress_us": round(c * 1e3, 2),
        "decompress_us": round(d * 1e3, 2),
        "compress_GBps": round(2 * bc.n / (c * 1e-3) / 1e9, 1),
        "decompress_GBps": round(2 * bc.n / (d * 1e-3) / 1e9, 1),
        "compress_hbm_frac": round(moved / (c * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "decompress_hbm_frac": round(moved / (d * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "ratio": round(2 * bc.n / (bc.static_bytes + n_esc), 5),
        "bits_per_value": round(8 * (bc.static_bytes + n_esc) / bc.n, 4),
        "escape_frac": round(n_esc / bc.n, 5),
    }


def bench_rs(torch, Z, W, iters):
    """Reduce-scatter receive share: 7 peer shards x 64 Mi, 32 chunks of 2 Mi values."""
    wl = W.rs_512m()
    P, chunk, n = wl.extra["peers"], wl.extra["chunk"], wl.extra["shard"]
    plans = [Z.plan(sigma=s) for s in wl.sigmas]
    peers = [to_dev(torch, s) for s in wl.segments]
    local = to_dev(torch, wl.extra["local"])
    dst = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    nch = n // chunk
    S = Z.static_size(chunk)
    # every chunk's compressed output kept (as a receiver would hold what arrived)
    static = torch.empty(nch * P * S, dtype=torch.uint8, device="cuda")
    esc = torch.empty(nch * P * chunk, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(Z.workspace_size(P * chunk, P), dtype=torch.uint8, device="cuda")
    n_esc = torch.zeros(nch, P + 1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    comp = [Z.PreparedCompress([p[c * chunk:(c + 1) * chunk] for p in peers], static[c * P * S:(c + 1) * P * S],
                               esc[c * P * chunk:(c + 1) * P * chunk], ws, n_esc[c], status) for c in range(nch)]
    # the same 32 calls through zipccl_compress_chunks: 8 chunks (56 segments) share a
    # launch, with a workspace that holds them (as the pipeline's does)
    ws2 = torch.zeros(Z.workspace_size(8 * P * chunk, 8 * P), dtype=torch.uint8, device="cuda")
    comp_seq = Z.PreparedCompressChunks([[p[c * chunk:(c + 1) * chunk] for p in peers] for c in range(nch)],
                                        [static[c * P * S:(c + 1) * P * S] for c in range(nch)],
                                        [esc[c * P * chunk:(c + 1) * P * chunk] for c in range(nch)], ws2,
                                        n_esc.view(-1), status)
    acc = [Z.PreparedAccumulate([static.data_ptr() + (c * P + p) * S for p in range(P)],
                                [esc.data_ptr() + c * P * chunk] * P, chunk, local[c * chunk:], dst[c * chunk:],
                                status, esc_bytes=[P * chunk] * P) for c in range(nch)]

    # the 32 decode-accumulates through zipccl_decompress_accumulate_chunks (18 chunks of
    # 7 peers per launch)
    acc_seq = Z.PreparedAccumulateChunks([static.data_ptr() + (c * P + p) * S for c in range(nch) for p in range(P)],
                                         [esc.data_ptr() + c * P * chunk for c in range(nch) for _ in range(P)],
                                         P, chunk, n, local, dst, status, esc_bytes=[P * chunk] * (P * nch))

    def compress_all():
        comp_seq.run(plans)

    def compress_calls():
        for c in range(nch):
            comp[c].run(plans)

    def accumulate_all():
        acc_seq.run()

    def accumulate_calls():
        for c in range(nch):
            acc[c].run()

    compress_all()
    accumulate_all()
    # per pass over the 32 chunks: back-to-back passes between two events, as the other
    # workloads are timed (launch ramp-up and drain amortised), and single passes
    c_ms = batched_ms(torch, lambda k: compress_all(), 1, iters)
    a_ms = batched_ms(torch, lambda k: accumulate_all(), 1, iters)
    tc, ta = Timer(torch), Timer(torch)
    for _ in range(iters):
        e = tc.start()
        compress_all()
        tc.stop(e)
        e = ta.start()
        accumulate_all()
        ta.stop(e)
    c1_ms, a1_ms = median(tc.ms()), median(ta.ms())
    tp, tq = Timer(torch), Timer(torch)
    for _ in range(iters):
        e = tp.start()
        compress_calls()
        tp.stop(e)
        e = tq.start()
        accumulate_calls()
        tq.stop(e)
    cp_ms, ap_ms = median(tp.ms()), median(tq.ms())
    total_esc = int(n_esc[:, -1].sum().item())
    static_total = nch * P * S
    comp_moved = 2 * P * n + static_total + total_esc
    acc_moved = static_total + total_esc + 2 * n + 2 * n
    # two-stream pipeline, wall time
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    pipe = Z.Pipeline(P, chunk, sa, sb)
    pipe.reduce(peers, plans, local, dst, status)
    torch.cuda.synchronize()
    walls = []
    for _ in range(iters):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pipe.reduce(peers, plans, local, dst, status)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    pipe.close()
    ok = int(status.item()) == 0
    wall = median(walls)
    return {
        "elements_per_peer": n, "peers": P, "chunk": chunk, "chunks": nch,
        "compress_us": round(c_ms * 1e3, 1),
        "compress_GBps": round(2 * P * n / (c_ms * 1e-3) / 1e9, 1),
        "compress_hbm_frac": round(comp_moved / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "compress_single_pass_us": round(c1_ms * 1e3, 1),
        "compress_separate_calls_us": round(cp_ms * 1e3, 1),
        "accumulate_us": round(a_ms * 1e3, 1),
        "accumulate_GBps_bf16_in": round(2 * P * n / (a_ms * 1e-3) / 1e9, 1),
        "accumulate_hbm_frac": round(acc_moved / (a_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "accumulate_single_pass_us": round(a1_ms * 1e3, 1),
        "accumulate_separate_calls_us": round(ap_ms * 1e3, 1),
        "pipeline_wall_us": round(wall * 1e6, 1),
        "pipeline_GBps_bf16_in": round(2 * P * n / wall / 1e9, 1),
        "ratio": round(2 * P * n / (static_total + total_esc), 5),
        "escape_frac": round(total_esc / (P * n), 5),
        "status_ok": ok,
    }


def bench_allgather(torch, Z, W, rounds):
    """All-gather receive side: the bucket's 16 layers as 16 ranks' shards, each
    compressed by its own call into its own buffers, all decoded by one
    zipccl_decompress_shards launch into the gathered 64 Mi tensor.  Two rotating sets
    (> 2 x 256 MB together) keep the inputs out of the Infinity Cache."""
    wl = W.bucket_64m()
    plans = [Z.plan(sigma=s) for s in wl.sigmas]
    sizes = [s.size for s in wl.segments]
    n = sum(sizes)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sets = []
    n_esc = 0
    for k in range(2):
        comp = [Z.compress_tensors([to_dev(torch, seg)], [pl]) for seg, pl in zip(wl.segments, plans)]
        torch.cuda.synchronize()
        if k == 0:
            n_esc = sum(int(c.n_esc[-1].item()) for c in comp)
        out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        call = Z.PreparedDecompressShards([c.static for c in comp], [c.esc for c in comp],
                                          list(torch.split(out, sizes)), status)
        sets.append(dict(out=out, call=call))
    d = batched_ms(torch, lambda k: sets[k % 2]["call"].run(), 2, rounds)
    want = torch.cat([to_dev(torch, seg) for seg in wl.segments])
    ok = int(status.item()) == 0
    ok = ok and all(bool(torch.equal(s["out"].view(torch.int16), want.view(torch.int16))) for s in sets)
    moved = sum(Z.static_size(m) for m in sizes) + n_esc + 2 * n
    return {
        "elements": n, "shards": len(sizes),
        "decompress_us": round(d * 1e3, 2),
        "decompress_GBps": round(2 * n / (d * 1e-3) / 1e9, 1),
        "decompress_hbm_frac": round(moved / (d * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "parity_round_trip": ok,
    }


def bench_moe_gather(torch, Z, W, rounds):
    """MoE dispatch from the unpermuted token matrix: the 8 destinations' rows compressed
    in one zipccl_compress_gather launch, against a permute copy (torch index_select)
    followed by zipccl_compress of the permuted buckets.  Two rotating sets."""
    import numpy as np
    wl = W.moe_routed_16384x7168()
    H, rows = wl.extra["hidden"], wl.extra["rows"]
    T = wl.segments[0].size // H
    plans = [Z.plan(sigma=s) for s in wl.sigmas]
    sizes = [len(r) * H for r in rows]
    n = sum(sizes)
    static_bytes = sum(Z.static_size(m) for m in sizes)
    ws = torch.zeros(Z.workspace_size(n, len(sizes)), dtype=torch.uint8, device="cuda")
    n_esc = torch.zeros(len(sizes) + 1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    order = torch.from_numpy(np.concatenate(rows).astype(np.int64)).cuda()
    sets = []
    for _ in range(2):
        mat = to_dev(torch, wl.segments[0]).view(T, H)
        rows_t = [torch.from_numpy(r).cuda() for r in rows]
        st = torch.empty(static_bytes, dtype=torch.uint8, device="cuda")
        esc = torch.empty(n, dtype=torch.uint8, device="cuda")
        perm = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        bufs = list(torch.split(perm, sizes))
        sets.append(dict(
            mat=mat, perm=perm, st=st, esc=esc,
            gather=Z.PreparedCompressGather(list(zip([mat] * len(rows_t), rows_t, plans)), st, esc, ws, n_esc, status),
            compress=Z.PreparedCompress(bufs, st, esc, ws, n_esc, status)))

    def permute(k):
        s = sets[k % 2]
        torch.index_select(s["mat"], 0, order, out=s["perm"].view(-1, H))

    g = batched_ms(torch, lambda k: sets[k % 2]["gather"].run(plans), 2, rounds)
    # parity: the gathered compress equals the compress of the permuted copy, byte for byte
    s0 = sets[0]
    s0["gather"].run(plans)
    torch.cuda.synchronize()
    st_g, esc_g = s0["st"].clone(), s0["esc"][:int(n_esc[-1].item())].clone()
    # torch's row gather, timed launch by launch (median); at the copy ceiling a permute
    # of these bytes could not take less than 2 x 235 MB / (5 TB/s), ~94 us
    pm_all = []
    for k in range(2 * rounds):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        permute(k)
        e1.record()
        torch.cuda.synchronize()
        pm_all.append(e0.elapsed_time(e1))
    pm = median(pm_all)
    cp = batched_ms(torch, lambda k: sets[k % 2]["compress"].run(plans), 2, rounds)
    permute(0)
    s0["compress"].run(plans)
    torch.cuda.synchronize()
    total_esc = int(n_esc[-1].item())
    ok = (int(status.item()) == 0 and bool(torch.equal(st_g, s0["st"]))
          and bool(torch.equal(esc_g, s0["esc"][:total_esc])))
    moved = compress_bytes(n, static_bytes, total_esc)
    return {
        "elements": n, "segments": len(sizes),
        "gather_compress_us": round(g * 1e3, 2),
        "gather_compress_GBps": round(2 * n / (g * 1e-3) / 1e9, 1),
        "gather_compress_hbm_frac": round(moved / (g * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "permute_us": round(pm * 1e3, 2),
        "compress_permuted_us": round(cp * 1e3, 2),
        "permute_plus_compress_us": round((pm + cp) * 1e3, 2),
        "parity_vs_permuted": ok,
    }


def bench_switcher(torch, Z, W):
    """The reduce-scatter switcher on this GPU: the codec profile on one 2 Mi-value chunk of
    the reduce-scatter share with 7 peers, and the choice for the share's full size
    (1 GiB of BF16 per rank over 8 ranks) on three kinds of link."""
    wl = W.rs_512m()
    x = to_dev(torch, wl.segments[0][:wl.extra["chunk"]])
    prof = Z.profile_codec(x, Z.plan(sigma=wl.sigmas[0]), wl.extra["peers"])
    links = {"xgmi_7x153GBps": Z.LinkT(153.0, 2.0, 7), "pcie5_x16_64GBps": Z.LinkT(64.0, 5.0, 1),
             "ib_ndr_50GBps": Z.LinkT(50.0, 5.0, 1)}
    out = {"compress_GBps": round(prof.compress_GBps, 1), "accumulate_GBps": round(prof.accumulate_GBps, 1),
           "compressed_fraction": round(prof.compressed_fraction, 5), "ranks": 8, "bytes_per_rank": 8 * wl.extra["shard"] * 2}
    for name, link in links.items():
        use, tn, tz = Z.rs_choose(prof, link, 8, out["bytes_per_rank"])
        out[name] = {"use_codec": use, "native_us": round(tn, 1), "zipped_us": round(tz, 1)}
    return out


def bench_estimated_plans(torch, Z, W, rounds):
    """The bucket coded with plans estimated on the device (every 16th tile of 512 values)
    instead of the layers' known sigmas: the estimate's launch time, the compress with
    device plans, and the compressed size against the known-sigma plans."""
    wl = W.bucket_64m()
    tens = [to_dev(torch, x) for x in wl.segments]
    n = wl.n_total
    k = len(tens)
    plans_dev = torch.empty(8 * k, dtype=torch.uint8, device="cuda")
    est_ws = torch.empty(Z.estimate_workspace_size(k), dtype=torch.uint8, device="cuda")
    static_bytes = sum(Z.static_size(x.size) for x in wl.segments)
    st = torch.empty(static_bytes, dtype=torch.uint8, device="cuda")
    esc = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(Z.workspace_size(n, k), dtype=torch.uint8, device="cuda")
    n_esc = torch.zeros(k + 1, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    # both calls marshalled once, so that the launch times are the GPU's
    import ctypes
    segs = Z._segment_array(tens)
    L = Z.lib()
    est_args = (segs, k, 16, ctypes.c_void_p(plans_dev.data_ptr()), ctypes.c_void_p(est_ws.data_ptr()),
                est_ws.numel(), None)
    comp_args = (segs, k, ctypes.c_void_p(plans_dev.data_ptr()), ctypes.c_void_p(st.data_ptr()), st.numel(),
                 ctypes.c_void_p(esc.data_ptr()), esc.numel(), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                 ctypes.c_void_p(n_esc.data_ptr()), ctypes.c_void_p(status.data_ptr()), None)
    # 4 launches per timed round on the same buffers (the compress then finds part of its
    # input in the 256 MB Infinity Cache: an indication, not a cold-HBM figure)
    est = batched_ms(torch, lambda _: L.zipccl_estimate_plans(*est_args), 4, rounds)
    comp = batched_ms(torch, lambda _: L.zipccl_compress_device_plans(*comp_args), 4, rounds)
    torch.cuda.synchronize()
    esc_est = int(n_esc[-1].item())
    raw = plans_dev.cpu().numpy().tobytes()
    same = sum(list(Z.PlanT.from_buffer_copy(raw[8 * i:8 * i + 8]).exponents) == Z.plan(sigma=s).exponents
               for i, s in enumerate(wl.sigmas))
    Z.compress(list(zip(tens, Z.plan_many(wl.sigmas))), st, esc, ws, n_esc, status)
    torch.cuda.synchronize()
    esc_known = int(n_esc[-1].item())
    return {"elements": n, "segments": k, "estimate_us": round(est * 1e3, 2),
            "compress_device_plans_us": round(comp * 1e3, 2),
            "ratio_estimated": round(2 * n / (static_bytes + esc_est), 5),
            "ratio_known_sigma": round(2 * n / (static_bytes + esc_known), 5),
            "tables_equal_to_known_sigma": f"{same}/{k}", "status_ok": int(status.item()) == 0}


def copy_ceiling(torch, iters=10):
    """A plain 1 GiB device-to-device copy: the practical HBM ceiling (read + write bytes / s)."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    t = Timer(torch)
    for _ in range(iters):
        e = t.start()
        b.copy_(a)
        t.stop(e)
    ms = median(t.ms())
    del a, b
    torch.cuda.empty_cache()
    return round(2 * (1 << 30) / (ms * 1e-3) / 1e9, 1)


def cpu_baseline(W, O, wl, reps):
    import numpy as np
    tables = [O.plan_sigma(s) for s in wl.sigmas]
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        st, esc, ne, rc = O.compress_batch(wl.segments, tables)
        t1 = time.perf_counter()
        off_st, off_esc = 0, 0
        for x in wl.segments:
            sz = O.static_size(x.size)
            O.decompress(st[off_st:off_st + sz], esc, x.size)
            off_st += sz
        t2 = time.perf_counter()
        times.append((t1 - t0, t2 - t1))
    c = median([t[0] for t in times])
    d = median([t[1] for t in times])
    n = wl.n_total
    out = {"value": round(4 * n / (c + d) / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{wl.name} full bucket ({n} values), compress + decompress, median of {reps}, 1 thread",
           "compress_GBps": round(2 * n / c / 1e9, 4), "decompress_GBps": round(2 * n / d / 1e9, 4),
           "host_cpus": os.cpu_count()}
    # the same oracle on every host thread (at most 16), one layer per task: the C calls
    # release the interpreter lock, and the layers are independent
    from concurrent.futures import ThreadPoolExecutor
    threads = max(1, min(16, os.cpu_count() or 1, len(wl.segments)))

    def one(k):
        x = wl.segments[k]
        st, esc, _ = O.compress(x, tables[k])
        O.decompress(st, esc, x.size)

    with ThreadPoolExecutor(threads) as pool:
        t0 = time.perf_counter()
        list(pool.map(one, range(len(wl.segments))))
        wall = time.perf_counter() - t0
    out["all_threads"] = {"threads": threads, "value": round(4 * n / wall / 1e9, 4), "unit": "GB/s",
                          "sample": "the same bucket, compress + decompress of each layer as one task"}
    return out


# ------------------------------------------------------------------------------------
# rocprofv3 summaries kept under profiles/ (text), and the measured HBM traffic
# ------------------------------------------------------------------------------------
KERNEL_SRC = os.path.join(ROOT, "lossless_bf16_exponent_codec_amd", "csrc", "zipccl_kernels.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "pmc_traffic_bucket_64m.txt")
TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/stats -o bench -- "
             "python3 bench.py --steps 20 --warmup 3 --no-cpu-baseline --no-extra")
PMC_CMD = ("rocprofv3 --pmc {counter} --output-format csv -d rocprof_out/pmc_{counter} -o run -- "
           "python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-extra")
RS_TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/stats_rs -o rs -- "
                "python3 bench.py --only rs_512m")
OUR_KERNELS = ("compress_single_kernel", "encode_kernel", "place_direct_kernel", "scan_kernel", "place_kernel",
               "decompress_kernel", "accumulate_kernel")
COPY_KERNEL = "__amd_rocclr_copyBuffer"
GIB = 1 << 30


def kernel_source_sha256():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def short_kernel_name(name):
    for k in OUR_KERNELS:
        if k in name:
            return k
    return COPY_KERNEL if COPY_KERNEL in name else None


def summarize_stats(csv_path, out_path, rs=False):
    """profiles/ text from rocprofv3 --stats (kernel_stats.csv) of TRACE_CMD (or, with rs,
    of RS_TRACE_CMD)."""
    import csv
    rows = [r for r in csv.DictReader(open(csv_path)) if short_kernel_name(r["Name"]) in OUR_KERNELS]
    title = ("# Kernel durations, rs_512m (7 peers x 64 Mi BF16 values in 32 chunks of 2 Mi)" if rs else
             "# Kernel durations, bucket_64m (16 x 4 Mi BF16 values, one table per layer)")
    lines = [title, "",
             "Command (from the repository root on the GPU host; rocprofv3's own averages):", "",
             "    " + (RS_TRACE_CMD if rs else TRACE_CMD), "",
             f"Kernel source sha256: `{kernel_source_sha256()}`", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {short_kernel_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    if rs:
        lines += ["", "The chunk compresses run as separate calls (compress_single_kernel, 7 segments of",
                  "2 Mi values each) and through zipccl_compress_chunks and the pipeline",
                  "(compress_single_kernel over 8 chunks, 56 segments, per launch); decode-accumulate",
                  "runs one chunk per launch and 18 chunks per launch (accumulate_kernel)."]
    else:
        lines += ["", "Calls include the warmup and verification round trips; all launches are of the",
                  "bucket workload (compress: compress_single_kernel, decompress: decompress_kernel)."]
    open(out_path, "w").write("\n".join(lines) + "\n")


def summarize_pmc(fetch_csv, write_csv, out_path, n_units=4096):
    """profiles/ text from two rocprofv3 --pmc runs of PMC_CMD (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch).  Each counter is scaled by what it reads for the
    bench's 1 GiB device-to-device copy (the copy reads and writes 1 GiB).  Bucket
    launches are told apart from others by grid size."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            k = short_kernel_name(r["Kernel_Name"])
            if k is None:
                continue
            grid = int(r["Grid_Size"])
            acc.setdefault((k, grid), []).append(float(r["Counter_Value"]))
        return {key: sum(v) / len(v) for key, v in acc.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy_f = max(v for (k, g), v in f.items() if k == COPY_KERNEL)
    copy_w = max(v for (k, g), v in w.items() if k == COPY_KERNEL)
    sf, sw = (GIB / 1024) / copy_f, (GIB / 1024) / copy_w      # true KiB per counted KiB
    cmp_ = ("compress_single_kernel", (n_units + (n_units + 7) // 8) * 512)
    dec = ("decompress_kernel", n_units * 512)
    kib = {k: (f[k] * sf, w[k] * sw) for k in (cmp_, dec)}
    comp = sum(kib[cmp_])
    decomp = sum(kib[dec])
    lines = ["# Measured HBM traffic, bucket_64m (16 x 4 Mi BF16 values)", "",
             "Commands (from the repository root on the GPU host), one run per counter:", "",
             "    " + PMC_CMD.format(counter="FETCH_SIZE"), "    " + PMC_CMD.format(counter="WRITE_SIZE"), "",
             f"Scale factors from the 1 GiB copy in the same runs: FETCH_SIZE x{sf:.4f}, WRITE_SIZE x{sw:.4f}",
             f"(the copy counted {copy_f:.0f} KiB fetched and {copy_w:.0f} KiB written per dispatch).", "",
             "| kernel | grid | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
             "|---|---|---|---|---|---|"]
    for k in (cmp_, dec):
        lines.append(f"| {k[0]} | {k[1]} | {f[k]:.1f} | {w[k]:.1f} | {kib[k][0] * 1024 / 1e6:.2f} | "
                     f"{kib[k][1] * 1024 / 1e6:.2f} |")
    lines += ["", "Machine-readable (bench.py reports these as roofline.traffic while the kernel",
              "source hash matches; bytes per launch):", "", "```",
              f"source_sha256={kernel_source_sha256()}",
              f"compress_traffic_bytes={int(comp * 1024)}",
              f"decompress_traffic_bytes={int(decomp * 1024)}", "```"]
    open(out_path, "w").write("\n".join(lines) + "\n")


RS_PMC_CMD = ("rocprofv3 --pmc {counter} --output-format csv -d rocprof_out/pmc_rs_{counter} -o run -- "
              "python3 bench.py --only rs_512m")


def summarize_pmc_rs(fetch_csv, write_csv, out_path):
    """profiles/ text from two rocprofv3 --pmc runs of RS_PMC_CMD (FETCH_SIZE, then
    WRITE_SIZE): HBM bytes per launch of the reduce-scatter share's kernels, per value,
    against the algorithmic bytes (decode-accumulate: 7 peers x ~1.40 B + 2 B local + 2 B
    out per output value; compress: 2 B in + ~1.40 B out per value).  Scaled by the
    counters' reading of the 1 GiB copy in the same runs.  A decode-accumulate launch has a
    workgroup per 4096 outputs; a compress launch ceil(units / 8) placing workgroups after
    its units of 16384 values."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            k = short_kernel_name(r["Kernel_Name"])
            if k is None:
                continue
            acc.setdefault((k, int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return {key: (sum(v) / len(v), len(v)) for key, v in acc.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy_f = max(v for (k, g), (v, c) in f.items() if k == COPY_KERNEL)
    copy_w = max(v for (k, g), (v, c) in w.items() if k == COPY_KERNEL)
    sf, sw = (GIB / 1024) / copy_f, (GIB / 1024) / copy_w
    lines = ["# Measured HBM traffic, rs_512m (7 peers x 64 Mi BF16 values, 32 chunks of 2 Mi)", "",
             "Commands (from the repository root on the GPU host), one run per counter:", "",
             "    " + RS_PMC_CMD.format(counter="FETCH_SIZE"), "    " + RS_PMC_CMD.format(counter="WRITE_SIZE"), "",
             f"Scale factors from the 1 GiB copy in the same runs: FETCH_SIZE x{sf:.4f}, WRITE_SIZE x{sw:.4f}.",
             f"Kernel source sha256: `{kernel_source_sha256()}`", "",
             "| kernel | grid | launches | values | read MB | write MB | B per value | algorithmic B per value |",
             "|---|---|---|---|---|---|---|---|"]
    for (k, grid) in sorted(set(f) & set(w)):
        if k == COPY_KERNEL:
            continue
        (fv, nl), (wv, _) = f[(k, grid)], w[(k, grid)]
        rd, wr = fv * sf * 1024, wv * sw * 1024
        wgs = grid // 512
        if k == "accumulate_kernel":
            vals, alg = wgs * 4096, "13.80 (per output)"
        elif k == "compress_single_kernel":
            units = wgs - (wgs + 8) // 9   # wgs = units + ceil(units / 8)
            while units + (units + 7) // 8 < wgs:
                units += 1
            vals, alg = units * 16384, "3.40"
        else:
            continue
        lines.append(f"| {k} | {grid} | {nl} | {vals} | {rd / 1e6:.2f} | {wr / 1e6:.2f} | "
                     f"{(rd + wr) / vals:.3f} | {alg} |")
    lines += ["", "Values per launch follow from the grid (the last chunk of a launch may be short, so",
              "they are upper bounds for the smaller launches)."]
    open(out_path, "w").write("\n".join(lines) + "\n")


SQ_COUNTERS = "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_BUSY_CYCLES"
SQ_CMD = ("rocprofv3 --pmc " + SQ_COUNTERS + " --output-format csv -d rocprof_out/pmc_sq_rs -o run -- "
          "python3 bench.py --only rs_512m")


def summarize_sq(csv_path, out_path):
    """profiles/ text from one rocprofv3 --pmc run of SQ_CMD: instruction counts per
    launch of the reduce-scatter kernels, and the VALU issue time they imply (a wave64
    VALU instruction occupies a SIMD for 4 cycles; 1024 SIMDs at 2.4 GHz)."""
    import csv
    acc = {}
    for r in csv.DictReader(open(csv_path)):
        k = short_kernel_name(r["Kernel_Name"])
        if k is None or k == COPY_KERNEL:
            continue
        grid = int(r.get("Grid_Size", 0) or 0)
        acc.setdefault((k, grid), {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = ["# Instruction counts, rs_512m kernels (rocprofv3 SQ counters, mean per launch)", "",
             "Command (from the repository root on the GPU host):", "", "    " + SQ_CMD, "",
             f"Kernel source sha256: `{kernel_source_sha256()}`", "",
             "| kernel | grid | launches | waves | VALU | SALU | LDS | VMEM rd | VMEM wr | VALU issue us |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for (k, grid), d in sorted(acc.items()):
        m = {c: sum(v) / len(v) for c, v in d.items()}
        n = len(next(iter(d.values())))
        valu_us = m.get("SQ_INSTS_VALU", 0) * 4 / 1024 / 2.4e3
        lines.append(f"| {k} | {grid} | {n} | {m.get('SQ_WAVES', 0):.0f} | {m.get('SQ_INSTS_VALU', 0):.0f} | "
                     f"{m.get('SQ_INSTS_SALU', 0):.0f} | {m.get('SQ_INSTS_LDS', 0):.0f} | "
                     f"{m.get('SQ_INSTS_VMEM_RD', 0):.0f} | {m.get('SQ_INSTS_VMEM_WR', 0):.0f} | {valu_us:.2f} |")
    lines += ["", "Counters are per launch (the profiler serialises launches).  VALU issue us = VALU",
              "instructions x 4 cycles / 1024 SIMDs / 2.4 GHz: the time the launch's VALU work",
              "needs if every SIMD issued one wave64 VALU instruction every 4 cycles."]
    open(out_path, "w").write("\n".join(lines) + "\n")


def measured_traffic():
    """Bytes per launch from the committed PMC summary, or {} if it is missing or was
    taken on another version of the kernels."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return {}
    kv = dict(line.split("=", 1) for line in text.splitlines() if "=" in line and " " not in line.strip())
    if kv.get("source_sha256") != kernel_source_sha256():
        return {}
    return {"compress": int(kv["compress_traffic_bytes"]), "decompress": int(kv["decompress_traffic_bytes"])}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=4, help="rotating buffer sets (> 2)")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--summarize-stats", nargs=2, metavar=("KERNEL_STATS_CSV", "OUT_MD"),
                    help="write a profiles/ summary of a rocprofv3 --stats run and exit")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD"),
                    help="write a profiles/ summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-rs-stats", nargs=2, metavar=("KERNEL_STATS_CSV", "OUT_MD"),
                    help="write a profiles/ summary of a rocprofv3 --stats run of --only rs_512m and exit")
    ap.add_argument("--summarize-rs-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD"),
                    help="write a profiles/ summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "--only rs_512m and exit")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("COUNTER_CSV", "OUT_MD"),
                    help="write a profiles/ summary of a rocprofv3 SQ-counter run of --only rs_512m and exit")
    ap.add_argument("--only", default=None,
                    help="run one of the other workloads alone (for profiling) and print its figures")
    args = ap.parse_args(argv)
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return 0
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return 0
    if args.summarize_rs_stats:
        summarize_stats(*args.summarize_rs_stats, rs=True)
        return 0
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq)
        return 0
    if args.summarize_rs_pmc:
        summarize_pmc_rs(*args.summarize_rs_pmc)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the codec's hot path is single-GPU and there is no "
              f"multi-GPU path; --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only (WORLD_SIZE > 1 given)", file=sys.stderr)
        return 2

    import torch
    from lossless_bf16_exponent_codec_amd import workloads as W
    from lossless_bf16_exponent_codec_amd import zipccl as Z
    torch.cuda.set_device(0)

    if args.only:
        runners = {"rs_512m": lambda: bench_rs(torch, Z, W, 5),
                   "rs_switcher": lambda: bench_switcher(torch, Z, W),
                   "bucket_64m_estimated_plans": lambda: bench_estimated_plans(torch, Z, W, 5),
                   "allgather_16x4m": lambda: bench_allgather(torch, Z, W, 5),
                   "moe_routed_16384x7168": lambda: bench_moe_gather(torch, Z, W, 5)}
        if args.only not in runners:
            print(f"--only takes one of {sorted(runners)}", file=sys.stderr)
            return 2
        res = runners[args.only]()
        # the 1 GiB copy whose counter readings scale a --pmc run of this command
        print(json.dumps({"workload": args.only, **res, "hbm_copy_GBps": copy_ceiling(torch)}), flush=True)
        return 0

    log("generating bucket_64m")
    wl = W.bucket_64m()
    bc = BatchCodec(torch, Z, wl.segments, wl.sigmas, args.sets)
    n = bc.n

    log(f"warmup {args.warmup}, timing {args.steps} steps")
    ms_per_step = run_codec(torch, bc, args.steps, args.warmup)
    value = 4 * n / (ms_per_step * 1e-3) / 1e9
    # per-launch averages (roofline, per-operation figures): back-to-back launches over
    # the rotating sets
    c_avg, d_avg = op_times(torch, bc, max(2, args.steps // len(bc.sets)))
    ok = bc.verify()
    rep = codec_report(bc, c_avg, d_avg)
    n_esc = bc.n_esc_total()
    moved = compress_bytes(n, bc.static_bytes, n_esc)

    traffic = measured_traffic()

    def roof(name, op, avg_ms, launches):
        ach = moved / (avg_ms * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": name, "launches": launches, "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                "bytes_per_launch": moved, "avg_launch_us": round(avg_ms * 1e3, 2), "traffic": traffic.get(op)}

    # the step's dominant operation: decompress is one launch; so is compress
    # (compress_single_kernel; encode_kernel, scan_kernel, place_kernel above 2^28 values)
    units = sum((m + 16383) // 16384 for m in bc.sizes)
    c_launches = (["compress_single_kernel"] if units <= 16384
                  else ["encode_kernel", "scan_kernel", "place_kernel"])
    roof_d = roof("decompress_kernel", "decompress", d_avg, ["decompress_kernel"])
    roof_c = roof("compress", "compress", c_avg, c_launches)
    primary, secondary = (roof_d, roof_c) if d_avg >= c_avg else (roof_c, roof_d)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": "bucket_64m: gradient bucket of 16 layers x 4194304 BF16 values, "
                               "N(0, sigma_l), sigma_l log-uniform in [1e-4, 1e-1], one table per layer",
                   "elements": n, "segments": len(bc.sizes), "rotating_sets": args.sets},
        "compress_GBps": rep["compress_GBps"],
        "decompress_GBps": rep["decompress_GBps"],
        "compress_hbm_frac": rep["compress_hbm_frac"],
        "decompress_hbm_frac": rep["decompress_hbm_frac"],
        "ratio": rep["ratio"],
        "bits_per_value": rep["bits_per_value"],
        "escape_frac": rep["escape_frac"],
        "parity_round_trip": ok,
        "roofline": primary,
        "roofline_other_op": secondary,
    }
    log("copy ceiling")
    out["hbm_copy_GBps"] = copy_ceiling(torch)
    out["roofline"]["frac_of_copy"] = round(out["roofline"]["achieved"] / out["hbm_copy_GBps"], 4)
    if not args.no_extra:
        per = {"bucket_64m": rep}
        for name in ("chunk_1m", "act_8192x7168", "moe_16384x7168"):
            log(f"workload {name}")
            w2 = W.get(name)
            sets = 8 if name == "chunk_1m" else 4
            b2 = BatchCodec(torch, Z, w2.segments, w2.sigmas, sets)
            run_codec(torch, b2, 3, 3)
            cm, dm = op_times(torch, b2, 5)
            r2 = codec_report(b2, cm, dm)
            r2["parity_round_trip"] = b2.verify()
            per[name] = r2
            del b2
            torch.cuda.empty_cache()
        log("workload moe_routed_16384x7168")
        per["moe_routed_16384x7168"] = bench_moe_gather(torch, Z, W, 5)
        torch.cuda.empty_cache()
        log("bucket with plans estimated on the device")
        per["bucket_64m_estimated_plans"] = bench_estimated_plans(torch, Z, W, 5)
        torch.cuda.empty_cache()
        log("workload allgather_16x4m")
        per["allgather_16x4m"] = bench_allgather(torch, Z, W, 5)
        torch.cuda.empty_cache()
        log("workload rs_512m")
        per["rs_512m"] = bench_rs(torch, Z, W, 5)
        log("reduce-scatter switcher")
        per["rs_switcher"] = bench_switcher(torch, Z, W)
        out["per_config"] = per
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, 1 thread)")
        from oracle import oracle as O
        out["cpu_baseline"] = cpu_baseline(W, O, wl, args.cpu_reps)
    print(json.dumps(out), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
