#!/usr/bin/env python3
"""Benchmark of the lossless BF16 exponent codec on one MI355X.

One step = the whole hot path over the reduce-scatter receive share, the largest
workload that fits one GPU: 7 peer shards of 64 Mi BF16 values (N(0, 1e-3)) and the
local shard.  Plan the 7 tables on the host, compress the peer shards in 32 chunks of
2 Mi values (one compress call per chunk, one segment per peer; 16 chunks share a
launch), then decode the 7 compressed shards of every chunk and add them in fp32, in
peer order, to the local shard, rounding once to BF16.  Inputs are resident in HBM
before the timed region; the step's working set (~1.7 GB) is far larger than the
256 MB Infinity Cache.  Every timed measurement comes after the same work has run
untimed for a few tenths of a second: an idle GPU sits at a low clock and the first
milliseconds of load run at ramping clocks.

Printed (one JSON line on stdout):
  value      BF16 bytes handled per second by the step: (2 x 7n compressed + 2 x 7n
             decoded) / step wall time, in GB/s;
  roofline   for the step's dominant kernel (compress_single_kernel): algorithmic
             HBM bytes per launch (2 B per value + static parts + escape bytes) /
             average launch time, from HIP events on the launch stream around
             back-to-back passes, against the 8 TB/s HBM peak; traffic: the HBM bytes
             per launch that rocprofv3's FETCH_SIZE and WRITE_SIZE counters measured
             (profiles/pmc_traffic_rs_512m.txt; null when that was taken on other kernel
             sources); roofline_other_op for decode-accumulate; each also beside the
             rate a plain streaming kernel of the same read/write mix reaches on this
             GPU (stream_ceiling_GBps; all the probes' rates in stream_ceilings_GBps);
  pipelined_step  the same step through the two-stream pipeline (zipccl_pipeline_reduce,
             calls back to back), beside the one-stream step;
  cpu_baseline  the plain C oracle on the host's cores, on a bounded sample of the
             same workload (4 of the 32 chunks), 1 thread and all threads;
  per_config every workload (1 Mi chunk, 64 Mi gradient bucket, activations with
             escapes and specials, MoE dispatch buckets, the same dispatch compressed
             from the unpermuted token matrix by row index, the all-gather receive side,
             the reduce-scatter share with its two-stream pipeline, plans estimated on
             the device, the switcher's profile), each with GB/s, HBM fraction and the
             oracle's time on the host beside it.
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
COMPRESS_CALLS_PER_LAUNCH = 16   # chunk calls that share one compress launch (the most the library
                                 # takes; launches of 8 took 4 % longer per pass)
ACC_SLOTS = 256                  # peer segments one decode-accumulate launch takes
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
    settle(torch, lambda k: (bc.compress(k % R, plans), bc.decompress((k - LAG) % R)))
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
    does not set the figure, and the fastest batch."""
    plans = bc.plans()
    cs, ds = [], []
    for _ in range(batches):
        cs.append(batched_ms(torch, lambda k: bc.compress(k, plans), len(bc.sets), rounds))
        ds.append(batched_ms(torch, bc.decompress, len(bc.sets), rounds))
    return median(cs), median(ds), min(cs), min(ds)


SETTLE_S = 0.3   # untimed work before each timed measurement, in seconds


def settle(torch, fn, seconds=SETTLE_S):
    """Run fn(k) back to back, untimed, for `seconds` of wall time.  An idle MI355X sits
    at a low shader clock (about 160 MHz read by amd-smi) and raises it only under
    sustained load; a batch timed right after host work (generating a workload) ran
    partly at ramping clocks, up to 38 % slower than the same kernels under continuous
    load, which held their time for 45 s.  The first launch of a kernel also loads it."""
    t_end = time.perf_counter() + seconds
    k = 0
    while True:
        fn(k)
        k += 1
        if k % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() >= t_end:
                break
    torch.cuda.synchronize()


def batched_ms(torch, fn, sets, rounds):
    """Average time of one launch of fn(k) over rounds x sets back-to-back launches on
    the rotating sets, from two HIP events on the launch stream around the whole batch
    (the events' own latency is then not counted per launch), after the same launches
    have run untimed until the clock has settled."""
    settle(torch, lambda k: fn(k % sets))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(rounds):
        for k in range(sets):
            fn(k)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (rounds * sets)


def codec_report(bc, c, d, c_min=None, d_min=None):
    """Per-operation figures from average launch times c, d (ms; medians over batches,
    with the fastest batch's c_min, d_min beside them)."""
    n_esc = bc.n_esc_total()
    moved = compress_bytes(bc.n, bc.static_bytes, n_esc)
    return {
        "elements": bc.n,
        "segments": len(bc.sizes),
        "compress_us": round(c * 1e3, 2),
        "decompress_us": round(d * 1e3, 2),
        "compress_us_min": None if c_min is None else round(c_min * 1e3, 2),
        "decompress_us_min": None if d_min is None else round(d_min * 1e3, 2),
        "compress_GBps": round(2 * bc.n / (c * 1e-3) / 1e9, 1),
        "decompress_GBps": round(2 * bc.n / (d * 1e-3) / 1e9, 1),
        "compress_hbm_frac": round(moved / (c * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "decompress_hbm_frac": round(moved / (d * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "ratio": round(2 * bc.n / (bc.static_bytes + n_esc), 5),
        "bits_per_value": round(8 * (bc.static_bytes + n_esc) / bc.n, 4),
        "escape_frac": round(n_esc / bc.n, 5),
    }



class RSShare:
    """The reduce-scatter receive share on the device: 7 peer shards and the local shard,
    the 32 chunks' compressed outputs (kept, as a receiver holds what arrived), and the
    compress and decode-accumulate sequences marshalled once."""

    def __init__(self, torch, Z, W):
        wl = W.rs_512m()
        self.torch, self.Z, self.wl = torch, Z, wl
        self.P, self.chunk, self.n = wl.extra["peers"], wl.extra["chunk"], wl.extra["shard"]
        P, chunk, n = self.P, self.chunk, self.n
        self.nch = n // chunk
        self.sigmas = wl.sigmas
        self.peers = [to_dev(torch, s) for s in wl.segments]
        self.local = to_dev(torch, wl.extra["local"])
        self.dst = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        self.S = S = Z.static_size(chunk)
        self.static = torch.empty(self.nch * P * S, dtype=torch.uint8, device="cuda")
        self.esc = torch.empty(self.nch * P * chunk, dtype=torch.uint8, device="cuda")
        self.n_esc = torch.zeros(self.nch, P + 1, dtype=torch.int64, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        # 16 chunks (112 segments) share a compress launch, with a workspace that holds them
        self.per_launch = COMPRESS_CALLS_PER_LAUNCH
        self.ws = torch.zeros(Z.workspace_size(self.per_launch * P * chunk, self.per_launch * P), dtype=torch.uint8,
                              device="cuda")
        self.comp_seq = Z.PreparedCompressChunks(
            [[p[c * chunk:(c + 1) * chunk] for p in self.peers] for c in range(self.nch)],
            [self.static[c * P * S:(c + 1) * P * S] for c in range(self.nch)],
            [self.esc[c * P * chunk:(c + 1) * P * chunk] for c in range(self.nch)], self.ws, self.n_esc.view(-1),
            self.status)
        self.acc_seq = Z.PreparedAccumulateChunks(
            [self.static.data_ptr() + (c * P + p) * S for c in range(self.nch) for p in range(P)],
            [self.esc.data_ptr() + c * P * chunk for c in range(self.nch) for _ in range(P)],
            P, chunk, n, self.local, self.dst, self.status, esc_bytes=[P * chunk] * (P * self.nch))

    def plans(self):
        return [self.Z.plan(sigma=s) for s in self.sigmas]

    def compress_all(self, plans=None):
        self.comp_seq.run(self.plans() if plans is None else plans)

    def accumulate_all(self):
        self.acc_seq.run()

    def step(self):
        self.compress_all()            # the 7 tables are planned on the host each step
        self.accumulate_all()

    def total_esc(self):
        return int(self.n_esc[:, -1].sum().item())

    def compress_bytes(self):
        return 2 * self.P * self.n + self.nch * self.P * self.S + self.total_esc()

    def accumulate_bytes(self):
        return self.nch * self.P * self.S + self.total_esc() + 2 * self.n + 2 * self.n

    def check(self):
        """The decode-accumulate output against torch on the device: fp32 adds in peer
        order, one rounding to BF16 (the inputs hold no NaN, so torch's NaN bits do not
        matter), and the status word."""
        torch = self.torch
        torch.cuda.synchronize()
        ok = int(self.status.item()) == 0
        for c0 in range(0, self.n, 1 << 24):
            sl = slice(c0, min(self.n, c0 + (1 << 24)))
            acc = self.local[sl].float()
            for p in self.peers:
                acc = acc + p[sl].float()
            ok = ok and bool(torch.equal(acc.to(torch.bfloat16).view(torch.int16), self.dst[sl].view(torch.int16)))
        return ok

    def accumulate_traffic_per_launch(self):
        """Measured HBM bytes of the decode-accumulate launches of one pass, per launch on
        average (the launches hold different numbers of chunks), or None."""
        per_acc = ACC_SLOTS // self.P
        grids = [(self.chunk // 4096) * 512 * min(per_acc, self.nch - c0) for c0 in range(0, self.nch, per_acc)]
        t = [measured_traffic("rs_512m", "accumulate_kernel", g) for g in grids]
        return None if None in t else int(sum(t) / len(t))

    def launches(self):
        """Kernel launches of one step, for the counter summaries: kernel, grid size in
        work-items, launches per step, algorithmic bytes per launch.  Decode-accumulate
        launches hold up to 256 / 7 = 36 chunks each (one launch for the 32 chunks)."""
        units = self.per_launch * self.P * ((self.chunk + 16383) // 16384)
        nl_c = self.nch // self.per_launch
        out = [{"kernel": "compress_single_kernel", "grid": (units + (units + 7) // 8) * 512, "per_step": nl_c,
                "bytes": self.compress_bytes() / nl_c, "values": self.per_launch * self.P * self.chunk}]
        per_acc = ACC_SLOTS // self.P
        shapes = {}
        for c0 in range(0, self.nch, per_acc):
            k = min(per_acc, self.nch - c0)
            shapes[k] = shapes.get(k, 0) + 1
        for k, count in shapes.items():
            out.append({"kernel": "accumulate_kernel", "grid": (self.chunk // 4096) * 512 * k, "per_step": count,
                        "bytes": self.accumulate_bytes() / self.nch * k, "values": k * self.chunk})
        return out

    def accumulate_launches_per_step(self):
        return -(-self.nch // (ACC_SLOTS // self.P))


def bench_rs_extra(torch, Z, rs, iters):
    """The reduce-scatter share's per-operation figures: each sequence alone, back to
    back (launch ramp-up and drain amortised), one pass between its own events, 32
    separate calls, and the two-stream pipeline's wall time."""
    P, chunk, n, nch = rs.P, rs.chunk, rs.n, rs.nch
    plans = rs.plans()
    comp = [Z.PreparedCompress([p[c * chunk:(c + 1) * chunk] for p in rs.peers],
                               rs.static[c * P * rs.S:(c + 1) * P * rs.S], rs.esc[c * P * chunk:(c + 1) * P * chunk],
                               rs.ws, rs.n_esc[c], rs.status) for c in range(nch)]
    acc = [Z.PreparedAccumulate([rs.static.data_ptr() + (c * P + p) * rs.S for p in range(P)],
                                [rs.esc.data_ptr() + c * P * chunk] * P, chunk, rs.local[c * chunk:],
                                rs.dst[c * chunk:], rs.status, esc_bytes=[P * chunk] * P) for c in range(nch)]
    rs.compress_all(plans)
    rs.accumulate_all()
    c_ms = batched_ms(torch, lambda k: rs.compress_all(plans), 1, iters)
    a_ms = batched_ms(torch, lambda k: rs.accumulate_all(), 1, iters)
    tc, ta = Timer(torch), Timer(torch)
    for _ in range(iters):
        e = tc.start()
        rs.compress_all(plans)
        tc.stop(e)
        e = ta.start()
        rs.accumulate_all()
        ta.stop(e)
    c1_ms, a1_ms = median(tc.ms()), median(ta.ms())
    tp, tq = Timer(torch), Timer(torch)
    for _ in range(iters):
        e = tp.start()
        for c in range(nch):
            comp[c].run(plans)
        tp.stop(e)
        e = tq.start()
        for c in range(nch):
            acc[c].run()
        tq.stop(e)
    cp_ms, ap_ms = median(tp.ms()), median(tq.ms())
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    pipe = Z.Pipeline(P, chunk, sa, sb)
    pipe.reduce(rs.peers, plans, rs.local, rs.dst, rs.status)
    torch.cuda.synchronize()
    walls = []
    for _ in range(iters):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pipe.reduce(rs.peers, plans, rs.local, rs.dst, rs.status)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    # calls back to back, as a training loop would issue them: host enqueue of one call
    # overlaps the GPU work of the one before
    settle(torch, lambda k: pipe.reduce(rs.peers, plans, rs.local, rs.dst, rs.status))
    t0 = time.perf_counter()
    for _ in range(4 * iters):
        pipe.reduce(rs.peers, plans, rs.local, rs.dst, rs.status)
    torch.cuda.synchronize()
    b2b = (time.perf_counter() - t0) / (4 * iters)
    pipe.close()
    ok = rs.check()     # the pipeline's output, against torch
    wall = median(walls)
    static_total = nch * P * rs.S
    total_esc = rs.total_esc()
    return {
        "elements_per_peer": n, "peers": P, "chunk": chunk, "chunks": nch,
        "compress_us": round(c_ms * 1e3, 1),
        "compress_GBps": round(2 * P * n / (c_ms * 1e-3) / 1e9, 1),
        "compress_hbm_frac": round(rs.compress_bytes() / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "compress_single_pass_us": round(c1_ms * 1e3, 1),
        "compress_separate_calls_us": round(cp_ms * 1e3, 1),
        "accumulate_us": round(a_ms * 1e3, 1),
        "accumulate_GBps_bf16_in": round(2 * P * n / (a_ms * 1e-3) / 1e9, 1),
        "accumulate_hbm_frac": round(rs.accumulate_bytes() / (a_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "accumulate_single_pass_us": round(a1_ms * 1e3, 1),
        "accumulate_separate_calls_us": round(ap_ms * 1e3, 1),
        "pipeline_wall_us": round(wall * 1e6, 1),
        "pipeline_GBps_bf16_in": round(2 * P * n / wall / 1e9, 1),
        "pipeline_back_to_back_us": round(b2b * 1e6, 1),
        "ratio": round(2 * P * n / (static_total + total_esc), 5),
        "escape_frac": round(total_esc / (P * n), 5),
        "parity_vs_torch_fp32": ok,
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
    blocks = sum((m + 4095) // 4096 for m in sizes)
    launches = [{"kernel": "decompress_kernel", "grid": blocks * 128, "per_step": 1, "bytes": moved, "values": n}]
    return {
        "elements": n, "shards": len(sizes),
        "decompress_us": round(d * 1e3, 2),
        "decompress_GBps": round(2 * n / (d * 1e-3) / 1e9, 1),
        "decompress_hbm_frac": round(moved / (d * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "parity_round_trip": ok,
    }, launches


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
    units = sum((m + 16383) // 16384 for m in sizes)
    launches = [{"kernel": "compress_single_kernel", "grid": (units + (units + 7) // 8) * 512, "per_step": 1,
                 "bytes": moved, "values": n,
                 "note": "the gathered compress and the compress of the permuted copy launch this kernel with "
                         "the same grid and move the same algorithmic bytes; the counters average both"}]
    return {
        "elements": n, "segments": len(sizes),
        "gather_compress_us": round(g * 1e3, 2),
        "gather_compress_GBps": round(2 * n / (g * 1e-3) / 1e9, 1),
        "gather_compress_hbm_frac": round(moved / (g * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "permute_us": round(pm * 1e3, 2),
        "compress_permuted_us": round(cp * 1e3, 2),
        "permute_plus_compress_us": round((pm + cp) * 1e3, 2),
        "parity_vs_permuted": ok,
    }, launches


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
    settle(torch, lambda k: b.copy_(a))
    t = Timer(torch)
    for _ in range(iters):
        e = t.start()
        b.copy_(a)
        t.stop(e)
    ms = median(t.ms())
    del a, b
    torch.cuda.empty_cache()
    return round(2 * (1 << 30) / (ms * 1e-3) / 1e9, 1)


# Streaming probes (libzcprobe.so, built beside the codec): plain kernels that move memory
# in the codec's shapes with nothing to compute.  Each rate is bytes read plus written per
# second over 1 GiB buffers: the rate the same GPU reaches for that mix.
PROBE_KINDS = {"copy": 0, "read": 1, "write": 2, "mix_16_12": 3, "acc_7": 4}


def stream_ceilings(torch, iters=10):
    import ctypes
    path = os.path.join(ROOT, "lossless_bf16_exponent_codec_amd", "libzcprobe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run python -m lossless_bf16_exponent_codec_amd.build")
    lib = ctypes.CDLL(path)
    lib.zcprobe_launch.restype = ctypes.c_int
    lib.zcprobe_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.zcprobe_moved_bytes.restype = ctypes.c_uint64
    lib.zcprobe_moved_bytes.argtypes = [ctypes.c_int, ctypes.c_uint64]
    nbytes = 1 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, kind in PROBE_KINDS.items():
        def launch(_k=None, kind=kind):
            r = lib.zcprobe_launch(kind, a.data_ptr(), b.data_ptr(), nbytes, stream)
            if r != 0:
                raise RuntimeError(f"zcprobe_launch({name}) returned {r}")
        settle(torch, launch)
        t = Timer(torch)
        for _ in range(iters):
            e = t.start()
            launch()
            t.stop(e)
        out[name] = round(lib.zcprobe_moved_bytes(kind, nbytes) / (median(t.ms()) * 1e-3) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------------------------
# the oracle on the host's cores, beside every workload (a baseline, not the target)
# ------------------------------------------------------------------------------------
def host_threads():
    return max(1, min(16, os.cpu_count() or 1))


def host_info():
    """The host the oracle runs on: logical CPUs, the CPU model and the NUMA nodes (Linux)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        numa = len([d for d in os.listdir("/sys/devices/system/node") if d.startswith("node") and d[4:].isdigit()])
    except OSError:
        numa = None
    return {"host_cpus": os.cpu_count(), "cpu_model": model, "numa_nodes": numa}


def oracle_codec(O, segments, sigmas, reps=1, sample=None):
    """The oracle's compress (one batch call) and decompress (one call per segment) of a
    workload's segments on one thread, median of reps; then the same values as at least
    host_threads() independent segments (each workload segment split in halves until
    there are enough), compress + decompress of each as one task on every thread."""
    from concurrent.futures import ThreadPoolExecutor
    tables = [O.plan_sigma(s if s is not None else 1.0) for s in sigmas]
    n = int(sum(x.size for x in segments))
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        st, esc, ne, rc = O.compress_batch(segments, tables)
        t1 = time.perf_counter()
        off_st = 0
        for x in segments:
            sz = O.static_size(x.size)
            O.decompress(st[off_st:off_st + sz], esc, x.size)
            off_st += sz
        times.append((t1 - t0, time.perf_counter() - t1))
    c, d = median([t[0] for t in times]), median([t[1] for t in times])
    threads = host_threads()
    pieces = list(zip(segments, tables))
    while len(pieces) < threads and max(p[0].size for p in pieces) > 8192:
        pieces = [q for x, t in pieces for q in ((x[:x.size // 2], t), (x[x.size // 2:], t))]

    def one(k):
        x, t = pieces[k]
        s, e, _ = O.compress(x, t)
        O.decompress(s, e, x.size)

    with ThreadPoolExecutor(threads) as pool:
        t0 = time.perf_counter()
        list(pool.map(one, range(len(pieces))))
        wall = time.perf_counter() - t0
    return {"value": round(4 * n / (c + d) / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "compress_GBps": round(2 * n / c / 1e9, 4), "decompress_GBps": round(2 * n / d / 1e9, 4),
            "sample": sample or f"all {n} values, compress + decompress, 1 thread" + (f", median of {reps}" if reps > 1 else ""),
            "all_threads": {"threads": threads, "value": round(4 * n / wall / 1e9, 4), "unit": "GB/s",
                            "sample": f"the same values as {len(pieces)} segments, compress + decompress of each as one task"}}


def oracle_rs(O, W, chunks=4, reps=3):
    """The oracle on a bounded sample of the reduce-scatter share: the first `chunks`
    chunks of the 7 peers (compress each peer's chunk, then decode-accumulate the chunk
    into the local shard), on one thread (median of reps), and 16 chunks as one task
    each on every thread."""
    from concurrent.futures import ThreadPoolExecutor
    wl = W.rs_512m()
    P, chunk = wl.extra["peers"], wl.extra["chunk"]
    tables = [O.plan_sigma(s) for s in wl.sigmas]
    local = wl.extra["local"]

    def do_chunk(c):
        t0 = time.perf_counter()
        comp = [O.compress(p[c * chunk:(c + 1) * chunk], t) for p, t in zip(wl.segments, tables)]
        t1 = time.perf_counter()
        O.decompress_accumulate([x[0] for x in comp], [x[1] for x in comp], chunk, local[c * chunk:(c + 1) * chunk])
        return t1 - t0, time.perf_counter() - t1

    times = []
    for _ in range(reps):
        ts = [do_chunk(c) for c in range(chunks)]
        times.append((sum(t[0] for t in ts), sum(t[1] for t in ts)))
    c, a = median([t[0] for t in times]), median([t[1] for t in times])
    v = P * chunk * chunks
    threads = host_threads()
    par = 16
    with ThreadPoolExecutor(threads) as pool:
        t0 = time.perf_counter()
        list(pool.map(do_chunk, range(par)))
        wall = time.perf_counter() - t0
    return {"value": round(4 * v / (c + a) / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "compress_GBps": round(2 * v / c / 1e9, 4), "accumulate_GBps_bf16_in": round(2 * v / a / 1e9, 4),
            "sample": f"rs_512m chunks 0..{chunks - 1} of the 7 peers ({chunks} x 7 x {chunk} values): compress + "
                      f"decode-accumulate, median of {reps}, 1 thread",
            **host_info(),
            "all_threads": {"threads": threads, "value": round(4 * P * chunk * par / wall / 1e9, 4), "unit": "GB/s",
                            "sample": f"rs_512m chunks 0..{par - 1}, compress + decode-accumulate of each chunk as one task"}}


# ------------------------------------------------------------------------------------
# one workload alone (for profiling), with the launches of one pass
# ------------------------------------------------------------------------------------
def codec_launches(bc, n_esc):
    """compress_single_kernel and decompress_kernel launches of one BatchCodec pass."""
    units = sum((m + 16383) // 16384 for m in bc.sizes)
    blocks = sum((m + 4095) // 4096 for m in bc.sizes)
    moved = compress_bytes(bc.n, bc.static_bytes, n_esc)
    return [{"kernel": "compress_single_kernel", "grid": (units + (units + 7) // 8) * 512, "per_step": 1,
             "bytes": moved, "values": bc.n},
            {"kernel": "decompress_kernel", "grid": blocks * 128, "per_step": 1, "bytes": moved, "values": bc.n}]


def bench_codec_workload(torch, Z, W, name, rounds=5):
    w2 = W.get(name)
    sets = 8 if name == "chunk_1m" else 4
    b2 = BatchCodec(torch, Z, w2.segments, w2.sigmas, sets)
    run_codec(torch, b2, 3, 3)
    cm, dm, cmin, dmin = op_times(torch, b2, rounds)
    r2 = codec_report(b2, cm, dm, cmin, dmin)
    r2["parity_round_trip"] = b2.verify()
    launches = codec_launches(b2, b2.n_esc_total())
    del b2
    torch.cuda.empty_cache()
    return r2, launches, w2

# ------------------------------------------------------------------------------------
# rocprofv3 summaries kept under profiles/ (text), and the measured HBM traffic
# ------------------------------------------------------------------------------------
KERNEL_SRC = os.path.join(ROOT, "lossless_bf16_exponent_codec_amd", "csrc", "zipccl_kernels.hip")
OUR_KERNELS = ("compress_single_kernel", "encode_kernel", "place_direct_kernel", "scan_kernel", "place_kernel",
               "decompress_kernel", "accumulate_kernel", "estimate_partial_kernel", "estimate_finish_kernel")
COPY_KERNEL = "__amd_rocclr_copyBuffer"
GIB = 1 << 30


def kernel_code_text(text):
    """The kernel source without its comments, trailing blanks and empty lines: what a
    profile was taken on, so that a change to comments alone keeps it valid (the source
    has no string literal holding "//")."""
    lines = []
    for line in text.splitlines():
        line = line.split("//", 1)[0].rstrip()
        if line:
            lines.append(line)
    return "\n".join(lines) + "\n"


def kernel_source_sha256():
    """sha256 of the kernel code (kernel_code_text of zipccl_kernels.hip)."""
    import hashlib
    with open(KERNEL_SRC, encoding="utf-8") as f:
        return hashlib.sha256(kernel_code_text(f.read()).encode()).hexdigest()


def short_kernel_name(name):
    for k in OUR_KERNELS:
        if k in name:
            return k
    return COPY_KERNEL if COPY_KERNEL in name else None


def summarize_stats_any(csv_path, out_path, title, command):
    """profiles/ text from rocprofv3 --kernel-trace --stats (kernel_stats.csv): rocprofv3's
    own per-kernel averages."""
    import csv
    rows = [r for r in csv.DictReader(open(csv_path)) if short_kernel_name(r["Name"]) in OUR_KERNELS]
    lines = [f"# Kernel durations, {title}", "",
             "Command (from the repository root on the GPU host; rocprofv3's own averages):", "",
             "    " + command, "",
             f"Kernel code sha256 (zipccl_kernels.hip without comments): `{kernel_source_sha256()}`", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {short_kernel_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    open(out_path, "w").write("\n".join(lines) + "\n")


def pmc_cmd(name, counter):
    return (f"rocprofv3 --pmc {counter} --output-format csv -d rocprof_out/pmc_{name}_{counter} -o run -- "
            f"python3 bench.py --only {name} --launches-out rocprof_out/launches_{name}.json")


def per_kernel_counter(path, counter):
    """Mean counter value per (kernel, grid) over the dispatches of a rocprofv3 --pmc CSV."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = short_kernel_name(r["Kernel_Name"])
        if k is None:
            continue
        acc.setdefault((k, int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
    return {key: (sum(v) / len(v), len(v)) for key, v in acc.items()}


def summarize_pmc_any(name, launches_json, fetch_csv, write_csv, out_path):
    """profiles/pmc_traffic_<name>.txt from two rocprofv3 --pmc runs of pmc_cmd(name, ...)
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch): HBM bytes per launch of each of the
    workload's kernels against its algorithmic bytes (launches_json, written by the same
    command).  Each counter is scaled by what it reads for the 1 GiB device copy at the end
    of the run (the copy reads and writes 1 GiB)."""
    launches = json.load(open(launches_json))
    f = per_kernel_counter(fetch_csv, "FETCH_SIZE")
    w = per_kernel_counter(write_csv, "WRITE_SIZE")
    copy_f = max(v for (k, g), (v, c) in f.items() if k == COPY_KERNEL)
    copy_w = max(v for (k, g), (v, c) in w.items() if k == COPY_KERNEL)
    sf, sw = (GIB / 1024) / copy_f, (GIB / 1024) / copy_w      # true KiB per counted KiB
    lines = [f"# Measured HBM traffic, {name}", "",
             "Commands (from the repository root on the GPU host), one run per counter:", "",
             "    " + pmc_cmd(name, "FETCH_SIZE"), "    " + pmc_cmd(name, "WRITE_SIZE"), "",
             f"Scale factors from the 1 GiB copy in the same runs: FETCH_SIZE x{sf:.4f}, WRITE_SIZE x{sw:.4f}",
             f"(the copy counted {copy_f:.0f} KiB fetched and {copy_w:.0f} KiB written per dispatch).",
             f"Kernel code sha256 (zipccl_kernels.hip without comments): `{kernel_source_sha256()}`", "",
             "| kernel | grid | dispatches | read MB | write MB | measured MB | algorithmic MB | measured / algorithmic |",
             "|---|---|---|---|---|---|---|---|"]
    mr = []
    for L in launches:
        key = (L["kernel"], L["grid"])
        if key not in f or key not in w:
            continue
        (fv, nd), (wv, _) = f[key], w[key]
        rd, wr = fv * sf * 1024, wv * sw * 1024
        lines.append(f"| {L['kernel']} | {L['grid']} | {nd} | {rd / 1e6:.2f} | {wr / 1e6:.2f} | {(rd + wr) / 1e6:.2f} | "
                     f"{L['bytes'] / 1e6:.2f} | {(rd + wr) / L['bytes']:.4f} |")
        mr.append(f"{L['kernel']}_{L['grid']}_traffic_bytes={int(rd + wr)}")
    lines += ["", "Machine-readable (bench.py reports these as roofline.traffic while the kernel source",
              "hash matches; bytes per launch):", "", "```", f"source_sha256={kernel_source_sha256()}"] + mr + ["```"]
    open(out_path, "w").write("\n".join(lines) + "\n")


TCC_PASSES = ("TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_BUBBLE_sum TCC_EA0_RDREQ_128B_sum",
              "TCC_EA0_RDREQ_DRAM_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum")


def tcc_cmd(k):
    return (f"rocprofv3 --pmc {TCC_PASSES[k]} --output-format csv -d rocprof_out/tcc{k} -o run -- "
            "python3 bench.py --only bucket_64m --launches-out rocprof_out/launches_bucket_64m.json")


def summarize_tcc(csv0, csv1, out_path):
    """Appends to out_path the read bytes of each kernel by three routes, from the raw TCC
    counters of two --pmc passes of tcc_cmd: FETCH_SIZE's own expression (128-byte requests
    taken from TCC_BUBBLE), the request counts by size (TCC_EA0_RDREQ_128B / 64B / 32B),
    and the DRAM read requests in 32-byte units (TCC_EA0_RDREQ_DRAM_32B)."""
    c = {}
    for path, names in ((csv0, TCC_PASSES[0]), (csv1, TCC_PASSES[1])):
        for cn in names.split():
            for key, (v, n) in per_kernel_counter(path, cn).items():
                c.setdefault(key, {})[cn] = v
    lines = ["", "## Cross-check of the FETCH_SIZE scale with raw TCC read-request counters", "",
             "Commands (two passes of four TCC counters each):", "", "    " + tcc_cmd(0), "    " + tcc_cmd(1), "",
             "Bytes read per dispatch: by FETCH_SIZE's expression (TCC_BUBBLE x 128 + other requests x 64, 32-byte "
             "ones x 32); by request size (RDREQ_128B x 128 + RDREQ_64B x 64 + RDREQ_32B x 32); and the DRAM "
             "read requests in 32-byte units (RDREQ_DRAM_32B x 32).  Write bytes: WRREQ_64B x 64 + other x 32.", "",
             "| kernel | grid | FETCH_SIZE-style MB | by request size MB | DRAM 32B units MB | write MB |",
             "|---|---|---|---|---|---|"]
    for (k, g), d in sorted(c.items()):
        if k not in (COPY_KERNEL, "compress_single_kernel", "decompress_kernel") or len(d) < 8:
            continue
        rd = d["TCC_EA0_RDREQ_sum"]
        fs = d["TCC_BUBBLE_sum"] * 128 + (rd - d["TCC_BUBBLE_sum"] - d["TCC_EA0_RDREQ_32B_sum"]) * 64 + \
            d["TCC_EA0_RDREQ_32B_sum"] * 32
        bs = d["TCC_EA0_RDREQ_128B_sum"] * 128 + d["TCC_EA0_RDREQ_64B_sum"] * 64 + d["TCC_EA0_RDREQ_32B_sum"] * 32
        dr = d["TCC_EA0_RDREQ_DRAM_32B_sum"] * 32
        wb = d["TCC_EA0_WRREQ_64B_sum"] * 64 + (d["TCC_EA0_WRREQ_sum"] - d["TCC_EA0_WRREQ_64B_sum"]) * 32
        lines.append(f"| {k} | {g} | {fs / 1e6:.2f} | {bs / 1e6:.2f} | {dr / 1e6:.2f} | {wb / 1e6:.2f} |")
    open(out_path, "a").write("\n".join(lines) + "\n")


def measured_traffic(name, kernel, grid):
    """Bytes per launch from profiles/pmc_traffic_<name>.txt, or None if it is missing, was
    taken on another version of the kernels, or has no row for this launch."""
    try:
        text = open(os.path.join(ROOT, "profiles", f"pmc_traffic_{name}.txt")).read()
    except OSError:
        return None
    kv = dict(line.split("=", 1) for line in text.splitlines() if "=" in line and " " not in line.strip())
    if kv.get("source_sha256") != kernel_source_sha256():
        return None
    v = kv.get(f"{kernel}_{grid}_traffic_bytes")
    return int(v) if v is not None else None

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
             f"Kernel code sha256 (zipccl_kernels.hip without comments): `{kernel_source_sha256()}`", "",
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



TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/stats -o bench -- "
             "python3 bench.py --steps 20 --warmup 3 --no-cpu-baseline --no-extra")


def only_cmd_stats(name):
    return (f"rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/stats_{name} -o run -- "
            f"python3 bench.py --only {name}")


_WL = {}


def workload(W, name):
    if name not in _WL:
        _WL[name] = W.get(name)
    return _WL[name]


def run_only(torch, Z, W, name):
    """One workload alone: its figures and the launches of one pass."""
    if name in ("chunk_1m", "bucket_64m", "act_8192x7168", "moe_16384x7168"):
        res, launches, _ = bench_codec_workload(torch, Z, W, name)
        return res, launches
    if name == "rs_512m":
        rs = RSShare(torch, Z, W)
        res = bench_rs_extra(torch, Z, rs, 5)
        return res, rs.launches()
    if name == "moe_routed_16384x7168":
        return bench_moe_gather(torch, Z, W, 5)
    if name == "allgather_16x4m":
        return bench_allgather(torch, Z, W, 5)
    if name == "bucket_64m_estimated_plans":
        return bench_estimated_plans(torch, Z, W, 5), []
    if name == "rs_switcher":
        return bench_switcher(torch, Z, W), []
    raise KeyError(name)


ONLY_NAMES = ("chunk_1m", "bucket_64m", "act_8192x7168", "moe_16384x7168", "moe_routed_16384x7168",
              "allgather_16x4m", "rs_512m", "bucket_64m_estimated_plans", "rs_switcher")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=4, help="rotating buffer sets of the bucket (> 2)")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--only", default=None, choices=ONLY_NAMES,
                    help="run one workload alone (for profiling) and print its figures")
    ap.add_argument("--launches-out", default=None, help="with --only: write the pass's launches (JSON) here")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("NAME", "KERNEL_STATS_CSV", "OUT_MD"),
                    help="profiles/ summary of a rocprofv3 --stats run (NAME: headline, or the --only workload)")
    ap.add_argument("--summarize-pmc", nargs=5, metavar=("NAME", "LAUNCHES_JSON", "FETCH_CSV", "WRITE_CSV", "OUT_MD"),
                    help="profiles/ summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of --only NAME")
    ap.add_argument("--summarize-tcc", nargs=3, metavar=("CSV0", "CSV1", "OUT_MD"),
                    help="append the raw TCC read-request cross-check to a traffic summary")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("COUNTER_CSV", "OUT_MD"),
                    help="profiles/ summary of a rocprofv3 SQ-counter run of --only rs_512m")
    args = ap.parse_args(argv)
    if args.summarize_stats:
        name, csv_path, out = args.summarize_stats
        if name == "headline":
            summarize_stats_any(csv_path, out, "headline step (rs_512m: 7 peers x 64 Mi values in 32 chunks of 2 Mi, "
                                "compress + decode-accumulate)", TRACE_CMD)
        else:
            summarize_stats_any(csv_path, out, name, only_cmd_stats(name))
        return 0
    if args.summarize_pmc:
        summarize_pmc_any(*args.summarize_pmc)
        return 0
    if args.summarize_tcc:
        summarize_tcc(*args.summarize_tcc)
        return 0
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq)
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
        res, launches = run_only(torch, Z, W, args.only)
        if args.launches_out:
            os.makedirs(os.path.dirname(os.path.abspath(args.launches_out)), exist_ok=True)
            json.dump(launches, open(args.launches_out, "w"))
        # the 1 GiB copy whose counter readings scale a --pmc run of this command
        print(json.dumps({"workload": args.only, **res, "hbm_copy_GBps": copy_ceiling(torch)}), flush=True)
        return 0

    # ---- the headline step: the reduce-scatter receive share ----
    log("generating rs_512m")
    rs = RSShare(torch, Z, W)
    P, n = rs.P, rs.n
    log(f"warmup {args.warmup}, timing {args.steps} steps")
    settle(torch, lambda k: rs.step(), 2 * SETTLE_S)   # untimed: the clock comes up first
    for _ in range(args.warmup):
        rs.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        rs.step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
    value = 4 * P * n / (ms_per_step * 1e-3) / 1e9
    ok = rs.check()
    # per-launch averages for the roofline: each sequence alone, back-to-back passes
    # between two HIP events on the launch stream (median of three batches)
    plans = rs.plans()
    rounds = max(2, args.steps // 3)
    c_all = [batched_ms(torch, lambda k: rs.compress_all(plans), 1, rounds) for _ in range(3)]
    a_all = [batched_ms(torch, lambda k: rs.accumulate_all(), 1, rounds) for _ in range(3)]
    c_ms, a_ms = median(c_all), median(a_all)
    lc = rs.launches()[0]
    nl_a = rs.accumulate_launches_per_step()
    c_launch_ms = c_ms / lc["per_step"]
    a_launch_ms = a_ms / nl_a
    c_bytes = rs.compress_bytes() / lc["per_step"]
    a_bytes = rs.accumulate_bytes() / nl_a
    roof_c = {"bound": "hbm", "kernel": "compress_single_kernel", "achieved": round(c_bytes / (c_launch_ms * 1e-3) / 1e9, 1),
              "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(c_bytes / (c_launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
              "traffic": measured_traffic("rs_512m", lc["kernel"], lc["grid"]),
              "bytes_per_launch": int(c_bytes), "avg_launch_us": round(c_launch_ms * 1e3, 2),
              "avg_launch_us_min": round(min(c_all) / lc["per_step"] * 1e3, 2),
              "launches_per_step": lc["per_step"], "values_per_launch": lc["values"]}
    roof_a = {"bound": "hbm", "kernel": "accumulate_kernel", "achieved": round(a_bytes / (a_launch_ms * 1e-3) / 1e9, 1),
              "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(a_bytes / (a_launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
              "traffic": rs.accumulate_traffic_per_launch(), "bytes_per_launch": int(a_bytes),
              "avg_launch_us": round(a_launch_ms * 1e3, 2), "avg_launch_us_min": round(min(a_all) / nl_a * 1e3, 2),
              "launches_per_step": nl_a,
              "note": "one launch holds all 32 chunks of 7 peers (up to 36 fit); bytes, time and traffic per launch"}
    total_esc = rs.total_esc()
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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "rs_512m: reduce-scatter receive share, 7 peer shards x 67108864 BF16 values "
                               "N(0, 1e-3) compressed in 32 chunks of 2097152 values (16 chunks per launch), then "
                               "decoded and added in fp32, peers in order, into the local shard N(0, 1e-3), one "
                               "BF16 rounding",
                   "elements_per_peer": n, "peers": P, "chunk": rs.chunk, "chunks": rs.nch},
        "compress_GBps": round(2 * P * n / (c_ms * 1e-3) / 1e9, 1),
        "accumulate_GBps_bf16_in": round(2 * P * n / (a_ms * 1e-3) / 1e9, 1),
        "compress_hbm_frac": roof_c["frac"],
        "accumulate_hbm_frac": roof_a["frac"],
        "ratio": round(2 * P * n / (rs.nch * P * rs.S + total_esc), 5),
        "bits_per_value": round(8 * (rs.nch * P * rs.S + total_esc) / (P * n), 4),
        "escape_frac": round(total_esc / (P * n), 5),
        "parity_vs_torch_fp32": ok,
        "roofline": roof_c,
        "roofline_other_op": roof_a,
    }
    log("copy ceiling")
    out["hbm_copy_GBps"] = copy_ceiling(torch)
    out["roofline"]["frac_of_copy"] = round(out["roofline"]["achieved"] / out["hbm_copy_GBps"], 4)
    log("streaming probes")
    ceil = stream_ceilings(torch)
    out["stream_ceilings_GBps"] = ceil
    # each kernel beside the probe of its own mix: compress reads 2 B and writes ~1.4 B per
    # value (probe: 16 B read, 12 B written); decode-accumulate reads each of 7 peers' A and
    # plane bytes of a tile plus the local values and writes the sum (probe: the same reads
    # and write in its workgroup and wave shape, escapes and arithmetic left out)
    for key, probe in (("roofline", "mix_16_12"), ("roofline_other_op", "acc_7")):
        out[key]["stream_ceiling_GBps"] = ceil[probe]
        out[key]["stream_ceiling_probe"] = probe
        out[key]["frac_of_stream_ceiling"] = round(out[key]["achieved"] / ceil[probe], 4)
    from oracle import oracle as O
    if not args.no_extra:
        per = {}
        log("workload bucket_64m")
        wl = workload(W, "bucket_64m")
        bc = BatchCodec(torch, Z, wl.segments, wl.sigmas, args.sets)
        step_ms = run_codec(torch, bc, 10, 3)
        cm, dm, cmin, dmin = op_times(torch, bc, max(2, args.steps // len(bc.sets)))
        r = codec_report(bc, cm, dm, cmin, dmin)
        r["step_GBps"] = round(4 * bc.n / (step_ms * 1e-3) / 1e9, 1)
        r["parity_round_trip"] = bc.verify()
        r["compress_traffic_bytes"] = measured_traffic("bucket_64m", *[(L["kernel"], L["grid"]) for L in
                                                                        codec_launches(bc, bc.n_esc_total())][0])
        r["decompress_traffic_bytes"] = measured_traffic("bucket_64m", *[(L["kernel"], L["grid"]) for L in
                                                                          codec_launches(bc, bc.n_esc_total())][1])
        per["bucket_64m"] = r
        del bc
        torch.cuda.empty_cache()
        for name in ("chunk_1m", "act_8192x7168", "moe_16384x7168"):
            log(f"workload {name}")
            r2, launches, w2 = bench_codec_workload(torch, Z, W, name)
            r2["compress_traffic_bytes"] = measured_traffic(name, launches[0]["kernel"], launches[0]["grid"])
            r2["decompress_traffic_bytes"] = measured_traffic(name, launches[1]["kernel"], launches[1]["grid"])
            _WL[name] = w2
            per[name] = r2
        log("workload moe_routed_16384x7168")
        r3, l3 = bench_moe_gather(torch, Z, W, 5)
        r3["gather_compress_traffic_bytes"] = measured_traffic("moe_routed_16384x7168", l3[0]["kernel"], l3[0]["grid"])
        per["moe_routed_16384x7168"] = r3
        torch.cuda.empty_cache()
        log("bucket with plans estimated on the device")
        per["bucket_64m_estimated_plans"] = bench_estimated_plans(torch, Z, W, 5)
        torch.cuda.empty_cache()
        log("workload allgather_16x4m")
        r4, l4 = bench_allgather(torch, Z, W, 5)
        r4["decompress_traffic_bytes"] = measured_traffic("allgather_16x4m", l4[0]["kernel"], l4[0]["grid"])
        per["allgather_16x4m"] = r4
        torch.cuda.empty_cache()
        log("workload rs_512m (per operation, pipeline)")
        per["rs_512m"] = bench_rs_extra(torch, Z, rs, 5)
        # the same step through the two-stream pipeline (zipccl_pipeline_reduce: compress on one
        # stream, decode-accumulate on the other, handed over in groups of chunks); on one GPU
        # there is no transfer for it to overlap, so the step above runs the chunk calls on one
        # stream and this figure stands beside it
        pb = per["rs_512m"]["pipeline_back_to_back_us"]
        out["pipelined_step"] = {"value": round(4 * P * n / (pb * 1e-6) / 1e9, 1), "unit": "GB/s",
                                 "ms_per_step": round(pb * 1e-3, 4), "streams": 2,
                                 "api": "zipccl_pipeline_reduce, calls back to back"}
        log("reduce-scatter switcher")
        per["rs_switcher"] = bench_switcher(torch, Z, W)
        out["per_config"] = per
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle): reduce-scatter share sample")
        out["cpu_baseline"] = oracle_rs(O, W, chunks=4, reps=args.cpu_reps)
        if "per_config" in out:
            out["per_config"]["rs_512m"]["oracle"] = out["cpu_baseline"]
            for name in ("chunk_1m", "bucket_64m", "act_8192x7168", "moe_16384x7168"):
                log(f"oracle on {name}")
                wl = workload(W, name)
                out["per_config"][name]["oracle"] = oracle_codec(O, wl.segments, wl.sigmas)
    print(json.dumps(out), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
