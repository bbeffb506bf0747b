"""Seeded synthetic inputs for the codec's five workloads.

This module draws random numbers and shapes them; it holds none of the codec's
arithmetic (no exponent tables, no codes, no sizes), so both the HIP path and the
CPU oracle can consume the same bits.  Values are drawn in fp32 on the CPU with a
seeded torch generator and rounded to BF16 (round to nearest even), and returned as
numpy uint16 arrays of BF16 bit patterns.

The method's premise is that communication tensors of LLM training are close to
Gaussian ("ZipCCL ..." gist.science explanation page, section 2.A); real Llama3 /
Qwen / DeepSeek tensors are not available here, so Gaussian draws with the stated
shapes stand in for them.

Workloads:
  chunk_1m     1 048 576 values from N(0, 0.02), seed 1, one segment.
  bucket_64m   a 64 Mi-value gradient bucket: 16 layers of 4 Mi values; layer l is
               N(0, sigma_l) with sigma_l = 10**U(-4, -1) (numpy default_rng(2)), drawn
               with seed 200 + l; one segment per layer.
  act_8192x7168  activation tensor: N(0, 1) base (seed 3); under a seeded permutation
               the first 5 % of positions are set to +0.0, the next 0.1 % are scaled by
               100 in fp32 before rounding, the next 1000 get special BF16 patterns
               (subnormals with random sign, -0, +-Inf, quiet, signalling and payload
               NaNs) in round-robin order.  One segment.
  moe_16384x7168 MoE dispatch payload N(0, 0.5) (seed 4), already permuted into 8
               contiguous destination buckets whose token counts follow Zipf(s=1.2)
               (largest-remainder rounding of 16384 * k**-1.2 / sum); one segment per
               bucket.
  moe_routed_16384x7168  the same token matrix before the permute: each of the 16384
               tokens is routed to one of 8 destinations with the same Zipf(1.2) counts
               by a seeded permutation (numpy default_rng(41)); destination b gets the
               tokens perm[c_0 + ... + c_(b-1) :][:c_b] in ascending order.  For the
               compress of rows gathered by index.
  rs_512m      reduce-scatter receive share: 7 peer shards of 64 Mi values from
               N(0, 1e-3) with seeds 500..506 and the local shard with seed 507;
               processed in chunks of 2 Mi values (4 MiB of BF16) per peer.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "gaussian_bf16", "chunk_1m", "bucket_64m", "act_8192x7168",
           "moe_16384x7168", "moe_routed_16384x7168", "rs_512m", "zipf_counts", "WORKLOADS", "get"]


@dataclass
class Workload:
    name: str
    segments: list            # list of np.uint16 arrays (BF16 bit patterns), one per segment
    sigmas: list              # the sigma each segment was drawn with (None: no Gaussian sigma)
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_total(self) -> int:
        return int(sum(s.size for s in self.segments))


def _bf16_bits(t32: torch.Tensor) -> np.ndarray:
    return t32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def gaussian_bf16(n: int, sigma: float, seed: int) -> np.ndarray:
    """n values of N(0, sigma^2), fp32 draws rounded to BF16, as uint16 bit patterns."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    t = torch.randn(n, generator=g, dtype=torch.float32)
    t.mul_(sigma)
    return _bf16_bits(t)


def chunk_1m() -> Workload:
    return Workload("chunk_1m", [gaussian_bf16(1 << 20, 0.02, 1)], [0.02],
                    "1 048 576 values, N(0, 0.02), seed 1")


def bucket_sigmas(layers: int = 16, seed: int = 2) -> list:
    rng = np.random.default_rng(seed)
    return [float(10.0 ** u) for u in rng.uniform(-4.0, -1.0, size=layers)]


def bucket_64m(layers: int = 16, per_layer: int = 1 << 22) -> Workload:
    sig = bucket_sigmas(layers)
    segs = [gaussian_bf16(per_layer, s, 200 + l) for l, s in enumerate(sig)]
    return Workload("bucket_64m", segs, sig,
                    f"{layers} layers x {per_layer} values, sigma_l log-uniform in [1e-4, 1e-1]")


SPECIAL_PATTERNS = [None, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x7FFF, 0xFFFF]


def act_8192x7168(rows: int = 8192, cols: int = 7168, seed: int = 3) -> Workload:
    n = rows * cols
    g = torch.Generator(device="cpu").manual_seed(seed)
    base = torch.randn(n, generator=g, dtype=torch.float32)
    perm = torch.randperm(n, generator=g)
    n_zero = n * 5 // 100
    n_out = n // 1000
    n_spec = 1000
    out_idx = perm[n_zero:n_zero + n_out]
    base[out_idx] *= 100.0
    bits = _bf16_bits(base)
    bits[perm[:n_zero].numpy()] = 0x0000
    spec_idx = perm[n_zero + n_out:n_zero + n_out + n_spec].numpy()
    sub_mant = torch.randint(1, 128, (n_spec,), generator=g).numpy().astype(np.uint16)
    sub_sign = torch.randint(0, 2, (n_spec,), generator=g).numpy().astype(np.uint16)
    for k, pos in enumerate(spec_idx):
        pat = SPECIAL_PATTERNS[k % len(SPECIAL_PATTERNS)]
        if pat is None:
            pat = int(sub_sign[k]) << 15 | int(sub_mant[k])
        bits[pos] = pat
    return Workload("act_8192x7168", [bits], [1.0],
                    "8192x7168, N(0,1), 5% zeros, 0.1% x100 outliers, 1000 special patterns",
                    {"zero_idx": perm[:n_zero].numpy(), "spec_idx": spec_idx})


def zipf_counts(total: int, buckets: int, s: float) -> list:
    """Largest-remainder split of `total` in proportion to k**-s, k = 1..buckets."""
    w = np.array([k ** -s for k in range(1, buckets + 1)], dtype=np.float64)
    q = w / w.sum() * total
    c = np.floor(q).astype(np.int64)
    rem = total - int(c.sum())
    order = np.argsort(-(q - c), kind="stable")
    c[order[:rem]] += 1
    return [int(v) for v in c]


def moe_16384x7168(tokens: int = 16384, hidden: int = 7168, buckets: int = 8, s: float = 1.2,
                   sigma: float = 0.5, seed: int = 4) -> Workload:
    flat = gaussian_bf16(tokens * hidden, sigma, seed)
    counts = zipf_counts(tokens, buckets, s)
    segs, r = [], 0
    for c in counts:
        segs.append(flat[r * hidden:(r + c) * hidden])
        r += c
    return Workload("moe_16384x7168", segs, [sigma] * buckets,
                    f"{tokens}x{hidden} N(0,{sigma}), {buckets} Zipf({s}) buckets {counts}",
                    {"counts": counts, "hidden": hidden})


def moe_routed_16384x7168(tokens: int = 16384, hidden: int = 7168, buckets: int = 8, s: float = 1.2,
                          sigma: float = 0.5, seed: int = 4, route_seed: int = 41) -> Workload:
    flat = gaussian_bf16(tokens * hidden, sigma, seed)
    counts = zipf_counts(tokens, buckets, s)
    perm = np.random.default_rng(route_seed).permutation(tokens)
    rows, r = [], 0
    for c in counts:
        rows.append(np.sort(perm[r:r + c]).astype(np.int32))
        r += c
    return Workload("moe_routed_16384x7168", [flat], [sigma] * buckets,
                    f"{tokens}x{hidden} N(0,{sigma}) tokens routed to {buckets} destinations, Zipf({s}) counts {counts}",
                    {"counts": counts, "hidden": hidden, "rows": rows})


def rs_512m(peers: int = 7, shard: int = 1 << 26, chunk: int = 1 << 21, sigma: float = 1e-3) -> Workload:
    segs = [gaussian_bf16(shard, sigma, 500 + p) for p in range(peers)]
    local = gaussian_bf16(shard, sigma, 500 + peers)
    return Workload("rs_512m", segs, [sigma] * peers,
                    f"{peers} peer shards x {shard} values N(0,{sigma}) + local shard, chunks of {chunk}",
                    {"local": local, "chunk": chunk, "shard": shard, "peers": peers})


WORKLOADS = {
    "chunk_1m": chunk_1m,
    "bucket_64m": bucket_64m,
    "act_8192x7168": act_8192x7168,
    "moe_16384x7168": moe_16384x7168,
    "moe_routed_16384x7168": moe_routed_16384x7168,
    "rs_512m": rs_512m,
}


def get(name: str) -> Workload:
    return WORKLOADS[name]()
