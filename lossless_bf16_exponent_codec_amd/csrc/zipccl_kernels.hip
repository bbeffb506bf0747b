// HIP kernels of the lossless BF16 exponent codec for CDNA4 (gfx950), wave64.
//
// Method: "ZipCCL: Efficient Lossless Data Compression of Communication Collectives
// for Accelerating LLM Training" (gist.science explanation page), S2.B (split into
// sign+mantissa and exponent; top-7 exponents -> 3-bit codes, others -> escape code 0
// with the exponent in a separate array), S2.C (128-byte aligned sections, codes as
// three 1-bit planes), S2.D (local reduction on the reduce-scatter receive side).
// The byte layout (format version 1) is documented in include/zipccl.h.
//
// Work decomposition.  A tile is 512 values: lane l of a wave holds values
// 8l..8l+7, one 16-byte load.  A block is 8 tiles (4096 values, one escape-offset
// entry) and belongs to one wave.  A workgroup of 4 waves handles a unit of 4 blocks.
//   * Plane word (p, j) of a tile is the wave ballot of "bit p of code(8l + j)", so
//     the 24 words of a tile come from 24 ballots and land in SGPRs; v_writelane moves
//     them into one VGPR (lane k gets 32-bit half k) for a 192-byte vector store.
//   * Escapes: per-column escape ballots, mbcnt gives each lane the number of escapes
//     in lower lanes, the lane's own escapes follow in column order.  Escape bytes are
//     staged in LDS per wave and copied out once the unit's global position is known.
//   * The global escape position of each unit comes from a single-pass decoupled
//     look-back scan (Merrill & Garland, "Single-pass Parallel Prefix Scan with
//     Decoupled Look-back", 2016) over per-unit status words in the workspace.  Units
//     are numbered by a ticket taken at workgroup start, so a unit only ever waits for
//     units that are already running; every wait is bounded.
#include "zipccl_internal.h"
#include "zipccl.h"

namespace zc {

namespace {

constexpr uint32_t kStAggregate = 1;   // status flag: the unit's own count is published
constexpr uint32_t kStInclusive = 2;   // status flag: count including all earlier units
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr uint32_t kTagMask = (1u << 30) - 1;

__device__ inline uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ inline uint64_t ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }

// Number of set bits of m in the lanes below this one, plus acc.
__device__ inline uint32_t mbcnt(uint64_t m, uint32_t acc)
{
    return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), acc));
}

__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) { return __builtin_amdgcn_perm(hi, lo, sel); }

// k if this lane's bit of the wave-uniform mask is set, else 0: one v_cndmask with the
// mask as its SGPR-pair condition.
__device__ inline uint32_t lane_select(uint64_t mask, uint32_t k) { return __builtin_amdgcn_inverse_ballot_w64(mask) ? k : 0u; }

// llvm.amdgcn.writelane: the compiler knows this instruction, so it also inserts the
// wait states its operands need (inline assembly would hide them from it).
__device__ int zc_writelane(int src, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// Writes the wave-uniform value v into lane k of w (v_writelane_b32).
template <int k>
__device__ inline uint32_t write_lane(uint32_t w, uint32_t v)
{
    return uint32_t(zc_writelane(int(v), k, int(w)));
}

__device__ inline uint64_t ld_agent(const uint64_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void st_agent(uint64_t* p, uint64_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline uint32_t ld_agent32(const uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void st_agent32(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline uint32_t add_agent32(uint32_t* p, uint32_t v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void or_status(uint32_t* s, uint32_t bits)
{
    if (s) __hip_atomic_fetch_or(s, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t pack_status(uint32_t tag, uint32_t flag, uint32_t value)
{
    return (uint64_t(tag) << 34) | (uint64_t(flag) << 32) | value;
}

__device__ inline uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Segment holding global unit u: the last s with seg[s].unit0 <= u (segments are in
// unit order, seg[0].unit0 == 0).
template <class Seg>
__device__ inline int find_segment(const Seg* seg, int nseg, uint32_t u)
{
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (seg[mid].unit0 <= u) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Loads the 8 values of this lane in tile t; values at or past n read as 0.
__device__ inline uint4 load_lane(const uint16_t* src, uint64_t t, uint32_t lane, uint32_t n)
{
    uint64_t i = t * kTile + 8ull * lane;
    if (i + 8 <= n) return *reinterpret_cast<const uint4*>(src + i);
    uint32_t v[4] = {0, 0, 0, 0};
    for (uint32_t j = 0; j < 8; j++)
        if (i + j < n) v[j >> 1] |= uint32_t(src[i + j]) << (16 * (j & 1));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// --------------------------------------------------------------------------------
// compress
// --------------------------------------------------------------------------------
// Lane 2k of w receives the low half of plane word k = 8p + j, lane 2k+1 the high half.
template <int k>
__device__ inline void write_planes(uint32_t& w, const uint64_t (&P)[3][8])
{
    if constexpr (k < 24) {
        w = write_lane<2 * k>(w, uint32_t(P[k / 8][k % 8]));
        w = write_lane<2 * k + 1>(w, uint32_t(P[k / 8][k % 8] >> 32));
        write_planes<k + 1>(w, P);
    }
}
// Encodes one tile held by the wave.  `full`: all 512 values exist.  Writes the 512
// A bytes and the 192 plane bytes; appends this tile's escape exponents to the wave's
// LDS staging area at run..; returns the tile's escape count.
template <bool kFull>
__device__ inline uint32_t encode_tile(uint4 v, uint32_t lane, uint32_t nvalid, const uint8_t* s_lut,
                                       uint8_t* A_tile, uint32_t* B_tile, uint8_t* s_esc, uint32_t run)
{
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint32_t e[8], c[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        e[j] = (d[j >> 1] >> (7 + 16 * (j & 1))) & 0xFFu;
        c[j] = s_lut[e[j]];
        if (!kFull && uint32_t(j) >= nvalid) c[j] = 8;   // not a value: no plane bits, no escape
    }
    // sign+mantissa bytes: low byte of a BF16 holds the mantissa (bits 0-6), high byte
    // the sign (bit 7).  Gather low and high bytes of 4 values, then merge.
    uint32_t lo0 = perm(d[1], d[0], 0x06040200u), hi0 = perm(d[1], d[0], 0x07050301u);
    uint32_t lo1 = perm(d[3], d[2], 0x06040200u), hi1 = perm(d[3], d[2], 0x07050301u);
    uint2 a;
    a.x = (lo0 & 0x7F7F7F7Fu) | (hi0 & 0x80808080u);
    a.y = (lo1 & 0x7F7F7F7Fu) | (hi1 & 0x80808080u);
    *reinterpret_cast<uint2*>(A_tile + 8 * lane) = a;

    // 24 plane words: ballot of code bit p in column j.
    uint64_t P[3][8];
#pragma unroll
    for (int p = 0; p < 3; p++)
#pragma unroll
        for (int j = 0; j < 8; j++) P[p][j] = ballot((c[j] >> p) & 1u);
    uint32_t w = 0;
    write_planes<0>(w, P);
    if (lane < 48) B_tile[lane] = w;

    // escapes, in value order: lower lanes first, then this lane's columns in order
    uint64_t Z[8];
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        if (kFull) Z[j] = ~(P[0][j] | P[1][j] | P[2][j]);
        else Z[j] = ballot(c[j] == 0);
        cnt += __builtin_popcountll(Z[j]);
    }
    uint32_t r = run;
#pragma unroll
    for (int j = 0; j < 8; j++) r = mbcnt(Z[j], r);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        if (c[j] == 0) {
            s_esc[r] = uint8_t(e[j]);
            r++;
        }
    }
    return cnt;
}

__global__ __launch_bounds__(kThreads) void compress_kernel(const CArgs a)
{
    __shared__ uint8_t s_lut[256];
    __shared__ uint8_t s_esc[kWaves][kBlock];
    __shared__ uint32_t s_cnt[kWaves];
    __shared__ uint32_t s_misc[4];

    const uint32_t tid = threadIdx.x, lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t* wsu = a.ws;
    uint64_t* seg_base = reinterpret_cast<uint64_t*>(a.ws + 4);
    uint64_t* ust = seg_base + kMaxSegs;

    if (tid == 0) {
        s_misc[0] = add_agent32(&wsu[1], 1u);   // ticket = unit number in launch order
        s_misc[1] = ld_agent32(&wsu[0]);        // generation of this launch's status words
    }
    __syncthreads();
    const uint32_t unit = __builtin_amdgcn_readfirstlane(s_misc[0]);
    const uint32_t gen = __builtin_amdgcn_readfirstlane(s_misc[1]);
    const uint32_t tag = (gen + 1) & kTagMask;
    if (unit >= a.total_units) {
        // only possible with a workspace that was not zero-filled or a call that was
        // aborted: touch nothing, report, and still count towards the reset
        if (tid == 0) {
            or_status(a.status, ZIPCCL_STATUS_SCAN_TIMEOUT);
            uint32_t done = add_agent32(&wsu[2], 1u);
            if (done == a.total_units - 1) {
                st_agent32(&wsu[1], 0u);
                st_agent32(&wsu[2], 0u);
                st_agent32(&wsu[0], gen + 1);
            }
        }
        return;
    }

    const int s = find_segment(a.seg, a.nseg, unit);
    const CSeg& sg = a.seg[s];
    const uint32_t n = sg.n;
    const uint32_t ui = unit - sg.unit0;                 // unit within the segment
    const uint32_t T = uint32_t(tiles_of(n));
    const uint32_t K = uint32_t(blocks_of(n));
    const uint32_t units = uint32_t(units_of(n));
    uint8_t* dst = sg.dst;
    uint8_t* A = dst + 128;
    uint32_t* B = reinterpret_cast<uint32_t*>(dst + planes_off(n));
    uint32_t* C = reinterpret_cast<uint32_t*>(dst + offsets_off(n));

    // this wave's block and tiles
    const uint32_t b = ui * kWaves + wave;
    const uint32_t t0 = b * 8;
    const uint32_t ntiles = t0 < T ? min(8u, T - t0) : 0u;
    const uint32_t nfull = t0 < T ? min(ntiles, n / kTile - min(n / kTile, t0)) : 0u;

    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; k++)
        if (uint32_t(k) < ntiles) v[k] = load_lane(sg.src, t0 + k, lane, n);

    {   // exponent -> code table for this segment
        uint32_t e = tid, code = 0;
#pragma unroll
        for (int r = 0; r < 7; r++) {
            uint32_t te = (r < 4 ? (sg.table_lo >> (8 * r)) : (sg.table_hi >> (8 * (r - 4)))) & 0xFFu;
            if (te == e) code = r + 1;
        }
        s_lut[tid] = uint8_t(code);
    }
    __syncthreads();

    uint32_t run = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        uint32_t t = t0 + k;
        if (uint32_t(k) < nfull) {
            run += encode_tile<true>(v[k], lane, 8, s_lut, A + 512ull * t, B + 48ull * t, s_esc[wave], run);
        } else if (uint32_t(k) < ntiles) {
            uint64_t i = uint64_t(t) * kTile + 8ull * lane;
            uint32_t nvalid = i >= n ? 0u : uint32_t(min<uint64_t>(8, n - i));
            run += encode_tile<false>(v[k], lane, nvalid, s_lut, A + 512ull * t, B + 48ull * t, s_esc[wave], run);
        }
    }
    if (lane == 0) s_cnt[wave] = run;
    __syncthreads();
    uint32_t before = 0, agg = 0;
#pragma unroll
    for (uint32_t w = 0; w < kWaves; w++) {
        uint32_t c = __builtin_amdgcn_readfirstlane(s_cnt[w]);
        if (w < wave) before += c;
        agg += c;
    }

    // ---- decoupled look-back: exclusive escape count of all earlier units ----
    if (wave == 0) {
        uint32_t excl = 0;
        if (unit == 0) {
            if (lane == 0) st_agent(&ust[0], pack_status(tag, kStInclusive, agg));
        } else {
            if (lane == 0) st_agent(&ust[unit], pack_status(tag, kStAggregate, agg));
            int64_t hi = int64_t(unit) - 1;
            uint32_t spins = 0;
            while (true) {
                int64_t idx = hi - int64_t(lane);
                uint64_t wv = idx >= 0 ? ld_agent(&ust[idx]) : pack_status(tag, kStInclusive, 0);
                uint32_t flag = uint32_t(wv >> 32) & 3u;
                bool ready = (uint32_t(wv >> 34) == tag) && flag != 0;
                uint64_t notready = ~ballot(ready);
                uint64_t incl = ballot(ready && flag == kStInclusive);
                if (incl) {
                    uint32_t L = __builtin_ctzll(incl);
                    uint64_t need = L == 63 ? ~0ull : ((2ull << L) - 1);
                    if ((notready & need) == 0) {
                        excl += wave_sum(lane <= L ? uint32_t(wv) : 0u);
                        break;
                    }
                } else if (notready == 0) {
                    excl += wave_sum(uint32_t(wv));
                    hi -= 64;
                    continue;
                }
                if (++spins > kSpinLimit) {
                    if (lane == 0) or_status(a.status, ZIPCCL_STATUS_SCAN_TIMEOUT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (lane == 0) st_agent(&ust[unit], pack_status(tag, kStInclusive, excl + agg));
        }
        // escape count before the segment's first unit
        uint32_t segbase = excl;
        if (ui == 0) {
            if (lane == 0) st_agent(&seg_base[s], pack_status(tag, kStInclusive, excl));
        } else {
            uint32_t spins = 0;
            while (true) {
                uint64_t wv = ld_agent(&seg_base[s]);
                if (uint32_t(wv >> 34) == tag && ((uint32_t(wv >> 32) & 3u) == kStInclusive)) {
                    segbase = uint32_t(wv);
                    break;
                }
                if (++spins > kSpinLimit) {
                    if (lane == 0) or_status(a.status, ZIPCCL_STATUS_SCAN_TIMEOUT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (lane == 0) {
            s_misc[2] = excl;
            s_misc[3] = segbase;
        }
    }
    __syncthreads();
    const uint32_t excl = __builtin_amdgcn_readfirstlane(s_misc[2]);
    const uint32_t segbase = __builtin_amdgcn_readfirstlane(s_misc[3]);

    // ---- outputs that need the position: offsets, escapes, header ----
    const uint32_t mine = s_cnt[wave];
    const uint64_t gpos = uint64_t(excl) + before;   // first escape of this wave, launch-wide
    if (b < K && lane == 0) C[b] = uint32_t(gpos - segbase);
    for (uint32_t k = lane; k < mine; k += 64) {
        uint64_t pos = gpos + k;
        if (pos < a.esc_cap) a.esc[pos] = s_esc[wave][k];
        else or_status(a.status, ZIPCCL_STATUS_ESC_OVERFLOW);
    }

    if (ui == units - 1) {
        const uint32_t n_esc = excl + agg - segbase;
        if (wave == 0 && lane < 32) {
            const uint64_t sb = static_bytes_of(n);
            uint32_t hv = 0;
            switch (lane) {
                case 0: hv = ZIPCCL_MAGIC; break;
                case 1: hv = 1u; break;                  // version 1, flags 0
                case 2: hv = n; break;
                case 4: hv = sg.table_lo; break;
                case 5: hv = sg.table_hi & 0x00FFFFFFu; break;
                case 6: hv = kBlock; break;
                case 7: hv = kTile; break;
                case 8: hv = n_esc; break;
                case 10: hv = segbase; break;
                case 12: hv = uint32_t(sb); break;
                case 13: hv = uint32_t(sb >> 32); break;
                default: hv = 0; break;
            }
            reinterpret_cast<uint32_t*>(dst)[lane] = hv;
            if (lane == 0 && a.n_esc_out) a.n_esc_out[s] = n_esc;
            if (lane == 0 && a.n_esc_out && unit == a.total_units - 1) a.n_esc_out[a.nseg] = excl + agg;
        }
        if (wave == 1) {   // zero padding of the plane and offset sections
            const uint32_t bpad = uint32_t(round128(192ull * T) - 192ull * T);
            uint8_t* bp = reinterpret_cast<uint8_t*>(B) + 192ull * T;
            for (uint32_t k = lane; k < bpad; k += 64) bp[k] = 0;
            const uint32_t cpad = uint32_t(round128(4ull * K) - 4ull * K);
            uint8_t* cp = reinterpret_cast<uint8_t*>(C) + 4ull * K;
            for (uint32_t k = lane; k < cpad; k += 64) cp[k] = 0;
        }
    }

    // ---- last workgroup to finish resets the counters and advances the generation ----
    if (tid == 0) {
        uint32_t done = add_agent32(&wsu[2], 1u);
        if (done == a.total_units - 1) {
            st_agent32(&wsu[1], 0u);
            st_agent32(&wsu[2], 0u);
            st_agent32(&wsu[0], gen + 1);
        }
    }
}

// --------------------------------------------------------------------------------
// decode helpers
// --------------------------------------------------------------------------------
struct SegHeader {
    bool ok;
    uint32_t tlo, thi;     // table bytes, byte 0 of tlo is the escape placeholder 0
    uint32_t n_esc;
    uint64_t esc_offset;
};

// Reads and validates a segment header against the expected n and buffer sizes.
__device__ inline SegHeader read_header(const uint8_t* st, uint32_t n, uint64_t esc_bytes)
{
    const uint32_t* h = reinterpret_cast<const uint32_t*>(st);
    SegHeader r;
    uint32_t magic = h[0], ver = h[1], nlo = h[2], nhi = h[3];
    uint32_t t0 = h[4], t1 = h[5];
    uint32_t blk = h[6], tile = h[7];
    uint64_t n_esc = uint64_t(h[8]) | (uint64_t(h[9]) << 32);
    uint64_t eoff = uint64_t(h[10]) | (uint64_t(h[11]) << 32);
    uint64_t sb = uint64_t(h[12]) | (uint64_t(h[13]) << 32);
    bool ok = magic == ZIPCCL_MAGIC && ver == 1u && nlo == n && nhi == 0 && blk == kBlock && tile == kTile &&
              sb == static_bytes_of(n) && n_esc <= n && eoff <= esc_bytes && n_esc <= esc_bytes - eoff;
    // table: 7 ascending values in 1..254 (byte 3 of t1 must be 0)
    uint32_t prev = 0;
    for (int r2 = 0; r2 < 7; r2++) {
        uint32_t e = (r2 < 4 ? (t0 >> (8 * r2)) : (t1 >> (8 * (r2 - 4)))) & 0xFFu;
        ok = ok && e > prev && e <= 254;
        prev = e;
    }
    ok = ok && (t1 >> 24) == 0;
    r.ok = ok;
    // 8-byte decode table for v_perm: byte 0 = placeholder for code 0, bytes 1..7 = table
    r.tlo = t0 << 8;
    r.thi = (t0 >> 24) | (t1 << 8);
    r.n_esc = uint32_t(n_esc);
    r.esc_offset = eoff;
    return r;
}

// Escape range of block b: [first, last) within the segment's escapes; false if the
// offset table is inconsistent.
__device__ inline bool block_escapes(const uint32_t* C, uint32_t b, uint32_t K, uint32_t n_esc, uint32_t nvals,
                                     uint32_t& first, uint32_t& last)
{
    first = C[b];
    last = (b + 1 < K) ? C[b + 1] : n_esc;
    return first <= last && last <= n_esc && last - first <= nvals;
}

__device__ inline uint32_t load_sgpr32(const uint32_t* p) { return __builtin_amdgcn_readfirstlane(*p); }

// Decodes one tile: returns the 8 BF16 values of this lane as 4 dwords.
//   Ap: this lane's 8 A bytes; P: the tile's 24 plane words; esc: the wave's staged
//   escape bytes starting at this tile's first escape; valid: values of this lane that
//   exist (8 for a full tile).  Returns the tile's escape count via *cnt.
template <bool kFull>
__device__ inline uint4 decode_tile(uint2 Ap, const uint64_t* P, uint32_t tlo, uint32_t thi, const uint8_t* s_esc,
                                    uint32_t run, uint32_t lane, uint32_t nvalid, uint32_t* cnt)
{
    // codes as bytes: C0 = columns 0..3, C1 = columns 4..7
    uint32_t C0 = 0, C1 = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        C0 |= lane_select(P[j], 1u << (8 * j)) | lane_select(P[8 + j], 2u << (8 * j)) |
              lane_select(P[16 + j], 4u << (8 * j));
        C1 |= lane_select(P[4 + j], 1u << (8 * j)) | lane_select(P[12 + j], 2u << (8 * j)) |
              lane_select(P[20 + j], 4u << (8 * j));
    }
    uint32_t E0 = perm(thi, tlo, C0), E1 = perm(thi, tlo, C1);

    // escapes of the tile: code 0 and inside the segment
    uint64_t Z[8];
    uint32_t total = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        Z[j] = ~(P[j] | P[8 + j] | P[16 + j]);
        if (!kFull) Z[j] &= ballot(uint32_t(j) < nvalid);
        total += __builtin_popcountll(Z[j]);
    }
    *cnt = total;
    if (total) {
        uint32_t r = run;
#pragma unroll
        for (int j = 0; j < 8; j++) r = mbcnt(Z[j], r);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            if ((Z[j] >> lane) & 1ull) {
                uint32_t x = s_esc[r++];
                if (j < 4) E0 = (E0 & ~(0xFFu << (8 * j))) | (x << (8 * j));
                else E1 = (E1 & ~(0xFFu << (8 * (j - 4)))) | (x << (8 * (j - 4)));
            }
        }
    }
    // reassemble: low byte = exponent bit 0 << 7 | mantissa, high byte = sign | exponent >> 1
    uint32_t lo0 = (Ap.x & 0x7F7F7F7Fu) | ((E0 << 7) & 0x80808080u);
    uint32_t hi0 = (Ap.x & 0x80808080u) | ((E0 >> 1) & 0x7F7F7F7Fu);
    uint32_t lo1 = (Ap.y & 0x7F7F7F7Fu) | ((E1 << 7) & 0x80808080u);
    uint32_t hi1 = (Ap.y & 0x80808080u) | ((E1 >> 1) & 0x7F7F7F7Fu);
    uint4 o;
    o.x = perm(hi0, lo0, 0x05010400u);
    o.y = perm(hi0, lo0, 0x07030602u);
    o.z = perm(hi1, lo1, 0x05010400u);
    o.w = perm(hi1, lo1, 0x07030602u);
    return o;
}

__device__ inline void load_planes(const uint8_t* Bt, uint64_t P[24])
{
    const uint64_t* q = reinterpret_cast<const uint64_t*>(Bt);
#pragma unroll
    for (int w = 0; w < 24; w++) P[w] = q[w];
}

// --------------------------------------------------------------------------------
// decompress
// --------------------------------------------------------------------------------
// Decodes block b of one segment.  `st` is only read in the kernel, so it is marked
// restrict: the plane words and the header then load through the scalar cache.
__device__ __forceinline__ void decode_block(const uint8_t* __restrict__ st, const uint8_t* __restrict__ esc_base,
                                          uint64_t esc_bytes, uint16_t* dst, uint32_t n, uint32_t b, uint32_t lane,
                                          uint8_t* s_esc, uint32_t* status)
{
    const uint32_t T = uint32_t(tiles_of(n)), K = uint32_t(blocks_of(n));
    const SegHeader h = read_header(st, n, esc_bytes);
    if (!h.ok) {
        if (lane == 0) or_status(status, ZIPCCL_STATUS_CORRUPT);
        return;
    }
    const uint8_t* A = st + 128;
    const uint8_t* B = st + planes_off(n);
    const uint32_t* C = reinterpret_cast<const uint32_t*>(st + offsets_off(n));
    const uint32_t nvals = min(kBlock, n - b * kBlock);
    uint32_t first, last;
    if (!block_escapes(C, b, K, h.n_esc, nvals, first, last)) {
        if (lane == 0) or_status(status, ZIPCCL_STATUS_CORRUPT);
        return;
    }
    const uint8_t* esc = esc_base + h.esc_offset + first;
    for (uint32_t k = lane; k < last - first; k += 64) s_esc[k] = esc[k];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const uint32_t t0 = b * 8;
    const uint32_t ntiles = min(8u, T - t0);
    uint32_t run = 0;
    for (uint32_t k = 0; k < ntiles; k++) {
        const uint32_t t = t0 + k;
        uint64_t P[24];
        load_planes(B + 192ull * t, P);
        uint2 Ap = *reinterpret_cast<const uint2*>(A + 512ull * t + 8 * lane);
        const uint64_t i = uint64_t(t) * kTile + 8ull * lane;
        uint32_t cnt;
        if ((uint64_t(t) + 1) * kTile <= n) {
            uint4 o = decode_tile<true>(Ap, P, h.tlo, h.thi, s_esc, run, lane, 8, &cnt);
            *reinterpret_cast<uint4*>(dst + i) = o;
        } else {
            uint32_t nvalid = i >= n ? 0u : uint32_t(min<uint64_t>(8, n - i));
            uint4 o = decode_tile<false>(Ap, P, h.tlo, h.thi, s_esc, run, lane, nvalid, &cnt);
            const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
            for (uint32_t j = 0; j < nvalid; j++) dst[i + j] = uint16_t(ov[j >> 1] >> (16 * (j & 1)));
        }
        run += cnt;
    }
    if (run != last - first && lane == 0) or_status(status, ZIPCCL_STATUS_CORRUPT);
}

__global__ __launch_bounds__(kThreads) void decompress_kernel(const DArgs a)
{
    __shared__ uint8_t s_esc[kWaves][kBlock];
    const uint32_t lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t unit = blockIdx.x;
    const int s = find_segment(a.seg, a.nseg, unit);
    const uint32_t n = a.seg[s].n;
    const uint32_t b = (unit - a.seg[s].unit0) * kWaves + wave;
    if (b >= blocks_of(n)) return;
    decode_block(a.seg[s].src, a.esc, a.esc_bytes, a.seg[s].dst, n, b, lane, s_esc[wave], a.status);
}

// --------------------------------------------------------------------------------
// decompress + fp32 accumulate + one rounding
// --------------------------------------------------------------------------------
__device__ inline uint32_t round_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kThreads) void accumulate_kernel(const AArgs a)
{
    __shared__ uint8_t s_esc[kWaves][kBlock];
    const uint32_t tid = threadIdx.x, lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t n = a.n;
    const uint32_t T = uint32_t(tiles_of(n)), K = uint32_t(blocks_of(n));
    const uint32_t b = blockIdx.x * kWaves + wave;
    if (b >= K) return;
    const uint32_t t0 = b * 8;
    const uint32_t ntiles = min(8u, T - t0);
    const uint32_t nvals = min(kBlock, n - b * kBlock);

    // acc = f32(local)
    float acc[8][8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        if (uint32_t(k) < ntiles) {
            uint4 v = load_lane(a.local, t0 + k, lane, n);
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 8; j++) acc[k][j] = __uint_as_float((j & 1) ? (d[j >> 1] & 0xFFFF0000u) : (d[j >> 1] << 16));
        }
    }
    bool bad = false;
    for (int p = 0; p < a.npeers; p++) {
        const uint8_t* st = a.st[p];
        const SegHeader h = read_header(st, n, a.esc_bytes[p]);
        const uint8_t* A = st + 128;
        const uint8_t* B = st + planes_off(n);
        const uint32_t* C = reinterpret_cast<const uint32_t*>(st + offsets_off(n));
        uint32_t first = 0, last = 0;
        if (!h.ok || !block_escapes(C, b, K, h.n_esc, nvals, first, last)) {
            bad = true;
            break;
        }
        const uint8_t* esc = a.esc[p] + h.esc_offset + first;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        for (uint32_t k = lane; k < last - first; k += 64) s_esc[wave][k] = esc[k];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint32_t run = 0;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            if (uint32_t(k) < ntiles) {
                const uint32_t t = t0 + k;
                uint64_t P[24];
                load_planes(B + 192ull * t, P);
                uint2 Ap = *reinterpret_cast<const uint2*>(A + 512ull * t + 8 * lane);
                uint32_t cnt;
                uint4 o;
                if ((uint64_t(t) + 1) * kTile <= n) {
                    o = decode_tile<true>(Ap, P, h.tlo, h.thi, s_esc[wave], run, lane, 8, &cnt);
                } else {
                    const uint64_t i = uint64_t(t) * kTile + 8ull * lane;
                    uint32_t nvalid = i >= n ? 0u : uint32_t(min<uint64_t>(8, n - i));
                    o = decode_tile<false>(Ap, P, h.tlo, h.thi, s_esc[wave], run, lane, nvalid, &cnt);
                }
                run += cnt;
                const uint32_t d[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int j = 0; j < 8; j++)
                    acc[k][j] = acc[k][j] + __uint_as_float((j & 1) ? (d[j >> 1] & 0xFFFF0000u) : (d[j >> 1] << 16));
            }
        }
        if (run != last - first) {
            bad = true;
            break;
        }
    }
    if (bad) {
        if (lane == 0) or_status(a.status, ZIPCCL_STATUS_CORRUPT);
        return;
    }
#pragma unroll
    for (int k = 0; k < 8; k++) {
        if (uint32_t(k) < ntiles) {
            const uint32_t t = t0 + k;
            const uint64_t i = uint64_t(t) * kTile + 8ull * lane;
            uint32_t r[8];
#pragma unroll
            for (int j = 0; j < 8; j++) r[j] = round_bf16_bits(acc[k][j]);
            if (i + 8 <= n) {
                uint4 o = make_uint4(r[0] | (r[1] << 16), r[2] | (r[3] << 16), r[4] | (r[5] << 16), r[6] | (r[7] << 16));
                *reinterpret_cast<uint4*>(a.dst + i) = o;
            } else {
                for (uint32_t j = 0; j < 8; j++)
                    if (i + j < n) a.dst[i + j] = uint16_t(r[j]);
            }
        }
    }
}

}  // namespace

hipError_t launch_compress(const CArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(compress_kernel, dim3(a.total_units), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decompress(const DArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(decompress_kernel, dim3(a.total_units), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_accumulate(const AArgs& a, hipStream_t s)
{
    uint32_t grid = uint32_t((blocks_of(a.n) + kWaves - 1) / kWaves);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(accumulate_kernel, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace zc
