// Host layer of libzipccl: plans, sizes, argument validation, launches, chunk
// sequences and the two-stream chunk pipeline.  Every device-side step runs in
// zipccl_kernels.hip.
//
// Method: "ZipCCL: Efficient Lossless Data Compression of Communication Collectives
// for Accelerating LLM Training" (gist.science explanation page), S2.A (sigma-derived
// exponent table), S2.B (3-bit codes + escapes), S2.D (two-phase MoE all-to-all and the
// reduce-scatter's local reduction), S4 (the all-gather); the chunked multi-stream
// pipeline follows the CCCL page's pipeline section.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>
#include <new>
#include <random>

#include "zipccl.h"
#include "zipccl_internal.h"

using namespace zc;

namespace {

// Where the window of 7 binades moves up by one: for log2(sigma) with fractional part
// c the lowest binade of the window and the binade just above it hold equal Gaussian
// mass.  Solved by bisection on 2[Phi(2^(k+1)/s) - Phi(2^k/s)] (continuous model).
constexpr double kSwitchPhase = 0.7195805543641254;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

zipccl_status hip_status(hipError_t e) { return e == hipSuccess ? ZIPCCL_OK : ZIPCCL_ERR_HIP; }

// Largest launch (in workgroup units) whose escape positions the place kernel computes
// itself.  ZIPCCL_DIRECT_PREFIX_MAX_UNITS lowers it, which tests use to exercise the
// scan-kernel path on small inputs.
uint64_t direct_prefix_max_units()
{
    const char* e = std::getenv("ZIPCCL_DIRECT_PREFIX_MAX_UNITS");
    if (!e || !*e) return kDirectPrefixMaxUnits;
    return std::min<uint64_t>(std::strtoull(e, nullptr, 10), kDirectPrefixMaxUnits);
}

// Tags of the single-launch compress: one per call, process-wide, 48 bits, never 0.  The
// ready words a call's encoders write carry its tag, so the placing workgroups tell them
// from words an earlier call left in the same workspace (no call repeats a tag in this
// process; the random start makes a match with memory another process left unlikely).
uint64_t next_tag()
{
    static std::atomic<uint64_t> counter{[] {
        std::random_device rd;
        const uint64_t t = uint64_t(std::chrono::steady_clock::now().time_since_epoch().count());
        return (uint64_t(rd()) << 32) ^ uint64_t(rd()) ^ (t * 0x9E3779B97F4A7C15ull);
    }()};
    for (;;) {
        const uint64_t t = counter.fetch_add(1, std::memory_order_relaxed) & ((1ull << (64 - kReadyCountBits)) - 1);
        if (t != 0) return t;
    }
}

// Whether a compress call runs as one launch: yes unless the positions need the scan
// kernel, the caller passed no status word, the stream is being captured into a graph (a
// replay would repeat the tag baked into the captured arguments), or
// ZIPCCL_SINGLE_LAUNCH=0 asks for the two-launch path.  The single launch's placing
// workgroups wait (bounded) for the encoders, and a wait that runs out is reported only
// through the status word; without one the two launches, which wait for nothing, run
// instead, so no call can end with unwritten headers that nobody is told about.
bool single_launch(const CArgs& a, hipStream_t stream)
{
    if (!a.direct || !a.status) return false;
    const char* e = std::getenv("ZIPCCL_SINGLE_LAUNCH");
    if (e && e[0] == '0' && e[1] == 0) return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return false;
    return cs == hipStreamCaptureStatusNone;
}

hipError_t compress_launch(CArgs& a, hipStream_t stream)
{
    const bool single = single_launch(a, stream);
    a.tag = single ? next_tag() : 0;
    a.wait_tag = a.tag;
    a.wait_polls = 1u << 16;
    // Test hook for the bounded wait's error path: the placing workgroups wait for a tag
    // no call uses, 4 polls per word, so every one gives up and reports
    // ZIPCCL_STATUS_WAIT_LIMIT (and writes nothing) within microseconds.
    const char* e = std::getenv("ZIPCCL_TEST_WAIT_LIMIT");
    if (single && e && e[0] == '1' && e[1] == 0) {
        a.wait_tag = (a.tag ^ (1ull << 47)) | 1u;   // never this call's tag, never 0
        a.wait_polls = 4;
    }
    return launch_compress(a, stream, single);
}

void pack_table(const zipccl_plan_t& p, uint32_t& lo, uint32_t& hi)
{
    lo = uint32_t(p.table[0]) | uint32_t(p.table[1]) << 8 | uint32_t(p.table[2]) << 16 | uint32_t(p.table[3]) << 24;
    hi = uint32_t(p.table[4]) | uint32_t(p.table[5]) << 8 | uint32_t(p.table[6]) << 16;
}

bool plan_valid(const zipccl_plan_t& p)
{
    for (int r = 0; r < 7; r++) {
        if (p.table[r] < 1 || p.table[r] > 254) return false;
        if (r > 0 && p.table[r] <= p.table[r - 1]) return false;   // strictly ascending
    }
    return true;
}

}  // namespace

extern "C" {

const char* zipccl_strerror(zipccl_status s)
{
    switch (s) {
        case ZIPCCL_OK: return "ok";
        case ZIPCCL_ERR_INVALID: return "invalid argument";
        case ZIPCCL_ERR_ALIGN: return "misaligned pointer";
        case ZIPCCL_ERR_SIZE: return "size limit exceeded or buffer too small";
        case ZIPCCL_ERR_HIP: return "HIP runtime error";
        case ZIPCCL_ERR_CORRUPT: return "corrupt data or a device status bit set";
    }
    return "unknown status";
}

zipccl_status zipccl_plan(double sigma, const uint8_t* table7, zipccl_plan_t* out)
{
    if (!out) return ZIPCCL_ERR_INVALID;
    zipccl_plan_t p{};
    if (table7) {
        uint8_t t[7];
        std::memcpy(t, table7, 7);
        std::sort(t, t + 7);
        std::memcpy(p.table, t, 7);
        if (!plan_valid(p)) return ZIPCCL_ERR_INVALID;   // also rejects duplicates
    } else {
        if (!(sigma > 0.0) || !std::isfinite(sigma)) return ZIPCCL_ERR_INVALID;
        double e0 = 123.0 + std::floor(std::log2(sigma) - kSwitchPhase);
        e0 = std::min(248.0, std::max(1.0, e0));
        for (int r = 0; r < 7; r++) p.table[r] = uint8_t(int(e0) + r);
    }
    *out = p;
    return ZIPCCL_OK;
}

zipccl_status zipccl_plan_many(const double* sigma, int n, zipccl_plan_t* out)
{
    if (n < 0 || (n > 0 && (!sigma || !out))) return ZIPCCL_ERR_INVALID;
    for (int i = 0; i < n; i++) {
        const zipccl_status r = zipccl_plan(sigma[i], nullptr, out + i);
        if (r != ZIPCCL_OK) return r;
    }
    return ZIPCCL_OK;
}

uint64_t zipccl_static_size(uint64_t n) { return static_bytes_of(n); }

uint64_t zipccl_compressed_size(uint64_t n, uint64_t n_esc) { return static_bytes_of(n) + n_esc; }

uint64_t zipccl_workspace_size(uint64_t total_n, int nseg)
{
    if (nseg < 1) nseg = 1;
    return ws_bytes(total_n / kUnit + uint64_t(nseg));   // bounds the sum of ceil(n_s / 16384)
}

namespace {

// Workspace sections of a launch of `units` units (the sizes depend on the count).
void set_workspace(CArgs& a, void* workspace, uint64_t units)
{
    uint8_t* w = static_cast<uint8_t*>(workspace);
    a.counts = reinterpret_cast<uint32_t*>(w);
    w += ws_counts_bytes(units);
    a.pos = reinterpret_cast<uint32_t*>(w);
    w += ws_pos_bytes(units);
    a.unit_counts = reinterpret_cast<uint32_t*>(w);
    w += ws_units_bytes(units);
    a.ready = reinterpret_cast<uint64_t*>(w);
    w += ws_ready_bytes(units);
    a.stage = w;
}

// Completes the compress arguments once a.seg[0..nseg) holds src, rows, row_len,
// src_rows, n and the table of each segment.
zipccl_status prepare_compress(CArgs& a, int nseg, void* static_out, uint64_t static_cap, void* esc_out,
                               uint64_t esc_cap, void* workspace, uint64_t workspace_bytes, uint64_t* n_esc_out,
                               uint32_t* status)
{
    uint64_t total = 0, units = 0, blocks = 0, st_off = 0;
    for (int s = 0; s < nseg; s++) {
        CSeg& c = a.seg[s];
        c.dst = static_cast<uint8_t*>(static_out) + st_off;
        c.unit0 = uint32_t(units);
        c.block0 = uint32_t(blocks);
        total += c.n;
        units += units_of(c.n);
        blocks += blocks_of(c.n);
        st_off += static_bytes_of(c.n);
    }
    if (total >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
    if (st_off > static_cap) return ZIPCCL_ERR_SIZE;
    if (ws_bytes(units) > workspace_bytes) return ZIPCCL_ERR_SIZE;
    if (esc_cap > 0 && !esc_out) return ZIPCCL_ERR_INVALID;
    CCall& c = a.call[0];
    c.esc = static_cast<uint8_t*>(esc_out);
    c.esc_cap = esc_out ? esc_cap : 0;
    c.n_esc_out = n_esc_out;
    c.seg0 = 0;
    c.nseg = uint32_t(nseg);
    c.unit0 = 0;
    c.block_end = uint32_t(blocks);
    for (int s = 0; s < nseg; s++) a.seg[s].call = 0;
    a.ncalls = 1;
    set_workspace(a, workspace, units);
    a.status = status;
    a.nseg = nseg;
    a.total_units = uint32_t(units);
    a.total_blocks = uint32_t(blocks);
    a.direct = (units > 0 && units <= direct_prefix_max_units()) ? 1u : 0u;
    return ZIPCCL_OK;
}

zipccl_status compress_segments(CArgs& a, int nseg, void* static_out, uint64_t static_cap, void* esc_out,
                                uint64_t esc_cap, void* workspace, uint64_t workspace_bytes, uint64_t* n_esc_out,
                                uint32_t* status, void* stream)
{
    if (zipccl_status r = prepare_compress(a, nseg, static_out, static_cap, esc_out, esc_cap, workspace,
                                           workspace_bytes, n_esc_out, status))
        return r;
    return hip_status(compress_launch(a, static_cast<hipStream_t>(stream)));
}

zipccl_status check_compress_buffers(int nseg, void* static_out, void* workspace, uint64_t* n_esc_out,
                                     uint32_t* status)
{
    if (nseg < 1 || nseg > kMaxSegs || !static_out || !workspace) return ZIPCCL_ERR_INVALID;
    if (!aligned(static_out, 128) || !aligned(workspace, 256) || (n_esc_out && !aligned(n_esc_out, 8)) ||
        (status && !aligned(status, 4)))
        return ZIPCCL_ERR_ALIGN;
    return ZIPCCL_OK;
}

}  // namespace

namespace {

// Segments of a plain (contiguous) compress call into a.seg (their plans are checked
// unless the tables come from device memory).
zipccl_status fill_segments(CArgs& a, const zipccl_segment_t* segs, int nseg, bool check_plans = true)
{
    std::memset(&a, 0, sizeof(a));
    for (int s = 0; s < nseg; s++) {
        const zipccl_segment_t& g = segs[s];
        if (g.n >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
        if (g.n > 0 && !g.src) return ZIPCCL_ERR_INVALID;
        if (!aligned(g.src, 16)) return ZIPCCL_ERR_ALIGN;
        if (check_plans && !plan_valid(g.plan)) return ZIPCCL_ERR_INVALID;
        CSeg& c = a.seg[s];
        c.src = static_cast<const uint16_t*>(g.src);
        c.n = uint32_t(g.n);
        pack_table(g.plan, c.table_lo, c.table_hi);
    }
    return ZIPCCL_OK;
}

// Launches prepared chunk calls in order on one stream.  Consecutive calls whose
// positions the place workgroups compute themselves (direct: at most
// kDirectPrefixMaxUnits units each) share a launch while the launch has room (kMaxCalls
// calls, kLaunchSegs segments) and the workspace holds all their units; each keeps its
// own outputs and escape numbering.
zipccl_status launch_chunks(const std::vector<CArgs>& calls, void* workspace, uint64_t workspace_bytes,
                            hipStream_t stream)
{
    size_t k = 0;
    while (k < calls.size()) {
        CArgs b = calls[k];
        size_t j = k + 1;
        if (b.direct && !b.dplans) {
            for (; j < calls.size() && b.ncalls < kMaxCalls; j++) {
                const CArgs& c = calls[j];
                const uint64_t units = uint64_t(b.total_units) + c.total_units;
                if (!c.direct || c.dplans || b.nseg + c.nseg > kLaunchSegs || units >= (1ull << 32) ||
                    ws_bytes(units) > workspace_bytes)
                    break;
                for (int s = 0; s < c.nseg; s++) {
                    CSeg g = c.seg[s];
                    g.unit0 += b.total_units;
                    g.block0 += b.total_blocks;
                    g.call = uint32_t(b.ncalls);
                    b.seg[b.nseg + s] = g;
                }
                CCall cc = c.call[0];
                cc.seg0 = uint32_t(b.nseg);
                cc.unit0 = b.total_units;
                cc.block_end = b.total_blocks + c.total_blocks;
                b.call[b.ncalls++] = cc;
                b.nseg += c.nseg;
                b.total_units = uint32_t(units);
                b.total_blocks += c.total_blocks;
            }
            set_workspace(b, workspace, b.total_units);
        }
        if (hipError_t e = compress_launch(b, stream)) return hip_status(e);
        k = j;
    }
    return ZIPCCL_OK;
}

}  // namespace

zipccl_status zipccl_compress(const zipccl_segment_t* segs, int nseg, void* static_out, uint64_t static_cap,
                              void* esc_out, uint64_t esc_cap, void* workspace, uint64_t workspace_bytes,
                              uint64_t* n_esc_out, uint32_t* status, void* stream)
{
    if (!segs) return ZIPCCL_ERR_INVALID;
    if (zipccl_status r = check_compress_buffers(nseg, static_out, workspace, n_esc_out, status)) return r;
    CArgs a;
    if (zipccl_status r = fill_segments(a, segs, nseg)) return r;
    return compress_segments(a, nseg, static_out, static_cap, esc_out, esc_cap, workspace, workspace_bytes,
                             n_esc_out, status, stream);
}

static_assert(kNoAllocMaxValues == ZIPCCL_NOALLOC_MAX_VALUES && kNoAllocScratchBytes == ZIPCCL_NOALLOC_SCRATCH_BYTES,
              "the header states the static workspace's limits");

zipccl_status zipccl_compress_noalloc(const zipccl_segment_t* segs, int nseg, void* static_out, uint64_t static_cap,
                                      void* esc_out, uint64_t esc_cap, uint64_t* n_esc_out, uint32_t* status,
                                      void* stream)
{
    if (!segs || nseg < 1 || nseg > kMaxSegs || !static_out) return ZIPCCL_ERR_INVALID;
    uint64_t total = 0;
    for (int s = 0; s < nseg; s++) {
        if (segs[s].n > kNoAllocMaxValues) return ZIPCCL_ERR_SIZE;
        total += segs[s].n;
    }
    if (total > kNoAllocMaxValues) return ZIPCCL_ERR_SIZE;   // beyond the static workspace
    if (!aligned(static_out, 128) || (n_esc_out && !aligned(n_esc_out, 8)) || (status && !aligned(status, 4)))
        return ZIPCCL_ERR_ALIGN;
    CArgs a;
    if (zipccl_status r = fill_segments(a, segs, nseg)) return r;
    void* ws = nullptr;   // the library's static device array on the stream's device
    if (hipError_t e = noalloc_workspace(static_cast<hipStream_t>(stream), &ws)) return hip_status(e);
    return compress_segments(a, nseg, static_out, static_cap, esc_out, esc_cap, ws, kNoAllocScratchBytes, n_esc_out,
                             status, stream);
}

uint64_t zipccl_estimate_workspace_size(int nseg)
{
    if (nseg < 1) nseg = 1;
    return uint64_t(nseg) * kEstParts * 16;
}

zipccl_status zipccl_estimate_plans(const zipccl_segment_t* segs, int nseg, uint32_t stride, zipccl_plan_t* plans_dev,
                                    void* workspace, uint64_t workspace_bytes, void* stream)
{
    if (!segs || nseg < 1 || nseg > kMaxSegs || stride < 1 || !plans_dev || !workspace) return ZIPCCL_ERR_INVALID;
    if (!aligned(plans_dev, 8) || !aligned(workspace, 16)) return ZIPCCL_ERR_ALIGN;
    if (workspace_bytes < zipccl_estimate_workspace_size(nseg)) return ZIPCCL_ERR_SIZE;
    EArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int s = 0; s < nseg; s++) {
        if (segs[s].n >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
        if (segs[s].n > 0 && !segs[s].src) return ZIPCCL_ERR_INVALID;
        if (!aligned(segs[s].src, 16)) return ZIPCCL_ERR_ALIGN;
        a.src[s] = static_cast<const uint16_t*>(segs[s].src);
        a.n[s] = uint32_t(segs[s].n);
    }
    a.plans = reinterpret_cast<uint8_t*>(plans_dev);
    a.partial = static_cast<double*>(workspace);
    a.stride = stride;
    a.nseg = nseg;
    return hip_status(launch_estimate_plans(a, static_cast<hipStream_t>(stream)));
}

zipccl_status zipccl_compress_device_plans(const zipccl_segment_t* segs, int nseg, const zipccl_plan_t* plans_dev,
                                           void* static_out, uint64_t static_cap, void* esc_out, uint64_t esc_cap,
                                           void* workspace, uint64_t workspace_bytes, uint64_t* n_esc_out,
                                           uint32_t* status, void* stream)
{
    if (!segs || !plans_dev) return ZIPCCL_ERR_INVALID;
    if (!aligned(plans_dev, 8)) return ZIPCCL_ERR_ALIGN;
    if (zipccl_status r = check_compress_buffers(nseg, static_out, workspace, n_esc_out, status)) return r;
    CArgs a;
    if (zipccl_status r = fill_segments(a, segs, nseg, false)) return r;
    a.dplans = reinterpret_cast<const uint8_t*>(plans_dev);
    return compress_segments(a, nseg, static_out, static_cap, esc_out, esc_cap, workspace, workspace_bytes,
                             n_esc_out, status, stream);
}

zipccl_status zipccl_compress_chunks(const zipccl_segment_t* segs, int nseg, int nchunks, void* const* static_out,
                                     const uint64_t* static_cap, void* const* esc_out, const uint64_t* esc_cap,
                                     void* workspace, uint64_t workspace_bytes, uint64_t* n_esc_out,
                                     uint32_t* status, void* stream)
{
    if (nchunks < 0 || nseg < 1 || nseg > kMaxPeers) return ZIPCCL_ERR_INVALID;
    if (nchunks == 0) return ZIPCCL_OK;
    if (!segs || !static_out || !static_cap || !esc_out || !esc_cap || !workspace) return ZIPCCL_ERR_INVALID;
    if (!aligned(workspace, 256)) return ZIPCCL_ERR_ALIGN;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    std::vector<CArgs> calls;   // every chunk is checked before anything is enqueued
    try {
        calls.resize(size_t(nchunks));
    } catch (...) {
        return ZIPCCL_ERR_SIZE;
    }
    for (int k = 0; k < nchunks; k++) {
        uint64_t* ne = n_esc_out ? n_esc_out + uint64_t(k) * (nseg + 1) : nullptr;
        if (zipccl_status r = check_compress_buffers(nseg, static_out[k], ws, ne, status)) return r;
        CArgs& a = calls[size_t(k)];
        if (zipccl_status r = fill_segments(a, segs + uint64_t(k) * nseg, nseg)) return r;
        if (zipccl_status r = prepare_compress(a, nseg, static_out[k], static_cap[k], esc_out[k], esc_cap[k],
                                               ws, workspace_bytes, ne, status))
            return r;
    }
    return launch_chunks(calls, ws, workspace_bytes, static_cast<hipStream_t>(stream));
}

zipccl_status zipccl_compress_gather(const zipccl_gather_segment_t* segs, int nseg, void* static_out,
                                     uint64_t static_cap, void* esc_out, uint64_t esc_cap, void* workspace,
                                     uint64_t workspace_bytes, uint64_t* n_esc_out, uint32_t* status, void* stream)
{
    if (!segs) return ZIPCCL_ERR_INVALID;
    if (zipccl_status r = check_compress_buffers(nseg, static_out, workspace, n_esc_out, status)) return r;
    CArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int s = 0; s < nseg; s++) {
        const zipccl_gather_segment_t& g = segs[s];
        if (g.row_len % 8 != 0 || g.row_len < 512 || g.row_len >= (1ull << 32)) return ZIPCCL_ERR_INVALID;
        if (g.src_rows >= (1ull << 32) || g.nrows >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
        const uint64_t n = g.nrows * g.row_len;
        if (n >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
        if (n > 0 && (!g.src || !g.rows || g.src_rows == 0)) return ZIPCCL_ERR_INVALID;
        if (!aligned(g.src, 16) || !aligned(g.rows, 4)) return ZIPCCL_ERR_ALIGN;
        if (!plan_valid(g.plan)) return ZIPCCL_ERR_INVALID;
        CSeg& c = a.seg[s];
        c.src = static_cast<const uint16_t*>(g.src);
        c.rows = n > 0 ? g.rows : nullptr;
        c.row_len = uint32_t(g.row_len);
        c.src_rows = uint32_t(g.src_rows);
        c.n = uint32_t(n);
        pack_table(g.plan, c.table_lo, c.table_hi);
    }
    return compress_segments(a, nseg, static_out, static_cap, esc_out, esc_cap, workspace, workspace_bytes,
                             n_esc_out, status, stream);
}

zipccl_status zipccl_decompress(const void* static_in, uint64_t static_bytes, const void* esc_in,
                                uint64_t esc_bytes, const zipccl_dsegment_t* segs, int nseg, uint32_t* status,
                                void* stream)
{
    if (!segs || nseg < 1 || nseg > kMaxSegs || !static_in) return ZIPCCL_ERR_INVALID;
    if (!aligned(static_in, 128) || (status && !aligned(status, 4))) return ZIPCCL_ERR_ALIGN;
    if (esc_bytes > 0 && !esc_in) return ZIPCCL_ERR_INVALID;
    DArgs a;
    std::memset(&a, 0, sizeof(a));
    uint64_t units = 0, st_off = 0;
    for (int s = 0; s < nseg; s++) {
        const zipccl_dsegment_t& g = segs[s];
        if (g.n >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
        if (g.n > 0 && !g.dst) return ZIPCCL_ERR_INVALID;
        if (!aligned(g.dst, 16)) return ZIPCCL_ERR_ALIGN;
        DSeg& d = a.seg[s];
        d.src = static_cast<const uint8_t*>(static_in) + st_off;
        // with no escape buffer no escape is ever read; any device address will do
        d.esc = static_cast<const uint8_t*>(esc_in ? esc_in : static_in);
        d.esc_bytes = esc_in ? esc_bytes : 0;
        d.dst = static_cast<uint16_t*>(g.dst);
        d.n = uint32_t(g.n);
        d.unit0 = uint32_t(units);
        units += blocks_of(g.n);   // one decompress workgroup per block
        st_off += static_bytes_of(g.n);
    }
    if (st_off > static_bytes) return ZIPCCL_ERR_SIZE;
    a.status = status;
    a.nseg = nseg;
    a.total_units = uint32_t(units);
    return hip_status(launch_decompress(a, static_cast<hipStream_t>(stream)));
}

zipccl_status zipccl_decompress_shards(const void* const* static_in, const void* const* esc_in,
                                       const uint64_t* esc_bytes, const zipccl_dsegment_t* segs, int nseg,
                                       uint32_t flags, uint32_t* status, void* stream)
{
    if (!segs || !static_in || !esc_in || !esc_bytes || nseg < 1 || nseg > kMaxSegs) return ZIPCCL_ERR_INVALID;
    if (flags & ~ZIPCCL_SHARDS_ESC_AT_FIRST) return ZIPCCL_ERR_INVALID;
    if (status && !aligned(status, 4)) return ZIPCCL_ERR_ALIGN;
    DArgs a;
    std::memset(&a, 0, sizeof(a));
    uint64_t units = 0;
    for (int s = 0; s < nseg; s++) {
        const zipccl_dsegment_t& g = segs[s];
        if (g.n >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
        if (!static_in[s] || (g.n > 0 && !g.dst) || (esc_bytes[s] > 0 && !esc_in[s])) return ZIPCCL_ERR_INVALID;
        if (!aligned(static_in[s], 128) || !aligned(g.dst, 16)) return ZIPCCL_ERR_ALIGN;
        DSeg& d = a.seg[s];
        d.src = static_cast<const uint8_t*>(static_in[s]);
        d.esc = static_cast<const uint8_t*>(esc_in[s] ? esc_in[s] : static_in[s]);
        d.esc_bytes = esc_in[s] ? esc_bytes[s] : 0;
        d.dst = static_cast<uint16_t*>(g.dst);
        d.n = uint32_t(g.n);
        d.unit0 = uint32_t(units);
        d.esc_at_first = (flags & ZIPCCL_SHARDS_ESC_AT_FIRST) ? 1u : 0u;
        units += blocks_of(g.n);   // one decompress workgroup per block
    }
    a.status = status;
    a.nseg = nseg;
    a.total_units = uint32_t(units);
    return hip_status(launch_decompress(a, static_cast<hipStream_t>(stream)));
}

zipccl_status zipccl_decompress_accumulate(const void* const* static_in, const void* const* esc_in,
                                           const uint64_t* esc_bytes, int npeers, uint64_t n, const void* local,
                                           void* dst, uint32_t* status, void* stream)
{
    if (npeers < 1 || npeers > kMaxPeers || !static_in || !esc_in || !esc_bytes) return ZIPCCL_ERR_INVALID;
    if (n >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
    if (n > 0 && (!local || !dst)) return ZIPCCL_ERR_INVALID;
    if (!aligned(local, 16) || !aligned(dst, 16) || (status && !aligned(status, 4))) return ZIPCCL_ERR_ALIGN;
    AArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int p = 0; p < npeers; p++) {
        if (!static_in[p]) return ZIPCCL_ERR_INVALID;
        if (!aligned(static_in[p], 128)) return ZIPCCL_ERR_ALIGN;
        if (esc_bytes[p] > 0 && !esc_in[p]) return ZIPCCL_ERR_INVALID;
        a.st[p] = static_cast<const uint8_t*>(static_in[p]);
        a.esc[p] = static_cast<const uint8_t*>(esc_in[p] ? esc_in[p] : static_in[p]);
        a.esc_bytes[p] = esc_in[p] ? esc_bytes[p] : 0;
    }
    a.local = static_cast<const uint16_t*>(local);
    a.dst = static_cast<uint16_t*>(dst);
    a.status = status;
    a.n = uint32_t(n);
    a.chunk = uint32_t(n);
    a.npeers = npeers;
    a.nchunks = 1;
    return hip_status(launch_accumulate(a, static_cast<hipStream_t>(stream)));
}

zipccl_status zipccl_decompress_accumulate_chunks(const void* const* static_in, const void* const* esc_in,
                                                  const uint64_t* esc_bytes, int npeers, uint64_t chunk, uint64_t n,
                                                  const void* local, void* dst, uint32_t* status, void* stream)
{
    if (npeers < 1 || npeers > kMaxPeers || chunk == 0 || chunk % kBlock != 0) return ZIPCCL_ERR_INVALID;
    if (n >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
    if (n == 0) return ZIPCCL_OK;
    if (!static_in || !esc_in || !esc_bytes || !local || !dst) return ZIPCCL_ERR_INVALID;
    if (!aligned(local, 16) || !aligned(dst, 16) || (status && !aligned(status, 4))) return ZIPCCL_ERR_ALIGN;
    const uint64_t nchunks = (n + chunk - 1) / chunk;
    for (uint64_t i = 0; i < nchunks * uint64_t(npeers); i++) {   // everything checked before any launch
        if (!static_in[i] || (esc_bytes[i] > 0 && !esc_in[i])) return ZIPCCL_ERR_INVALID;
        if (!aligned(static_in[i], 128)) return ZIPCCL_ERR_ALIGN;
    }
    // as many chunks per launch as the kernel arguments hold
    const uint64_t per_launch = uint64_t(kMaxAccSlots / npeers);
    for (uint64_t c0 = 0; c0 < nchunks; c0 += per_launch) {
        const uint64_t c1 = std::min(nchunks, c0 + per_launch);
        AArgs a;
        std::memset(&a, 0, sizeof(a));
        for (uint64_t c = c0; c < c1; c++) {
            for (int p = 0; p < npeers; p++) {
                const uint64_t i = c * npeers + p, j = (c - c0) * npeers + p;
                a.st[j] = static_cast<const uint8_t*>(static_in[i]);
                a.esc[j] = static_cast<const uint8_t*>(esc_in[i] ? esc_in[i] : static_in[i]);
                a.esc_bytes[j] = esc_in[i] ? esc_bytes[i] : 0;
            }
        }
        const uint64_t first = c0 * chunk;
        a.local = static_cast<const uint16_t*>(local) + first;
        a.dst = static_cast<uint16_t*>(dst) + first;
        a.status = status;
        a.n = uint32_t(std::min(n, c1 * chunk) - first);
        a.chunk = uint32_t(chunk);
        a.npeers = npeers;
        a.nchunks = int32_t(c1 - c0);
        if (hipError_t e = launch_accumulate(a, static_cast<hipStream_t>(stream))) return hip_status(e);
    }
    return ZIPCCL_OK;
}

// ---------------------------------------------------------------------------------
// reduce-scatter switcher: device profile and host cost model
// ---------------------------------------------------------------------------------
namespace {

struct ProfileLayout {
    uint64_t ws, st, esc, ne, status, dst, total;
};

ProfileLayout profile_layout(uint64_t n, int npeers)
{
    auto r256 = [](uint64_t v) { return (v + 255) & ~uint64_t(255); };
    ProfileLayout l;
    l.ws = 0;
    l.st = l.ws + r256(zipccl_workspace_size(n * uint64_t(npeers), npeers));
    l.esc = l.st + r256(uint64_t(npeers) * static_bytes_of(n));
    l.ne = l.esc + r256(uint64_t(npeers) * n);
    l.status = l.ne + r256(8 * uint64_t(npeers + 1));
    l.dst = l.status + 256;
    l.total = l.dst + r256(2 * n);
    return l;
}

}  // namespace

uint64_t zipccl_profile_scratch_size(uint64_t n, int npeers)
{
    if (npeers < 1 || npeers > kMaxPeers) return 0;
    return profile_layout(n, npeers).total;
}

zipccl_status zipccl_profile_codec(const void* sample, uint64_t n, zipccl_plan_t plan, int npeers, void* scratch,
                                   uint64_t scratch_bytes, void* stream, zipccl_codec_profile_t* out)
{
    if (!sample || !scratch || !out || n == 0 || npeers < 1 || npeers > kMaxPeers || !plan_valid(plan))
        return ZIPCCL_ERR_INVALID;
    if (n * uint64_t(npeers) >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
    if (!aligned(sample, 16) || !aligned(scratch, 256)) return ZIPCCL_ERR_ALIGN;
    const ProfileLayout l = profile_layout(n, npeers);
    if (scratch_bytes < l.total) return ZIPCCL_ERR_SIZE;
    uint8_t* base = static_cast<uint8_t*>(scratch);
    hipStream_t s = static_cast<hipStream_t>(stream);
    zipccl_segment_t segs[kMaxPeers];
    const void* sin[kMaxPeers];
    const void* ein[kMaxPeers];
    uint64_t eb[kMaxPeers];
    for (int p = 0; p < npeers; p++) {
        segs[p].src = sample;
        segs[p].n = n;
        segs[p].plan = plan;
        sin[p] = base + l.st + uint64_t(p) * static_bytes_of(n);
        ein[p] = base + l.esc;
        eb[p] = uint64_t(npeers) * n;
    }
    uint64_t* ne_dev = reinterpret_cast<uint64_t*>(base + l.ne);
    // a status word of its own: the profile is timed on the same launches callers get
    // (the single-launch compress needs one), and a set bit fails the call
    uint32_t* st_dev = reinterpret_cast<uint32_t*>(base + l.status);
    if (hipMemsetAsync(st_dev, 0, sizeof(uint32_t), s) != hipSuccess) return ZIPCCL_ERR_HIP;
    auto compress = [&]() {
        return zipccl_compress(segs, npeers, base + l.st, uint64_t(npeers) * static_bytes_of(n), base + l.esc,
                               uint64_t(npeers) * n, base + l.ws, l.st - l.ws, ne_dev, st_dev, stream);
    };
    auto accumulate = [&]() {
        return zipccl_decompress_accumulate(sin, ein, eb, npeers, n, sample, base + l.dst, st_dev, stream);
    };
    hipEvent_t e[4] = {};
    for (auto& ev : e)
        if (hipEventCreate(&ev) != hipSuccess) {
            for (auto& x : e)
                if (x) (void)hipEventDestroy(x);
            return ZIPCCL_ERR_HIP;
        }
    zipccl_status r = compress();   // warm-up, and the compressed size
    if (r == ZIPCCL_OK) r = accumulate();
    constexpr int kReps = 3;
    bool ok = r == ZIPCCL_OK && hipEventRecord(e[0], s) == hipSuccess;
    for (int k = 0; ok && k < kReps; k++) ok = compress() == ZIPCCL_OK;
    ok = ok && hipEventRecord(e[1], s) == hipSuccess && hipEventRecord(e[2], s) == hipSuccess;
    for (int k = 0; ok && k < kReps; k++) ok = accumulate() == ZIPCCL_OK;
    ok = ok && hipEventRecord(e[3], s) == hipSuccess && hipEventSynchronize(e[3]) == hipSuccess;
    float tc = 0, ta = 0;
    uint64_t total_esc = 0;
    ok = ok && hipEventElapsedTime(&tc, e[0], e[1]) == hipSuccess && hipEventElapsedTime(&ta, e[2], e[3]) == hipSuccess;
    ok = ok && hipMemcpy(&total_esc, ne_dev + npeers, sizeof(total_esc), hipMemcpyDeviceToHost) == hipSuccess;
    uint32_t dev_status = 0;
    ok = ok && hipMemcpy(&dev_status, st_dev, sizeof(dev_status), hipMemcpyDeviceToHost) == hipSuccess;
    for (auto& ev : e) (void)hipEventDestroy(ev);
    if (r != ZIPCCL_OK) return r;
    if (!ok || tc <= 0 || ta <= 0) return ZIPCCL_ERR_HIP;
    if (dev_status != 0) return ZIPCCL_ERR_CORRUPT;   // the device reported a status bit
    const double bf16 = 2.0 * double(n) * npeers;   // bytes of one launch
    out->compress_GBps = bf16 / (tc * 1e-3 / kReps) / 1e9;
    out->accumulate_GBps = bf16 / (ta * 1e-3 / kReps) / 1e9;
    out->compressed_fraction = (double(npeers) * double(static_bytes_of(n)) + double(total_esc)) / bf16;
    return ZIPCCL_OK;
}

zipccl_status zipccl_rs_choose(const zipccl_codec_profile_t* prof, const zipccl_link_t* link, int ranks,
                               uint64_t bytes, int* use_codec, double* native_us, double* zipped_us)
{
    if (!prof || !link || ranks < 2 || link->links < 1 || !(link->bw_GBps > 0) || !(link->latency_us >= 0) ||
        !(prof->compress_GBps > 0) || !(prof->accumulate_GBps > 0) || !(prof->compressed_fraction > 0))
        return ZIPCCL_ERR_INVALID;
    const double m = ranks - 1;
    const double shard = double(bytes) / ranks;
    const double rounds = std::ceil(m / link->links);
    const double native = rounds * (link->latency_us + shard / (link->bw_GBps * 1e3));
    const double zipped = m * shard / (prof->compress_GBps * 1e3) +
                          rounds * (link->latency_us + prof->compressed_fraction * shard / (link->bw_GBps * 1e3)) +
                          m * shard / (prof->accumulate_GBps * 1e3);
    const bool raw = bytes < (1ull << 20) || prof->compressed_fraction >= 1.0;
    if (use_codec) *use_codec = (!raw && zipped < native) ? 1 : 0;
    if (native_us) *native_us = native;
    if (zipped_us) *zipped_us = zipped;
    return ZIPCCL_OK;
}

// ---------------------------------------------------------------------------------
// two-stream chunk pipeline
// ---------------------------------------------------------------------------------
struct zipccl_pipeline {
    int npeers;
    uint64_t chunk;
    uint32_t group;            // chunks per hand-off between the streams
    uint8_t* scratch;
    uint64_t slot_static, slot_esc, ws_size;   // bytes per chunk slot and of one workspace
    hipStream_t sa, sb;
    hipEvent_t compressed[2], reduced[2];      // one per half of the ring
    bool reduced_recorded[2];
};

namespace {

// Chunks per hand-off: an event record or wait costs the host a few microseconds and
// leaves the waiting stream idle for ~11 us of GPU time (kernel trace), and each
// hand-off splits the launches the chunks could share, so the streams hand over groups
// of chunks holding at least 2^27 values (each chunk is still its own compress call and
// its own segments).  Measured on 7 x 2 Mi-value chunks, 32 chunks: groups of 8 took
// 509.7 us, groups of 16 489.0 us, with a ring of 2 x 16 chunk buffers (1.35 GB of
// scratch; 0.68 GB for 8).
uint32_t pipeline_group(int npeers, uint64_t chunk)
{
    uint32_t g = 1;
    while (g < 16 && uint64_t(g) * uint64_t(npeers) * chunk < (1ull << 27)) g *= 2;
    return g;
}

// Scratch layout: one compress workspace that holds as many chunks as share a compress
// launch (at most kMaxCalls, kLaunchSegs segments), then
// 2 * group chunk slots (a ring of two groups), each holding the chunk's npeers static
// parts and room for all its escapes.
void pipeline_layout(int npeers, uint64_t chunk, uint64_t& slot_static, uint64_t& slot_esc, uint64_t& ws)
{
    slot_static = uint64_t(npeers) * static_bytes_of(chunk);
    slot_esc = (uint64_t(npeers) * chunk + 255) & ~uint64_t(255);
    const uint64_t b = std::min<uint64_t>({uint64_t(pipeline_group(npeers, chunk)), uint64_t(kMaxCalls),
                                           uint64_t(kLaunchSegs / npeers)});
    ws = (zipccl_workspace_size(b * uint64_t(npeers) * chunk, int(b) * npeers) + 255) & ~uint64_t(255);
}

}  // namespace

uint64_t zipccl_pipeline_scratch_size(int npeers, uint64_t chunk)
{
    if (npeers < 1 || npeers > kMaxPeers || chunk == 0) return 0;
    uint64_t ss, se, ws;
    pipeline_layout(npeers, chunk, ss, se, ws);
    return ws + 2ull * pipeline_group(npeers, chunk) * (ss + se);
}

zipccl_status zipccl_pipeline_create(int npeers, uint64_t chunk, void* scratch, uint64_t scratch_bytes,
                                     void* stream_a, void* stream_b, zipccl_pipeline** out)
{
    if (!out || npeers < 1 || npeers > kMaxPeers || chunk == 0 || chunk % kBlock != 0 || !scratch)
        return ZIPCCL_ERR_INVALID;
    if (chunk * uint64_t(npeers) >= (1ull << 32)) return ZIPCCL_ERR_INVALID;
    if (!aligned(scratch, 256)) return ZIPCCL_ERR_ALIGN;
    if (scratch_bytes < zipccl_pipeline_scratch_size(npeers, chunk)) return ZIPCCL_ERR_SIZE;
    zipccl_pipeline* p = new (std::nothrow) zipccl_pipeline();
    if (!p) return ZIPCCL_ERR_INVALID;
    p->npeers = npeers;
    p->chunk = chunk;
    p->scratch = static_cast<uint8_t*>(scratch);
    pipeline_layout(npeers, chunk, p->slot_static, p->slot_esc, p->ws_size);
    p->group = pipeline_group(npeers, chunk);
    p->sa = static_cast<hipStream_t>(stream_a);
    p->sb = static_cast<hipStream_t>(stream_b);
    for (int k = 0; k < 2; k++) {
        p->reduced_recorded[k] = false;
        if (hipEventCreateWithFlags(&p->compressed[k], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&p->reduced[k], hipEventDisableTiming) != hipSuccess) {
            zipccl_pipeline_destroy(p);
            return ZIPCCL_ERR_HIP;
        }
    }
    *out = p;
    return ZIPCCL_OK;
}

zipccl_status zipccl_pipeline_reduce(zipccl_pipeline* pipe, const void* const* peer_src,
                                     const zipccl_plan_t* plans, uint64_t n, const void* local, void* dst,
                                     uint32_t* status)
{
    if (!pipe || !peer_src || !plans) return ZIPCCL_ERR_INVALID;
    if (n >= (1ull << 32)) return ZIPCCL_ERR_SIZE;
    if (n > 0 && (!local || !dst)) return ZIPCCL_ERR_INVALID;
    if (!aligned(local, 16) || !aligned(dst, 16)) return ZIPCCL_ERR_ALIGN;
    const int P = pipe->npeers;
    for (int p = 0; p < P; p++) {
        if (n > 0 && !peer_src[p]) return ZIPCCL_ERR_INVALID;
        if (!aligned(peer_src[p], 16)) return ZIPCCL_ERR_ALIGN;
        if (!plan_valid(plans[p])) return ZIPCCL_ERR_INVALID;
    }
    const uint64_t nchunks = (n + pipe->chunk - 1) / pipe->chunk;
    const uint64_t G = pipe->group;
    hipStream_t sa = pipe->sa, sb = pipe->sb;
    uint8_t* slots = pipe->scratch + pipe->ws_size;
    const uint64_t slot_bytes = pipe->slot_static + pipe->slot_esc;
    for (uint64_t c0 = 0; c0 < nchunks; c0 += G) {
        const int half = int((c0 / G) & 1);   // which half of the ring this group uses
        const uint64_t c1 = std::min(nchunks, c0 + G);
        // the group two hand-offs back used these slots: its reduction must be done
        if (pipe->reduced_recorded[half] && hipStreamWaitEvent(sa, pipe->reduced[half], 0) != hipSuccess)
            return ZIPCCL_ERR_HIP;
        // compress the group on stream a (its chunks share launches: up to kMaxCalls each)
        zipccl_segment_t segs[16 * kMaxPeers];
        void* st_out[16];
        void* esc_out[16];
        uint64_t st_cap[16], esc_cap[16];
        for (uint64_t c = c0; c < c1; c++) {
            const uint64_t k = c - c0, off = c * pipe->chunk;
            const uint64_t m = std::min(pipe->chunk, n - off);
            uint8_t* st = slots + (uint64_t(half) * G + k) * slot_bytes;
            for (int p = 0; p < P; p++) {
                zipccl_segment_t& g = segs[k * P + p];
                g.src = static_cast<const uint16_t*>(peer_src[p]) + off;
                g.n = m;
                g.plan = plans[p];
            }
            st_out[k] = st;
            st_cap[k] = pipe->slot_static;
            esc_out[k] = st + pipe->slot_static;
            esc_cap[k] = pipe->slot_esc;
        }
        if (zipccl_status r = zipccl_compress_chunks(segs, P, int(c1 - c0), st_out, st_cap, esc_out, esc_cap,
                                                     pipe->scratch, pipe->ws_size, nullptr, status, sa))
            return r;
        if (hipEventRecord(pipe->compressed[half], sa) != hipSuccess ||
            hipStreamWaitEvent(sb, pipe->compressed[half], 0) != hipSuccess)
            return ZIPCCL_ERR_HIP;
        // reduce the group on stream b: one decode-accumulate launch for its chunks
        const void* sin[16 * kMaxPeers];
        const void* ein[16 * kMaxPeers];
        uint64_t eb[16 * kMaxPeers];
        for (uint64_t c = c0; c < c1; c++) {
            const uint64_t k = c - c0;
            const uint64_t m = std::min(pipe->chunk, n - c * pipe->chunk);
            uint8_t* st = slots + (uint64_t(half) * G + k) * slot_bytes;
            for (int p = 0; p < P; p++) {
                sin[k * P + p] = st + uint64_t(p) * static_bytes_of(m);
                ein[k * P + p] = st + pipe->slot_static;
                eb[k * P + p] = pipe->slot_esc;
            }
        }
        const uint64_t first = c0 * pipe->chunk, m_all = std::min(n, c1 * pipe->chunk) - first;
        if (zipccl_status r = zipccl_decompress_accumulate_chunks(
                sin, ein, eb, P, pipe->chunk, m_all, static_cast<const uint16_t*>(local) + first,
                static_cast<uint16_t*>(dst) + first, status, sb))
            return r;
        if (hipEventRecord(pipe->reduced[half], sb) != hipSuccess) return ZIPCCL_ERR_HIP;
        pipe->reduced_recorded[half] = true;
    }
    return ZIPCCL_OK;
}

void zipccl_pipeline_destroy(zipccl_pipeline* pipe)
{
    if (!pipe) return;
    for (int k = 0; k < 2; k++) {
        if (pipe->compressed[k]) (void)hipEventDestroy(pipe->compressed[k]);
        if (pipe->reduced[k]) (void)hipEventDestroy(pipe->reduced[k]);
    }
    delete pipe;
}

}  // extern "C"
