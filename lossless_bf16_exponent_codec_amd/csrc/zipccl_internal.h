// Internal definitions shared by the HIP kernels and the host layer of libzipccl.
// Kernel arguments travel by value in the kernel-argument segment: up to 4 KiB for
// the per-call tables; the compress and decode-accumulate launches that several calls
// share carry larger tables (about 8 and 6 KiB; this runtime passes 16000 bytes intact).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zc {

constexpr uint32_t kTile = 512;               // values per tile: 64 lanes x 8 values
constexpr uint32_t kBlock = 4096;             // values per escape-offset entry (8 tiles)
constexpr uint32_t kWaves = 4;                // waves per workgroup
constexpr uint32_t kThreads = 64 * kWaves;    // 256
constexpr uint32_t kUnit = kBlock * kWaves;   // values per workgroup: one block per wave
constexpr int kMaxSegs = 64;       // segments of one call
constexpr int kLaunchSegs = 128;   // segments of one compress launch (several calls)
constexpr int kMaxPeers = 16;
constexpr uint64_t kMaxKernelArgs = 12288;   // bytes; 16000 measured to arrive intact

// Uncoded blocks: the plane bytes of a tile (3 planes x 8 columns x 64 bits) hold the
// exponents of its first 192 values; the rest of the tile's exponents go to the escape
// buffer.
constexpr uint32_t kUncodedPlaneBytes = 192;
constexpr uint32_t kBlockOverflow = (kBlock / kTile) * (kTile - kUncodedPlaneBytes);   // of a full block: 2560

// Encode granule: half a block (4 tiles, 2048 values) per wave, 8 waves per workgroup.
constexpr uint32_t kHalf = kBlock / 2;
constexpr uint32_t kEncWaves = 8;
constexpr uint32_t kEncThreads = 64 * kEncWaves;
constexpr uint32_t kStageHead = 2 * kEncWaves;   // bytes: a unit's slot counts in its staged record

// Compress workspace, by half-block slot: slot 8u + w belongs to wave w of workgroup
// unit u (slots past a segment's end hold 0 escapes).  A u32 escape count per slot,
// the launch-wide position of each slot's first escape (one more entry for the total;
// used only when the positions come from the scan kernel), a u32 escape count per
// unit, a u64 ready word per unit (the single-launch compress: the call's tag above
// the unit's escape count), then kUnit staging bytes per unit that hold its escape
// exponents, contiguous in value order, until their positions are known.  The
// single-launch compress leaves the per-slot counts alone: a unit's staging bytes open
// with its 8 slot counts (u16 each, kStageHead bytes) and its escapes follow them.
__host__ __device__ constexpr uint64_t ws_counts_bytes(uint64_t units) { return (32 * units + 255) & ~uint64_t(255); }
__host__ __device__ constexpr uint64_t ws_pos_bytes(uint64_t units) { return (4 * (8 * units + 1) + 255) & ~uint64_t(255); }
__host__ __device__ constexpr uint64_t ws_units_bytes(uint64_t units) { return (4 * (units + 1) + 255) & ~uint64_t(255); }
__host__ __device__ constexpr uint64_t ws_ready_bytes(uint64_t units) { return (8 * units + 255) & ~uint64_t(255); }
__host__ __device__ constexpr uint64_t ws_bytes(uint64_t units)
{
    return ws_counts_bytes(units) + ws_pos_bytes(units) + ws_units_bytes(units) + ws_ready_bytes(units) +
           uint64_t(kHalf) * 8 * units;
}

// The no-allocation compress: its workspace is a static device array sized for calls of
// up to kNoAllocMaxValues values in at most kMaxSegs segments (each segment adds at most
// one partial unit).
constexpr uint64_t kNoAllocMaxValues = 1ull << 26;
constexpr uint64_t kNoAllocMaxUnits = kNoAllocMaxValues / kUnit + kMaxSegs;
constexpr uint64_t kNoAllocScratchBytes = ws_bytes(kNoAllocMaxUnits);
// Device address of this library's static compress workspace on the device that runs
// `stream` (looked up once per device, with that device current).
hipError_t noalloc_workspace(hipStream_t stream, void** out);

// Ready word of a unit in the single-launch compress: the call's tag (48 bits, drawn
// per call by the host, never 0) above the unit's escape count (at most kUnit).
constexpr uint32_t kReadyCountBits = 16;

// Up to this many workgroup units (2^28 values) in a call the place kernel sums the unit
// counts of the call before its unit itself; above, a one-workgroup scan kernel computes
// the positions (and the call has a launch of its own).
constexpr uint32_t kDirectPrefixMaxUnits = 16384;

struct CSeg {              // compress: one segment
    const uint16_t* src;   // n BF16 values, or the matrix the rows are gathered from
    uint8_t* dst;          // static part of this segment
    const int32_t* rows;   // gathered segment: n / row_len row indices; null: src is contiguous
    uint32_t n;
    uint32_t unit0;        // first encode workgroup of the segment (units of kUnit values)
    uint32_t block0;       // first block of the segment in launch-wide block numbering
    uint32_t table_lo;     // table[0..3]
    uint32_t table_hi;     // table[4..6], byte 3 = 0
    uint32_t row_len;      // gathered segment: values per row (a multiple of 8, >= 512)
    uint32_t src_rows;     // gathered segment: rows of the matrix (indices must be below)
    uint32_t call;         // the compress call (CCall) the segment belongs to
};

// One compress call of a launch: a launch may compress several independent calls (the
// chunks of a sequence), each with its own escape buffer, escape positions counted from
// its own first escape, and its own escape-count output.  Its segments, units and
// blocks are consecutive in the launch.
struct CCall {
    uint8_t* esc;
    uint64_t esc_cap;
    uint64_t* n_esc_out;   // nseg + 1 entries or null
    uint32_t seg0;         // first segment of the call
    uint32_t nseg;
    uint32_t unit0;        // first unit of the call
    uint32_t block_end;    // one past the call's last block (launch-wide numbering)
};
constexpr int kMaxCalls = 16;

struct CArgs {
    CSeg seg[kLaunchSegs];
    CCall call[kMaxCalls];
    uint32_t* counts;      // workspace: escapes per half-block slot
    uint32_t* pos;         // workspace: launch-wide position of each slot's first escape
    uint32_t* unit_counts; // workspace: escapes per workgroup unit
    uint8_t* stage;        // workspace: kUnit bytes per unit
    uint64_t* ready;       // workspace: a ready word per unit (single-launch compress)
    uint64_t tag;          // this launch's tag in the ready words (single-launch compress)
    uint64_t wait_tag;     // the tag the placing workgroups wait for (== tag; tests force a mismatch)
    uint32_t wait_polls;   // polls of one ready word before a placing workgroup gives up
    uint32_t* status;      // or null
    const uint8_t* dplans; // device plans (8 bytes per segment) replacing the segments' tables, or null
    int32_t nseg;
    int32_t ncalls;        // 1 unless direct
    uint32_t total_units;
    uint32_t total_blocks;
    uint32_t direct;       // 1: the place kernel computes positions from unit_counts
};

static_assert(sizeof(CArgs) <= kMaxKernelArgs, "kernel arguments of a compress launch");

struct DSeg {              // decompress: one segment
    const uint8_t* src;    // static part
    const uint8_t* esc;    // escape buffer the header's esc_offset refers to
    uint64_t esc_bytes;
    uint16_t* dst;
    uint32_t n;
    uint32_t unit0;        // first decompress workgroup of the segment (one per block of kBlock values)
    uint32_t esc_at_first; // 1: esc points at the segment's first escape (header esc_offset ignored)
    uint32_t pad;
};

struct DArgs {
    DSeg seg[kMaxSegs];
    uint32_t* status;
    int32_t nseg;
    uint32_t total_units;  // decompress workgroups: blocks of all segments
};
static_assert(sizeof(DArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// Decompress + accumulate over nchunks consecutive chunks of `chunk` values (the last
// may be shorter; chunk is a multiple of kBlock unless nchunks == 1): chunk c covers
// values [c * chunk, min(n, (c + 1) * chunk)) of local / dst and has one compressed
// segment per peer, at st[c * npeers + p] with escapes in esc[c * npeers + p].
constexpr int kMaxAccSlots = 256;

struct AArgs {
    const uint8_t* st[kMaxAccSlots];
    const uint8_t* esc[kMaxAccSlots];
    uint64_t esc_bytes[kMaxAccSlots];
    const uint16_t* local;
    uint16_t* dst;
    uint32_t* status;
    uint32_t n;             // values of all chunks together
    uint32_t chunk;
    int32_t npeers;
    int32_t nchunks;
};
static_assert(sizeof(AArgs) <= kMaxKernelArgs, "kernel arguments of a decode-accumulate launch");

__host__ __device__ inline uint64_t round128(uint64_t v) { return (v + 127) & ~uint64_t(127); }
__host__ __device__ inline uint64_t tiles_of(uint64_t n) { return (n + kTile - 1) / kTile; }
__host__ __device__ inline uint64_t blocks_of(uint64_t n) { return (n + kBlock - 1) / kBlock; }
__host__ __device__ inline uint64_t units_of(uint64_t n) { return (n + kUnit - 1) / kUnit; }
__host__ __device__ inline uint64_t planes_off(uint64_t n) { return 128 + 512 * tiles_of(n); }
__host__ __device__ inline uint64_t offsets_off(uint64_t n) { return planes_off(n) + round128(192 * tiles_of(n)); }
__host__ __device__ inline uint64_t static_bytes_of(uint64_t n) { return offsets_off(n) + round128(4 * blocks_of(n)); }

// Encode + place.  single: one launch whose last workgroups place the units once their
// encoders have published their ready words (a.ready, a.tag); else encode, then place
// (or scan + place) in launches of their own.  single needs direct == 1.
hipError_t launch_compress(const CArgs& a, hipStream_t s, bool single);
hipError_t launch_decompress(const DArgs& a, hipStream_t s);
// Plans from a strided sample of each segment (one workgroup per segment).
constexpr uint32_t kEstParts = 16;   // workgroups per segment in the estimate
struct EArgs {
    const uint16_t* src[kMaxSegs];
    uint32_t n[kMaxSegs];
    uint8_t* plans;        // device, 8 bytes per segment
    double* partial;       // device scratch: kEstParts (sum, count) pairs per segment
    uint32_t stride;       // every stride-th tile of 512 values is sampled
    int32_t nseg;
};
static_assert(sizeof(EArgs) <= 4096, "kernel arguments are limited to 4 KiB");
hipError_t launch_estimate_plans(const EArgs& a, hipStream_t s);
hipError_t launch_accumulate(const AArgs& a, hipStream_t s);

}  // namespace zc
