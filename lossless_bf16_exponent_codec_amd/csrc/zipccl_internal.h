// Internal definitions shared by the HIP kernels and the host layer of libzipccl.
// Kernel arguments travel by value in the kernel-argument segment (< 4 KiB each).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zc {

constexpr uint32_t kTile = 512;               // values per tile: 64 lanes x 8 values
constexpr uint32_t kBlock = 4096;             // values per escape-offset entry (8 tiles)
constexpr uint32_t kWaves = 4;                // waves per workgroup
constexpr uint32_t kThreads = 64 * kWaves;    // 256
constexpr uint32_t kUnit = kBlock * kWaves;   // values per workgroup: one block per wave
constexpr int kMaxSegs = 64;
constexpr int kMaxPeers = 16;

// Workspace layout (32-bit words): [0] generation, [1] ticket counter, [2] finished
// counter, [3] 0; then kMaxSegs u64 segment-base slots; then one u64 status word per
// workgroup unit of the launch.
constexpr uint64_t kWsHeaderBytes = 16;
constexpr uint64_t kWsSegBytes = 8ull * kMaxSegs;

struct CSeg {              // compress: one segment
    const uint16_t* src;   // n BF16 values
    uint8_t* dst;          // static part of this segment
    uint32_t n;
    uint32_t unit0;        // first workgroup unit of the segment in launch order
    uint32_t table_lo;     // table[0..3]
    uint32_t table_hi;     // table[4..6], byte 3 = 0
};

struct CArgs {
    CSeg seg[kMaxSegs];
    uint8_t* esc;
    uint64_t esc_cap;
    uint32_t* ws;
    uint64_t* n_esc_out;   // nseg + 1 entries or null
    uint32_t* status;      // or null
    int32_t nseg;
    uint32_t total_units;
};

struct DSeg {              // decompress: one segment
    const uint8_t* src;    // static part
    uint16_t* dst;
    uint32_t n;
    uint32_t unit0;
};

struct DArgs {
    DSeg seg[kMaxSegs];
    const uint8_t* esc;
    uint64_t esc_bytes;
    uint32_t* status;
    int32_t nseg;
    uint32_t total_units;
};

struct AArgs {             // decompress + accumulate
    const uint8_t* st[kMaxPeers];
    const uint8_t* esc[kMaxPeers];
    uint64_t esc_bytes[kMaxPeers];
    const uint16_t* local;
    uint16_t* dst;
    uint32_t* status;
    uint32_t n;
    int32_t npeers;
};

__host__ __device__ inline uint64_t round128(uint64_t v) { return (v + 127) & ~uint64_t(127); }
__host__ __device__ inline uint64_t tiles_of(uint64_t n) { return (n + kTile - 1) / kTile; }
__host__ __device__ inline uint64_t blocks_of(uint64_t n) { return (n + kBlock - 1) / kBlock; }
__host__ __device__ inline uint64_t units_of(uint64_t n) { return n == 0 ? 1 : (n + kUnit - 1) / kUnit; }
__host__ __device__ inline uint64_t planes_off(uint64_t n) { return 128 + 512 * tiles_of(n); }
__host__ __device__ inline uint64_t offsets_off(uint64_t n) { return planes_off(n) + round128(192 * tiles_of(n)); }
__host__ __device__ inline uint64_t static_bytes_of(uint64_t n) { return offsets_off(n) + round128(4 * blocks_of(n)); }

hipError_t launch_compress(const CArgs& a, hipStream_t s);
hipError_t launch_decompress(const DArgs& a, hipStream_t s);
hipError_t launch_accumulate(const AArgs& a, hipStream_t s);

}  // namespace zc
