// Streaming probes for the benchmark (not part of the codec): plain kernels that move
// memory in the shapes the codec's kernels do, so that a launch's HBM rate can be set
// beside what a kernel with nothing to compute reaches on the same GPU.
//
// Every probe uses 16-byte non-temporal lane accesses over buffers of `bytes` bytes
// (src read, dst written; both at least `bytes` long, 256-byte aligned, bytes a multiple
// of 2^20), in the shape that measured fastest: one 16-byte access per lane and stream
// (the read probe: four per lane, equal to one); four per lane, spread over a block,
// wrote at 6.0 instead of 6.7 TB/s and mixed at 6.0 instead of 6.4 TB/s:
//   ZCPROBE_COPY        read src, write dst (1 : 1)
//   ZCPROBE_READ        read src (a word is written only if an impossible xor comes out)
//   ZCPROBE_WRITE       write dst
//   ZCPROBE_MIX_16_12   compress-like: per 16 bytes read from the first half of src, 8 + 4
//                       bytes written to two sections of dst
//   ZCPROBE_ACC_7       decode-accumulate-like: one 512-thread workgroup per block of 8
//                       tiles, one tile per wave; per tile it reads, from each of 7 peer
//                       regions of src, 512 A bytes (8 per lane) and 192 plane bytes (a
//                       dword in 48 of 64 lanes) from a separate plane section, plus 16
//                       bytes per lane of a local region, and writes 16 bytes per lane
// zcprobe_moved_bytes(kind, bytes) gives the bytes one launch reads plus writes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int ZCPROBE_COPY = 0, ZCPROBE_READ = 1, ZCPROBE_WRITE = 2, ZCPROBE_MIX_16_12 = 3, ZCPROBE_ACC_7 = 4;
constexpr int kAccPeers = 7;
constexpr uint64_t kAccPeerTileBytes = 512 + 192;   // a tile's A and plane bytes in one peer region
constexpr uint64_t kAccTileBytes = kAccPeers * kAccPeerTileBytes + 1024;   // of src per tile, local included

// Tiles of the ACC_7 probe over buffers of `bytes` bytes (a multiple of 8).
uint64_t acc_tiles(uint64_t bytes) { return (bytes / kAccTileBytes) & ~uint64_t(7); }

__global__ __launch_bounds__(256) void copy_k(const v4u* __restrict__ a, v4u* __restrict__ b, uint64_t n4)
{
    const uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n4) __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

__global__ __launch_bounds__(256) void read_k(const v4u* __restrict__ a, uint32_t* __restrict__ out, uint64_t n4)
{
    const uint64_t i = uint64_t(blockIdx.x) * 1024 + threadIdx.x;
    v4u v[4];
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = i + 256 * k < n4 ? __builtin_nontemporal_load(a + i + 256 * k) : v4u{0, 0, 0, 0};
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    if (acc == 0x9E3779B9u && v[0].x == 0x7F4A7C15u) out[0] = acc;   // keeps the loads; never true for the filled input
}

__global__ __launch_bounds__(256) void write_k(v4u* __restrict__ b, uint64_t n4)
{
    const uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n4) __builtin_nontemporal_store(v4u{unsigned(i), 1u, 2u, 3u}, b + i);
}

__global__ __launch_bounds__(256) void mix_k(const v4u* __restrict__ a, uint8_t* __restrict__ b, uint64_t m4)
{
    const uint64_t j = uint64_t(blockIdx.x) * 256 + threadIdx.x;
    if (j >= m4) return;
    const v4u v = __builtin_nontemporal_load(a + j);
    __builtin_nontemporal_store(v2u{v.x, v.y}, reinterpret_cast<v2u*>(b) + j);           // 8 B: A-like
    __builtin_nontemporal_store(v.z ^ v.w, reinterpret_cast<uint32_t*>(b + 8 * m4) + j);   // 4 B: plane-like
}

// src: 7 peer regions of T * 704 bytes (A section of 512 T, then plane section of 192 T),
// then the local region (1024 T); dst: T * 1024 bytes.  Grid: T / 8 workgroups.
__global__ __launch_bounds__(512) void acc_k(const uint8_t* __restrict__ src, v4u* __restrict__ dst, uint64_t T)
{
    const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint64_t t = uint64_t(blockIdx.x) * 8 + wave;
    const uint32_t c = lane & 31, q = c & 3;
    const uint32_t pdw = q < 3 ? 2 * (8 * q + (c >> 2)) + (lane >> 5) : 0u;   // 48 lanes, 192 bytes
    uint32_t acc = 0;
#pragma unroll
    for (int p = 0; p < kAccPeers; p++) {
        const uint8_t* base = src + p * kAccPeerTileBytes * T;
        const v2u A = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(base + 512 * t) + lane);
        const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(base + 512 * T + 192 * t) + pdw);
        acc ^= A.x ^ A.y ^ w;
    }
    const v4u* local = reinterpret_cast<const v4u*>(src + kAccPeers * kAccPeerTileBytes * T);
    v4u v = __builtin_nontemporal_load(local + 64 * t + lane);
    v.x ^= acc;
    __builtin_nontemporal_store(v, dst + 64 * t + lane);
}

bool valid(int kind, const void* src, void* dst, uint64_t bytes)
{
    if (kind < ZCPROBE_COPY || kind > ZCPROBE_ACC_7) return false;
    if (bytes == 0 || bytes % (1u << 20) != 0) return false;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 256 != 0) return false;
    return dst != nullptr && (kind == ZCPROBE_WRITE || src != nullptr);   // every probe writes dst
}

}  // namespace

// Bytes one launch of `kind` over buffers of `bytes` bytes reads plus writes (0: invalid kind).
extern "C" uint64_t zcprobe_moved_bytes(int kind, uint64_t bytes)
{
    const uint64_t n4 = bytes / 16;
    switch (kind) {
        case ZCPROBE_COPY: return 2 * bytes;
        case ZCPROBE_READ: return bytes;
        case ZCPROBE_WRITE: return bytes;
        case ZCPROBE_MIX_16_12: return (n4 / 2) * 28;
        case ZCPROBE_ACC_7: return acc_tiles(bytes) * (kAccPeers * kAccPeerTileBytes + 2 * 1024);
        default: return 0;
    }
}

// Launches one probe on `stream` (a hipStream_t; null: the default stream).  READ writes
// at most one word, at dst (at least 4 bytes).  Returns a hipError_t value (0: launched);
// an invalid kind, size or alignment returns hipErrorInvalidValue and launches nothing.
extern "C" int zcprobe_launch(int kind, const void* src, void* dst, uint64_t bytes, void* stream)
{
    if (!valid(kind, src, dst, bytes)) return int(hipErrorInvalidValue);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint64_t n4 = bytes / 16;
    const v4u* a = static_cast<const v4u*>(src);
    switch (kind) {
        case ZCPROBE_COPY:
            hipLaunchKernelGGL(copy_k, dim3(uint32_t((n4 + 255) / 256)), dim3(256), 0, s, a, static_cast<v4u*>(dst), n4);
            break;
        case ZCPROBE_READ:
            hipLaunchKernelGGL(read_k, dim3(uint32_t((n4 + 1023) / 1024)), dim3(256), 0, s, a, static_cast<uint32_t*>(dst), n4);
            break;
        case ZCPROBE_WRITE:
            hipLaunchKernelGGL(write_k, dim3(uint32_t((n4 + 255) / 256)), dim3(256), 0, s, static_cast<v4u*>(dst), n4);
            break;
        case ZCPROBE_MIX_16_12: {   // reads the first half of src; writes 12 / 16 of that to dst
            const uint64_t m4 = n4 / 2;
            hipLaunchKernelGGL(mix_k, dim3(uint32_t((m4 + 255) / 256)), dim3(256), 0, s, a, static_cast<uint8_t*>(dst), m4);
            break;
        }
        case ZCPROBE_ACC_7: {
            const uint64_t T = acc_tiles(bytes);
            hipLaunchKernelGGL(acc_k, dim3(uint32_t(T / 8)), dim3(512), 0, s, static_cast<const uint8_t*>(src),
                               static_cast<v4u*>(dst), T);
            break;
        }
    }
    return int(hipGetLastError());
}
