// HIP kernels of the lossless BF16 exponent codec for CDNA4 (gfx950), wave64.
//
// Method: "ZipCCL: Efficient Lossless Data Compression of Communication Collectives
// for Accelerating LLM Training" (gist.science explanation page), S2.B (split into
// sign+mantissa and exponent; top-7 exponents -> 3-bit codes, others -> escape code 0
// with the exponent in a separate array), S2.C (128-byte aligned sections, codes as
// three 1-bit planes), S2.D (local reduction on the reduce-scatter receive side; the
// MoE dispatch, whose token rows the encoder can read by index).
// The byte layout (format version 1) is documented in include/zipccl.h.
//
// Work decomposition.  A tile is 512 values: lane l of a wave holds values 8l..8l+7,
// one 16-byte load.  A block is 8 tiles (4096 values, one escape-offset entry); a unit
// is 4 blocks (one encoding workgroup, one half block per wave).
//   * Planes.  A lane looks up, per value, a one-byte code entry (3-bit code plus an
//     escape flag) and ORs the 8 entries, the one of column j shifted by 4j, into one
//     32-bit row.  A 32x32 bit transpose inside each half-wave (5 stages: a lane
//     exchange by DPP or ds_swizzle, v_alignbit, v_bfi) turns the rows of 32 lanes into
//     plane dwords, each lane holding one bit position of the rows.  The decoders load
//     the plane dwords in an order chosen so that the same transpose (its own inverse)
//     gives each lane a row with the codes of its columns b and b+4 in byte b.
//   * Escapes.  A DPP prefix scan over the wave's per-lane escape counts gives each
//     lane the position of its first escape; a lane's escapes follow in column order.
//     Decoding replaces the code-0 byte of the v_perm table with the lane's first
//     escape of each group of 4 columns; a second escape in a group is placed by masks,
//     and only a third or fourth is patched byte by byte.
//   * Uncoded blocks.  A block whose escapes would reach its overflow (the values past
//     the first 192 of each tile) is rewritten by its encoding waves: plane bytes hold
//     the first 192 exponents of each tile, the rest go where the escapes would have
//     gone.  Decoders recognise such a block from its offset-table entries alone.
//   * Compress is one launch (compress_single_kernel) when the caller passes a status
//     word: encoding workgroups write the A bytes and planes, stage each unit's half-block
//     counts and escapes in the workspace as one record (whole 8-byte words) and then
//     publish the unit's escape count in a ready word tagged with the call's tag; placing
//     workgroups, interleaved in the grid about
//     one generation of encoders behind the units they place, wait (bounded) for the
//     ready words of their call's units up to theirs, then compute escape positions,
//     compact the escapes and write offset tables and headers.  What one workgroup
//     hands to another goes through agent-scope (write-through) stores and loads, so no
//     cache-wide write-back or invalidate is needed.  Without a status word (a wait that
//     ran out could not be reported) and under graph capture the same work is two launches
//     that wait for nothing (encode_kernel, place_direct_kernel); above 2^28 values in a
//     call a one-workgroup scan kernel computes the positions and a per-block place
//     kernel follows.
//     One launch may compress several independent calls (the chunks of a sequence):
//     each segment names its call, and positions, offsets and headers count from the
//     first escape of the call.
//   * Decompress: one workgroup per block, one half block per wave, one barrier to share
//     the escape count of the first half; each segment has its own escape buffer.
//     Decode-accumulate: one workgroup per block, one wave per tile, all peers of a
//     tile in one wave; the A bytes wait in LDS so that 4 workgroups fit per CU; its
//     decode table and staged escapes hold exponents rotated by one bit, so a lane's
//     bytes assemble without shifts; one launch may cover several chunks, each with its
//     own peers.
#include "zipccl_internal.h"
#include "zipccl.h"

#include <mutex>

namespace zc {

namespace {

__device__ inline uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ inline uint64_t ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }

// Number of set bits of m in the lanes below this one, plus acc.
__device__ inline uint32_t mbcnt(uint64_t m, uint32_t acc)
{
    return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), acc));
}

// Streaming accesses (each byte is read or written once per launch): non-temporal loads
// of the codec's inputs and stores of its outputs.  On the 64 Mi bucket they took ~8 %
// off a compress + decompress step, most of it from the decompressed output.
typedef unsigned int zc_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int zc_u32x4 __attribute__((ext_vector_type(4)));
__device__ inline void store_nt(uint2* p, uint2 v)
{
    zc_u32x2 x = {v.x, v.y};
    __builtin_nontemporal_store(x, reinterpret_cast<zc_u32x2*>(p));
}
__device__ inline void store_nt(uint4* p, uint4 v)
{
    zc_u32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<zc_u32x4*>(p));
}
__device__ inline void store_nt(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ inline uint4 load_nt(const uint4* p)
{
    const zc_u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const zc_u32x4*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ inline uint2 load_nt(const uint2* p)
{
    const zc_u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const zc_u32x2*>(p));
    return make_uint2(x.x, x.y);
}
__device__ inline uint32_t load_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }

// Agent-scope accesses for what one workgroup hands to another inside a launch (the
// single-launch compress): stores written through to memory, loads that bypass the
// non-coherent caches, so no cache-wide write-back or invalidate is needed.
template <class T>
__device__ inline void store_agent(T* p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <class T>
__device__ inline T load_agent(const T* p) { return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Waits until this wave's memory accesses have completed (agent-scope stores included).
__device__ inline void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0); expcnt, lgkmcnt untouched

__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) { return __builtin_amdgcn_perm(hi, lo, sel); }

// ORs bits into the status word; skips the atomic when they are set already (on bad
// input every workgroup may report, and atomics on one address are serialised).
__device__ inline void or_status(uint32_t* s, uint32_t bits)
{
    if (!s) return;
    if ((__hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & bits) == bits) return;
    __hip_atomic_fetch_or(s, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Segment holding launch-wide index u: the last s with seg[s].*first <= u (segments
// are in launch order and seg[0].*first == 0).
template <auto First, class Seg>
__device__ inline int find_segment(const Seg* seg, int nseg, uint32_t u)
{
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (seg[mid].*First <= u) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The same lookup by the whole wave at once, for code where every lane of the wave is
// active and u is the same in all of them: lane s compares segments s and s + 64 (nseg <=
// 128), and the last segment whose first index is at most u is the highest lane of the
// ballots.  One load round trip instead of one per binary-search step (with 1 or 2
// segments the binary search needs none or one).
template <auto First, class Seg>
__device__ inline int find_segment_wave(const Seg* seg, int nseg, uint32_t u)
{
    static_assert(kLaunchSegs <= 128 && kMaxSegs <= 128, "two segments per lane at most");
    if (nseg <= 2) return find_segment<First>(seg, nseg, u);   // no load, or one
    u = __builtin_amdgcn_readfirstlane(u);
    const int lane = int(lane_id());
    const bool lo = lane < nseg && seg[lane].*First <= u;   // seg[0] starts at 0
    const uint64_t m = __builtin_amdgcn_ballot_w64(lo);
    if (nseg > 64) {   // only in tables of more than 64 entries
        const bool hi = lane + 64 < nseg && seg[lane + 64].*First <= u;
        const uint64_t mh = __builtin_amdgcn_ballot_w64(hi);
        if (mh != 0) return 127 - __builtin_clzll(mh);
    }
    return 63 - __builtin_clzll(m | 1ull);
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

// Gathered segments (CSeg::rows set): value i of the segment is column i % row_len of
// matrix row rows[i / row_len].  row_len is a multiple of 8 and at least 512, so a
// lane's 8 values lie in one row and a tile spans at most two.  A row index outside the
// matrix is replaced by 0 and reported through `bad`.
//
// Address of this lane's 8 values in the tile that starts at value i0 (all 512 exist):
// the tile's rows are read with scalar loads, the lane picks one by its column.
__device__ inline const uint16_t* gathered_lane_ptr(const CSeg& sg, uint32_t i0, uint32_t lane, bool& bad)
{
    const uint32_t L = sg.row_len;
    const uint32_t r0 = __builtin_amdgcn_readfirstlane(i0 / L);
    const uint32_t c0 = i0 - r0 * L;
    const uint32_t split = L - c0;   // values of the tile still in row r0
    const uint32_t r1 = __builtin_amdgcn_readfirstlane(min(r0 + 1, sg.n / L - 1));
    // both indices are the same for the whole wave: scalar loads
    const uint32_t x0 = __builtin_amdgcn_readfirstlane(sg.rows[r0]);
    const uint32_t x1 = __builtin_amdgcn_readfirstlane(sg.rows[r1]);
    const uint32_t j = 8 * lane;
    const bool second = j >= split;
    uint32_t x = second ? x1 : x0;
    const uint32_t col = second ? j - split : c0 + j;
    const bool b = x >= sg.src_rows;   // negative indices compare as large
    bad = bad || b;
    return sg.src + uint64_t(b ? 0u : x) * L + col;
}

// This lane's 8 values of tile t of a gathered segment (0 past n; n is a multiple of 8).
__device__ inline uint4 load_lane_rows(const CSeg& sg, uint32_t t, uint32_t lane, bool& bad)
{
    const uint64_t i = uint64_t(t) * kTile + 8ull * lane;
    if (i >= sg.n) return make_uint4(0, 0, 0, 0);
    const uint32_t L = sg.row_len;
    const uint32_t r = uint32_t(i) / L;
    const uint32_t x = uint32_t(sg.rows[r]);
    const bool b = x >= sg.src_rows;
    bad = bad || b;
    return load_nt(reinterpret_cast<const uint4*>(sg.src + uint64_t(b ? 0u : x) * L + (uint32_t(i) - r * L)));
}

// --------------------------------------------------------------------------------
// compress
// --------------------------------------------------------------------------------
// Per-lane constants of the 32x32 bit transpose within each half-wave (stage s =
// 16, 8, 4, 2, 1): lanes whose bit s is clear keep the bit columns of mask M_s and
// take their partner's columns rotated left by s; the others keep ~M_s and take the
// partner's columns rotated right by s.
struct Transpose32 {
    uint32_t keep[5];
    uint32_t rot[5];   // rotate-right amount for v_alignbit
};

__device__ inline Transpose32 transpose_consts(uint32_t lane)
{
    const uint32_t M[5] = {0x0000FFFFu, 0x00FF00FFu, 0x0F0F0F0Fu, 0x33333333u, 0x55555555u};
    Transpose32 c;
#pragma unroll
    for (int k = 0; k < 5; k++) {
        const uint32_t sft = 16u >> k;
        const bool upper = (lane & sft) != 0;
        c.keep[k] = upper ? ~M[k] : M[k];
        c.rot[k] = upper ? sft : 32u - sft;
    }
    return c;
}

// The word of lane ^ sft.  xor 8, 2 and 1 stay inside a row of 16 lanes and are DPP
// moves (row_ror:8, quad_perm [2,3,0,1], quad_perm [1,0,3,2]): a few cycles on the
// VALU.  xor 16 and 4 go through ds_swizzle's bit mode (groups of 32 lanes).
template <int sft>
__device__ inline uint32_t partner(uint32_t x)
{
    if constexpr (sft == 8) return uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x128, 0xF, 0xF, true));
    else if constexpr (sft == 2) return uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x4E, 0xF, 0xF, true));
    else if constexpr (sft == 1) return uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0xB1, 0xF, 0xF, true));
    else return uint32_t(__builtin_amdgcn_ds_swizzle(int(x), 0x1F | (sft << 10)));
}

// One transpose stage: exchange with lane ^ sft, rotate the partner's word, keep this
// lane's own columns.
template <int k>
__device__ inline uint32_t transpose_stage(uint32_t x, const Transpose32& c)
{
    constexpr int sft = 16 >> k;
    const uint32_t y = partner<sft>(x);
    const uint32_t t = __builtin_amdgcn_alignbit(y, y, c.rot[k]);
    // (x & keep) | (t & ~keep) as one v_bfi_b32: the compiler emits v_and + v_and_or here,
    // one VALU instruction more per stage (decode-accumulate 1.6 % faster, A/B)
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(c.keep[k]), "v"(x), "v"(t));
    return r;
}

// Transposes the 32x32 bit matrix held by each half-wave (row = lane, column = bit):
// afterwards bit i of lane c (within the half) is bit c of lane i.
__device__ inline uint32_t transpose32(uint32_t x, const Transpose32& c)
{
    x = transpose_stage<0>(x, c);
    x = transpose_stage<1>(x, c);
    x = transpose_stage<2>(x, c);
    x = transpose_stage<3>(x, c);
    return transpose_stage<4>(x, c);
}

// Inclusive prefix sum over the 64 lanes of the wave (every lane active): running sums
// inside each row of 16 lanes by DPP row shifts, then the totals of rows 0 and 2, and
// of rows 0-1, added to the rows after them (DPP row broadcasts).
__device__ inline uint32_t wave_scan_incl(uint32_t x)
{
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x111, 0xF, 0xF, true));    // row_shr:1
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x112, 0xF, 0xF, true));    // row_shr:2
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x114, 0xF, 0xF, true));    // row_shr:4
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x118, 0xF, 0xF, true));    // row_shr:8
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x142, 0xA, 0xF, false));   // row_bcast:15
    x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x143, 0xC, 0xF, false));   // row_bcast:31
    return x;
}

// Escape ranks for kN counts per lane (kN even; each count at most 512, so two share a
// dword as 16-bit fields and one scan serves both).  excl[i]: escapes of count i in
// the lanes below this one; total[i]: of the whole wave.  Counts from `live` on are 0
// and skipped (live is the same in every lane).
template <int kN>
__device__ inline void wave_ranks(const uint32_t (&cnt)[kN], uint32_t (&excl)[kN], uint32_t (&total)[kN],
                                  uint32_t live = kN)
{
#pragma unroll
    for (int i = 0; i < kN; i += 2) {
        excl[i] = excl[i + 1] = total[i] = total[i + 1] = 0;
        if (uint32_t(i) >= live) continue;
        const uint32_t x = cnt[i] | (cnt[i + 1] << 16);
        const uint32_t incl = wave_scan_incl(x);
        const uint32_t t = uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
        const uint32_t e = incl - x;   // no borrow between the fields: incl >= x in each
        excl[i] = e & 0xFFFFu;
        excl[i + 1] = e >> 16;
        total[i] = t & 0xFFFFu;
        total[i + 1] = t >> 16;
    }
}

// Ranks of a wave's escapes over its 4 tiles in value order (tile by tile, lanes in
// order inside a tile): start[k] = position of this lane's first escape of tile k.
// Returns the escapes of all 4 tiles.
__device__ inline uint32_t half_ranks(const uint32_t (&cnt)[4], uint32_t (&start)[4])
{
    uint32_t excl[4], total[4];
    wave_ranks<4>(cnt, excl, total);
    uint32_t base = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        start[k] = base + excl[k];
        base += total[k];
    }
    return base;
}

// Orders LDS writes of the wave's lanes before the reads of other lanes of the wave.
__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Code table entry of an exponent (one byte): the 3-bit code in bits 0-2, bit 3 set
// when the code is 0 (an escape).  Encoder row of a lane: the entry of column j shifted
// left by 4j, so bit 4j + p is plane p of column j and bit 4j + 3 flags an escape.
__device__ inline uint32_t code_entry(uint32_t code) { return code | (code == 0 ? 8u : 0u); }

// Plane dword stored by a lane after the encoder's transpose: lane c of half h holds
// row bit c = 4j + p, i.e. bit p of column j for the 32 lanes of the half, which is
// dword h of plane word 8p + j; lanes with p = 3 hold escape flags and store nothing.
__device__ inline uint32_t encoder_plane_dword(uint32_t lane)
{
    const uint32_t c = lane & 31u, p = c & 3u;
    return p < 3 ? 2 * (8 * p + (c >> 2)) + (lane >> 5) : ~0u;
}

// What one tile leaves for the escape pass: the lane's escape flags (bit 4j + 3 for
// column j) and the 8 exponents of the lane (columns 0-3 in e0, 4-7 in e1, one byte
// each).
struct TileEsc {
    uint32_t m, e0, e1;
};

// Encodes one tile held by the wave.  kFull: all 512 values exist (else `nvalid` of
// this lane's 8 values do).  Writes the 512 A bytes and the 192 plane bytes.
template <bool kFull>
__device__ inline TileEsc encode_tile(uint4 v, uint32_t lane, uint32_t nvalid, const uint8_t* s_lut,
                                      const Transpose32& tc, uint32_t bdw, uint8_t* A_tile, uint32_t* B_tile)
{
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint32_t row = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        uint32_t ent = s_lut[(d[j >> 1] >> (7 + 16 * (j & 1))) & 0xFFu];
        if (!kFull && uint32_t(j) >= nvalid) ent = 0;   // not a value: no plane bits, no escape
        row |= ent << (4 * j);
    }
    // sign+mantissa bytes: low byte of a BF16 holds the mantissa (bits 0-6), high byte
    // the sign (bit 7).  Gather low and high bytes of 4 values, then merge.
    const uint32_t lo0 = perm(d[1], d[0], 0x06040200u), hi0 = perm(d[1], d[0], 0x07050301u);
    const uint32_t lo1 = perm(d[3], d[2], 0x06040200u), hi1 = perm(d[3], d[2], 0x07050301u);
    uint2 a;
    a.x = (lo0 & 0x7F7F7F7Fu) | (hi0 & 0x80808080u);
    a.y = (lo1 & 0x7F7F7F7Fu) | (hi1 & 0x80808080u);
    store_nt(reinterpret_cast<uint2*>(A_tile + 8 * lane), a);

    const uint32_t col = transpose32(row, tc);
    if (bdw != ~0u) store_nt(B_tile + bdw, col);

    TileEsc r;
    r.m = row & 0x88888888u;
    // exponent = low 7 bits of the high byte, then bit 7 of the low byte
    r.e0 = ((hi0 << 1) & 0xFEFEFEFEu) | ((lo0 >> 7) & 0x01010101u);
    r.e1 = ((hi1 << 1) & 0xFEFEFEFEu) | ((lo1 >> 7) & 0x01010101u);
    return r;
}

// Writes the lane's escape exponents of one tile to s_esc from position r on, in
// column order.  Most lanes have none or one, so the loop is short.
__device__ inline void stage_tile_escapes(const TileEsc& te, uint32_t r, uint8_t* s_esc)
{
    for (uint32_t m = te.m; m; m &= m - 1) s_esc[r++] = uint8_t(perm(te.e1, te.e0, __builtin_ctz(m) >> 2));
}

// The 16-byte loads of this lane's values in half block hb (all 2048 values exist):
// addresses first (a gathered segment reads its row indices with scalar loads), then the
// 4 loads in straight-line code.
__device__ inline void load_full_half(const CSeg& sg, uint32_t hb, uint32_t lane, uint4 (&v)[4], bool& bad_row)
{
    const uint16_t* src[4];
    if (sg.rows == nullptr) {
#pragma unroll
        for (int k = 0; k < 4; k++) src[k] = sg.src + uint64_t(hb) * kHalf + k * kTile + 8 * lane;
    } else {
#pragma unroll
        for (int k = 0; k < 4; k++) src[k] = gathered_lane_ptr(sg, hb * kHalf + k * kTile, lane, bad_row);
    }
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = load_nt(reinterpret_cast<const uint4*>(src[k]));
}

// The same for the segment's last, partial half block (values past n read as 0).
__device__ inline void load_partial_half(const CSeg& sg, uint32_t hb, uint32_t lane, uint4 (&v)[4], bool& bad_row)
{
    if (sg.rows == nullptr) {
#pragma unroll
        for (int k = 0; k < 4; k++) v[k] = load_lane(sg.src, hb * 4 + k, lane, sg.n);
    } else {
#pragma unroll
        for (int k = 0; k < 4; k++) v[k] = load_lane_rows(sg, hb * 4 + k, lane, bad_row);
    }
}

// Values of a segment of n values that lie past the first 192 of their tile, among the
// m values from the start of a tile on (every tile full but the last): what a stretch
// of an uncoded block puts in the escape buffer.  32-bit scalar arithmetic, no branch.
__device__ inline uint32_t overflow_of(uint32_t m)
{
    return (m / kTile) * (kTile - kUncodedPlaneBytes) + max(m % kTile, kUncodedPlaneBytes) - kUncodedPlaneBytes;
}

// The same for half block hb of the segment (0 past the segment).
__device__ inline uint32_t half_overflow(uint32_t n, uint32_t hb)
{
    const uint32_t full = n / kHalf;   // half blocks with all their values
    const uint32_t m = hb < full ? kHalf : (hb == full ? n % kHalf : 0u);
    return overflow_of(m);
}

// Half block hb of an uncoded block (v: this lane's values of its 4 tiles): the
// exponents of each tile's values 0..191 replace the tile's 192 plane bytes (lanes
// 0..23, 8 bytes each; 0 past n), and those of values 192.. are staged in s_esc tile
// after tile, in value order, in place of the coded escapes.  The plane dwords this
// wave stored before are overwritten, so it first waits for them to complete.
__device__ inline void store_uncoded_half(const CSeg& sg, uint32_t hb, uint32_t lane, const uint4 (&v)[4],
                                          uint8_t* s_esc)
{
    const uint32_t n = sg.n;
    const uint32_t T = uint32_t(tiles_of(n));
    uint8_t* B = sg.dst + planes_off(n);
    wait_vm();
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t t = hb * 4 + k;
        if (t >= T) break;
        const uint64_t i = uint64_t(t) * kTile + 8ull * lane;
        const uint32_t nvalid = i >= n ? 0u : uint32_t(min<uint64_t>(8, n - i));
        const uint32_t d[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; j++) e[j] = uint32_t(j) < nvalid ? (d[j >> 1] >> (7 + 16 * (j & 1))) & 0xFFu : 0u;
        if (8 * lane < kUncodedPlaneBytes) {
            const uint2 w = make_uint2(e[0] | e[1] << 8 | e[2] << 16 | e[3] << 24, e[4] | e[5] << 8 | e[6] << 16 | e[7] << 24);
            *reinterpret_cast<uint2*>(B + 192ull * t + 8 * lane) = w;
        } else {
            // earlier tiles of the half are full: each put kTile - 192 bytes before this one
            uint8_t* q = s_esc + k * (kTile - kUncodedPlaneBytes) + (8 * lane - kUncodedPlaneBytes);
            for (uint32_t j = 0; j < nvalid; j++) q[j] = uint8_t(e[j]);
        }
    }
    wave_lds_sync();
}

// Encodes half block hb of a segment (tiles 4hb .. 4hb+3, those that exist): A bytes,
// planes, the escape count (to workspace slot gh) and the escape exponents in value
// order in s_esc; zero padding after the segment's last half block.
// The code table of segment s: the segment descriptor's, or the plan the caller left in
// device memory (8 bytes per segment: 7 ascending exponents and a zero byte).
template <class Args>
__device__ inline void seg_table(const Args& a, int s, uint32_t& lo, uint32_t& hi)
{
    if (a.dplans) {
        const uint32_t* t = reinterpret_cast<const uint32_t*>(a.dplans + 8 * s);
        lo = __builtin_amdgcn_readfirstlane(t[0]);
        hi = __builtin_amdgcn_readfirstlane(t[1]) & 0x00FFFFFFu;
    } else {
        lo = a.seg[s].table_lo;
        hi = a.seg[s].table_hi;
    }
}

template <bool kFull, bool kPublish, class Args>
__device__ inline uint32_t encode_half(const Args& a, const CSeg& sg, uint32_t hb, uint32_t gh, const uint4 (&v)[4],
                                       uint32_t lane, const uint8_t* lut, const Transpose32& tc, uint8_t* s_esc)
{
    const uint32_t n = sg.n;
    const uint32_t T = uint32_t(tiles_of(n)), K = uint32_t(blocks_of(n));
    uint8_t* dst = sg.dst;
    uint8_t* A = dst + 128;
    uint32_t* B = reinterpret_cast<uint32_t*>(dst + planes_off(n));
    const uint32_t bdw = encoder_plane_dword(lane);
    const uint32_t t0 = hb * 4;
    TileEsc te[4];
    if constexpr (kFull) {   // all 2048 values exist
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t t = t0 + k;
            te[k] = encode_tile<true>(v[k], lane, 8, lut, tc, bdw, A + 512ull * t, B + 48ull * t);
        }
    } else {
        const uint32_t ntiles = t0 < T ? min(4u, T - t0) : 0u;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t t = t0 + k;
            te[k] = TileEsc{0, 0, 0};
            if (uint32_t(k) < ntiles) {
                const uint64_t i = uint64_t(t) * kTile + 8ull * lane;
                const uint32_t nvalid = i >= n ? 0u : uint32_t(min<uint64_t>(8, n - i));
                te[k] = encode_tile<false>(v[k], lane, nvalid, lut, tc, bdw, A + 512ull * t, B + 48ull * t);
            }
        }
    }
    // escapes in value order: tile by tile, lower lanes first, a lane's columns in order
    uint32_t cnt[4], start[4];
#pragma unroll
    for (int k = 0; k < 4; k++) cnt[k] = __builtin_popcount(te[k].m);
    const uint32_t run = min(half_ranks(cnt, start), kHalf);
#pragma unroll
    for (int k = 0; k < 4; k++) stage_tile_escapes(te[k], start[k], s_esc);
    if constexpr (!kPublish) {   // the single launch puts the count in the unit's staged record
        if (lane == 0) a.counts[gh] = run;
    }
    if (hb == 2 * K - 1) {   // zero padding of the plane and offset sections
        const uint32_t bpad = uint32_t(round128(192ull * T) - 192ull * T);
        uint8_t* bp = reinterpret_cast<uint8_t*>(B) + 192ull * T;
        for (uint32_t k = lane; k < bpad; k += 64) bp[k] = 0;
        const uint32_t cpad = uint32_t(round128(4ull * K) - 4ull * K);
        uint8_t* cp = dst + offsets_off(n) + 4ull * K;
        for (uint32_t k = lane; k < cpad; k += 64) cp[k] = 0;
    }
    return run;
}

// Encode: one workgroup per unit of 4 blocks, one half block per wave.  No workgroup
// waits for another: each wave writes its tiles' A bytes and planes and its escape
// count; the unit's escape exponents go, in value order, to the unit's staging area.
// kPublish (single-launch compress): the unit's ready word is written last, after every
// wave's counts and staged escapes have reached memory.
template <bool kPublish, class Args>
__device__ inline void encode_unit(const Args& a, uint32_t unit)
{
    __shared__ uint8_t s_lut[256];
    __shared__ __attribute__((aligned(16))) uint8_t s_esc[kEncWaves][kHalf];

    const uint32_t tid = threadIdx.x, lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = find_segment_wave<&CSeg::unit0>(a.seg, a.nseg, unit);
    const CSeg& sg = a.seg[s];
    const uint32_t n = sg.n;
    const uint32_t hb = (unit - sg.unit0) * kEncWaves + wave;   // half block within the segment
    const bool active = hb < 2 * blocks_of(n);

    // Every load of the half block first.  A half block with all 2048 values loads in
    // straight-line code before the code table is built; the segment's last, partial half
    // block loads after the barrier (values past n read as 0).  The compiler emits these
    // loads as flat loads (their addresses come from the segment table), and a flat load
    // also counts on the LDS/scalar counter, so the wave's first wait for a scalar result
    // waits for all four.  Loads through global-space pointers, which let each tile wait
    // for its own, measured 0.9-1.6 % slower, and issuing the fourth only after the first
    // tile's stores slower still; the decoders, whose loads are global, lose 19-30 % when
    // they wait for all of theirs at once.
    const bool full = active && uint64_t(hb + 1) * kHalf <= n;
    bool bad_row = false;   // a gathered row index outside the matrix
    uint4 v[4];
    if (full) load_full_half(sg, hb, lane, v, bad_row);
    __shared__ uint32_t s_hcnt[kEncWaves];
    uint32_t table_lo, table_hi;
    seg_table(a, s, table_lo, table_hi);
    if (tid < 256) {   // exponent -> code entry of this segment
        uint32_t code = 0;
#pragma unroll
        for (int r = 0; r < 7; r++) {
            const uint32_t te = (r < 4 ? (table_lo >> (8 * r)) : (table_hi >> (8 * (r - 4)))) & 0xFFu;
            if (te == tid) code = r + 1;
        }
        s_lut[tid] = uint8_t(code_entry(code));
    }
    const Transpose32 tc = transpose_consts(lane);
    __syncthreads();
    uint32_t run = 0;
    const uint32_t slot = unit * kEncWaves + wave;
    if (full) {
        run = encode_half<true, kPublish>(a, sg, hb, slot, v, lane, s_lut, tc, s_esc[wave]);
    } else if (active) {
        load_partial_half(sg, hb, lane, v, bad_row);
        run = encode_half<false, kPublish>(a, sg, hb, slot, v, lane, s_lut, tc, s_esc[wave]);
    }
    if (lane == 0) s_hcnt[wave] = run;
    __syncthreads();
    // Blocks stored uncoded: a block (waves 2k, 2k + 1) whose escapes reach its overflow
    // (its values past the first 192 of each tile) puts exactly those values' exponents
    // in the escape buffer instead.  Every wave works out the escape-buffer bytes of all
    // 8 half blocks from the counts, so no second barrier is needed.
    const uint32_t hb0 = (unit - sg.unit0) * kEncWaves;   // first half block of the unit
    uint32_t before = 0, total = 0;
#pragma unroll
    for (uint32_t w = 0; w < kEncWaves; w++) {
        const uint32_t c = s_hcnt[w];
        if (w < wave) before += c;
        total += c;
    }
    bool my_uncoded = false;
    // a block of 4096 values overflows 2560; only a segment's last unit has shorter ones
    const bool maybe_uncoded = total >= kBlockOverflow || hb0 + kEncWaves > n / kHalf;
    if (__builtin_amdgcn_readfirstlane(maybe_uncoded)) {
        before = total = 0;
#pragma unroll
        for (uint32_t k = 0; k < kEncWaves / 2; k++) {
            const uint32_t c0 = s_hcnt[2 * k], c1 = s_hcnt[2 * k + 1];
            const uint32_t o0 = half_overflow(n, hb0 + 2 * k), o1 = half_overflow(n, hb0 + 2 * k + 1);
            const bool unc = o0 + o1 > 0 && c0 + c1 >= o0 + o1;
            const uint32_t b0 = unc ? o0 : c0, b1 = unc ? o1 : c1;
            if (2 * k < wave) before += b0;
            if (2 * k + 1 < wave) before += b1;
            total += b0 + b1;
            if (wave >> 1 == k) {
                my_uncoded = unc && active;
                if (unc) run = (wave & 1) ? o1 : o0;
            }
        }
    }
    before = __builtin_amdgcn_readfirstlane(before);
    total = __builtin_amdgcn_readfirstlane(total);
    if (__builtin_amdgcn_readfirstlane(my_uncoded)) {   // rare: the wave's block is uncoded
        bool ignore = false;                           // bad rows were reported by the first pass
        if (full) load_full_half(sg, hb, lane, v, ignore);
        else load_partial_half(sg, hb, lane, v, ignore);
        store_uncoded_half(sg, hb, lane, v, s_esc[wave]);
        if constexpr (!kPublish) {
            if (lane == 0) a.counts[slot] = run;
        }
    }
    if (!kPublish && tid == 0) a.unit_counts[unit] = total;   // for the place kernel's prefix sums
    // the unit's escapes, contiguous in value order: one run per unit for the place kernel
    const uint8_t* esc_lds = s_esc[wave];
    if constexpr (kPublish) {
        // The unit's staged record, assembled in LDS: its 8 half-block counts (u16), then
        // its escapes.  It is written through to memory (agent scope) as whole 8-byte words,
        // consecutive across the workgroup's lanes: per-wave byte runs written through cost
        // each unit several partial-line writes (3.5 % of a 64 Mi-value launch with 2.4 %
        // escapes, 7 % with 7.5 %).  A block holds at most kBlockOverflow escape bytes.
        __shared__ __attribute__((aligned(16))) uint8_t s_rec[kStageHead + 4 * kBlockOverflow];
        if (lane == 0) reinterpret_cast<uint16_t*>(s_rec)[wave] = uint16_t(run);
        for (uint32_t k = lane; k < run; k += 64) s_rec[kStageHead + before + k] = esc_lds[k];
        __syncthreads();
        const uint32_t words = (kStageHead + min(total, 4 * kBlockOverflow) + 7) / 8;
        uint64_t* rec = reinterpret_cast<uint64_t*>(a.stage + uint64_t(unit) * kUnit);
        for (uint32_t k = tid; k < words; k += kEncThreads)
            store_agent(rec + k, reinterpret_cast<const uint64_t*>(s_rec)[k]);
    } else {
        uint8_t* stage = a.stage + uint64_t(unit) * kUnit + before;
        for (uint32_t k = lane; k < run; k += 64) stage[k] = esc_lds[k];
        if (!active && lane == 0) a.counts[slot] = 0;   // the scan kernel reads every slot
    }
    if (ballot(bad_row) && lane == 0) or_status(a.status, ZIPCCL_STATUS_BAD_INDEX);
    if constexpr (kPublish) {
        // What the placing workgroup reads (the staged record) was stored at agent scope,
        // i.e. written through to memory; each wave waits for its stores to complete, and
        // after the barrier the ready word is written.  (A release fence would write back
        // the XCD's whole L2 per wave: ~20x slower.)
        wait_vm();
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(a.ready + unit, (a.tag << kReadyCountBits) | total, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ __launch_bounds__(kEncThreads) void encode_kernel(const CArgs a) { encode_unit<false>(a, blockIdx.x); }

// Writes the 128-byte header block of a segment (lanes 0..31 of one wave).
__device__ inline void write_header(const CSeg& sg, uint32_t table_lo, uint32_t table_hi, uint32_t lane,
                                    uint32_t n_esc, uint32_t esc_offset)
{
    if (lane >= 32) return;
    const uint32_t n = sg.n;
    const uint64_t sbytes = static_bytes_of(n);
    uint32_t hv = 0;
    switch (lane) {
        case 0: hv = ZIPCCL_MAGIC; break;
        case 1: hv = 1u; break;                  // version 1, flags 0
        case 2: hv = n; break;
        case 4: hv = table_lo; break;
        case 5: hv = table_hi & 0x00FFFFFFu; break;
        case 6: hv = kBlock; break;
        case 7: hv = kTile; break;
        case 8: hv = n_esc; break;
        case 10: hv = esc_offset; break;
        case 12: hv = uint32_t(sbytes); break;
        case 13: hv = uint32_t(sbytes >> 32); break;
        default: hv = 0; break;
    }
    reinterpret_cast<uint32_t*>(sg.dst)[lane] = hv;
}

constexpr uint32_t kScanThreads = 1024;
constexpr uint32_t kScanPer = 16;                       // counts per thread per round
constexpr uint32_t kScanRound = kScanThreads * kScanPer;

// Header of segment s: its escape count and where its escapes start (for an empty
// segment, where they would start).
template <class Args>
__device__ inline void write_seg_header(const Args& a, int s, uint32_t lane, uint32_t n_esc, uint32_t esc_offset)
{
    uint32_t lo, hi;
    seg_table(a, s, lo, hi);
    write_header(a.seg[s], lo, hi, lane, n_esc, esc_offset);
}

// Scan: one workgroup turns the per-slot escape counts into launch-wide positions:
// pos[h] = escapes of all slots before h, pos[8 * total_units] = all escapes.  Rounds of 16 consecutive counts per thread keep loads and stores 16 bytes
// wide.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const CArgs a)
{
    __shared__ uint32_t s_wtot[kScanThreads / 64];
    const uint32_t tid = threadIdx.x, lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t Kt = kEncWaves * a.total_units;   // half-block slots
    uint32_t carry = 0;
    for (uint32_t r0 = 0; r0 < Kt; r0 += kScanRound) {
        const uint32_t lo = r0 + tid * kScanPer;
        uint32_t c[kScanPer];
        if (lo + kScanPer <= Kt) {
            const uint4* q = reinterpret_cast<const uint4*>(a.counts + lo);
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint4 v = q[k];
                c[4 * k] = v.x; c[4 * k + 1] = v.y; c[4 * k + 2] = v.z; c[4 * k + 3] = v.w;
            }
        } else {
#pragma unroll
            for (uint32_t k = 0; k < kScanPer; k++) c[k] = lo + k < Kt ? a.counts[lo + k] : 0u;
        }
        uint32_t mine = 0;
#pragma unroll
        for (uint32_t k = 0; k < kScanPer; k++) mine += c[k];
        uint32_t incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            uint32_t y = __shfl_up(incl, o, 64);
            if (lane >= uint32_t(o)) incl += y;
        }
        __syncthreads();                       // previous round's readers of s_wtot are done
        if (lane == 63) s_wtot[wave] = incl;
        __syncthreads();
        uint32_t base = carry, total = 0;
        for (uint32_t w = 0; w < kScanThreads / 64; w++) {
            const uint32_t t = s_wtot[w];
            if (w < wave) base += t;
            total += t;
        }
        uint32_t run = base + incl - mine;
        uint32_t p[kScanPer];
#pragma unroll
        for (uint32_t k = 0; k < kScanPer; k++) {
            p[k] = run;
            run += c[k];
        }
        if (lo + kScanPer <= Kt) {
            uint4* q = reinterpret_cast<uint4*>(a.pos + lo);
#pragma unroll
            for (int k = 0; k < 4; k++) q[k] = make_uint4(p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]);
        } else {
#pragma unroll
            for (uint32_t k = 0; k < kScanPer; k++)
                if (lo + k < Kt) a.pos[lo + k] = p[k];
        }
        carry += total;
    }
    if (tid == 0) a.pos[Kt] = carry;
    uint64_t* const ne = a.call[0].n_esc_out;   // the scan path has one call
    if (tid == 0 && ne && Kt == 0) ne[a.nseg] = 0;
    if (Kt == 0 && wave == 0) {   // only empty segments: every header says offset 0
        for (int s = 0; s < a.nseg; s++) {
            write_seg_header(a, s, lane, 0u, 0u);
            if (lane == 0 && ne) ne[s] = 0;
        }
    }
}

// Copies len bytes from LDS (src, 4-byte aligned, with at least len rounded up to 4 bytes
// readable) to esc[p + off ...].  The dwords of the destination that the run covers
// whole are written as dwords (lane l: dwords l, l + 64, ...; each a v_alignbyte of two
// LDS dwords), the at most 3 bytes before and after them byte by byte: the units on
// either side own the rest of those dwords.  Bytes at or past esc_cap are dropped
// (returns true if there were any), byte by byte.
__device__ inline bool copy_run(const CCall& c, const uint8_t* src, uint32_t p, uint32_t off, uint32_t len,
                                uint32_t lane)
{
    uint8_t* dst = c.esc + p + off;
    if (uint64_t(p) + off + len <= c.esc_cap) {   // the common case: no per-byte check
        const uint32_t h = min(len, uint32_t(0u - uint32_t(reinterpret_cast<uintptr_t>(dst))) & 3u);
        const uint32_t nd = (len - h) / 4, t0 = h + 4 * nd;   // whole dwords, then the tail
        if (lane < h) dst[lane] = src[lane];
        if (lane < len - t0) dst[t0 + lane] = src[t0 + lane];
        uint32_t* dw = reinterpret_cast<uint32_t*>(dst + h);
        const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
        if (h == 0) {
            for (uint32_t i = lane; i < nd; i += 64) dw[i] = s32[i];
        } else {   // dword i holds source bytes h + 4i .. h + 4i + 3 (all before t0 <= len)
            for (uint32_t i = lane; i < nd; i += 64) dw[i] = __builtin_amdgcn_alignbyte(s32[i + 1], s32[i], h);
        }
        return false;
    }
    bool over = false;
    for (uint32_t k = lane; k < len; k += 64) {
        if (uint64_t(p) + off + k < c.esc_cap) dst[k] = src[k];
        else over = true;
    }
    return over;
}

// Copies the m staged escapes of one unit to its call's esc[p ...] (every lane of one wave).  lds:
// the wave's 1 KB LDS buffer, holding the first 512 bytes of the unit's staging area
// (stage), where the escapes start `skip` bytes in; more are brought from the staging
// area 1 KB at a time, 16 bytes per lane.  Returns true if a byte fell at or past esc_cap.
template <bool kAgent>
__device__ inline bool place_unit_escapes(const CCall& c, uint8_t* lds, const uint8_t* stage, uint32_t skip,
                                          uint32_t p, uint32_t m, uint32_t lane)
{
    const uint32_t head = 512 - skip;   // escapes in the first 512 bytes
    bool over = copy_run(c, lds + skip, p, 0, min(m, head), lane);
    for (uint32_t c0 = head; c0 < m; c0 += 1024) {   // more than `head` escapes in the unit
        const uint32_t o = skip + c0 + 16 * lane;      // byte of the staging area, a multiple of 16
        uint4 x = make_uint4(0, 0, 0, 0);
        if (o + 16 <= kUnit) {
            const uint4* q = reinterpret_cast<const uint4*>(stage + o);
            if constexpr (kAgent) {
                const uint64_t* q2 = reinterpret_cast<const uint64_t*>(q);
                const uint64_t x0 = load_agent(q2), x1 = load_agent(q2 + 1);
                x = make_uint4(uint32_t(x0), uint32_t(x0 >> 32), uint32_t(x1), uint32_t(x1 >> 32));
            } else {
                x = q[0];
            }
        }
        wave_lds_sync();   // earlier reads of the buffer are done
        reinterpret_cast<uint4*>(lds)[lane] = x;
        wave_lds_sync();
        over = copy_run(c, lds, p, c0, min(m - c0, 1024u), lane) || over;
    }
    return over;
}

// Offset-table entry of block gb (launch-wide) of segment sg (index s, of call c), whose
// escapes occupy [p0, p2) of the call's escapes (base = the segment's first escape); the
// segment header from the segment's last block, and the headers of the call's empty
// segments next to it.
template <class Args>
__device__ inline void place_block_tables(const Args& a, const CCall& c, const CSeg& sg, int s, uint32_t gb,
                                          uint32_t p0, uint32_t p2, uint32_t base, uint32_t lane)
{
    const uint32_t K = uint32_t(blocks_of(sg.n));
    const int e0 = int(c.seg0), e1 = int(c.seg0 + c.nseg);   // the call's segments
    if (lane == 0) reinterpret_cast<uint32_t*>(sg.dst + offsets_off(sg.n))[gb - sg.block0] = p0 - base;
    if (gb == sg.block0 + K - 1) {
        write_seg_header(a, s, lane, p2 - base, base);
        if (lane == 0 && c.n_esc_out) c.n_esc_out[s - e0] = p2 - base;
    }
    // empty segments just before this one start where it starts; those after the
    // call's last block start at the end
    if (gb == sg.block0) {
        for (int e = s - 1; e >= e0 && a.seg[e].n == 0; e--) {
            write_seg_header(a, e, lane, 0u, p0);
            if (lane == 0 && c.n_esc_out) c.n_esc_out[e - e0] = 0;
        }
    }
    if (gb + 1 == c.block_end) {
        for (int e = s + 1; e < e1; e++) {
            write_seg_header(a, e, lane, 0u, p2);
            if (lane == 0 && c.n_esc_out) c.n_esc_out[e - e0] = 0;
        }
        if (lane == 0 && c.n_esc_out) c.n_esc_out[c.nseg] = p2;
    }
}

// Workspace slot of the first half of block gb (launch-wide) of segment s.
__device__ inline uint32_t block_slot(const CSeg& sg, uint32_t gb)
{
    const uint32_t lb = gb - sg.block0;
    return (sg.unit0 + lb / kWaves) * kEncWaves + (lb % kWaves) * 2;
}

// Place, after the scan kernel: one wave per block, positions from pos[]; the block's
// escapes are copied from its unit's staging area byte by byte.
__global__ __launch_bounds__(kThreads) void place_kernel(const CArgs a)
{
    const uint32_t lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t gb = blockIdx.x * kWaves + wave;
    if (gb >= a.total_blocks) return;
    const int s = find_segment<&CSeg::block0>(a.seg, a.nseg, gb);
    const CSeg sg = a.seg[s];
    const uint32_t slot = block_slot(sg, gb);
    const uint32_t unit = slot / kEncWaves;
    const uint32_t p0 = a.pos[slot], p2 = a.pos[slot + 2], pu = a.pos[unit * kEncWaves];
    const uint8_t* stage = a.stage + uint64_t(unit) * kUnit + (p0 - pu);
    bool over = false;
    const CCall& c = a.call[0];   // the scan path has one call, starting at unit 0
    for (uint32_t k = lane; k < p2 - p0; k += 64) {
        const uint64_t at = uint64_t(p0) + k;
        if (at < c.esc_cap) c.esc[at] = stage[k];
        else over = true;
    }
    if (ballot(over) && lane == 0) or_status(a.status, ZIPCCL_STATUS_ESC_OVERFLOW);
    place_block_tables(a, c, sg, s, gb, p0, p2, a.pos[sg.unit0 * kEncWaves], lane);
}

// Place without the scan kernel: one workgroup per 8 encode units, one unit (4 blocks)
// per wave.  Escape positions count from the first escape of a unit's call, so the
// workgroup sums the escape counts of the units of its first unit's call before its
// first unit (and before the first unit of that unit's segment) from unit_counts[], a
// few kilobytes read from L2; each wave then copies its unit's escapes (staged
// contiguous, the first 512 bytes requested up front) in one run and derives its
// blocks' offsets from the unit's 8 half-block counts.  A call has at most
// kDirectPrefixMaxUnits units; a launch of several calls may have more.
constexpr uint32_t kPlaceUnits = 8;
constexpr uint32_t kPlaceThreads = 64 * kPlaceUnits;
// uint4 loads per thread: the call's units before the group, from a multiple of 4 on
constexpr uint32_t kPrefixLoads = (kDirectPrefixMaxUnits + 3 + 4 * kPlaceThreads - 1) / (4 * kPlaceThreads);

// Bounded wait of the single-launch compress: polls for the ready word of unit u of this
// call (tag) and returns its escape count; after `polls` polls (2^16 by default, about
// 0.1 s) sets `late` and returns 0.  A placing workgroup comes after every encoder whose
// word it waits for in the grid (workgroups are dispatched in grid order), and encoders
// wait for nothing, so the wait ends long before the limit.
__device__ inline uint32_t wait_ready(const uint64_t* ready, uint32_t u, uint64_t tag, uint32_t polls, uint64_t w,
                                      bool& late)
{
    for (uint32_t k = 0; (w >> kReadyCountBits) != tag; k++) {
        if (late || k >= polls) {   // once one wait has run out, the thread waits no more
            late = true;
            return 0;
        }
        __builtin_amdgcn_s_sleep(8);
        w = __hip_atomic_load(ready + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return uint32_t(w & ((1u << kReadyCountBits) - 1u));
}

// Unit counts of the single-launch compress, from the ready words of units [c0, u_end)
// (c0: the first unit of the call of the group's first unit; each thread takes every
// kPlaceThreads-th, 4 loads in flight): the escapes from c0 to u_first (acc) and to u0
// (accs); the counts of the group's own units go to s_ucnt.
template <class Args>
__device__ inline bool wait_unit_counts(const Args& a, uint32_t c0, uint32_t u_first, uint32_t u_end, uint32_t u0,
                                        uint32_t tid, uint32_t* s_ucnt, uint32_t& acc, uint32_t& accs)
{
    constexpr uint32_t kPer = 4;
    bool late = false;
    acc = accs = 0;
    for (uint32_t base = c0; base < u_end; base += kPer * kPlaceThreads) {
        uint64_t w[kPer];
#pragma unroll
        for (uint32_t k = 0; k < kPer; k++) {
            const uint32_t u = base + tid + k * kPlaceThreads;
            w[k] = u < u_end ? __hip_atomic_load(a.ready + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
        }
#pragma unroll
        for (uint32_t k = 0; k < kPer; k++) {
            const uint32_t u = base + tid + k * kPlaceThreads;
            if (u >= u_end) break;
            const uint32_t c = wait_ready(a.ready, u, a.wait_tag, a.wait_polls, w[k], late);
            if (u < u_first) acc += c;
            else s_ucnt[u - u_first] = c;
            if (u < u0) accs += c;
        }
    }
    return late;
}

// Positions count from the first escape of the unit's call: each workgroup sums the
// unit counts of its first unit's call before its first unit and before the first unit
// of that unit's segment (a call or segment that starts inside the group starts at the
// counts of the group's units before it).
// kWait (single-launch compress): the counts come from the encoders' ready words, waited
// for; the encoder output read after that (half-block counts, staged escapes) is read
// with agent-scope loads.
template <bool kWait, class Args>
__device__ inline void place_group(const Args& a, uint32_t group, bool one_call)
{
    __shared__ uint32_t s_red[2][kPlaceUnits];
    __shared__ uint32_t s_ucnt[kPlaceUnits];
    __shared__ uint32_t s_late;
    __shared__ __attribute__((aligned(16))) uint8_t s_head[kPlaceUnits][1024];   // staged escapes, per wave
    const uint32_t tid = threadIdx.x, lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t u_first = group * kPlaceUnits;
    const uint32_t unit = u_first + wave;
    const bool active = unit < a.total_units;
    const uint32_t slot0 = unit * kEncWaves;
    const uint8_t* stage = a.stage + uint64_t(unit) * kUnit;   // the unit's escapes, contiguous
    uint2 head = make_uint2(0, 0);
    uint32_t hc[2 * kWaves];   // the unit's half-block escape counts
    uint32_t acc = 0, accs = 0;
    const int s = find_segment<&CSeg::unit0>(a.seg, a.nseg, active ? unit : a.total_units - 1);
    const int s_first = find_segment<&CSeg::unit0>(a.seg, a.nseg, u_first);
    const uint32_t u0 = a.seg[s_first].unit0;             // first unit of the first unit's segment
    // ... and of its call (0 in a launch of one call, which the caller read with the
    // launch's first arguments: no dependent argument loads before the first ready words
    // are requested)
    const uint32_t c0 = one_call ? 0u : a.call[a.seg[s_first].call].unit0;
    if constexpr (!kWait) {
        head = active ? reinterpret_cast<const uint2*>(stage)[lane] : make_uint2(0, 0);
#pragma unroll
        for (uint32_t k = 0; k < 2 * kWaves; k++) hc[k] = active ? a.counts[slot0 + k] : 0u;
        if (lane == 0) s_ucnt[wave] = active ? a.unit_counts[unit] : 0u;
        // unit_counts[c0 .. u_first), 4 per load from the multiple of 4 at or below c0
        // (u_first is a multiple of 8)
        const uint32_t q0 = c0 & ~3u;
        uint4 q[kPrefixLoads];
#pragma unroll
        for (uint32_t r = 0; r < kPrefixLoads; r++) {
            const uint32_t i = q0 + 4 * (tid + r * kPlaceThreads);
            q[r] = i < u_first ? *reinterpret_cast<const uint4*>(a.unit_counts + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (uint32_t r = 0; r < kPrefixLoads; r++) {
            const uint32_t i = q0 + 4 * (tid + r * kPlaceThreads);
            const uint32_t v[4] = {q[r].x, q[r].y, q[r].z, q[r].w};
#pragma unroll
            for (uint32_t k = 0; k < 4; k++) {
                if (i + k >= c0) acc += v[k];
                if (i + k >= c0 && i + k < u0) accs += v[k];
            }
        }
    } else {
        const uint32_t u_end = min(u_first + kPlaceUnits, a.total_units);
        if (tid == 0) s_late = 0;
        if (tid < kPlaceUnits && u_first + tid >= u_end) s_ucnt[tid] = 0;
        __syncthreads();
        const bool late = wait_unit_counts(a, c0, u_first, u_end, u0, tid, s_ucnt, acc, accs);
        if (late) s_late = 1;   // any thread; read after the barrier below
    }
    const CSeg sg = a.seg[s];
    const uint32_t K = uint32_t(blocks_of(sg.n));
    const uint32_t b0 = (unit - sg.unit0) * kWaves;   // first block of the unit within the segment

#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        acc += __shfl_xor(acc, o, 64);
        accs += __shfl_xor(accs, o, 64);
    }
    if (lane == 0) {
        s_red[0][wave] = acc;
        s_red[1][wave] = accs;
    }
    if constexpr (!kWait) reinterpret_cast<uint2*>(s_head[wave])[lane] = head;
    __syncthreads();
    if constexpr (kWait) {
        if (s_late) {   // an encoder's count never arrived: place nothing, report it
            if (tid == 0) or_status(a.status, ZIPCCL_STATUS_WAIT_LIMIT);
            return;
        }
        if (!active) return;
        // the encoder's agent-scope stores completed before its ready word was written:
        // agent-scope loads see them (an acquire fence would invalidate the L2 per wave)
        const uint64_t h = load_agent(reinterpret_cast<const uint64_t*>(stage) + lane);
        head = make_uint2(uint32_t(h), uint32_t(h >> 32));
        // the unit's 8 half-block counts, u16 each, open its staged record (lanes 0 and 1)
#pragma unroll
        for (uint32_t k = 0; k < 2 * kWaves; k += 2) {
            const uint32_t q = __builtin_amdgcn_readlane(k & 2 ? head.y : head.x, k >> 2);
            hc[k] = q & 0xFFFFu;
            hc[k + 1] = q >> 16;
        }
        reinterpret_cast<uint2*>(s_head[wave])[lane] = head;
        wave_lds_sync();
    }
    if (!active) return;
    uint32_t pre = 0, first_base = 0;
#pragma unroll
    for (uint32_t w = 0; w < kPlaceUnits; w++) {
        pre += s_red[0][w];
        first_base += s_red[1][w];
    }
    // escapes before this unit, before its segment's first unit and before its call's
    // first unit, counted from the first escape of the group's first call: a segment or
    // call that starts inside the group starts at `pre` plus the units of the group
    // before it; otherwise it holds the group's first unit, and its start was summed
    // above (0 for the call)
    const CCall& c = a.call[sg.call];
    uint32_t upos = pre;
    for (uint32_t w = 0; w < wave; w++) upos += s_ucnt[w];
    uint32_t base = first_base;
    if (sg.unit0 >= u_first) {
        base = pre;
        for (uint32_t w = 0; w < sg.unit0 - u_first; w++) base += s_ucnt[w];
    }
    uint32_t cbase = 0;
    if (c.unit0 >= u_first) {
        cbase = pre;
        for (uint32_t w = 0; w < c.unit0 - u_first; w++) cbase += s_ucnt[w];
    }
    upos -= cbase;   // positions within the call's escapes
    base -= cbase;
    // the unit's escapes in one run; its blocks' positions from its 8 half-block counts
    if (ballot(place_unit_escapes<kWait>(c, s_head[wave], stage, kWait ? kStageHead : 0u, upos, s_ucnt[wave], lane)) &&
        lane == 0)
        or_status(a.status, ZIPCCL_STATUS_ESC_OVERFLOW);
    uint32_t p = upos;
#pragma unroll
    for (uint32_t k = 0; k < kWaves; k++) {
        if (b0 + k >= K) break;
        const uint32_t p0 = p, p2 = p0 + hc[2 * k] + hc[2 * k + 1];
        place_block_tables(a, c, sg, s, sg.block0 + b0 + k, p0, p2, base, lane);
        p = p2;
    }
}

__global__ __launch_bounds__(kPlaceThreads) void place_direct_kernel(const CArgs a)
{
    place_group<false>(a, blockIdx.x, a.ncalls <= 1);
}

// Compress in one launch: total_units workgroups encode (as encode_kernel) and publish
// each unit's escape count in its ready word; ceil(total_units / 8) place (as
// place_direct_kernel) once the ready words they need carry this call's tag.
// The grid interleaves the two roles, in unit order: the workgroup that places group c
// (units 8c .. 8c + 7) comes right after the encoder of unit 8c + 8 + kPlaceLag, so its
// units were encoded about one generation of workgroups earlier and it finds their
// counts ready while later units are still being encoded.  The last kTailGroups groups
// (all of them in a launch of up to 4096 units) are placed after the last encoder, last
// group first: they fill the slots the last generation of encoders frees, and the last
// group, which has the most ready words of its call to read, starts while the last
// encoders still run.  Every placer comes after every encoder it waits for, and encoders
// wait for nothing, so every wait ends.
// Measured on 32 chunk calls of 7 x 2 Mi values: launches of 8 calls with every placer
// at the end took 317.9 us, interleaved launches of 16 calls 306.2 us (32 calls per
// launch were no faster than 16).  A lag of 512 units left placers waiting in slots the
// encoders needed (336 us); 1024 to 2048 measured alike.  No tail groups: 310.1 us.
constexpr uint32_t kPlaceLag = 1024;   // units: about one generation of encoders
constexpr uint32_t kTailGroups = 512;  // groups placed after the last encoder (all, if fewer)

__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu(8)))
void compress_single_kernel(const CArgs a)
{
    static_assert(kEncThreads == kPlaceThreads, "both roles use the same workgroup size");
    constexpr uint32_t L = kPlaceLag, Q = kPlaceUnits;
    const uint32_t E = a.total_units, b = blockIdx.x;
    const bool one_call = a.ncalls <= 1;   // next to total_units in the arguments: one load
    const uint32_t groups = (E + Q - 1) / Q;
    // groups placed before the last encoder: 0 .. interleaved - 1
    const uint32_t interleaved = min(E >= L + Q ? (E - L) / Q : 0u, groups > kTailGroups ? groups - kTailGroups : 0u);
    bool place = false;
    uint32_t idx = b;                              // the unit or group of this workgroup
    if (b >= E + interleaved) {                    // after the last encoder, last group first
        place = true;
        idx = groups - 1 - (b - E - interleaved);
    } else if (b >= L + Q) {
        const uint32_t r = b - L - Q;
        if (r >= (Q + 1) * interleaved) {          // encoders after the interleaved placers
            idx = b - interleaved;
        } else {                                   // cycles of one placer then Q encoders
            const uint32_t cycle = r / (Q + 1), pos = r % (Q + 1);
            place = pos == 0;
            idx = place ? cycle : L + Q + Q * cycle + pos - 1;
        }
    }
    // one call site per role: the kernel's code stays the size of the two roles
    if (place) place_group<true>(a, idx, one_call);
    else encode_unit<true>(a, idx);
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

// Reads and validates a segment header against the expected n and buffer sizes.  With
// at_first the escape buffer starts at the segment's first escape, whatever esc_offset
// the header records (a shard received on its own).
__device__ inline SegHeader read_header(const uint8_t* st, uint32_t n, uint64_t esc_bytes, bool at_first = false)
{
    const uint32_t* h = reinterpret_cast<const uint32_t*>(st);
    SegHeader r;
    uint32_t magic = h[0], ver = h[1], nlo = h[2], nhi = h[3];
    uint32_t t0 = h[4], t1 = h[5];
    uint32_t blk = h[6], tile = h[7];
    uint64_t n_esc = uint64_t(h[8]) | (uint64_t(h[9]) << 32);
    uint64_t eoff = at_first ? 0ull : (uint64_t(h[10]) | (uint64_t(h[11]) << 32));
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

// --------------------------------------------------------------------------------
// decompress + fp32 accumulate + one rounding
// --------------------------------------------------------------------------------
// Two fp32 sums rounded once to BF16 (round to nearest, ties to even), packed low/high:
// one v_cvt_pk_bf16_f32.  On every non-NaN fp32 pattern tried (2^24 random patterns plus
// ties, near-ties and specials in every binade, denormals included) it gives the bits of
// the integer rule (u + 0x7FFF + ((u >> 16) & 1)) >> 16; a NaN comes out as a NaN that
// keeps sign and payload bits, which fix_nan_bf16x2 replaces.
typedef __bf16 zc_bf16x2 __attribute__((ext_vector_type(2)));
typedef float zc_f32x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2_rne(float lo, float hi)
{
    const zc_f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, zc_bf16x2));
}

// Bit 15 / 31 set where the low / high BF16 half is a NaN: (h & 0x7FFF) > 0x7F80, i.e.
// (h & 0x7FFF) + 0x7F reaches 0x8000 (no carry crosses into the other half).
__device__ inline uint32_t nan_halves(uint32_t x) { return ((x & 0x7FFF7FFFu) + 0x007F007Fu) & 0x80008000u; }

// Every NaN half becomes the canonical 0x7FC0.
__device__ inline uint32_t fix_nan_bf16x2(uint32_t x)
{
    const uint32_t m = nan_halves(x);
    if (m & 0x8000u) x = (x & 0xFFFF0000u) | 0x7FC0u;
    if (m & 0x80000000u) x = (x & 0x0000FFFFu) | 0x7FC00000u;
    return x;
}

// Plane dword a lane loads in the decoders, chosen so that after the half-wave transpose
// byte b of the lane's row holds the code of column b in bits 0-2 and the code of
// column b + 4 in bits 4-6: lane c = 8b + 4g + p of half h takes dword h of plane word
// 8p + b + 4g; lanes with p = 3 take nothing (their row bits stay 0).
__device__ inline uint32_t decoder_plane_dword(uint32_t lane)
{
    const uint32_t c = lane & 31u, p = c & 3u;
    return p < 3 ? 2 * (8 * p + (c >> 3) + 4 * ((c >> 2) & 1u)) + (lane >> 5) : ~0u;
}

// Escape flags of the valid columns of a decoder row: column b at bit 8b, column b + 4
// at bit 8b + 4 (0x11111111 when all 8 exist).
__device__ inline uint32_t valid_flags(uint32_t nvalid)
{
    if (nvalid >= 8) return 0x11111111u;
    const uint32_t lo = nvalid >= 4 ? 0x01010101u : 0x01010101u & ((1u << (8 * nvalid)) - 1u);
    const uint32_t hi = nvalid > 4 ? (0x01010101u & ((1u << (8 * (nvalid - 4))) - 1u)) << 4 : 0u;
    return lo | hi;
}

__device__ inline uint32_t escape_flags(uint32_t row, uint32_t vflags)
{
    return ~(row | (row >> 1) | (row >> 2)) & vflags;
}

// A lane's 8 decoded values as the low and high bytes of their BF16 bits (values 0-3 in
// lo0/hi0, 4-7 in lo1/hi1).  row: the lane's decoder row; z: its escape flags; r: the
// position of its first escape in esc_lds; tlo/thi: the 8-byte decode table (byte 0 is
// the code-0 placeholder, 0).
struct LaneBytes {
    uint32_t lo0, hi0, lo1, hi1;
};

// A group of 4 columns whose escape flags z (bit 8c for column c) hold two or more set
// bits: the byte of the second flagged column becomes x (the group's second escape).
// With fewer than two flags, E is returned unchanged.
__device__ inline uint32_t patch_second_escape(uint32_t E, uint32_t z, uint32_t x)
{
    const uint32_t rest = z & (z - 1);          // flags after the first
    const uint32_t second = rest & (0u - rest); // the lowest of them (0 if none)
    // its byte as (second << 8) - second: the empty asm keeps the compiler from folding
    // it into a multiply by 255, a quarter-rate instruction
    uint32_t up = second << 8;
    asm("" : "+v"(up));
    const uint32_t mask = up - second;
    return (E & ~mask) | (perm(x, x, 0u) & mask);   // x in every byte
}

// BF16 low byte = exponent bit 0 << 7 | mantissa, high byte = sign | exponent >> 1, from
// the lane's A bytes and exponent bytes (values 0-3 in .x / E0, 4-7 in .y / E1).
__device__ inline LaneBytes assemble_lane(uint2 A, uint32_t E0, uint32_t E1)
{
    LaneBytes o;
    o.lo0 = (A.x & 0x7F7F7F7Fu) | ((E0 << 7) & 0x80808080u);
    o.hi0 = (A.x & 0x80808080u) | ((E0 >> 1) & 0x7F7F7F7Fu);
    o.lo1 = (A.y & 0x7F7F7F7Fu) | ((E1 << 7) & 0x80808080u);
    o.hi1 = (A.y & 0x80808080u) | ((E1 >> 1) & 0x7F7F7F7Fu);
    return o;
}

// Every byte rotated right by one bit: exponent bit 0 to bit 7, bits 1-7 down by one,
// i.e. the bits of the BF16 low byte's top bit and of the high byte's low 7 bits.
__device__ inline uint32_t rotr1_bytes(uint32_t x) { return ((x >> 1) & 0x7F7F7F7Fu) | ((x << 7) & 0x80808080u); }
// the low byte of x twice (v_perm), shifted right by one
__device__ inline uint8_t rotr1_byte(uint32_t x) { return uint8_t(perm(x, x, 0x0C0C0000u) >> 1); }

// The same from exponent bytes already rotated by rotr1 (R0 / R1): each output byte is a
// bit select of an A byte and a rotated exponent byte, with no shift.
__device__ inline LaneBytes assemble_lane_rot(uint2 A, uint32_t R0, uint32_t R1)
{
    LaneBytes o;
    o.lo0 = (A.x & 0x7F7F7F7Fu) | (R0 & 0x80808080u);
    o.hi0 = (A.x & 0x80808080u) | (R0 & 0x7F7F7F7Fu);
    o.lo1 = (A.y & 0x7F7F7F7Fu) | (R1 & 0x80808080u);
    o.hi1 = (A.y & 0x80808080u) | (R1 & 0x7F7F7F7Fu);
    return o;
}

// Exponent bytes of this lane's 8 values in a tile of an uncoded block (values 0-3 in
// .x, 4-7 in .y): those of the tile's first 192 values from its 192 plane bytes (lanes
// 0..23), the others from the escape buffer, where the tile's bytes start at esc (byte by
// byte: the escape buffer has no alignment).  nvalid: values of the lane that exist.
__device__ inline uint2 uncoded_exponents(const uint8_t* tile_planes, const uint8_t* esc, uint32_t lane,
                                          uint32_t nvalid)
{
    if (8 * lane < kUncodedPlaneBytes) return *reinterpret_cast<const uint2*>(tile_planes + 8 * lane);
    const uint8_t* q = esc + (8 * lane - kUncodedPlaneBytes);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (uint32_t j = 0; j < 4; j++) {
        if (j < nvalid) w0 |= uint32_t(q[j]) << (8 * j);
        if (j + 4 < nvalid) w1 |= uint32_t(q[j + 4]) << (8 * j);
        __builtin_amdgcn_sched_barrier(0);   // two loads in flight: few live registers (a rare path)
    }
    return make_uint2(w0, w1);
}

// Escape-buffer bytes of block b of a segment of n values when the block is uncoded.
__device__ inline uint32_t block_overflow(uint32_t n, uint32_t b)
{
    const uint32_t full = n / kBlock;   // blocks with all their values
    return overflow_of(b < full ? kBlock : (b == full ? n % kBlock : 0u));
}

template <bool kRot = false>
__device__ inline LaneBytes decode_lane(uint32_t row, uint32_t z, uint2 A, uint32_t tlo, uint32_t thi, uint32_t r,
                                        const uint8_t* esc_lds)
{
    // byte b of z holds column b's flag in bit 0 and column b + 4's in bit 4, so the sum
    // of z's bytes (one v_sad_u8 against 0) is n0 + 16 n1: the escapes of each group of
    // 4 columns, at most 4 each
    const uint32_t s = __builtin_amdgcn_sad_u8(z, 0u, 0u);
    const uint32_t n0 = s & 0xFu;
    // a code 0 selects table byte 0: the first escape of each group of 4 columns goes
    // there, so a group with at most one escape decodes with one v_perm
    const uint32_t x0 = esc_lds[r], x1 = esc_lds[r + n0];
    uint32_t E0 = perm(thi, tlo | x0, row & 0x07070707u);
    uint32_t E1 = perm(thi, tlo | x1, (row >> 4) & 0x07070707u);
    if (s & 0x66u) {   // rare: n0 or n1 is 2, 3 or 4 (several escapes among 4 columns of the lane)
        const uint32_t z0 = z & 0x01010101u, z1 = (z >> 4) & 0x01010101u;
        const uint32_t n1 = s >> 4;
        // the second escape of each group goes to the column of its second flag, by masks
        E0 = patch_second_escape(E0, z0, esc_lds[r + 1]);
        E1 = patch_second_escape(E1, z1, esc_lds[r + n0 + 1]);
        if (n0 > 2 || n1 > 2) {   // rarer still: a third or fourth escape, byte by byte
            uint32_t rr = r + 2;
            uint32_t m = z0 & (z0 - 1);
            for (m &= m - 1; m; m &= m - 1) {
                const uint32_t sh = __builtin_ctz(m);   // 8 * column
                E0 = (E0 & ~(0xFFu << sh)) | (uint32_t(esc_lds[rr++]) << sh);
            }
            rr = r + n0 + 2;
            m = z1 & (z1 - 1);
            for (m &= m - 1; m; m &= m - 1) {
                const uint32_t sh = __builtin_ctz(m);
                E1 = (E1 & ~(0xFFu << sh)) | (uint32_t(esc_lds[rr++]) << sh);
            }
        }
    }
    return kRot ? assemble_lane_rot(A, E0, E1) : assemble_lane(A, E0, E1);
}

// acc[j] += the lane's decoded value j (f32 bits = BF16 bits << 16: bytes [0, 0, low, high])
__device__ inline void add_lane(float (&acc)[8], const LaneBytes& o)
{
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t sel = 0x0C0Cu | ((j & 3u) << 16) | ((4u + (j & 3u)) << 24);
        const uint32_t f = j < 4 ? perm(o.hi0, o.lo0, sel) : perm(o.hi1, o.lo1, sel);
        acc[j] = acc[j] + __uint_as_float(f);
    }
}

constexpr uint32_t kAccWaves = 8;                  // one wave per tile of a block
constexpr uint32_t kAccThreads = 64 * kAccWaves;
constexpr uint32_t kAccBlkHead = 512;              // escape bytes per peer fetched for a block before the barrier
constexpr uint32_t kEscPad = 16;                   // decode_lane may read esc_lds[total]

// What decode-accumulate needs of a peer's header for the workgroup's block, checked by
// one wave and shared through LDS: the v_perm decode table, where the block's escapes
// start in the peer's escape buffer and how many there are.
struct PeerBlock {
    uint32_t tlo, thi;         // the v_perm decode table, each byte rotated right by one bit
    uint32_t esc_lo, esc_hi;   // escape-buffer offset of the block's first escape
    uint32_t count;            // the block's bytes in the escape buffer
    uint32_t state;            // kPeerCorrupt, kPeerCoded or kPeerUncoded
};
constexpr uint32_t kPeerCorrupt = 0, kPeerCoded = 1, kPeerUncoded = 2;

// Decode-accumulate: one workgroup per block, one wave per tile.  Every peer's bytes
// for the tile are requested up front; wave p checks peer p's header and offset-table
// entries (one chain of scalar loads per wave instead of one per peer in every wave)
// and leaves what the others need in LDS; each wave counts its tile's escapes per peer
// from the plane rows, one barrier shares the counts and the peer records so that every
// wave knows where its tile's escapes start, then the peers are decoded and added in
// order.
template <int kPeers>
// Up to 7 peers the kernel fits 64 VGPRs without spills (the A bytes wait in LDS, not in
// registers), so 4 workgroups run per CU.  At low occupancy it was latency-bound (at 2
// workgroups per CU it took 1.77x as long as at 3, and 4 took 7-peer launches 12 % below
// 3); at 4 it is bound by VALU issue (~124 instructions per wave plus ~80 per peer).
// With 8 peers the LDS allows 3 workgroups per CU (6 waves per SIMD).
__global__ __launch_bounds__(kAccThreads)
__attribute__((amdgpu_waves_per_eu(kPeers <= 7 ? 8 : (kPeers <= 8 ? 6 : 4))))
void accumulate_kernel(const AArgs a)
{
    __shared__ uint32_t s_cnt[kPeers][kAccWaves];
    __shared__ PeerBlock s_peer[kPeers];
    __shared__ __attribute__((aligned(16))) uint8_t s_blk[kPeers][kAccBlkHead + kEscPad];   // each peer's first escapes of the block
    __shared__ uint8_t s_esc[kAccWaves][kTile + kEscPad];      // a tile's escapes when they lie further on
    __shared__ uint2 s_A[kAccWaves][kPeers][64];                 // the tile's A bytes per peer, parked until decode
    const uint32_t lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the workgroup's chunk, and its block within the chunk
    const uint32_t P = uint32_t(a.npeers);
    const uint32_t c = blockIdx.y, b = blockIdx.x;   // one grid row per chunk
    const uint64_t first = uint64_t(c) * a.chunk;
    const uint32_t n = uint32_t(min<uint64_t>(a.chunk, a.n - first));
    if (b >= uint32_t(blocks_of(n))) return;         // the last chunk's row is longer than it
    const uint8_t* const* peer_st = a.st + c * P;
    const uint8_t* const* peer_esc = a.esc + c * P;
    const uint64_t* peer_eb = a.esc_bytes + c * P;
    const uint16_t* local = a.local + first;
    uint16_t* dst = a.dst + first;
    const uint32_t T = uint32_t(tiles_of(n)), K = uint32_t(blocks_of(n));
    const uint32_t t = b * 8 + wave;
    const bool has_tile = t < T;
    const uint64_t i0 = uint64_t(t) * kTile + 8ull * lane;
    const uint32_t rem = has_tile ? n - t * kTile : 0u;   // values from the tile's start on (32-bit, no overflow)
    const uint32_t nvalid = rem > 8 * lane ? min(8u, rem - 8 * lane) : 0u;
    const uint32_t pdw = decoder_plane_dword(lane);

    // ---- requests ----
    // Every lane issues the same vector loads, unconditionally (addresses of what does
    // not exist are clamped into peer 0's static part of the chunk, which is at least 896 bytes), so
    // that the compiler can wait for exactly the loads each step needs: the transposes
    // start once the plane dwords are in while the A bytes, the local values and the
    // escape heads are still on their way.  Plane dwords first, then A bytes, then local.
    const uint8_t* const safe = peer_st[0];
    const uint32_t tl = has_tile ? t : T - 1;   // T >= 1: a launch has at least one block
    const uint32_t pdl = pdw == ~0u ? 0u : 4 * pdw;   // byte offset; lanes with p = 3: any dword (bits unused)
    // Up to 8 peers the launch picks the instance of exactly npeers: every slot exists, so
    // the peers' pointers are read with no clamp and their loads go out together rather
    // than one after another.
    const uint8_t* stp[kPeers];
#pragma unroll
    for (int p = 0; p < kPeers; p++) stp[p] = peer_st[kPeers <= 8 || uint32_t(p) < P ? p : 0];
    uint32_t pw[kPeers];
    uint2 Ap[kPeers];
#pragma unroll
    for (int p = 0; p < kPeers; p++)
        pw[p] = load_nt(reinterpret_cast<const uint32_t*>(stp[p] + planes_off(n) + 192ull * tl + pdl));
#pragma unroll
    for (int p = 0; p < kPeers; p++)
        Ap[p] = load_nt(reinterpret_cast<const uint2*>(stp[p] + 128 + 512ull * tl + 8 * lane));
    uint4 lv = load_nt(reinterpret_cast<const uint4*>(nvalid == 8 ? reinterpret_cast<const uint8_t*>(local + i0)
                                                                    : safe));

    // ---- this wave's share of the header checks: peers wave, wave + 8 ----
    constexpr int kMine = (kPeers + kAccWaves - 1) / kAccWaves;   // peers checked per wave
    uint32_t head[kMine][kAccBlkHead / 64];                       // their blocks' first escapes
    // a block is uncoded when it puts exactly its overflow in the escape buffer (a coded
    // block puts fewer escapes there)
    const uint32_t ovf = block_overflow(n, b);
#pragma unroll
    for (int i = 0; i < kMine; i++) {
        const uint32_t p = wave + i * kAccWaves;
        const uint8_t* src = safe;   // with m = 0 every lane reads byte 0 of it
        uint32_t m = 0;
        if (p < P) {
            const uint8_t* st = peer_st[p];
            const SegHeader hd = read_header(st, n, peer_eb[p]);
            const uint32_t* C = reinterpret_cast<const uint32_t*>(st + offsets_off(n));
            uint32_t first = 0, last = 0;
            const bool ok = hd.ok && block_escapes(C, b, K, hd.n_esc, min(kBlock, n - b * kBlock), first, last);
            const uint64_t e = hd.esc_offset + first;
            const uint32_t state = !ok ? kPeerCorrupt : (ovf > 0 && last - first == ovf ? kPeerUncoded : kPeerCoded);
            // the decode table with every exponent rotated (rotr1): decoding then assembles
            // each lane's bytes without shifts (escape bytes are rotated where they are staged)
            if (lane == 0)
                s_peer[p] = PeerBlock{rotr1_bytes(hd.tlo), rotr1_bytes(hd.thi), uint32_t(e), uint32_t(e >> 32),
                                      last - first, state};
            m = ok ? min(last - first, kAccBlkHead) : 0u;
            if (m > 0) src = peer_esc[p] + e;
        }
        // the block's first escapes, requested now so that they arrive while the tiles
        // are transposed (written to LDS just before the barrier): lane l fetches bytes
        // l, l + 64, ... (indexes past m re-read byte m - 1)
        const uint32_t last_i = m > 0 ? m - 1 : 0u;
#pragma unroll
        for (uint32_t k = 0; k < kAccBlkHead / 64; k++) head[i][k] = src[min(64 * k + lane, last_i)];
    }

    // ---- per peer: plane rows, escape flags, escape ranks within the tile ----
    const Transpose32 tc = transpose_consts(lane);
    const uint32_t vf = valid_flags(nvalid);   // 0 in a wave without a tile
    constexpr int kPairs = (kPeers + 1) & ~1;   // the rank scans take counts in pairs
    uint32_t rows[kPeers], zf[kPeers], cnt[kPairs], rank[kPairs], total[kPairs];
#pragma unroll
    for (int p = 0; p < kPairs; p++) {
        cnt[p] = 0;
        if (p < kPeers) {
            rows[p] = zf[p] = 0;
            if (kPeers <= 8 || uint32_t(p) < P) {   // no branch up to 8 peers: transposes interleave
                rows[p] = transpose32(pw[p], tc);
                zf[p] = escape_flags(rows[p], vf);
            }
            cnt[p] = __builtin_popcount(zf[p]);
        }
    }
    wave_ranks<kPairs>(cnt, rank, total, P);
    // the A bytes (requested right after the plane dwords, so in by now) wait in LDS until
    // their peer is decoded: 2 x kPeers fewer live registers
#pragma unroll
    for (int p = 0; p < kPeers; p++) s_A[wave][p][lane] = Ap[p];
    if (lane == 0) {
#pragma unroll
        for (int p = 0; p < kPeers; p++) s_cnt[p][wave] = total[p];
    }
#pragma unroll
    for (int i = 0; i < kMine; i++) {
        const uint32_t p = wave + i * kAccWaves;
        if (p < P) {
#pragma unroll
            for (uint32_t k = 0; k < kAccBlkHead / 64; k++) s_blk[p][64 * k + lane] = uint8_t(head[i][k]);
            // rotated (rotr1) in place, 4 bytes per dword: the decode table's form
            wave_lds_sync();
            uint32_t* w = reinterpret_cast<uint32_t*>(s_blk[p]);
#pragma unroll
            for (uint32_t k = 0; k < kAccBlkHead / 256; k++) w[64 * k + lane] = rotr1_bytes(w[64 * k + lane]);
        }
    }
    __syncthreads();

    // ---- where each peer's escapes of this tile start within the block ----
    // Lane 8p + w reads tile w's count of peer p; one prefix sum over the wave then
    // gives every peer's count before this wave's tile and its block total by readlane.
    static_assert(kAccWaves == 8, "one lane per (peer, tile) pair in groups of 8");
    uint32_t before[kPeers], mine[kPeers];
    uint64_t odd = 0;   // nonzero: a peer that is not a coded block agreeing with its offsets
#pragma unroll
    for (int h = 0; h < (kPeers * kAccWaves + 63) / 64; h++) {
        const uint32_t idx = 64 * h + lane;
        const uint32_t v = idx < uint32_t(kPeers * kAccWaves) ? (&s_cnt[0][0])[idx] : 0u;
        const uint32_t incl = wave_scan_incl(v), excl = incl - v;
#pragma unroll
        for (int q = 0; q < 8 && 8 * h + q < kPeers; q++) {
            const int p = 8 * h + q;
            before[p] = mine[p] = 0;
            if (kPeers <= 8 || uint32_t(p) < P) {
                const uint32_t base = uint32_t(__builtin_amdgcn_readlane(int(excl), 8 * q));
                const uint32_t next = q < 7 ? uint32_t(__builtin_amdgcn_readlane(int(excl), 8 * q + 8))
                                            : uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
                before[p] = uint32_t(__builtin_amdgcn_readlane(int(excl), int(8 * q + wave))) - base;
                mine[p] = total[p];
                // the offset table must agree with the planes of a coded block (no branch per
                // peer: the peers' LDS records are read together; the conditions stay lane
                // masks in scalar registers)
                odd |= ballot(s_peer[p].state != kPeerCoded) | ballot(next - base != s_peer[p].count);
            }
        }
    }
    // rare: a corrupt peer, or one whose block is uncoded (its planes hold exponents, so
    // they are not checked against its offsets)
    bool bad = false;
    uint32_t uncoded = 0;
    if (odd != 0) {
        for (int p = 0; p < kPeers; p++) {
            if (kPeers > 8 && uint32_t(p) >= P) break;
            const uint32_t state = s_peer[p].state;
            uint32_t planes = 0;   // the block's escapes according to its planes
            for (uint32_t w = 0; w < kAccWaves; w++) planes += s_cnt[p][w];
            bad = bad || state == kPeerCorrupt || (state == kPeerCoded && planes != s_peer[p].count);
            if (state == kPeerUncoded) uncoded |= 1u << p;
        }
        bad = __builtin_amdgcn_readfirstlane(bad);
        uncoded = __builtin_amdgcn_readfirstlane(uncoded);
        // an uncoded peer takes the decode loop's rare branch, as a tile whose escapes go
        // past the block's first 512 does
#pragma unroll
        for (int p = 0; p < kPeers; p++)
            if (uncoded & (1u << p)) mine[p] = kAccBlkHead + 1;
    }
    // a lane holding the last values of the segment (fewer than 8) reads them now
    if (nvalid > 0 && nvalid < 8) lv = load_lane(local, t, lane, n);

    // ---- decode and add, peers in order ----
    float acc[8];
    {
        const uint32_t d[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
        for (int j = 0; j < 8; j++) acc[j] = __uint_as_float((j & 1) ? (d[j >> 1] & 0xFFFF0000u) : (d[j >> 1] << 16));
    }
    uint8_t* esc_lds = s_esc[wave];
#pragma unroll
    for (int p = 0; p < kPeers; p++) {
        if ((kPeers <= 8 || uint32_t(p) < P) && !bad && has_tile) {
            if (before[p] + mine[p] > kAccBlkHead) {
                // rare: the tile's escapes go past the block's first 512 (escape-heavy
                // tables), or the peer's block is uncoded; stage what the tile needs in the
                // wave's own LDS slot
                const uint64_t e = uint64_t(s_peer[p].esc_hi) << 32 | s_peer[p].esc_lo;
                const bool unc = (uncoded >> p) & 1u;
                if (unc) {
                    // the tile's exponents in value order: the first 192 from its plane
                    // bytes, the rest from the escape buffer, where earlier tiles of the
                    // block (all full) put kTile - 192 bytes each
                    const uint8_t* pl = peer_st[p] + planes_off(n) + 192ull * t;
                    const uint8_t* ex = peer_esc[p] + e + wave * (kTile - kUncodedPlaneBytes);
                    const uint32_t m = uint32_t(min<uint64_t>(kTile, n - uint64_t(t) * kTile));
#pragma unroll 1
                    for (uint32_t k = lane; k < m; k += 64)
                        esc_lds[k] = rotr1_byte(k < kUncodedPlaneBytes ? pl[k] : ex[k - kUncodedPlaneBytes]);
                } else {
                    const uint8_t* esc = peer_esc[p] + e + before[p];
#pragma unroll 1
                    for (uint32_t k = lane; k < mine[p]; k += 64) esc_lds[k] = rotr1_byte(esc[k]);
                }
                wave_lds_sync();
                // an uncoded tile decodes as if every value escaped: codes 0, this lane's
                // exponents at 8 * lane
                add_lane(acc, decode_lane<true>(unc ? 0u : rows[p], unc ? valid_flags(nvalid) : zf[p], s_A[wave][p][lane],
                                          s_peer[p].tlo, s_peer[p].thi, unc ? 8 * lane : rank[p], esc_lds));
            } else {
                add_lane(acc, decode_lane<true>(rows[p], zf[p], s_A[wave][p][lane], s_peer[p].tlo, s_peer[p].thi, rank[p],
                                          s_blk[p] + before[p]));
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
    }
    if (bad) {
        if (lane == 0 && wave == 0) or_status(a.status, ZIPCCL_STATUS_CORRUPT);
        return;
    }
    if (nvalid == 0) return;
    // one rounding per value (RNE), NaN -> 0x7FC0; the fix-up only runs in a lane that
    // holds a NaN
    uint32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; q++) r[q] = pack_bf16x2_rne(acc[2 * q], acc[2 * q + 1]);
    if (nan_halves(r[0]) | nan_halves(r[1]) | nan_halves(r[2]) | nan_halves(r[3])) {
#pragma unroll
        for (int q = 0; q < 4; q++) r[q] = fix_nan_bf16x2(r[q]);
    }
    if (nvalid == 8) {
        store_nt(reinterpret_cast<uint4*>(dst + i0), make_uint4(r[0], r[1], r[2], r[3]));
    } else {
        for (uint32_t j = 0; j < nvalid; j++) dst[i0 + j] = uint16_t(r[j >> 1] >> (16 * (j & 1)));
    }
}

// Decompress: one workgroup per block, one half block (4 tiles) per wave, as in the
// encoder.  Each wave requests the A bytes and one plane dword per lane of its 4 tiles
// at once, turns the planes back into per-lane rows with the half-wave bit transpose
// (its own inverse), ranks its escapes, learns through one barrier how many escapes the
// first half of its block holds, then fetches its half block's escapes and writes its
// 2048 values.  Workgroups of one block (rather than 4) shorten the launch's last
// generation: the bucket decompress took 3 % less time.
constexpr uint32_t kDecHalfTiles = 4;
constexpr uint32_t kDecWaves = 2;                       // the two half blocks of one block
constexpr uint32_t kDecThreads = 64 * kDecWaves;

__global__ __launch_bounds__(kDecThreads) void decompress_kernel(const DArgs a)
{
    __shared__ uint32_t s_cnt[kDecWaves];
    __shared__ uint8_t s_esc[kDecWaves][kHalf + kEscPad];
    const uint32_t lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t unit = blockIdx.x;
    const int s = find_segment_wave<&DSeg::unit0>(a.seg, a.nseg, unit);
    const DSeg& sg = a.seg[s];
    const uint32_t n = sg.n;
    const uint32_t T = uint32_t(tiles_of(n)), K = uint32_t(blocks_of(n));
    const uint32_t hb = (unit - sg.unit0) * kDecWaves + wave;   // half block within the segment
    const uint32_t b = hb >> 1, half = hb & 1;
    const bool active = b < K;
    const bool full = uint64_t(hb + 1) * kHalf <= n;          // all 2048 values exist
    const uint32_t pdw = decoder_plane_dword(lane);
    const uint8_t* st = sg.src;

    // A and plane addresses follow from n alone, so these loads are issued before (and
    // independently of) the header checks; escapes are read only once the header and
    // offset table have been validated.  Every wave issues the same loads, plane dwords
    // first, in straight-line code (tiles past the segment's last re-read it, lanes with
    // no plane dword read dword 0), so each transpose waits only for its own dword.
    const uint32_t T1 = T - 1;   // n >= 1: a segment with no values has no units
    const uint32_t pdl = pdw == ~0u ? 0u : 4 * pdw;   // byte offset
    uint2 Ap[kDecHalfTiles];
    uint32_t pw[kDecHalfTiles];
#pragma unroll
    for (int k = 0; k < int(kDecHalfTiles); k++) {
        const uint32_t t = min(hb * kDecHalfTiles + k, T1);
        pw[k] = load_nt(reinterpret_cast<const uint32_t*>(st + planes_off(n) + 192ull * t + pdl));
    }
#pragma unroll
    for (int k = 0; k < int(kDecHalfTiles); k++) {
        const uint32_t t = min(hb * kDecHalfTiles + k, T1);
        Ap[k] = load_nt(reinterpret_cast<const uint2*>(st + 128 + 512ull * t + 8 * lane));
    }
    bool bad = false;
    uint32_t first = 0, last = 0;
    SegHeader hd = {};
    if (active) {
        hd = read_header(st, n, sg.esc_bytes, sg.esc_at_first != 0);
        const uint32_t* C = reinterpret_cast<const uint32_t*>(st + offsets_off(n));
        bad = !hd.ok || !block_escapes(C, b, K, hd.n_esc, min(kBlock, n - b * kBlock), first, last);
    }
    if (active && !bad && last > first && last - first == block_overflow(n, b)) {
        // rare: an uncoded block (a coded one puts fewer bytes in the escape buffer).  Both
        // waves of the workgroup hold the same block, so both take this path (and neither
        // reaches the barrier below).
        const uint8_t* esc = sg.esc + hd.esc_offset + first + (half ? half_overflow(n, 2 * b) : 0u);
#pragma unroll
        for (int k = 0; k < int(kDecHalfTiles); k++) {
            const uint32_t t = hb * kDecHalfTiles + k;
            const uint64_t i0 = uint64_t(t) * kTile + 8ull * lane;
            const uint32_t nvalid = (t >= T || i0 >= n) ? 0u : uint32_t(min<uint64_t>(8, n - i0));
            const uint2 E = t < T ? uncoded_exponents(st + planes_off(n) + 192ull * t, esc + k * (kTile - kUncodedPlaneBytes),
                                                      lane, nvalid)
                                  : make_uint2(0, 0);
            if (nvalid == 0) continue;
            const LaneBytes y = assemble_lane(Ap[k], E.x, E.y);
            const uint32_t ov[4] = {perm(y.hi0, y.lo0, 0x05010400u), perm(y.hi0, y.lo0, 0x07030602u),
                                    perm(y.hi1, y.lo1, 0x05010400u), perm(y.hi1, y.lo1, 0x07030602u)};
            if (nvalid == 8) store_nt(reinterpret_cast<uint4*>(sg.dst + i0), make_uint4(ov[0], ov[1], ov[2], ov[3]));
            else
                for (uint32_t j = 0; j < nvalid; j++) sg.dst[i0 + j] = uint16_t(ov[j >> 1] >> (16 * (j & 1)));
        }
        return;
    }
    // rows, escape flags and the ranks of this lane's escapes within the half block
    const Transpose32 tc = transpose_consts(lane);
    uint32_t rows[kDecHalfTiles], zf[kDecHalfTiles], cnt[kDecHalfTiles], start[kDecHalfTiles];
#pragma unroll
    for (int k = 0; k < int(kDecHalfTiles); k++) {
        uint32_t vf = 0x11111111u;
        if (!full) {
            const uint32_t t = hb * kDecHalfTiles + k;
            const uint64_t i0 = uint64_t(t) * kTile + 8ull * lane;
            vf = valid_flags((!active || t >= T || i0 >= n) ? 0u : uint32_t(min<uint64_t>(8, n - i0)));
        }
        rows[k] = transpose32(pw[k], tc);
        zf[k] = escape_flags(rows[k], vf);
        cnt[k] = __builtin_popcount(zf[k]);
    }
    const uint32_t half_total = half_ranks(cnt, start);
    if (lane == 0) s_cnt[wave] = half_total;
    __syncthreads();
    if (!active) return;
    const uint32_t other = s_cnt[wave ^ 1u];
    const uint32_t half_start = half ? other : 0u;
    bad = bad || half_total + other != last - first;   // the offset table must agree with the planes
    if (bad) {
        if (lane == 0) or_status(a.status, ZIPCCL_STATUS_CORRUPT);
        return;
    }
    // every lane of the wave helps stage the half block's escapes: 4 bytes per lane in
    // flight per round of 256 (indexes past the last escape re-read it), so that a half
    // block with up to 256 escapes waits for one memory round trip rather than one per 64
    const uint8_t* esc = sg.esc + hd.esc_offset + first + half_start;
    uint8_t* esc_lds = s_esc[wave];
    for (uint32_t k0 = 0; k0 < half_total; k0 += 256) {
        uint32_t x[4];
#pragma unroll
        for (uint32_t j = 0; j < 4; j++) x[j] = esc[min(k0 + 64 * j + lane, half_total - 1)];
#pragma unroll
        for (uint32_t j = 0; j < 4; j++)
            if (k0 + 64 * j + lane < half_total) esc_lds[k0 + 64 * j + lane] = uint8_t(x[j]);
    }
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < int(kDecHalfTiles); k++) {
        const uint32_t t = hb * kDecHalfTiles + k;
        const uint64_t i0 = uint64_t(t) * kTile + 8ull * lane;
        const uint32_t nvalid = (t >= T || i0 >= n) ? 0u : uint32_t(min<uint64_t>(8, n - i0));
        if (nvalid == 0) continue;
        const LaneBytes y = decode_lane(rows[k], zf[k], Ap[k], hd.tlo, hd.thi, start[k], esc_lds);
        uint4 o;
        o.x = perm(y.hi0, y.lo0, 0x05010400u);
        o.y = perm(y.hi0, y.lo0, 0x07030602u);
        o.z = perm(y.hi1, y.lo1, 0x05010400u);
        o.w = perm(y.hi1, y.lo1, 0x07030602u);
        if (nvalid == 8) {
            store_nt(reinterpret_cast<uint4*>(sg.dst + i0), o);
        } else {
            const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
            for (uint32_t j = 0; j < nvalid; j++) sg.dst[i0 + j] = uint16_t(ov[j >> 1] >> (16 * (j & 1)));
        }
    }
}

}  // namespace

hipError_t launch_compress(const CArgs& a, hipStream_t s, bool single)
{
    if (single && a.direct) {
        const uint32_t groups = (a.total_units + kPlaceUnits - 1) / kPlaceUnits;
        hipLaunchKernelGGL(compress_single_kernel, dim3(a.total_units + groups), dim3(kEncThreads), 0, s, a);
        return hipGetLastError();
    }
    if (a.total_units > 0) hipLaunchKernelGGL(encode_kernel, dim3(a.total_units), dim3(kEncThreads), 0, s, a);
    if (a.direct) {
        hipLaunchKernelGGL(place_direct_kernel, dim3((a.total_units + kPlaceUnits - 1) / kPlaceUnits),
                           dim3(kPlaceThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
        if (a.total_blocks > 0)
            hipLaunchKernelGGL(place_kernel, dim3((a.total_blocks + kWaves - 1) / kWaves), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

// --------------------------------------------------------------------------------
// workspace of the no-allocation compress
// --------------------------------------------------------------------------------
// For callers that cannot allocate device memory: the compress workspace as a
// file-scope device array.  Each GPU the library runs on holds its own copy from the time
// the library's code is loaded on it until the process ends; every call on that GPU
// shares it.  In host code `scratch` is only a handle for the runtime, not a device
// address: the address that kernels are given comes from hipGetSymbolAddress, looked up
// once per device with that device current, and kept.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

hipError_t noalloc_workspace(hipStream_t stream, void** out)
{
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

// --------------------------------------------------------------------------------
// plans from the data: sigma estimated on the device
// --------------------------------------------------------------------------------
// The sample is every stride-th tile of 512 values: sample k is tile k * stride.  Each
// segment is split over kEstParts workgroups of 4 waves; part p takes samples p, p + 16,
// p + 32, ...; its wave w takes that list's entries w, w + 4, ..., 8 of them at a time,
// lane l the 16 bytes of values 8l .. 8l + 7 (one coalesced 1 KB load per wave and
// sample).  Each thread sums, in fp64, the squares of its finite values and counts them;
// the workgroup adds its 256 partial sums in a fixed order and stores (sum, count) in the
// caller's scratch.  A second launch adds each segment's 16 pairs in part order, so the
// estimate is the same on every run.  sigma = sqrt(sum / count) (the model's mean is 0;
// no finite sample, or sigma 0, counts as sigma 1), then the plan's closed form:
// e0 = 123 + floor(log2(sigma) - c), clamped to 1..248, table e0 .. e0 + 6.
constexpr uint32_t kEstThreads = 256;
constexpr uint32_t kEstWaves = kEstThreads / 64;
constexpr uint32_t kEstBatch = 8;   // samples in flight per wave
constexpr double kSwitchPhaseDev = 0.7195805543641254;   // where the 7-binade window moves up

namespace {

__global__ __launch_bounds__(kEstThreads) void estimate_partial_kernel(const EArgs a)
{
    __shared__ double s_sum[kEstThreads];
    __shared__ uint32_t s_cnt[kEstThreads];
    const uint32_t tid = threadIdx.x, lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t s = blockIdx.x / kEstParts, part = blockIdx.x % kEstParts;
    const uint16_t* src = a.src[s];
    const uint32_t n = a.n[s];
    const uint64_t T = tiles_of(n);
    double sum = 0.0;
    uint32_t cnt = 0;
    for (uint64_t j0 = wave; (part + uint64_t(kEstParts) * j0) * a.stride < T; j0 += uint64_t(kEstBatch) * kEstWaves) {
        uint4 v[kEstBatch];
#pragma unroll
        for (uint32_t b = 0; b < kEstBatch; b++) {
            const uint64_t k = part + uint64_t(kEstParts) * (j0 + uint64_t(b) * kEstWaves);
            const uint64_t i = k * a.stride * kTile + 8ull * lane;
            if (i + 8 <= n) {
                v[b] = load_nt(reinterpret_cast<const uint4*>(src + i));
            } else {   // the segment's ragged end, or past it: missing values read as NaN
                uint32_t w[4];
                for (uint32_t j = 0; j < 4; j++) {
                    const uint64_t q = i + 2 * j;
                    w[j] = (q < n ? uint32_t(src[q]) : 0x7FC0u) | (q + 1 < n ? uint32_t(src[q + 1]) << 16 : 0x7FC00000u);
                }
                v[b] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
#pragma unroll
        for (uint32_t b = 0; b < kEstBatch; b++) {
            const uint32_t w[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float f = __uint_as_float((j & 1) ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16));
                if (__builtin_isfinite(f)) {
                    const double d = double(f);
                    sum += d * d;
                    cnt++;
                }
            }
        }
    }
    s_sum[tid] = sum;
    s_cnt[tid] = cnt;
    __syncthreads();
    for (uint32_t h = kEstThreads / 2; h > 0; h >>= 1) {
        if (tid < h) {
            s_sum[tid] += s_sum[tid + h];
            s_cnt[tid] += s_cnt[tid + h];
        }
        __syncthreads();
    }
    if (tid == 0) {
        double* out = a.partial + 2 * (uint64_t(s) * kEstParts + part);
        out[0] = s_sum[0];
        out[1] = double(s_cnt[0]);
    }
}

// One thread per segment: the 16 partial pairs in part order, then the plan.
__global__ __launch_bounds__(64) void estimate_finish_kernel(const EArgs a)
{
    const uint32_t s = threadIdx.x;
    if (s >= uint32_t(a.nseg)) return;
    const double* in = a.partial + 2 * uint64_t(s) * kEstParts;
    double sum = 0.0, cnt = 0.0;
    for (uint32_t p = 0; p < kEstParts; p++) {
        sum += in[2 * p];
        cnt += in[2 * p + 1];
    }
    double sigma = cnt > 0.0 ? sqrt(sum / cnt) : 1.0;
    if (!(sigma > 0.0) || !__builtin_isfinite(sigma)) sigma = 1.0;
    const double e = 123.0 + floor(log2(sigma) - kSwitchPhaseDev);
    const uint32_t e0 = uint32_t(fmin(248.0, fmax(1.0, e)));
    const uint32_t lo = e0 | (e0 + 1) << 8 | (e0 + 2) << 16 | (e0 + 3) << 24;
    const uint32_t hi = (e0 + 4) | (e0 + 5) << 8 | (e0 + 6) << 16;
    reinterpret_cast<uint2*>(a.plans)[s] = make_uint2(lo, hi);
}

}  // namespace

static_assert(kMaxSegs <= 64, "the finishing launch takes one thread per segment");

hipError_t launch_estimate_plans(const EArgs& a, hipStream_t s)
{
    if (a.nseg < 1) return hipSuccess;
    hipLaunchKernelGGL(estimate_partial_kernel, dim3(a.nseg * kEstParts), dim3(kEstThreads), 0, s, a);
    hipLaunchKernelGGL(estimate_finish_kernel, dim3(1), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decompress(const DArgs& a, hipStream_t s)
{
    if (a.total_units == 0) return hipSuccess;
    hipLaunchKernelGGL(decompress_kernel, dim3(a.total_units), dim3(kDecThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_accumulate(const AArgs& a, hipStream_t s)
{
    if (a.n == 0 || a.nchunks < 1) return hipSuccess;
    // one grid row per chunk; a row holds a full chunk's blocks (the last chunk's surplus
    // workgroups return at once)
    const dim3 grid(uint32_t(blocks_of(a.nchunks > 1 ? a.chunk : a.n)), uint32_t(a.nchunks));
    // every peer slot of the instance issues its loads, so up to 8 peers the instance
    // holds exactly npeers
    switch (a.npeers) {
        case 1: hipLaunchKernelGGL(accumulate_kernel<1>, grid, dim3(kAccThreads), 0, s, a); break;
        case 2: hipLaunchKernelGGL(accumulate_kernel<2>, grid, dim3(kAccThreads), 0, s, a); break;
        case 3: hipLaunchKernelGGL(accumulate_kernel<3>, grid, dim3(kAccThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL(accumulate_kernel<4>, grid, dim3(kAccThreads), 0, s, a); break;
        case 5: hipLaunchKernelGGL(accumulate_kernel<5>, grid, dim3(kAccThreads), 0, s, a); break;
        case 6: hipLaunchKernelGGL(accumulate_kernel<6>, grid, dim3(kAccThreads), 0, s, a); break;
        case 7: hipLaunchKernelGGL(accumulate_kernel<7>, grid, dim3(kAccThreads), 0, s, a); break;
        case 8: hipLaunchKernelGGL(accumulate_kernel<8>, grid, dim3(kAccThreads), 0, s, a); break;
        default: hipLaunchKernelGGL(accumulate_kernel<kMaxPeers>, grid, dim3(kAccThreads), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace zc
