/*
 * zipccl.h -- C ABI of the lossless BF16 exponent codec for AMD Instinct MI355X
 * (gfx950).
 *
 * The codec follows "ZipCCL: Efficient Lossless Data Compression of Communication
 * Collectives for Accelerating LLM Training" (gist.science explanation page):
 *   S2.A  a table of the 7 most frequent exponents predicted from the tensor's
 *         standard deviation sigma with a Gaussian model, no online histogram;
 *   S2.B  each BF16 value is split into a sign+mantissa byte and an 8-bit exponent;
 *         a table exponent becomes a 3-bit code 001..111, any other exponent the
 *         escape code 000 with the full exponent appended to a separate array;
 *   S2.C  sections padded to 128 bytes; the 3-bit codes stored as three 1-bit planes;
 *   S2.D  the reduce-scatter receive side decodes and reduces locally;
 *   S4    the all-gather measured there: one compressed shard per rank, decoded by all.
 *
 * Compressed format, version 1 (all integers little-endian).  One segment of n values,
 * T = ceil(n/512) tiles, K = ceil(n/4096) blocks, R128 = round up to 128:
 *   [0,128)   header: u32 magic 0x3143435A, u16 version 1, u16 flags 0, u64 n,
 *             u8 table[7] (ascending), u8 0, u32 4096, u32 512, u64 n_esc,
 *             u64 esc_offset, u64 static_bytes, u64 0, 64 zero bytes
 *   A         512*T bytes: A[i] = sign << 7 | 7-bit mantissa of value i (0 past n)
 *   B         R128(192*T) bytes: u64 plane word 24*t + 8*p + j holds, in bit l,
 *             bit p of the code of value 512*t + 8*l + j (0 past n)
 *   C         R128(4*K) bytes: u32 off[b] = escape-buffer bytes of blocks 0..b-1
 *   static_bytes = 128 + 512*T + R128(192*T) + R128(4*K)
 * Escapes: one exponent byte per code-0 value, in index order, stored in a separate
 * escape buffer from byte esc_offset on.  code(e) = 1 + rank of e in the ascending
 * table, 0 if e is not in it; exponents 0 and 255 are never in a table.
 * Uncoded blocks, the fallback to no compression (CCCL page: adaptive compression
 * strategy; fall back when the ratio reaches 1): a tile of m values overflows
 * max(0, m - 192) values (those past the 192 its plane bytes can hold), a block the sum
 * over its tiles (2560 for 4096 values).  A block with overflow O > 0 whose code-0 values
 * number at least O is stored uncoded: A as usual; the 192 plane bytes of each tile hold
 * the exponents of its first 192 values (0 past the tile's end); the exponents of its
 * other values go to the escape buffer, tile after tile.  off[] and n_esc count escape-
 * buffer bytes, so an uncoded block has exactly O of them and a coded block fewer.
 * Random bits thus take 2n bytes plus header and offsets instead of about 2.38n.
 *
 * Conventions.
 *   - All data pointers are device pointers unless stated.  The caller owns every
 *     buffer; the library allocates no device memory.  Its only global state is the
 *     static workspace of zipccl_compress_noalloc (one per device, with its address
 *     looked up once per device).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only enqueues
 *     work on it and returns; nothing synchronises the host.
 *   - Argument errors are returned before anything is enqueued.  Data-dependent
 *     conditions found on the device are OR-ed into the optional device word
 *     `status` (ZIPCCL_STATUS_*); kernels never trap.
 *   - BF16 pointers must be 16-byte aligned, static sections 128-byte aligned.
 *   - One call may hold at most ZIPCCL_MAX_SEGMENTS segments and fewer than 2^32
 *     values in total.
 */
#ifndef ZIPCCL_H
#define ZIPCCL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZIPCCL_FORMAT_VERSION 1
#define ZIPCCL_MAGIC 0x3143435Au
#define ZIPCCL_MAX_SEGMENTS 64
#define ZIPCCL_MAX_PEERS 16

typedef enum zipccl_status {
    ZIPCCL_OK = 0,
    ZIPCCL_ERR_INVALID = 1,   /* bad argument: NULL pointer, bad sigma or table, nseg range */
    ZIPCCL_ERR_ALIGN = 2,     /* a pointer is not aligned as required */
    ZIPCCL_ERR_SIZE = 3,      /* a size limit is exceeded or a buffer is too small */
    ZIPCCL_ERR_HIP = 4,       /* the HIP runtime reported an error */
    ZIPCCL_ERR_CORRUPT = 5    /* a host-side check of device results failed (zipccl_profile_codec) */
} zipccl_status;

/* Bits OR-ed into the optional device status word. */
#define ZIPCCL_STATUS_ESC_OVERFLOW 1u  /* escapes did not fit esc_cap; those past it were dropped */
#define ZIPCCL_STATUS_CORRUPT 2u       /* decode: header or offset table inconsistent; not decoded */
#define ZIPCCL_STATUS_BAD_INDEX 4u     /* gathered compress: a row index outside the matrix (row 0 was read) */
#define ZIPCCL_STATUS_WAIT_LIMIT 8u    /* compress: a placing workgroup gave up waiting for an encoder's
                                          count (bounded wait); that unit's escapes, offsets and headers
                                          were not written */

/* A coding plan: 7 distinct exponents in 1..254, ascending; code(table[r]) = r + 1. */
typedef struct zipccl_plan_t {
    uint8_t table[7];
    uint8_t reserved; /* 0 */
} zipccl_plan_t;

/* One segment to compress: n BF16 values at src (device, 16-byte aligned). */
typedef struct zipccl_segment_t {
    const void* src;
    uint64_t n;
    zipccl_plan_t plan;
} zipccl_segment_t;

/* One segment to decompress: n values written to dst (device, 16-byte aligned). */
typedef struct zipccl_dsegment_t {
    void* dst;
    uint64_t n;
} zipccl_dsegment_t;

/* Plan (S2.A).  With table7 == NULL: the 7 exponents whose binades hold the most
 * mass of N(0, sigma^2), a contiguous window e0..e0+6 with
 * e0 = 123 + floor(log2(sigma) - 0.7195805543641254) clamped to 1..248 (the phase
 * constant is where the lowest and the next binade above the window carry equal
 * mass).  sigma must be finite and > 0.  With table7 != NULL: those 7 exponents
 * (distinct, 1..254) sorted ascending; sigma is ignored.  Host only.
 * Returns ZIPCCL_ERR_INVALID on a bad sigma or table, or a NULL out. */
zipccl_status zipccl_plan(double sigma, const uint8_t* table7, zipccl_plan_t* out);

/* Plans for n tensors at once (S2.A): out[i] = zipccl_plan(sigma[i], NULL, ...).  sigma
 * and out are host arrays of n entries (n >= 0).  On a bad sigma returns
 * ZIPCCL_ERR_INVALID; out[i] is then written for the sigmas before it only.  Host only. */
zipccl_status zipccl_plan_many(const double* sigma, int n, zipccl_plan_t* out);

/* Bytes of the fixed-size part of one segment of n values (format above). */
uint64_t zipccl_static_size(uint64_t n);

/* static_size(n) + n_esc: the whole compressed size of one segment (S2.B: 11 bits per
 * value plus 8 bits per escape-buffer byte plus metadata).  The escape-buffer bytes of a
 * segment never exceed its values (n_esc = n is a safe capacity); with uncoded blocks
 * they are at most 5n/8 + 192. */
uint64_t zipccl_compressed_size(uint64_t n, uint64_t n_esc);

/* Device workspace bytes needed by zipccl_compress for up to nseg segments holding
 * at most total_n values (about one byte per value: a 4-byte escape count per 2048-value
 * half block and a 16384-byte escape staging area per 16384 values).  The workspace
 * carries nothing from one call to the next and needs no initialisation (each call tags
 * what it publishes there with a value no earlier call in the process used); it must be
 * 256-byte aligned.
 * Calls that run concurrently need separate workspaces. */
uint64_t zipccl_workspace_size(uint64_t total_n, int nseg);

/* Compress nseg segments in one launch (S2.B, S2.C; two-phase layout of S2.D).
 *   static_out  device, 128-byte aligned, static_cap bytes >= sum of static_size(n_s);
 *               segment s is written at the sum of the static sizes before it.
 *   esc_out     device, esc_cap bytes; escapes of segment s follow those of segments
 *               0..s-1; header field esc_offset records where they start.  Escapes
 *               beyond esc_cap are dropped and ZIPCCL_STATUS_ESC_OVERFLOW is set; the
 *               headers still carry the true counts.
 *   workspace   device scratch, see zipccl_workspace_size.
 * With a status word the work is one kernel launch on `stream`: its encoding
 * workgroups write the fixed-size sections, stage each unit's escapes and publish the
 * unit's escape count in the workspace; its placing workgroups, each behind the encoders
 * of the units it places in the launch's grid, compute the escape positions from those
 * counts (bounded wait; a wait that runs out sets ZIPCCL_STATUS_WAIT_LIMIT), write the
 * offset tables and headers and compact the escapes.  Without a status word,
 * while `stream` is being captured into a graph, or with ZIPCCL_SINGLE_LAUNCH=0 in the
 * environment, the same work is two launches (encode, then place) in which nothing
 * waits, so nothing can time out unreported; above 2^28 values in one call it is encode,
 * a one-workgroup scan launch, then place.
 *   n_esc_out   optional device u64[nseg + 1]: per-segment escape counts, then the total.
 *   status      optional device u32, bits OR-ed in (NULL: the two-launch path).
 * Errors: INVALID (NULL pointers, nseg outside 1..ZIPCCL_MAX_SEGMENTS, bad table),
 * ALIGN, SIZE (segment n >= 2^32, sum >= 2^32, static_cap or workspace too small),
 * HIP (launch failure). */
zipccl_status zipccl_compress(const zipccl_segment_t* segs, int nseg, void* static_out, uint64_t static_cap,
                              void* esc_out, uint64_t esc_cap, void* workspace, uint64_t workspace_bytes,
                              uint64_t* n_esc_out, uint32_t* status, void* stream);

/* zipccl_compress for callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same outputs,
 * launches and errors, with the workspace taken from a static device array inside the
 * library (ZIPCCL_NOALLOC_SCRATCH_BYTES = 68 474 112 bytes, held by each GPU the library
 * runs on until the process ends) instead of a caller buffer.  The call allocates nothing;
 * its first call on a device looks the array's address up.  At most
 * ZIPCCL_NOALLOC_MAX_VALUES values in total per call; more returns ZIPCCL_ERR_SIZE before
 * anything is enqueued.  Every call on one GPU uses the same array: calls on one GPU that
 * can overlap (on different streams, or from different host threads) race and must be
 * ordered by the caller.  The array keeps what the last call left; no call depends on it.
 * Errors: as zipccl_compress (INVALID, ALIGN, SIZE, HIP). */
#define ZIPCCL_NOALLOC_MAX_VALUES (1ull << 26)
#define ZIPCCL_NOALLOC_SCRATCH_BYTES 68474112ull
zipccl_status zipccl_compress_noalloc(const zipccl_segment_t* segs, int nseg, void* static_out, uint64_t static_cap,
                                      void* esc_out, uint64_t esc_cap, uint64_t* n_esc_out, uint32_t* status,
                                      void* stream);

/* Device scratch bytes zipccl_estimate_plans needs for nseg segments (16 partial sums of
 * 16 bytes per segment). */
uint64_t zipccl_estimate_workspace_size(int nseg);

/* Plans estimated on the device, for tensors whose sigma the caller does not know
 * (S2.A's Gaussian model; the pages derive sigma from the layer's weights instead): for
 * each segment, sigma = sqrt(mean of x^2) over the finite values of every stride-th tile
 * of 512 values (tiles k * stride, k = 0, 1, ...), summed in fp64 in a fixed order (16
 * workgroups per segment each add their share, a second launch adds the 16 partial sums
 * in order), then the table of zipccl_plan(sigma, NULL) (no finite value, or sigma 0:
 * sigma = 1) written to plans_dev[s].  segs[s].plan is ignored.  Two launches on
 * `stream`; nothing returns to the host, and the result is the same on every run.
 *   plans_dev   device, 8-byte aligned, nseg entries
 *   workspace   device scratch, 16-byte aligned, zipccl_estimate_workspace_size(nseg) bytes
 * Errors: INVALID (NULL pointers with n > 0, nseg outside 1..ZIPCCL_MAX_SEGMENTS,
 * stride 0), ALIGN, SIZE (n >= 2^32, workspace too small), HIP. */
zipccl_status zipccl_estimate_plans(const zipccl_segment_t* segs, int nseg, uint32_t stride, zipccl_plan_t* plans_dev,
                                    void* workspace, uint64_t workspace_bytes, void* stream);

/* zipccl_compress with segment s coded by the plan in device memory at plans_dev[s]
 * (written by zipccl_estimate_plans, or by the caller: 7 distinct ascending exponents in
 * 1..254, then a zero byte) instead of segs[s].plan.  Same outputs and errors as
 * zipccl_compress; ALIGN also for plans_dev not 8-byte aligned.  A device plan that is not
 * a valid table gives a segment whose header the decoders reject. */
zipccl_status zipccl_compress_device_plans(const zipccl_segment_t* segs, int nseg, const zipccl_plan_t* plans_dev,
                                           void* static_out, uint64_t static_cap, void* esc_out, uint64_t esc_cap,
                                           void* workspace, uint64_t workspace_bytes, uint64_t* n_esc_out,
                                           uint32_t* status, void* stream);

/* A sequence of nchunks independent compress calls on one stream, as the chunked
 * pipeline of the CCCL page's pipeline section issues them: chunk k is what
 *   zipccl_compress(segs + k * nseg, nseg, static_out[k], static_cap[k], esc_out[k],
 *                   esc_cap[k], ..., n_esc_out + k * (nseg + 1), status, stream)
 * writes, byte for byte (each chunk's escapes and esc_offsets are its own), but
 * consecutive chunks share a kernel launch (up to 16 chunks and 128 segments per launch)
 * while the workspace holds them all, so that a launch has enough work to fill the GPU.
 * A chunk of more than 2^28 values has a launch of its own.
 *   segs        host array of nchunks * nseg segments, chunk after chunk; 1 <= nseg <=
 *               ZIPCCL_MAX_PEERS
 *   static_out, static_cap, esc_out, esc_cap   host arrays of nchunks entries
 *   workspace   device, 256-byte aligned, at least zipccl_workspace_size(v, nseg) bytes
 *               where v is the most values in one chunk; chunks k .. j share a launch
 *               when it holds zipccl_workspace_size(their values, their segments)
 *   n_esc_out   optional device u64[nchunks * (nseg + 1)]
 * Every chunk is checked before anything is enqueued.  nchunks == 0 does nothing.
 * Errors: as zipccl_compress, per chunk; INVALID also for nseg outside 1..ZIPCCL_MAX_PEERS
 * or nchunks < 0. */
zipccl_status zipccl_compress_chunks(const zipccl_segment_t* segs, int nseg, int nchunks, void* const* static_out,
                                     const uint64_t* static_cap, void* const* esc_out, const uint64_t* esc_cap,
                                     void* workspace, uint64_t workspace_bytes, uint64_t* n_esc_out,
                                     uint32_t* status, void* stream);

/* One segment whose values are rows of a row-major BF16 matrix picked by index: the
 * MoE all-to-all dispatch payload of one destination (S2.D), compressed where the
 * tokens lie instead of after a permute copy.  The segment's values are rows
 * rows[0], rows[1], ..., rows[nrows - 1] of src, each row_len values, in that order
 * (n = nrows * row_len); its compressed form is the one zipccl_compress gives for those
 * values laid out contiguously.
 *   src       device, 16-byte aligned: the matrix, src_rows rows of row_len values
 *   rows      device, 4-byte aligned: nrows row indices; an index outside [0, src_rows)
 *             sets ZIPCCL_STATUS_BAD_INDEX and row 0 is read in its place
 *   row_len   a multiple of 8, at least 512 */
typedef struct zipccl_gather_segment_t {
    const void* src;
    uint64_t src_rows;
    uint64_t row_len;
    const int32_t* rows;
    uint64_t nrows;
    zipccl_plan_t plan;
} zipccl_gather_segment_t;

/* zipccl_compress over gathered segments: the same outputs, layout, workspace and
 * launches (the encoder reads each tile's row indices with scalar loads).
 * Errors: as zipccl_compress; INVALID also for row_len not a multiple of 8 or below 512,
 * or NULL src / rows with nrows > 0; ALIGN for rows not 4-byte aligned; SIZE for
 * nrows * row_len >= 2^32 or src_rows >= 2^32. */
zipccl_status zipccl_compress_gather(const zipccl_gather_segment_t* segs, int nseg, void* static_out,
                                     uint64_t static_cap, void* esc_out, uint64_t esc_cap, void* workspace,
                                     uint64_t workspace_bytes, uint64_t* n_esc_out, uint32_t* status, void* stream);

/* Decompress nseg segments whose static parts lie back to back at static_in (as
 * zipccl_compress writes them; static_bytes = their total size) and whose escapes are
 * in esc_in (esc_bytes long; each header's esc_offset is relative to it).  Exact
 * inverse of zipccl_compress.  A segment whose header or offset table is inconsistent
 * with segs[s].n or the buffer sizes is not decoded and ZIPCCL_STATUS_CORRUPT is set;
 * no read leaves the given buffers.
 * Errors: INVALID, ALIGN, SIZE (static_bytes smaller than the segments need), HIP. */
zipccl_status zipccl_decompress(const void* static_in, uint64_t static_bytes, const void* esc_in,
                                uint64_t esc_bytes, const zipccl_dsegment_t* segs, int nseg,
                                uint32_t* status, void* stream);

/* All-gather receive side (the all-gather measurement of S4; each rank's shard is
 * compressed once and every receiver decodes all of them): decodes nseg one-segment
 * compressed shards that lie in separate buffers, in one launch, to segs[s].dst (the
 * slices of the gathered tensor).  static_in, esc_in and esc_bytes are host arrays of
 * nseg entries: static_in[s] is the shard's static part (device, 128-byte aligned,
 * static_size(segs[s].n) bytes as zipccl_compress wrote it) and esc_in[s] (esc_bytes[s]
 * long, NULL when 0) the escape buffer its header's esc_offset refers to, or, with
 * ZIPCCL_SHARDS_ESC_AT_FIRST in flags, a buffer that starts at the shard's first escape
 * (the two-phase all-to-all of S2.D: a receiver gets each sender's static part and that
 * segment's escape bytes, esc_offset .. esc_offset + n_esc of the sender's escape buffer,
 * and keeps them on their own).  A shard whose header or offset table is inconsistent
 * with segs[s].n or esc_bytes[s] is not decoded and ZIPCCL_STATUS_CORRUPT is set; no read
 * leaves the given buffers.
 * Errors: INVALID (NULL arrays or pointers, nseg outside 1..ZIPCCL_MAX_SEGMENTS, unknown
 * flags), ALIGN, SIZE (a segment n >= 2^32), HIP. */
#define ZIPCCL_SHARDS_ESC_AT_FIRST 1u
zipccl_status zipccl_decompress_shards(const void* const* static_in, const void* const* esc_in,
                                       const uint64_t* esc_bytes, const zipccl_dsegment_t* segs, int nseg,
                                       uint32_t flags, uint32_t* status, void* stream);

/* Reduce-scatter receive side (S2.D): for i < n
 *   dst[i] = bf16_rne( (((f32(local[i]) + f32(peer_0[i])) + f32(peer_1[i])) + ...) )
 * where peer_p is the one-segment compressed shard at static_in[p] with escapes in
 * esc_in[p] (esc_bytes[p] long), each of n values; fp32 additions in peer order
 * 0..npeers-1, round to nearest even, subnormals kept, one rounding to BF16 at the end
 * (a NaN sum gives 0x7FC0).  static_in, esc_in and esc_bytes are host arrays of
 * npeers entries (1..ZIPCCL_MAX_PEERS).  dst may equal local.  A corrupt shard sets
 * ZIPCCL_STATUS_CORRUPT and its blocks are left unwritten.
 * Errors: INVALID, ALIGN, SIZE (n >= 2^32), HIP. */
zipccl_status zipccl_decompress_accumulate(const void* const* static_in, const void* const* esc_in,
                                           const uint64_t* esc_bytes, int npeers, uint64_t n,
                                           const void* local, void* dst, uint32_t* status, void* stream);

/* zipccl_decompress_accumulate over consecutive chunks, in as few launches as the kernel
 * arguments allow (256 / npeers chunks each): chunk c covers values [c * chunk,
 * min(n, (c + 1) * chunk)) of local and dst, and peer p's compressed segment of it is at
 * static_in[c * npeers + p] with escapes in esc_in[c * npeers + p] (esc_bytes[...] long).
 * The result is that of one zipccl_decompress_accumulate call per chunk.  static_in,
 * esc_in and esc_bytes are host arrays of ceil(n / chunk) * npeers entries; chunk is a
 * multiple of 4096.  Every entry is checked before anything is enqueued; n == 0 does
 * nothing.  Errors: INVALID (npeers outside 1..ZIPCCL_MAX_PEERS, chunk 0 or not a
 * multiple of 4096, NULL pointers), ALIGN, SIZE (n >= 2^32), HIP. */
zipccl_status zipccl_decompress_accumulate_chunks(const void* const* static_in, const void* const* esc_in,
                                                  const uint64_t* esc_bytes, int npeers, uint64_t chunk, uint64_t n,
                                                  const void* local, void* dst, uint32_t* status, void* stream);

/* Chunked two-stream pipeline over a reduce-scatter receive share (S2.D; the chunked
 * multi-stream overlap of the CCCL page's pipeline section).  Chunks of `chunk` values
 * of every peer shard are compressed on stream_a (one compress call per chunk, one
 * segment per peer) and decoded + accumulated into dst on stream_b.  The streams hand
 * chunks over in groups of G (a power of two, at most 16, the smallest with
 * G * npeers * chunk >= 2^27 values, since each event record or wait costs the host
 * microseconds); a ring of two groups of chunk buffers lets group g + 1 compress while
 * group g is reduced.  Each group is compressed by one zipccl_compress_chunks call (its
 * chunks share launches) and reduced by one zipccl_decompress_accumulate_chunks call.
 * The scratch memory is caller-owned device memory of zipccl_pipeline_scratch_size()
 * bytes: a compress workspace for the chunks that share a launch plus 2 * G chunk
 * buffers of npeers * (static_size(chunk) + chunk) bytes.
 * Overlapping transfers of the compressed chunks would sit between the two streams. */
typedef struct zipccl_pipeline zipccl_pipeline;

uint64_t zipccl_pipeline_scratch_size(int npeers, uint64_t chunk);

/* Creates the host-side object (HIP events only; no device allocation).
 * Errors: INVALID (npeers outside 1..ZIPCCL_MAX_PEERS, chunk 0 or not a multiple of
 * 4096, chunk >= 2^32 / npeers, NULL out), ALIGN (scratch not 256-byte aligned),
 * SIZE (scratch too small), HIP. */
zipccl_status zipccl_pipeline_create(int npeers, uint64_t chunk, void* scratch, uint64_t scratch_bytes,
                                     void* stream_a, void* stream_b, zipccl_pipeline** out);

/* dst = bf16_rne(f32(local) + sum_p f32(peer_src[p])) over n values, through the
 * codec, chunk by chunk.  peer_src is a host array of npeers device pointers; plans is
 * a host array of npeers plans.  Inputs must be ready in stream_a's order; dst is
 * complete in stream_b's order when the enqueued work finishes.  dst may equal local.
 * Errors: INVALID, ALIGN, SIZE, HIP. */
zipccl_status zipccl_pipeline_reduce(zipccl_pipeline* pipe, const void* const* peer_src,
                                     const zipccl_plan_t* plans, uint64_t n, const void* local, void* dst,
                                     uint32_t* status);

void zipccl_pipeline_destroy(zipccl_pipeline* pipe);

/* ---- Reduce-scatter switcher (S2.D): profile once, then choose per call ----
 * The pages' switcher measures the cluster at start-up (bandwidth, latency, compression
 * ratio) and then picks, per reduce-scatter, the native collective or the zipped
 * all-to-all followed by the local decode-accumulate.  The pages give no formula; the
 * cost model below is this library's reading of that choice. */
typedef struct zipccl_codec_profile_t {
    double compress_GBps;     /* BF16 bytes compressed per second on this GPU */
    double accumulate_GBps;   /* BF16 bytes of peer shards decoded and accumulated per second */
    double compressed_fraction; /* compressed bytes / BF16 bytes of the sample (below 1 saves) */
} zipccl_codec_profile_t;

typedef struct zipccl_link_t {
    double bw_GBps;           /* bandwidth of one link from this rank */
    double latency_us;        /* per message */
    int links;                /* peers a rank sends to at once (xGMI in one node: 7; a ring: 1) */
} zipccl_link_t;

/* Device scratch bytes zipccl_profile_codec needs for a sample of n values and npeers. */
uint64_t zipccl_profile_scratch_size(uint64_t n, int npeers);

/* Measures this GPU's codec on a caller's sample (device BF16, n values, 16-byte aligned,
 * compressed with `plan`): a compress of npeers segments (all the sample) and a
 * decode-accumulate of npeers peer shards, each timed with HIP events over 3 launches
 * after one warm-up, and the compressed size.  Synchronises `stream` (an initialisation
 * call).  scratch: device, 256-byte aligned, zipccl_profile_scratch_size() bytes; it also
 * holds the status word of the profiled calls.
 * Errors: INVALID (NULL pointers, n == 0, npeers outside 1..ZIPCCL_MAX_PEERS, bad plan),
 * ALIGN, SIZE (n * npeers >= 2^32, scratch too small), HIP, CORRUPT (a profiled call set
 * a device status bit; the profile is not written). */
zipccl_status zipccl_profile_codec(const void* sample, uint64_t n, zipccl_plan_t plan, int npeers, void* scratch,
                                   uint64_t scratch_bytes, void* stream, zipccl_codec_profile_t* out);

/* Chooses for a reduce-scatter of `bytes` BF16 bytes per rank over `ranks` ranks (each
 * rank keeps bytes / ranks).  With shard = bytes / ranks and m = ranks - 1 peers:
 *   native  = ceil(m / links) * (latency + shard / bw)        (the reduction rides along)
 *   zipped  = m * shard / compress + ceil(m / links) * (latency + compressed_fraction * shard / bw)
 *             + m * shard / accumulate
 * use_codec = zipped < native, except that tensors under 1 MiB and compressed fractions of 1 or more
 * always take the native path.  Host only; any output pointer may be NULL.
 * Errors: INVALID (NULL prof or link, ranks < 2, links < 1, non-positive rates). */
zipccl_status zipccl_rs_choose(const zipccl_codec_profile_t* prof, const zipccl_link_t* link, int ranks,
                               uint64_t bytes, int* use_codec, double* native_us, double* zipped_us);

/* Static text for a status code. */
const char* zipccl_strerror(zipccl_status s);

#ifdef __cplusplus
}
#endif

#endif /* ZIPCCL_H */
