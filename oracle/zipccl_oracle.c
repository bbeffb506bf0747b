/*
 * zipccl_oracle.c -- plain, slow, single-threaded CPU reference of the lossless
 * BF16 exponent codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, link or call
 * this file.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or constant generator with the HIP
 * library: every rule below is written out again from the method description.
 *
 * Method source (cited by page and section, never by line):
 *   "ZipCCL: Efficient Lossless Data Compression of Communication Collectives for
 *   Accelerating LLM Training" -- gist.science explanation page.
 *     S2.A  LLM tensors are close to Gaussian; in BF16 the exponent values pile up,
 *           the 7 most frequent exponents cover more than 97 %; the table is derived
 *           from the standard deviation sigma, with no online histogram or sort.
 *     S2.B  split each value into sign+mantissa bits and exponent bits; an exponent
 *           among the top 7 becomes a 3-bit code 001..111; any other exponent gets
 *           the escape code 000 and its full 8-bit exponent goes to a separate array;
 *           16 -> 11 bits.
 *     S2.C  blocks padded to 128-byte boundaries; the 3-bit codes kept as three
 *           separate 1-bit arrays.
 *     S2.D  reduce-scatter: zipped all-to-all followed by a local reduction.
 *
 * The pages do not fix a byte layout.  The layout implemented here is this codec's
 * own reading (format version 1), stated in full so that a reader can check every
 * byte against it:
 *
 *   One segment of n BF16 values x[0..n).  T = ceil(n/512) tiles, K = ceil(n/4096)
 *   blocks, R128(v) = v rounded up to a multiple of 128.  Little-endian integers.
 *
 *   [0,128)          header: u32 magic 0x3143435A, u16 version 1, u16 flags 0,
 *                    u64 n, u8 table[7], u8 0, u32 4096, u32 512, u64 n_esc,
 *                    u64 esc_offset, u64 static_bytes, u64 0, then 64 zero bytes.
 *   A: 128, 512*T    sign+mantissa byte per value: A[i] = sign<<7 | mantissa(7 bits);
 *                    0 for n <= i < 512*T.
 *   B: next, R128(192*T)
 *                    bit planes.  64-bit word w = 24*t + 8*p + j (p = 0..2 is the code
 *                    bit, j = 0..7 the column).  Bit l (0..63) of that word is bit p of
 *                    code(512*t + 8*l + j); 0 past n; padding 0.
 *   C: next, R128(4*K)
 *                    u32 off[b] = number of escapes among x[0 .. 4096*b); padding 0.
 *   static_bytes = 128 + 512*T + R128(192*T) + R128(4*K).
 *
 *   Escapes: the exponent bytes of the values with code 0, in increasing index
 *   order, written to a separate buffer starting at esc_offset.
 *
 *   Uncoded blocks (the fallback to no compression where coding would not pay: the
 *   CCCL page's adaptive strategy section and its advice to fall back when the ratio
 *   reaches 1).  A tile of m values has m - 192 values (if positive) that do not fit its
 *   192 plane bytes; summed over the tiles of a block this is the block's overflow O.  A
 *   block with O > 0 whose coded form would put at least O exponents in the escape buffer
 *   is stored uncoded instead: its A bytes as usual; the 192 plane bytes of each of its
 *   tiles hold the exponents of the tile's first 192 values in index order (0 past the
 *   tile's last value); the exponents of the rest of each tile's values go, tile after
 *   tile in index order, to the escape buffer.  off[] counts the bytes each block puts
 *   in the escape buffer, so an uncoded block has exactly O of them and a coded block
 *   fewer: a decoder tells the two apart from off[] alone.
 *
 *   code(e) = 1 + r when e equals table[r] (table sorted ascending, 7 distinct values
 *   in 1..254), otherwise 0.  Exponents 0 (zero, subnormal) and 255 (Inf, NaN) are
 *   never in a table, so they always escape.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

#define ZO_OK 0
#define ZO_ERR_INVALID 1
#define ZO_ERR_SIZE 3
#define ZO_ERR_CORRUPT 5
#define ZO_ERR_OVERFLOW 7

#define ZO_MAGIC 0x3143435Au
#define ZO_TILE 512u
#define ZO_BLOCK 4096u

/* ------------------------------------------------------------------------- */
/* little-endian helpers                                                      */
/* ------------------------------------------------------------------------- */
static void put_u16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t* p, uint32_t v) { for (int k = 0; k < 4; k++) p[k] = (uint8_t)(v >> (8 * k)); }
static void put_u64(uint8_t* p, uint64_t v) { for (int k = 0; k < 8; k++) p[k] = (uint8_t)(v >> (8 * k)); }
static uint32_t get_u32(const uint8_t* p) { uint32_t v = 0; for (int k = 3; k >= 0; k--) v = (v << 8) | p[k]; return v; }
static uint64_t get_u64(const uint8_t* p) { uint64_t v = 0; for (int k = 7; k >= 0; k--) v = (v << 8) | p[k]; return v; }
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

/* ------------------------------------------------------------------------- */
/* sizes                                                                      */
/* ------------------------------------------------------------------------- */
uint64_t zo_tiles(uint64_t n) { return (n + ZO_TILE - 1) / ZO_TILE; }
uint64_t zo_blocks(uint64_t n) { return (n + ZO_BLOCK - 1) / ZO_BLOCK; }

uint64_t zo_static_size(uint64_t n)
{
    uint64_t T = zo_tiles(n), K = zo_blocks(n);
    return 128 + 512 * T + round_up(192 * T, 128) + round_up(4 * K, 128);
}

/* ------------------------------------------------------------------------- */
/* plan: sigma -> 7 most frequent exponents (S2.A)                            */
/* ------------------------------------------------------------------------- */

/* Probability that |X| lies in the binade of exponent field e, X ~ N(0, sigma^2):
 * P(2^(e-127) <= |X| < 2^(e-126)) = erfc(lo/(sigma*sqrt2)) - erfc(hi/(sigma*sqrt2)).
 * Continuous Gaussian model; BF16 rounding of the values is not modelled. */
double zo_binade_mass(int e, double sigma)
{
    double lo = ldexp(1.0, e - 127), hi = ldexp(1.0, e - 126);
    double s = sigma * sqrt(2.0);
    return erfc(lo / s) - erfc(hi / s);
}

static void sort7(uint8_t t[7])
{
    for (int a = 1; a < 7; a++)
        for (int b = a; b > 0 && t[b - 1] > t[b]; b--) {
            uint8_t tmp = t[b]; t[b] = t[b - 1]; t[b - 1] = tmp;
        }
}

/* The 7 exponent fields in 1..254 with the largest model mass; ties go to the lower
 * exponent.  Output sorted ascending.  Every candidate is ranked, no shortcut. */
int zo_plan_sigma(double sigma, uint8_t table_out[7])
{
    if (!(sigma > 0.0) || isinf(sigma) || isnan(sigma)) return ZO_ERR_INVALID;
    double m[255];
    int taken[255];
    for (int e = 1; e <= 254; e++) { m[e] = zo_binade_mass(e, sigma); taken[e] = 0; }
    for (int r = 0; r < 7; r++) {
        int best = -1;
        for (int e = 1; e <= 254; e++) {
            if (taken[e]) continue;
            if (best < 0 || m[e] > m[best]) best = e;   /* strict '>' keeps the lower e on ties */
        }
        taken[best] = 1;
        table_out[r] = (uint8_t)best;
    }
    sort7(table_out);
    return ZO_OK;
}

/* sigma of a tensor whose sigma the caller does not know.  S2.A models the values as
 * N(0, sigma^2) and takes sigma from the layer's weights; with no weights at hand the
 * plainest estimate under that model (mean 0) is the root mean square of the values.
 * It is taken over a sample: the tiles of 512 values with index 0, stride, 2*stride,
 * ... (the last may be short), skipping Inf and NaN, summed one value after another in
 * index order in fp64.  With no finite value, or a mean square of 0, sigma is 1. */
double zo_sample_sigma(const uint16_t* x, uint64_t n, uint64_t stride)
{
    double sum = 0.0;
    uint64_t count = 0;
    if (stride == 0) stride = 1;
    for (uint64_t t = 0; t * ZO_TILE < n; t += stride) {
        for (uint64_t i = t * ZO_TILE; i < n && i < (t + 1) * ZO_TILE; i++) {
            uint32_t u = (uint32_t)x[i] << 16;
            float f;
            memcpy(&f, &u, 4);
            if (isinf(f) || isnan(f)) continue;
            double d = (double)f;
            sum += d * d;
            count++;
        }
    }
    if (count == 0) return 1.0;
    double s = sqrt(sum / (double)count);
    if (!(s > 0.0) || isinf(s)) return 1.0;
    return s;
}

/* A caller-given table: exactly 7 distinct values in 1..254. */
int zo_plan_table(const uint8_t in[7], uint8_t table_out[7])
{
    for (int r = 0; r < 7; r++) {
        if (in[r] < 1 || in[r] > 254) return ZO_ERR_INVALID;
        for (int q = 0; q < r; q++)
            if (in[q] == in[r]) return ZO_ERR_INVALID;
        table_out[r] = in[r];
    }
    sort7(table_out);
    return ZO_OK;
}

/* ------------------------------------------------------------------------- */
/* field split and code (S2.B)                                                */
/* ------------------------------------------------------------------------- */
static unsigned sign_of(uint16_t x) { return (x >> 15) & 1u; }
static unsigned exponent_of(uint16_t x) { return (x >> 7) & 0xFFu; }
static unsigned mantissa_of(uint16_t x) { return x & 0x7Fu; }

static unsigned code_of(unsigned e, const uint8_t table[7])
{
    for (int r = 0; r < 7; r++)
        if (table[r] == e) return (unsigned)(r + 1);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* compress one segment                                                       */
/* ------------------------------------------------------------------------- */
/* Writes the static part (zo_static_size(n) bytes) to st and the escapes to
 * esc[esc_offset ...].  Escapes at positions >= esc_cap are counted but not stored;
 * the return is then ZO_ERR_OVERFLOW. */
int zo_compress(const uint16_t* x, uint64_t n, const uint8_t table_in[7], uint64_t esc_offset,
                uint8_t* st, uint8_t* esc, uint64_t esc_cap, uint64_t* n_esc_out)
{
    uint8_t table[7];
    if (zo_plan_table(table_in, table) != ZO_OK) return ZO_ERR_INVALID;
    if (n >= ((uint64_t)1 << 32)) return ZO_ERR_SIZE;
    uint64_t T = zo_tiles(n), K = zo_blocks(n);
    uint64_t sz = zo_static_size(n);
    uint8_t* A = st + 128;
    uint8_t* B = A + 512 * T;
    uint8_t* C = B + round_up(192 * T, 128);
    memset(st, 0, sz);

    uint64_t count = 0;   /* bytes in the escape buffer so far */
    int overflow = 0;
    for (uint64_t b = 0; b < K; b++) {
        uint64_t i0 = b * ZO_BLOCK, i1 = i0 + ZO_BLOCK < n ? i0 + ZO_BLOCK : n;
        put_u32(C + 4 * b, (uint32_t)count);
        /* the block's coded escapes and its overflow */
        uint64_t escapes = 0, ovf = 0;
        for (uint64_t i = i0; i < i1; i++) {
            if (code_of(exponent_of(x[i]), table) == 0) escapes++;
            if (i % 512 >= 192) ovf++;
        }
        int uncoded = ovf > 0 && escapes >= ovf;
        for (uint64_t i = i0; i < i1; i++) {
            uint16_t v = x[i];
            unsigned s = sign_of(v), e = exponent_of(v), m = mantissa_of(v);
            A[i] = (uint8_t)((s << 7) | m);
            uint64_t t = i / 512, l = (i % 512) / 8, j = i % 8;
            int to_esc;
            if (uncoded) {
                if (i % 512 < 192) B[192 * t + i % 512] = (uint8_t)e;   /* the tile's plane bytes */
                to_esc = i % 512 >= 192;
            } else {
                unsigned c = code_of(e, table);
                for (unsigned p = 0; p < 3; p++) {
                    if ((c >> p) & 1u) {
                        uint64_t w = 24 * t + 8 * p + j;      /* word index */
                        uint64_t bit = w * 64 + l;            /* bit index in B */
                        B[bit / 8] |= (uint8_t)(1u << (bit % 8));
                    }
                }
                to_esc = c == 0;
            }
            if (to_esc) {
                if (esc_offset + count < esc_cap) esc[esc_offset + count] = (uint8_t)e;
                else overflow = 1;
                count++;
            }
        }
    }

    put_u32(st + 0, ZO_MAGIC);
    put_u16(st + 4, 1);
    put_u16(st + 6, 0);
    put_u64(st + 8, n);
    memcpy(st + 16, table, 7);
    st[23] = 0;
    put_u32(st + 24, ZO_BLOCK);
    put_u32(st + 28, ZO_TILE);
    put_u64(st + 32, count);
    put_u64(st + 40, esc_offset);
    put_u64(st + 48, sz);
    put_u64(st + 56, 0);
    if (n_esc_out) *n_esc_out = count;
    return overflow ? ZO_ERR_OVERFLOW : ZO_OK;
}

/* Batch: segment s's static part follows those of segments 0..s-1; its escapes follow
 * theirs in the one escape buffer.  tables holds 7 bytes per segment. */
int zo_compress_batch(int nseg, const uint16_t* const* src, const uint64_t* n, const uint8_t* tables,
                      uint8_t* static_out, uint8_t* esc_out, uint64_t esc_cap, uint64_t* n_esc_out)
{
    uint64_t st_off = 0, esc_off = 0;
    int rc_all = ZO_OK;
    for (int s = 0; s < nseg; s++) {
        uint64_t ne = 0;
        int rc = zo_compress(src[s], n[s], tables + 7 * s, esc_off, static_out + st_off, esc_out,
                             esc_cap, &ne);
        if (rc == ZO_ERR_OVERFLOW) rc_all = rc;
        else if (rc != ZO_OK) return rc;
        if (n_esc_out) n_esc_out[s] = ne;
        st_off += zo_static_size(n[s]);
        esc_off += ne;
    }
    return rc_all;
}

/* ------------------------------------------------------------------------- */
/* decompress one segment: the exact inverse                                  */
/* ------------------------------------------------------------------------- */
/* st_bytes / esc_bytes are the sizes of the buffers the caller holds; every read is
 * checked against them.  n_expected is the length the caller expects. */
int zo_decompress(const uint8_t* st, uint64_t st_bytes, const uint8_t* esc, uint64_t esc_bytes,
                  uint64_t n_expected, uint16_t* out)
{
    if (st_bytes < 128) return ZO_ERR_CORRUPT;
    if (get_u32(st) != ZO_MAGIC || get_u16(st + 4) != 1 || get_u16(st + 6) != 0) return ZO_ERR_CORRUPT;
    uint64_t n = get_u64(st + 8);
    if (n != n_expected || n >= ((uint64_t)1 << 32)) return ZO_ERR_CORRUPT;
    if (get_u32(st + 24) != ZO_BLOCK || get_u32(st + 28) != ZO_TILE) return ZO_ERR_CORRUPT;
    uint8_t table[7];
    if (zo_plan_table(st + 16, table) != ZO_OK) return ZO_ERR_CORRUPT;
    if (memcmp(table, st + 16, 7) != 0) return ZO_ERR_CORRUPT;   /* stored sorted */
    uint64_t n_esc = get_u64(st + 32), esc_offset = get_u64(st + 40);
    if (get_u64(st + 48) != zo_static_size(n) || zo_static_size(n) > st_bytes) return ZO_ERR_CORRUPT;
    if (n_esc > n || esc_offset > esc_bytes || n_esc > esc_bytes - esc_offset) return ZO_ERR_CORRUPT;

    uint64_t T = zo_tiles(n);
    const uint8_t* A = st + 128;
    const uint8_t* B = A + 512 * T;
    const uint8_t* C = B + round_up(192 * T, 128);

    uint64_t K = zo_blocks(n);
    uint64_t used = 0;          /* escape-buffer bytes used so far in the whole segment */
    for (uint64_t b = 0; b < K; b++) {
        uint64_t i0 = b * ZO_BLOCK, i1 = i0 + ZO_BLOCK < n ? i0 + ZO_BLOCK : n;
        uint64_t first = get_u32(C + 4 * b);
        uint64_t last = b + 1 < K ? get_u32(C + 4 * (b + 1)) : n_esc;
        if (first != used || last < first) return ZO_ERR_CORRUPT;
        uint64_t ovf = 0;
        for (uint64_t i = i0; i < i1; i++)
            if (i % 512 >= 192) ovf++;
        int uncoded = ovf > 0 && last - first == ovf;
        uint64_t in_block = 0;  /* escape-buffer bytes of this block used so far */
        for (uint64_t i = i0; i < i1; i++) {
            uint64_t t = i / 512, l = (i % 512) / 8, j = i % 8;
            unsigned e;
            int from_esc;
            if (uncoded) {
                from_esc = i % 512 >= 192;
                e = from_esc ? 0u : B[192 * t + i % 512];
            } else {
                unsigned c = 0;
                for (unsigned p = 0; p < 3; p++) {
                    uint64_t bit = (24 * t + 8 * p + j) * 64 + l;
                    c |= (unsigned)((B[bit / 8] >> (bit % 8)) & 1u) << p;
                }
                from_esc = c == 0;
                e = from_esc ? 0u : table[c - 1];
            }
            if (from_esc) {
                uint64_t k = first + in_block;
                if (k >= last) return ZO_ERR_CORRUPT;
                e = esc[esc_offset + k];
                in_block++;
                used++;
            }
            unsigned a = A[i];
            unsigned s = (a >> 7) & 1u, m = a & 0x7Fu;
            out[i] = (uint16_t)((s << 15) | (e << 7) | m);
        }
        if (used != last) return ZO_ERR_CORRUPT;
    }
    if (used != n_esc) return ZO_ERR_CORRUPT;
    return ZO_OK;
}

/* ------------------------------------------------------------------------- */
/* fp32 accumulation and one rounding to BF16 (S2.D local reduction)          */
/* ------------------------------------------------------------------------- */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* Round a binary32 value to the nearest BF16, ties to the even significand, by the
 * definition: of the two BF16 neighbours choose the nearer one.  Overflow is decided
 * against 2^128, the value the next binade would start at.  NaN -> 0x7FC0. */
uint16_t zo_round_bf16(float f)
{
    if (isnan(f)) return 0x7FC0;
    uint32_t u = f32_bits(f);
    uint32_t lo = u & 0xFFFF0000u;                 /* toward zero */
    if (lo == u) return (uint16_t)(u >> 16);       /* exactly representable */
    uint32_t hi = lo + 0x10000u;                   /* away from zero, same sign */
    double vf = fabs((double)f);
    double vlo = fabs((double)bf16_to_f32((uint16_t)(lo >> 16)));
    double vhi;
    if ((hi & 0x7FFFFFFFu) == 0x7F800000u) vhi = ldexp(1.0, 128);
    else vhi = fabs((double)bf16_to_f32((uint16_t)(hi >> 16)));
    double dlo = vf - vlo, dhi = vhi - vf;
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

/* out[i] = round_bf16( (((f32(local[i]) + f32(d_0[i])) + f32(d_1[i])) + ...) ), each '+'
 * one IEEE binary32 addition rounded to nearest even, no flush of subnormals, peers
 * in array order; d_p is the decompressed segment of peer p.  out may equal local. */
int zo_decompress_accumulate(int npeers, const uint8_t* const* st, const uint64_t* st_bytes,
                             const uint8_t* const* esc, const uint64_t* esc_bytes, uint64_t n,
                             const uint16_t* local, uint16_t* out)
{
    uint16_t** d = (uint16_t**)calloc((size_t)(npeers > 0 ? npeers : 1), sizeof(uint16_t*));
    if (!d) return ZO_ERR_INVALID;
    int rc = ZO_OK;
    for (int p = 0; p < npeers && rc == ZO_OK; p++) {
        d[p] = (uint16_t*)malloc((size_t)(n > 0 ? n : 1) * 2);
        if (!d[p]) { rc = ZO_ERR_INVALID; break; }
        rc = zo_decompress(st[p], st_bytes[p], esc[p], esc_bytes[p], n, d[p]);
    }
    if (rc == ZO_OK) {
        unsigned csr = _mm_getcsr();
        _mm_setcsr(csr & ~0x8040u);            /* clear FTZ and DAZ: keep subnormals */
        for (uint64_t i = 0; i < n; i++) {
            volatile float acc = bf16_to_f32(local[i]);
            for (int p = 0; p < npeers; p++) acc = acc + bf16_to_f32(d[p][i]);
            out[i] = zo_round_bf16(acc);
        }
        _mm_setcsr(csr);
    }
    for (int p = 0; p < npeers; p++) free(d[p]);
    free(d);
    return rc;
}

/* Single fp32 sum of two BF16 values, exported for the rounding pins. */
uint16_t zo_add2_bf16(uint16_t a, uint16_t b)
{
    unsigned csr = _mm_getcsr();
    _mm_setcsr(csr & ~0x8040u);
    volatile float acc = bf16_to_f32(a);
    acc = acc + bf16_to_f32(b);
    uint16_t r = zo_round_bf16(acc);
    _mm_setcsr(csr);
    return r;
}

uint16_t zo_round_bits(uint32_t f32bits)
{
    float f;
    memcpy(&f, &f32bits, 4);
    return zo_round_bf16(f);
}
