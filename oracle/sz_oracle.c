/*
 * sz_oracle.c -- plain, slow, scalar CPU oracle of the SplitZip-style
 * exponent codec stream (format v1).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this file's library.  The GPU
 * library never links, includes or calls it, and it shares no code, header
 * or constant table with the GPU library: every constant below is written
 * out here on its own.
 *
 * What the method computes (SplitZip project page):
 *   - "Abstract": the most frequent exponent values of a BF16 tensor get a
 *     constant-width 4-bit code, sign and mantissa bits are kept as they
 *     are, and rare
 *     exponent values are routed through a separate escape stream.
 *   - FAQ "Is SplitZip lossy?": sign and mantissa are stored unchanged and
 *     decoding reproduces the input bit for bit.
 *   - FAQ "Does it work with an FP8 KV cache?": the same scheme applies to
 *     FP8 E5M2 and gains at most 1.14x.
 * The pages fix no byte layout.  The readings taken where they are silent:
 *   R1  16 code values; codes 0..14 name the 15 most frequent exponents,
 *       code 15 means "escape" (no extra flag bit: that would break the
 *       page's 1.14x ceiling for E5M2, which is exactly 8 bits / 7 bits).
 *   R2  ranking key: count descending, then exponent value ascending; the
 *       whole exponent domain takes part (256 values for BF16, 32 for E5M2),
 *       so zero-count values fill the table when fewer than 15 occur.
 *   R3  BF16 sign|mantissa byte = sign in bit 7, 7 mantissa bits in 6..0.
 *       E5M2 sign|mantissa field = 3 bits (sign<<2 | 2 mantissa bits),
 *       packed LSB-first: element i occupies stream bits [3i, 3i+3).
 *   R4  code plane: element 2i in the low nibble of byte i, element 2i+1 in
 *       the high nibble; an odd tail leaves a zero high nibble.
 *   R5  escape record = one byte holding the raw biased exponent; escapes
 *       are stored in element order; their positions are implied by code 15.
 *   R6  per-block escape offsets: format blocks of 4096 elements; a table of
 *       B = ceil(n/4096) u32 exclusive prefix counts of escapes.
 *   R7  exponent = the raw bit field (zero, subnormals, Inf and NaN are
 *       ordinary symbols; NaN payloads live in the mantissa field).
 *   R8  one histogram and one codebook per encoded tensor.
 *
 * Stream layout, little-endian, A(x) = x rounded up to a multiple of 256:
 *   0   u8[4]  magic 'S','Z','K','V'
 *   4   u8     version = 1
 *   5   u8     dtype (1 = BF16, 2 = FP8 E5M2)
 *   6   u8     log2 of the format block = 12
 *   7   u8     number of coded exponents = 15
 *   8   u64    n (element count)
 *   16  u64    E (escape count)
 *   24  u8[16] codebook cb[0..14], cb[15] = 0
 *   40  u64    C, total stream bytes
 *   48  u8[16] reserved, zero
 *   64  u32[B] escape offsets, then zeros up to H = A(64 + 4B)
 *   H          sign|mantissa plane, S bytes (BF16: n; E5M2: ceil(3n/8)),
 *              then zeros up to H + A(S)
 *   H + A(S)   code plane, ceil(n/2) bytes, then zeros up to A(ceil(n/2))
 *   ...        E escape bytes, no trailing padding
 *   C = H + A(S) + A(ceil(n/2)) + E.
 *
 * Decoding accepts a stream iff (checked in this order): src_bytes >= 64;
 * magic, version, dtype, block size, code count and n match; cb[15] = 0;
 * the reserved bytes are zero; E <= n; C = H + A(S) + A(ceil(n/2)) + E and
 * C <= src_bytes; off[0] = 0; every block's count of code-15 nibbles equals
 * its offset span (the next offset, or E after the last block).  Exponent
 * bytes are masked to the field width on reassembly.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SZO_OK 0
#define SZO_INVALID_ARGUMENT 1
#define SZO_BUFFER_TOO_SMALL 2
#define SZO_CORRUPT_STREAM 3

#define SZO_BF16 1
#define SZO_E5M2 2

#define SZO_BLOCK 4096u
#define SZO_ESC 15u
#define SZO_NCODES 15u

static uint64_t round256(uint64_t x) { return (x + 255u) / 256u * 256u; }

static int dtype_ok(int dt) { return dt == SZO_BF16 || dt == SZO_E5M2; }

/* number of distinct exponent values of the type */
static unsigned exponent_domain(int dt) { return dt == SZO_BF16 ? 256u : 32u; }

static uint64_t n_blocks(uint64_t n) { return (n + SZO_BLOCK - 1u) / SZO_BLOCK; }

static uint64_t header_region(uint64_t n) { return round256(64u + 4u * n_blocks(n)); }

static uint64_t sm_plane_bytes(uint64_t n, int dt) {
    return dt == SZO_BF16 ? n : (3u * n + 7u) / 8u;
}

static uint64_t code_plane_bytes(uint64_t n) { return (n + 1u) / 2u; }

/* everything but the escape bytes */
static uint64_t fixed_bytes(uint64_t n, int dt) {
    return header_region(n) + round256(sm_plane_bytes(n, dt)) + round256(code_plane_bytes(n));
}

/* raw element i as an unsigned integer */
static unsigned element(const uint8_t* src, uint64_t i, int dt) {
    if (dt == SZO_BF16) return (unsigned)src[2 * i] | ((unsigned)src[2 * i + 1] << 8);
    return src[i];
}

static unsigned exponent_of(unsigned u, int dt) {
    if (dt == SZO_BF16) return (u >> 7) & 0xFFu;   /* bits 14..7 */
    return (u >> 2) & 0x1Fu;                        /* bits 6..2 */
}

static unsigned signmant_of(unsigned u, int dt) {
    if (dt == SZO_BF16) return ((u >> 8) & 0x80u) | (u & 0x7Fu); /* s | m7 */
    return ((u >> 5) & 0x4u) | (u & 0x3u);                       /* s | m2 */
}

static unsigned reassemble(unsigned sm, unsigned e, int dt) {
    if (dt == SZO_BF16) return ((sm & 0x80u) << 8) | ((e & 0xFFu) << 7) | (sm & 0x7Fu);
    return ((sm & 0x4u) << 5) | ((e & 0x1Fu) << 2) | (sm & 0x3u);
}

static void put_u64(uint8_t* p, uint64_t v) {
    for (int k = 0; k < 8; k++) p[k] = (uint8_t)(v >> (8 * k));
}
static void put_u32(uint8_t* p, uint32_t v) {
    for (int k = 0; k < 4; k++) p[k] = (uint8_t)(v >> (8 * k));
}
static uint64_t get_u64(const uint8_t* p) {
    uint64_t v = 0;
    for (int k = 0; k < 8; k++) v |= (uint64_t)p[k] << (8 * k);
    return v;
}
static uint32_t get_u32(const uint8_t* p) {
    uint32_t v = 0;
    for (int k = 0; k < 4; k++) v |= (uint32_t)p[k] << (8 * k);
    return v;
}

/* ---- public entry points (C ABI, loaded with ctypes) ------------------- */

/* Largest stream for any codebook: with a caller-given codebook every
 * element may escape, so the bound takes E = n.  (With the tensor's own
 * codebook the 15 fullest of D exponent bins hold at least ceil(15n/D)
 * elements, so E <= floor((D-15)n/D); the tests check that tighter bound.) */
uint64_t szo_max_bytes(uint64_t n, int dt) {
    if (!dtype_ok(dt) || n >= ((uint64_t)1 << 32)) return 0;
    return fixed_bytes(n, dt) + n;
}

uint64_t szo_exact_bytes(uint64_t n, int dt, uint64_t escapes) {
    if (!dtype_ok(dt)) return 0;
    return fixed_bytes(n, dt) + escapes;
}

/* hist[v] = number of elements whose exponent field equals v (Abstract:
 * the method starts from how often each exponent value occurs). */
int szo_histogram(const void* src, uint64_t n, int dt, uint64_t* hist) {
    if (!dtype_ok(dt) || !hist || (n && !src)) return SZO_INVALID_ARGUMENT;
    for (unsigned v = 0; v < 256; v++) hist[v] = 0;
    for (uint64_t i = 0; i < n; i++) hist[exponent_of(element((const uint8_t*)src, i, dt), dt)]++;
    return SZO_OK;
}

/* Histogram over a block sample (an extension; the pages define no
 * sampling): only elements of 4096-element blocks b with b % stride == 0. */
int szo_histogram_sampled(const void* src, uint64_t n, int dt, uint64_t stride, uint64_t* hist) {
    if (!dtype_ok(dt) || !hist || (n && !src) || stride == 0) return SZO_INVALID_ARGUMENT;
    for (unsigned v = 0; v < 256; v++) hist[v] = 0;
    for (uint64_t i = 0; i < n; i++)
        if ((i / SZO_BLOCK) % stride == 0) hist[exponent_of(element((const uint8_t*)src, i, dt), dt)]++;
    return SZO_OK;
}

struct ranked { uint64_t count; unsigned value; };

static int by_count_then_value(const void* a, const void* b) {
    const struct ranked* x = (const struct ranked*)a;
    const struct ranked* y = (const struct ranked*)b;
    if (x->count != y->count) return x->count > y->count ? -1 : 1;
    if (x->value != y->value) return x->value < y->value ? -1 : 1;
    return 0;
}

/* Codebook (Abstract: "most frequent exponent values" get the codes):
 * order the whole exponent domain by (count desc, value asc) and give code c
 * to the c-th value, c = 0..14.  cb[15] = 0. */
int szo_codebook(const uint64_t* hist, int dt, uint8_t* cb) {
    if (!dtype_ok(dt) || !hist || !cb) return SZO_INVALID_ARGUMENT;
    unsigned d = exponent_domain(dt);
    struct ranked r[256];
    for (unsigned v = 0; v < d; v++) { r[v].count = hist[v]; r[v].value = v; }
    qsort(r, d, sizeof r[0], by_count_then_value);
    for (unsigned c = 0; c < SZO_NCODES; c++) cb[c] = (uint8_t)r[c].value;
    cb[SZO_ESC] = 0;
    return SZO_OK;
}

/* Encode one tensor.  cb may be NULL (then the histogram and codebook are
 * built here) or any 16 bytes; a value listed twice takes its lowest code. */
int szo_encode(const void* src_, uint64_t n, int dt, const uint8_t* cb_in,
               uint8_t* dst, uint64_t capacity, uint64_t* out_bytes) {
    const uint8_t* src = (const uint8_t*)src_;
    if (!dtype_ok(dt) || !dst || (n && !src) || n >= ((uint64_t)1 << 32)) return SZO_INVALID_ARGUMENT;
    if (capacity < szo_max_bytes(n, dt)) return SZO_BUFFER_TOO_SMALL;

    uint8_t cb[16];
    if (cb_in) {
        memcpy(cb, cb_in, 16);
    } else {
        uint64_t hist[256];
        szo_histogram(src, n, dt, hist);
        szo_codebook(hist, dt, cb);
    }
    cb[SZO_ESC] = 0;

    /* code of each exponent value: the first c whose entry is that value */
    unsigned code_of[256];
    for (unsigned v = 0; v < 256; v++) code_of[v] = SZO_ESC;
    for (unsigned c = 0; c < SZO_NCODES; c++)
        if (code_of[cb[c]] == SZO_ESC) code_of[cb[c]] = c;

    uint64_t h = header_region(n);
    uint64_t s = sm_plane_bytes(n, dt);
    uint64_t sm_at = h;
    uint64_t code_at = h + round256(s);
    uint64_t esc_at = code_at + round256(code_plane_bytes(n));

    memset(dst, 0, esc_at);

    uint64_t escapes = 0;
    for (uint64_t i = 0; i < n; i++) {
        if (i % SZO_BLOCK == 0) put_u32(dst + 64 + 4 * (i / SZO_BLOCK), (uint32_t)escapes);
        unsigned u = element(src, i, dt);
        unsigned e = exponent_of(u, dt);
        unsigned code = code_of[e];
        unsigned sm = signmant_of(u, dt);
        if (dt == SZO_BF16) {
            dst[sm_at + i] = (uint8_t)sm;
        } else {
            for (unsigned k = 0; k < 3; k++) {
                uint64_t bit = 3 * i + k;
                if ((sm >> k) & 1u) dst[sm_at + bit / 8] |= (uint8_t)(1u << (bit % 8));
            }
        }
        dst[code_at + i / 2] |= (uint8_t)(code << (4 * (i % 2)));
        if (code == SZO_ESC) {
            dst[esc_at + escapes] = (uint8_t)e;
            escapes++;
        }
    }

    uint64_t total = esc_at + escapes;
    dst[0] = 'S'; dst[1] = 'Z'; dst[2] = 'K'; dst[3] = 'V';
    dst[4] = 1;
    dst[5] = (uint8_t)dt;
    dst[6] = 12;
    dst[7] = SZO_NCODES;
    put_u64(dst + 8, n);
    put_u64(dst + 16, escapes);
    memcpy(dst + 24, cb, 16);
    put_u64(dst + 40, total);
    if (out_bytes) *out_bytes = total;
    return SZO_OK;
}

/* Decode (FAQ "Is SplitZip lossy?": the output equals the input bit for
 * bit).  Validates the whole stream before writing any output. */
int szo_decode(const uint8_t* src, uint64_t src_bytes, uint64_t n, int dt, void* dst_) {
    uint8_t* dst = (uint8_t*)dst_;
    if (!dtype_ok(dt) || !src || (n && !dst) || n >= ((uint64_t)1 << 32)) return SZO_INVALID_ARGUMENT;
    if (src_bytes < 64) return SZO_CORRUPT_STREAM;
    if (src[0] != 'S' || src[1] != 'Z' || src[2] != 'K' || src[3] != 'V') return SZO_CORRUPT_STREAM;
    if (src[4] != 1 || src[5] != dt || src[6] != 12 || src[7] != SZO_NCODES) return SZO_CORRUPT_STREAM;
    if (get_u64(src + 8) != n) return SZO_CORRUPT_STREAM;
    if (src[24 + SZO_ESC] != 0) return SZO_CORRUPT_STREAM;
    for (unsigned k = 48; k < 64; k++)
        if (src[k] != 0) return SZO_CORRUPT_STREAM;
    uint64_t escapes = get_u64(src + 16);
    if (escapes > n) return SZO_CORRUPT_STREAM;
    uint64_t total = get_u64(src + 40);
    if (total != fixed_bytes(n, dt) + escapes || total > src_bytes) return SZO_CORRUPT_STREAM;

    uint8_t cb[16];
    memcpy(cb, src + 24, 16);
    uint64_t nb = n_blocks(n);
    uint64_t h = header_region(n);
    uint64_t sm_at = h;
    uint64_t code_at = h + round256(sm_plane_bytes(n, dt));
    uint64_t esc_at = code_at + round256(code_plane_bytes(n));

    /* offsets must start at 0 and each block's span must equal the number
     * of escape codes it holds */
    if (nb && get_u32(src + 64) != 0) return SZO_CORRUPT_STREAM;
    for (uint64_t b = 0; b < nb; b++) {
        uint64_t first = get_u32(src + 64 + 4 * b);
        uint64_t next = (b + 1 < nb) ? get_u32(src + 64 + 4 * (b + 1)) : escapes;
        uint64_t hi = (b + 1) * SZO_BLOCK < n ? (b + 1) * SZO_BLOCK : n;
        uint64_t count = 0;
        for (uint64_t i = b * SZO_BLOCK; i < hi; i++)
            if (((src[code_at + i / 2] >> (4 * (i % 2))) & 0xFu) == SZO_ESC) count++;
        if (next < first || next - first != count) return SZO_CORRUPT_STREAM;
    }

    uint64_t j = 0;
    for (uint64_t i = 0; i < n; i++) {
        unsigned code = (src[code_at + i / 2] >> (4 * (i % 2))) & 0xFu;
        unsigned e = code == SZO_ESC ? src[esc_at + j++] : cb[code];
        unsigned sm;
        if (dt == SZO_BF16) {
            sm = src[sm_at + i];
        } else {
            sm = 0;
            for (unsigned k = 0; k < 3; k++) {
                uint64_t bit = 3 * i + k;
                sm |= ((src[sm_at + bit / 8] >> (bit % 8)) & 1u) << k;
            }
        }
        unsigned u = reassemble(sm, e, dt);
        if (dt == SZO_BF16) {
            dst[2 * i] = (uint8_t)(u & 0xFFu);
            dst[2 * i + 1] = (uint8_t)(u >> 8);
        } else {
            dst[i] = (uint8_t)u;
        }
    }
    return SZO_OK;
}
