/* lc_oracle.c -- plain scalar CPU oracle of the LC-style comparison codec.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests and by the benchmark's CPU
 * baseline through ctypes.  It shares no code with the GPU library.
 *
 * Source: FastKVComp companion page, "Inside an LC-style pipeline": three
 * stages, TUPL8_1 then BIT_8 (size-preserving bit permutations) then RZE_2
 * (leaves out zero words).  The page gives no stage internals, so the
 * plainest reading of each stage name is taken (readings L1..L6), written
 * out below and in the header of include/lc_codec.h:
 *
 *  L1 chunking: the input (n bytes, n < 2^31) is cut into chunks of 16384
 *     bytes (the last one shorter); each chunk is coded on its own.
 *  L2 TUPL8_1 (tuples of eight 1-byte values -> eight streams): with
 *     q = floor(L/8), byte 8i+j goes to j*q + i (i < q, j < 8); the last
 *     L mod 8 bytes stay where they are.
 *  L3 BIT_8 (bit planes of 8-byte words): with W = floor(L/8) little-endian
 *     64-bit words and G = floor(W/8), plane b (b < 64) is G bytes; bit a of
 *     plane byte s is bit b of word 8s+a.  Bytes from 64G on stay put.
 *  L4 RZE_2 (zero elimination on 2-byte words): with V = floor(L/2)
 *     little-endian 16-bit words, a bitmap of ceil(V/8) bytes (bit m%8 of
 *     byte m/8 set iff word m is non-zero), then the non-zero words in
 *     order, then the last byte if L is odd.
 *  L5 a chunk whose RZE_2 output is not shorter than the chunk is stored
 *     raw (the input bytes); its stored size then equals its length.
 *  L6 container, little-endian: 64-byte header
 *       0 "LCKV", 4 version 1, 5 pipeline 1 (TUPL8_1/BIT_8/RZE_2),
 *       6 log2 chunk bytes 14, 7 zero, 8 u64 n, 16 u64 chunk count C,
 *       24 u64 total stream bytes, 32..63 zero;
 *     at 64 a table of C (u32 offset, u32 size) pairs; the data region
 *     starts at D = 64 + 8C rounded up to 256; chunk c's payload sits at
 *     D + offset_c, offsets start at 0 and advance by size rounded up to 16,
 *     padding bytes are zero; total = D + sum of the rounded sizes.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LCO_OK 0
#define LCO_INVALID_ARGUMENT 1
#define LCO_BUFFER_TOO_SMALL 2
#define LCO_CORRUPT_STREAM 3

#define LCO_CHUNK 16384u

static uint64_t up16(uint64_t x) { return (x + 15u) / 16u * 16u; }
static uint64_t up256(uint64_t x) { return (x + 255u) / 256u * 256u; }
static uint64_t chunks_of(uint64_t n) { return (n + LCO_CHUNK - 1u) / LCO_CHUNK; }
static uint64_t data_region(uint64_t n) { return up256(64u + 8u * chunks_of(n)); }
static uint64_t chunk_len(uint64_t n, uint64_t c) {
    return c + 1u < chunks_of(n) ? LCO_CHUNK : n - c * LCO_CHUNK;
}

static void put_u32(uint8_t* p, uint32_t v) { for (int k = 0; k < 4; k++) p[k] = (uint8_t)(v >> (8 * k)); }
static void put_u64(uint8_t* p, uint64_t v) { for (int k = 0; k < 8; k++) p[k] = (uint8_t)(v >> (8 * k)); }
static uint32_t get_u32(const uint8_t* p) {
    uint32_t v = 0;
    for (int k = 0; k < 4; k++) v |= (uint32_t)p[k] << (8 * k);
    return v;
}
static uint64_t get_u64(const uint8_t* p) {
    uint64_t v = 0;
    for (int k = 0; k < 8; k++) v |= (uint64_t)p[k] << (8 * k);
    return v;
}
static unsigned bit_of(const uint8_t* p, uint64_t byte, unsigned bit) { return (p[byte] >> bit) & 1u; }

/* ---- the three stages and their inverses (each on one chunk of L bytes) */

/* L2: byte 8i+j -> j*q+i */
void lco_tupl8_1(const uint8_t* x, uint64_t L, uint8_t* y) {
    uint64_t q = L / 8u;
    for (uint64_t i = 0; i < q; i++)
        for (uint64_t j = 0; j < 8; j++) y[j * q + i] = x[8 * i + j];
    for (uint64_t p = 8 * q; p < L; p++) y[p] = x[p];
}

void lco_untupl8_1(const uint8_t* y, uint64_t L, uint8_t* x) {
    uint64_t q = L / 8u;
    for (uint64_t i = 0; i < q; i++)
        for (uint64_t j = 0; j < 8; j++) x[8 * i + j] = y[j * q + i];
    for (uint64_t p = 8 * q; p < L; p++) x[p] = y[p];
}

/* L3: plane b byte s bit a = bit b of word 8s+a; bit b of a word is bit
 * b%8 of its byte b/8 */
void lco_bit8(const uint8_t* y, uint64_t L, uint8_t* z) {
    uint64_t G = (L / 8u) / 8u;
    for (uint64_t b = 0; b < 64; b++)
        for (uint64_t s = 0; s < G; s++) {
            unsigned v = 0;
            for (unsigned a = 0; a < 8; a++) v |= bit_of(y, 8 * (8 * s + a) + b / 8, (unsigned)(b % 8)) << a;
            z[b * G + s] = (uint8_t)v;
        }
    for (uint64_t p = 64 * G; p < L; p++) z[p] = y[p];
}

void lco_unbit8(const uint8_t* z, uint64_t L, uint8_t* y) {
    uint64_t G = (L / 8u) / 8u;
    memset(y, 0, 64 * G);
    for (uint64_t b = 0; b < 64; b++)
        for (uint64_t s = 0; s < G; s++)
            for (unsigned a = 0; a < 8; a++)
                y[8 * (8 * s + a) + b / 8] |= (uint8_t)(bit_of(z, b * G + s, a) << (b % 8));
    for (uint64_t p = 64 * G; p < L; p++) y[p] = z[p];
}

/* L4: bitmap of non-zero 16-bit words, the non-zero words, the odd byte.
 * Returns the output length. */
uint64_t lco_rze2(const uint8_t* z, uint64_t L, uint8_t* out) {
    uint64_t V = L / 2u, nb = (V + 7u) / 8u, at = nb;
    memset(out, 0, nb);
    for (uint64_t m = 0; m < V; m++) {
        if (z[2 * m] | z[2 * m + 1]) {
            out[m / 8] |= (uint8_t)(1u << (m % 8));
            out[at++] = z[2 * m];
            out[at++] = z[2 * m + 1];
        }
    }
    if (L & 1u) out[at++] = z[L - 1];
    return at;
}

/* Inverse of L4; `len` is the stored length, which must match the bitmap.
 * Returns 0 on success, -1 if the lengths disagree. */
int lco_unrze2(const uint8_t* in, uint64_t len, uint64_t L, uint8_t* z) {
    uint64_t V = L / 2u, nb = (V + 7u) / 8u, nz = 0;
    if (len < nb) return -1;
    for (uint64_t m = 0; m < V; m++) nz += bit_of(in, m / 8, (unsigned)(m % 8));
    if (len != nb + 2 * nz + (L & 1u)) return -1;
    uint64_t at = nb;
    for (uint64_t m = 0; m < V; m++) {
        if (bit_of(in, m / 8, (unsigned)(m % 8))) {
            z[2 * m] = in[at++];
            z[2 * m + 1] = in[at++];
        } else {
            z[2 * m] = z[2 * m + 1] = 0;
        }
    }
    if (L & 1u) z[L - 1] = in[at];
    return 0;
}

/* ---- container ---------------------------------------------------------- */

uint64_t lco_max_bytes(uint64_t n) {
    if (n >= ((uint64_t)1 << 31)) return 0;
    uint64_t total = data_region(n);
    for (uint64_t c = 0; c < chunks_of(n); c++) total += up16(chunk_len(n, c));
    return total;
}

/* one chunk: coded payload into out (capacity >= L), returns its size */
static uint64_t code_chunk(const uint8_t* x, uint64_t L, uint8_t* out) {
    uint8_t* y = malloc(L ? L : 1);
    uint8_t* z = malloc(L ? L : 1);
    uint8_t* r = malloc(L + L / 16u + 16u);   /* bitmap + every word + odd byte */
    lco_tupl8_1(x, L, y);
    lco_bit8(y, L, z);
    uint64_t len = lco_rze2(z, L, r);
    if (len < L) {
        memcpy(out, r, len);
    } else {
        memcpy(out, x, L);
        len = L;
    }
    free(y);
    free(z);
    free(r);
    return len;
}

int lco_encode(const void* src_, uint64_t n, uint8_t* dst, uint64_t capacity, uint64_t* out_bytes) {
    const uint8_t* src = (const uint8_t*)src_;
    if (!dst || (n && !src) || n >= ((uint64_t)1 << 31)) return LCO_INVALID_ARGUMENT;
    if (capacity < lco_max_bytes(n)) return LCO_BUFFER_TOO_SMALL;
    uint64_t C = chunks_of(n), D = data_region(n), off = 0;
    memset(dst, 0, D);
    for (uint64_t c = 0; c < C; c++) {
        uint64_t L = chunk_len(n, c);
        uint64_t size = code_chunk(src + c * LCO_CHUNK, L, dst + D + off);
        memset(dst + D + off + size, 0, up16(size) - size);
        put_u32(dst + 64 + 8 * c, (uint32_t)off);
        put_u32(dst + 64 + 8 * c + 4, (uint32_t)size);
        off += up16(size);
    }
    memcpy(dst, "LCKV", 4);
    dst[4] = 1;
    dst[5] = 1;
    dst[6] = 14;
    dst[7] = 0;
    put_u64(dst + 8, n);
    put_u64(dst + 16, C);
    put_u64(dst + 24, D + off);
    if (out_bytes) *out_bytes = D + off;
    return LCO_OK;
}

/* Validates the header and the whole table before writing any output. */
int lco_decode(const uint8_t* src, uint64_t src_bytes, uint64_t n, void* dst_) {
    uint8_t* dst = (uint8_t*)dst_;
    if (!src || (n && !dst) || n >= ((uint64_t)1 << 31)) return LCO_INVALID_ARGUMENT;
    if (src_bytes < 64) return LCO_CORRUPT_STREAM;
    if (memcmp(src, "LCKV", 4) != 0 || src[4] != 1 || src[5] != 1 || src[6] != 14 || src[7] != 0)
        return LCO_CORRUPT_STREAM;
    for (unsigned k = 32; k < 64; k++)
        if (src[k]) return LCO_CORRUPT_STREAM;
    uint64_t C = chunks_of(n), D = data_region(n);
    if (get_u64(src + 8) != n || get_u64(src + 16) != C) return LCO_CORRUPT_STREAM;
    uint64_t total = get_u64(src + 24);
    if (src_bytes < D || total > src_bytes) return LCO_CORRUPT_STREAM;
    uint64_t off = 0;
    for (uint64_t c = 0; c < C; c++) {
        uint64_t L = chunk_len(n, c);
        uint64_t o = get_u32(src + 64 + 8 * c), size = get_u32(src + 64 + 8 * c + 4);
        if (o != off || size > L) return LCO_CORRUPT_STREAM;
        off += up16(size);
    }
    if (total != D + off) return LCO_CORRUPT_STREAM;
    /* every coded chunk's size must match its bitmap (L4) */
    for (uint64_t c = 0; c < C; c++) {
        uint64_t L = chunk_len(n, c), size = get_u32(src + 64 + 8 * c + 4);
        const uint8_t* p = src + D + get_u32(src + 64 + 8 * c);
        uint64_t V = L / 2u, nb = (V + 7u) / 8u, nz = 0;
        if (size == L) continue;
        if (size < nb) return LCO_CORRUPT_STREAM;
        for (uint64_t m = 0; m < V; m++) nz += bit_of(p, m / 8, (unsigned)(m % 8));
        if (size != nb + 2 * nz + (L & 1u)) return LCO_CORRUPT_STREAM;
    }
    uint8_t* z = malloc(LCO_CHUNK);
    uint8_t* y = malloc(LCO_CHUNK);
    int rc = LCO_OK;
    for (uint64_t c = 0; c < C && rc == LCO_OK; c++) {
        uint64_t L = chunk_len(n, c);
        const uint8_t* p = src + D + get_u32(src + 64 + 8 * c);
        uint64_t size = get_u32(src + 64 + 8 * c + 4);
        if (size == L) {
            memcpy(dst + c * LCO_CHUNK, p, L);
        } else if (lco_unrze2(p, size, L, z) != 0) {
            rc = LCO_CORRUPT_STREAM;
        } else {
            lco_unbit8(z, L, y);
            lco_untupl8_1(y, L, dst + c * LCO_CHUNK);
        }
    }
    free(z);
    free(y);
    return rc;
}
