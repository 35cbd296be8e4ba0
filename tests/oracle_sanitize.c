/* Drives both CPU oracles under AddressSanitizer and UBSan (built by
 * tests/test_oracle_sanitized.py with gcc; CPU only): random inputs of many
 * lengths round-trip, and every decode of a stream with one random byte
 * flipped, or cut short, returns without reading outside its buffers. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint64_t szo_max_bytes(uint64_t n, int dt);
int szo_encode(const void* src, uint64_t n, int dt, const uint8_t* cb, uint8_t* dst, uint64_t cap, uint64_t* out);
int szo_decode(const uint8_t* src, uint64_t src_bytes, uint64_t n, int dt, void* dst);
uint64_t lco_max_bytes(uint64_t n);
int lco_encode(const void* src, uint64_t n, uint8_t* dst, uint64_t cap, uint64_t* out);
int lco_decode(const uint8_t* src, uint64_t src_bytes, uint64_t n, void* dst);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {            /* xorshift64* */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return state * 0x2545F4914F6CDD1Dull;
}

/* a copy of exactly `len` bytes, so that any over-read is caught */
static uint8_t* exact_copy(const uint8_t* p, uint64_t len) {
    uint8_t* q = malloc(len ? len : 1);
    memcpy(q, p, len);
    return q;
}

static int check_sz(uint64_t n, int dt, int mode) {
    uint64_t w = dt == 1 ? 2 : 1, bytes = n * w;
    uint8_t* x = malloc(bytes ? bytes : 1);
    for (uint64_t i = 0; i < bytes; i++) x[i] = (uint8_t)next();
    if (mode == 1 && dt == 1)          /* few exponents: mostly coded, some escapes */
        for (uint64_t i = 0; i < n; i++) x[2 * i + 1] = (uint8_t)((x[2 * i + 1] & 0x80) | (0x3C + next() % 6));
    uint64_t cap = szo_max_bytes(n, dt), size = 0;
    uint8_t* s = malloc(cap);
    if (szo_encode(n ? x : NULL, n, dt, NULL, s, cap, &size) != 0) return 1;
    uint8_t* y = malloc(bytes ? bytes : 1);
    uint8_t* t = exact_copy(s, size);
    if (szo_decode(t, size, n, dt, y) != 0 || memcmp(x, y, bytes) != 0) return 2;
    for (int k = 0; k < 8 && size; k++) {            /* one byte flipped: any status, no bad access */
        uint64_t at = next() % size;
        t[at] ^= (uint8_t)(1u + next() % 255);
        (void)szo_decode(t, size, n, dt, y);
        memcpy(t, s, size);
    }
    uint8_t* cut = exact_copy(s, size / 2);          /* cut short */
    if (size && szo_decode(cut, size / 2, n, dt, y) == 0) return 3;
    free(cut); free(t); free(y); free(s); free(x);
    return 0;
}

static int check_lc(uint64_t n, int mode) {
    uint8_t* x = malloc(n ? n : 1);
    for (uint64_t i = 0; i < n; i++) {
        uint8_t v = (uint8_t)next();
        x[i] = mode == 0 ? v : mode == 1 ? (uint8_t)(v & 0x0F) : (next() % 16 ? 0 : v);
    }
    uint64_t cap = lco_max_bytes(n), size = 0;
    uint8_t* s = malloc(cap);
    if (lco_encode(n ? x : NULL, n, s, cap, &size) != 0) return 1;
    uint8_t* y = malloc(n ? n : 1);
    uint8_t* t = exact_copy(s, size);
    if (lco_decode(t, size, n, y) != 0 || memcmp(x, y, n) != 0) return 2;
    for (int k = 0; k < 8; k++) {
        uint64_t at = next() % size;
        t[at] ^= (uint8_t)(1u + next() % 255);
        (void)lco_decode(t, size, n, y);
        memcpy(t, s, size);
    }
    uint8_t* cut = exact_copy(s, size / 2);
    if (lco_decode(cut, size / 2, n, y) == 0) return 3;
    free(cut); free(t); free(y); free(s); free(x);
    return 0;
}

int main(void) {
    const uint64_t sizes[] = {0, 1, 2, 3, 15, 16, 17, 4095, 4096, 4097, 8191, 12289, 16383, 16384, 16385, 40000, 70001};
    for (unsigned i = 0; i < sizeof sizes / sizeof sizes[0]; i++) {
        for (int dt = 1; dt <= 2; dt++)
            for (int mode = 0; mode < 2; mode++) {
                int rc = check_sz(sizes[i], dt, mode);
                if (rc) { printf("exponent codec n=%llu dt=%d mode=%d failed %d\n", (unsigned long long)sizes[i], dt, mode, rc); return 1; }
            }
        for (int mode = 0; mode < 3; mode++) {
            int rc = check_lc(sizes[i], mode);
            if (rc) { printf("lc n=%llu mode=%d failed %d\n", (unsigned long long)sizes[i], mode, rc); return 1; }
        }
    }
    printf("ok\n");
    return 0;
}
