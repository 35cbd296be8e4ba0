// Host-side checks of the C ABI under AddressSanitizer and UBSan.
//
// Built by tests/test_api_sanitized.py from fp8_kv_cache_amd/csrc/api.cpp and
// lc_api.cpp (host code instrumented, device code as usual) with this file,
// which replaces every kernel launcher by a stub that only counts its calls.
// Nothing touches a GPU: the device pointers below are never dereferenced.
// Each case states the status the header documents and whether the call
// may reach a launcher: argument errors must return before any launch, and
// valid calls must reach one.  The size queries are swept over the edges of
// their domains (n up to 2^64 - 1, count up to 2^32 - 1), where a wrapped
// product would be a bug.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lc_codec.h"
#include "lc_internal.h"
#include "splitzip.h"
#include "sz_internal.h"

// The same entry points seen from C, where an enum argument is any int:
// declared with int parameters and bound to the same symbols, so that the
// calls below pass raw ints as a C caller would.
extern "C" {
const char* c_status_string(int status) __asm__("sz_status_string");
uint64_t c_max_compressed_bytes(uint64_t n, int dtype) __asm__("sz_max_compressed_bytes");
uint64_t c_encode_workspace_bytes(uint64_t n, int dtype) __asm__("sz_encode_workspace_bytes");
uint64_t c_compress_workspace_bytes(uint64_t n, int dtype) __asm__("sz_compress_workspace_bytes");
int c_build_codebook(const uint64_t* d_hist, int dtype, uint8_t* d_codebook, hipStream_t stream)
    __asm__("sz_build_codebook");
int c_histogram(const void* d_src, uint64_t n, int dtype, uint64_t* d_hist, hipStream_t stream)
    __asm__("sz_histogram");
}

static int g_launches = 0;
static int g_failures = 0;

namespace sz {
hipError_t launch_fill_u64(uint64_t*, uint64_t, uint64_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fill_i32(int32_t*, uint64_t, int32_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_histogram(const HistArgs& a, uint32_t, hipStream_t) {
    ++g_launches;
    return a.count && a.n ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_codebook(const CodebookArgs& a, uint32_t, hipStream_t) {
    ++g_launches;
    return a.count ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_encode(const EncodeArgs& a, uint32_t, hipStream_t) {
    ++g_launches;
    return a.count && a.n && a.counts && a.staging ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_encode_empty(const EncodeArgs&, uint32_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_compress(const CompressArgs& a, uint32_t, hipStream_t) {
    ++g_launches;
    return a.enc.count && a.enc.n && a.sync && a.sample_items ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_decode(const DecodeArgs& a, uint32_t, hipStream_t) {
    ++g_launches;
    return a.count && a.n ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_decode_empty(const DecodeArgs&, uint32_t, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace sz

namespace lc {
hipError_t launch_encode(const EncodeArgs& a, hipStream_t) {
    ++g_launches;
    return a.count ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
    ++g_launches;
    return a.count ? hipSuccess : hipErrorInvalidValue;
}
}  // namespace lc

#define EXPECT(call, want_status, want_launch)                                                           \
    do {                                                                                                 \
        const int before = g_launches;                                                                   \
        const int got = static_cast<int>(call);                                                          \
        const bool launched = g_launches != before;                                                      \
        if (got != static_cast<int>(want_status) || launched != (want_launch)) {                         \
            printf("FAIL line %d: %s -> status %d (want %d), launched %d (want %d)\n", __LINE__, #call, got, \
                   static_cast<int>(want_status), launched, static_cast<int>(want_launch));              \
            ++g_failures;                                                                                \
        }                                                                                                \
    } while (0)

int main() {
    // device pointers: 16-byte aligned, never dereferenced
    char* const F = reinterpret_cast<char*>(0x7F0000000000ull);
    void* const P = F;
    void* const M = F + 2;   // misaligned
    const void* const* T = reinterpret_cast<const void* const*>(F + 0x1000);
    void* const* D = reinterpret_cast<void* const*>(F + 0x2000);
    uint64_t* const H = reinterpret_cast<uint64_t*>(F + 0x3000);
    uint8_t* const C = reinterpret_cast<uint8_t*>(F + 0x4000);
    uint64_t* const O = reinterpret_cast<uint64_t*>(F + 0x5000);
    int32_t* const S = reinterpret_cast<int32_t*>(F + 0x6000);
    const sz_dtype B = SZ_DTYPE_BF16, E = SZ_DTYPE_FP8_E5M2, BAD = static_cast<sz_dtype>(3);
    const uint64_t BIG = uint64_t(1) << 40;   // a capacity or workspace size that always suffices
    const uint64_t n = 5000;

    // ---- size queries over the edges of their domains
    const uint64_t ns[] = {0, 1, 4095, 4096, 4097, (uint64_t(1) << 24), (uint64_t(1) << 32) - 1, uint64_t(1) << 32,
                           ~uint64_t(0)};
    const uint32_t counts[] = {0, 1, 2, 64, 1u << 16, 0xFFFFFFFFu};
    for (uint64_t x : ns) {
        for (sz_dtype dt : {B, E, BAD}) {
            const uint64_t m = sz_max_compressed_bytes(x, dt);
            if ((dt == BAD || x >= (uint64_t(1) << 32)) != (m == 0)) {
                printf("FAIL max bytes n=%llu dt=%d -> %llu\n", (unsigned long long)x, (int)dt, (unsigned long long)m);
                ++g_failures;
            }
            for (uint32_t c : counts) {
                const uint64_t w = sz_encode_workspace_bytes_batched(c, x, dt);
                const uint64_t cw = sz_compress_workspace_bytes_batched(c, x, dt);
                const uint64_t blocks = x < (uint64_t(1) << 32) ? (x + 4095) / 4096 : 0;
                const bool fits = dt != BAD && c && x && x < (uint64_t(1) << 32) &&
                                  static_cast<double>(c) * static_cast<double>(blocks) < 2147483648.0;
                if (fits && (w == 0 || w < static_cast<uint64_t>(c) * blocks * 4096)) {
                    printf("FAIL encode workspace c=%u n=%llu -> %llu\n", c, (unsigned long long)x,
                           (unsigned long long)w);
                    ++g_failures;
                }
                if (!fits && w != 0) {
                    printf("FAIL encode workspace c=%u n=%llu not rejected -> %llu\n", c, (unsigned long long)x,
                           (unsigned long long)w);
                    ++g_failures;
                }
                if (cw && cw < w) {
                    printf("FAIL compress workspace below encode workspace c=%u n=%llu\n", c, (unsigned long long)x);
                    ++g_failures;
                }
            }
        }
        for (uint32_t c : counts) (void)lc_encode_workspace_bytes_batched(c, x);
        (void)lc_max_compressed_bytes(x);
    }
    // enum arguments a C caller can pass: any int, in or out of the enumerators' range
    const int odd[] = {-1, 0, 1, 2, 3, 6, 7, 100, 0x7FFFFFFF};
    for (int v : odd) {
        const bool valid = v == 1 || v == 2;
        (void)c_status_string(v);
        if ((c_max_compressed_bytes(4096, v) != 0) != valid || (c_encode_workspace_bytes(4096, v) != 0) != valid ||
            (c_compress_workspace_bytes(4096, v) != 0) != valid) {
            printf("FAIL dtype %d in the size queries\n", v);
            ++g_failures;
        }
        EXPECT(c_build_codebook(reinterpret_cast<const uint64_t*>(0x7F0000000000ull), v,
                                reinterpret_cast<uint8_t*>(0x7F0000001000ull), nullptr),
               valid ? SZ_OK : SZ_ERR_INVALID_ARGUMENT, valid);
        EXPECT(c_histogram(reinterpret_cast<const void*>(0x7F0000000000ull), 100, v,
                           reinterpret_cast<uint64_t*>(0x7F0000001000ull), nullptr),
               valid ? SZ_OK : SZ_ERR_INVALID_ARGUMENT, valid);
    }
    if (sz_abi_version() != SZ_ABI_VERSION) {
        printf("FAIL abi version\n");
        ++g_failures;
    }

    const uint64_t cap = sz_max_compressed_bytes(n, B);
    const uint64_t ws = sz_encode_workspace_bytes(n, B);
    const uint64_t cws = sz_compress_workspace_bytes(n, B);
    const sz_compress_options bad_opts = {0, 0, 1};
    const sz_compress_options fuse_all = {1, 0, 0};

    // ---- histogram
    EXPECT(sz_histogram(P, n, B, H, nullptr), SZ_OK, true);
    EXPECT(sz_histogram(P, 0, B, H, nullptr), SZ_OK, true);            // fills the histogram with zeros
    EXPECT(sz_histogram(nullptr, 0, B, H, nullptr), SZ_OK, true);
    EXPECT(sz_histogram(nullptr, n, B, H, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_histogram(M, n, B, H, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_histogram(P, n, BAD, H, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_histogram(P, uint64_t(1) << 32, B, H, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_histogram(P, n, B, nullptr, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_histogram_sampled(P, n, E, 64, H, nullptr), SZ_OK, true);
    EXPECT(sz_histogram_sampled(P, n, E, 0, H, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_histogram_batched(T, 2, n, B, H, nullptr), SZ_OK, true);
    EXPECT(sz_histogram_batched(T, 0, n, B, H, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_histogram_batched(T, 0xFFFFFFFFu, n, B, H, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_histogram_batched(nullptr, 2, n, B, H, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_histogram_sampled_batched(T, 2, n, B, 8, H, nullptr), SZ_OK, true);
    EXPECT(sz_histogram_sampled_batched(T, 2, n, B, 0, H, nullptr), SZ_ERR_INVALID_ARGUMENT, false);

    // ---- codebook
    EXPECT(sz_build_codebook(H, B, C, nullptr), SZ_OK, true);
    EXPECT(sz_build_codebook(H, BAD, C, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_build_codebook(nullptr, B, C, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_build_codebook_batched(H, 0, B, C, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_build_codebook_batched(H, 3, E, C, nullptr), SZ_OK, true);

    // ---- encode
    EXPECT(sz_encode(P, n, B, C, P, cap, O, P, ws, nullptr), SZ_OK, true);
    EXPECT(sz_encode(P, 0, B, C, P, cap, O, nullptr, 0, nullptr), SZ_OK, true);   // header only
    EXPECT(sz_encode(P, n, B, C, P, cap - 1, O, P, ws, nullptr), SZ_ERR_BUFFER_TOO_SMALL, false);
    EXPECT(sz_encode(P, n, B, C, P, cap, O, P, ws - 1, nullptr), SZ_ERR_BUFFER_TOO_SMALL, false);
    EXPECT(sz_encode(P, n, B, C, P, cap, O, nullptr, ws, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_encode(P, n, B, C, P, cap, reinterpret_cast<uint64_t*>(F + 4), P, ws, nullptr),
           SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_encode(P, n, B, nullptr, P, cap, O, P, ws, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_encode(P, n, B, C, M, cap, O, P, ws, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_encode(P, uint64_t(1) << 32, B, C, P, BIG, O, P, BIG, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_encode_batched(T, 2, n, E, C, D, sz_max_compressed_bytes(n, E), O, P,
                             sz_encode_workspace_bytes_batched(2, n, E), nullptr),
           SZ_OK, true);
    EXPECT(sz_encode_batched(T, 2, n, E, C, D, sz_max_compressed_bytes(n, E), O, P,
                             sz_encode_workspace_bytes_batched(2, n, E) - 1, nullptr),
           SZ_ERR_BUFFER_TOO_SMALL, false);
    EXPECT(sz_encode_batched(T, 0x80000000u, 4096, B, C, D, BIG, O, P, BIG, nullptr), SZ_ERR_INVALID_ARGUMENT, false);

    // ---- compress (one launch, or the separate kernels below the fused size)
    EXPECT(sz_compress(P, n, B, H, C, P, cap, O, S, P, cws, nullptr, nullptr), SZ_OK, true);
    EXPECT(sz_compress(P, n, B, H, C, P, cap, O, S, P, cws, &fuse_all, nullptr), SZ_OK, true);
    EXPECT(sz_compress(P, 0, B, H, C, P, cap, O, S, P, cws, nullptr, nullptr), SZ_OK, true);
    EXPECT(sz_compress(P, n, B, H, C, P, cap, O, S, P, cws, &bad_opts, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_compress(P, n, B, H, C, P, cap, O, S, P, cws - 1, nullptr, nullptr), SZ_ERR_BUFFER_TOO_SMALL, false);
    EXPECT(sz_compress(P, n, B, H, C, P, cap, O, reinterpret_cast<int32_t*>(F + 2), P, cws, nullptr, nullptr),
           SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_compress(P, n, B, H, C, P, cap, O, S, nullptr, cws, nullptr, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_compress_batched(T, 3, n, B, H, C, D, cap, O, S, P, sz_compress_workspace_bytes_batched(3, n, B),
                               &fuse_all, nullptr),
           SZ_OK, true);
    EXPECT(sz_compress_batched(T, 3, n, B, H, C, D, cap, O, S, P, sz_compress_workspace_bytes_batched(3, n, B) - 1,
                               nullptr, nullptr),
           SZ_ERR_BUFFER_TOO_SMALL, false);
    EXPECT(sz_compress_batched(T, 0, n, B, H, C, D, cap, O, S, P, BIG, nullptr, nullptr), SZ_ERR_INVALID_ARGUMENT,
           false);
    EXPECT(sz_compress_noalloc(P, (uint64_t(1) << 24) + 1, B, H, C, P, BIG, O, S, nullptr, nullptr),
           SZ_ERR_BUFFER_TOO_SMALL, false);
    EXPECT(sz_compress_noalloc(P, n, B, H, C, P, cap, O, S, &bad_opts, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_compress_noalloc(P, n, B, H, C, P, cap - 1, O, S, nullptr, nullptr), SZ_ERR_BUFFER_TOO_SMALL, false);

    // ---- decode
    EXPECT(sz_decode(P, cap, n, B, P, S, nullptr), SZ_OK, true);
    EXPECT(sz_decode(P, 64, n, B, P, S, nullptr), SZ_ERR_CORRUPT_STREAM, false);
    EXPECT(sz_decode(P, cap, 0, B, nullptr, S, nullptr), SZ_OK, true);
    EXPECT(sz_decode(nullptr, cap, n, B, P, S, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_decode(P, cap, n, B, P, reinterpret_cast<int32_t*>(F + 1), nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(sz_decode_batched(T, O, 2, n, E, D, S, nullptr), SZ_OK, true);
    EXPECT(sz_decode_batched(T, nullptr, 2, n, E, D, S, nullptr), SZ_ERR_INVALID_ARGUMENT, false);

    // ---- the LC-style comparison codec
    const uint64_t lcap = lc_max_compressed_bytes(100000), lws = lc_encode_workspace_bytes(100000);
    EXPECT(lc_encode(P, 100000, P, lcap, O, P, lws, nullptr), SZ_OK, true);
    EXPECT(lc_encode(P, 100000, P, lcap - 1, O, P, lws, nullptr), SZ_ERR_BUFFER_TOO_SMALL, false);
    EXPECT(lc_encode(P, 100000, P, lcap, O, P, lws - 1, nullptr), SZ_ERR_BUFFER_TOO_SMALL, false);
    EXPECT(lc_encode(P, uint64_t(1) << 31, P, BIG, O, P, BIG, nullptr), SZ_ERR_INVALID_ARGUMENT, false);
    EXPECT(lc_decode(P, lcap, 100000, P, S, nullptr), SZ_OK, true);
    EXPECT(lc_decode(P, 10, 100000, P, S, nullptr), SZ_ERR_CORRUPT_STREAM, false);
    EXPECT(lc_encode_batched(T, 2, 100000, D, lcap, O, P, lc_encode_workspace_bytes_batched(2, 100000), nullptr),
           SZ_OK, true);
    EXPECT(lc_decode_batched(T, O, 2, 100000, D, S, nullptr), SZ_OK, true);
    EXPECT(lc_decode_batched(T, O, 0, 100000, D, S, nullptr), SZ_ERR_INVALID_ARGUMENT, false);

    if (g_failures) {
        printf("%d failure(s)\n", g_failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
