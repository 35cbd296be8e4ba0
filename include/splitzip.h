/*
 * splitzip.h -- C ABI of the MI355X (gfx950) lossless exponent codec for
 * BF16 and FP8-E5M2 KV-cache tensors.
 *
 * The method is SplitZip's (SplitZip project page, "Abstract"): the most
 * frequent exponent values of a tensor get constant-width 4-bit codes, sign and
 * mantissa bits are kept as they are, and rare exponent values are routed
 * through a separate escape stream; decoding is bit-exact (FAQ "Is
 * SplitZip lossy?"), also for FP8 E5M2 KV caches (FAQ "Does it work with
 * an FP8 KV cache?").
 *
 * ---- Stream format v1 (little-endian; A(x) = x rounded up to 256) -------
 *   0   u8[4]  'S','Z','K','V'          24  u8[16] codebook cb[0..14], cb[15]=0
 *   4   u8     version = 1              40  u64    C, total stream bytes
 *   5   u8     dtype (sz_dtype)         48  u8[16] reserved, zero
 *   6   u8     log2 block size = 12     64  u32[B] escape offsets (B = ceil(n/4096)),
 *   7   u8     coded exponents = 15                zeros up to H = A(64 + 4B)
 *   8   u64    n                        H   sign|mantissa plane, S bytes, zeros to A(S)
 *   16  u64    E, number of escapes     ..  code plane, ceil(n/2) bytes, zeros to A(.)
 *                                       ..  E escape bytes
 *   C = H + A(S) + A(ceil(n/2)) + E.
 *   BF16: exponent = bits 14..7 (8 bits); plane byte = sign<<7 | mantissa (7).
 *         S = n.
 *   E5M2: exponent = bits 6..2 (5 bits); plane field = sign<<2 | mantissa (2),
 *         3 bits per element packed LSB-first (element i at bits 3i..3i+2).
 *         S = ceil(3n/8).
 *   Codes: cb[c] is the exponent of code c (c < 15); code 15 is the escape.
 *         Element 2i is the low nibble of code byte i, 2i+1 the high nibble.
 *   Escapes: one byte per escaped element (its raw exponent), element order.
 *         off[b] = escapes before element 4096*b.
 *   Codebook built by sz_build_codebook: all exponent values of the type
 *         (256 for BF16, 32 for E5M2) ranked by count, descending, ties to
 *         the smaller exponent; code c = rank c.
 *
 * ---- Conventions ---------------------------------------------------------
 *   Pointers named d_* are HIP device memory owned by the caller.  Element,
 *   stream and workspace buffers must be 16-byte aligned.  Every call is
 *   asynchronous on `stream` (may be NULL for the null stream); the library
 *   never allocates, frees or synchronises.  Argument errors detectable on
 *   the host are returned before anything is enqueued.  A launch failure
 *   returns SZ_ERR_HIP.  0 <= n < 2^32 for every call.
 *   Calls sharing a workspace or output buffer must not overlap in time.
 */
#ifndef SPLITZIP_H
#define SPLITZIP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SZ_DTYPE_BF16 = 1,
    SZ_DTYPE_FP8_E5M2 = 2
} sz_dtype;

typedef enum {
    SZ_OK = 0,
    SZ_ERR_INVALID_ARGUMENT = 1,  /* null/misaligned pointer, bad dtype, n >= 2^32 */
    SZ_ERR_BUFFER_TOO_SMALL = 2,  /* output or workspace capacity below the bound */
    SZ_ERR_CORRUPT_STREAM = 3,    /* stream does not match n / dtype or its own header */
    SZ_ERR_HIP = 4,               /* a kernel launch failed */
    SZ_ERR_TIMEOUT = 5            /* sz_compress*: gave up waiting for a tensor's codebook */
} sz_status;

/* Largest stream sz_encode can write for n elements with ANY codebook
 * (every element may escape): H + A(S) + A(ceil(n/2)) + n.  Pure host
 * function; returns 0 for an invalid dtype or n >= 2^32. */
uint64_t sz_max_compressed_bytes(uint64_t n, sz_dtype dtype);

/* Workspace sz_encode needs: a u32 escape count per 4096-element block
 * (rounded up to 256 bytes), then 4096 staging bytes per block -- about one
 * byte per element.  Escapes are staged per block so that no workgroup ever
 * waits for another.  Pure host function; 0 on bad input or n = 0. */
uint64_t sz_encode_workspace_bytes(uint64_t n, sz_dtype dtype);

/* Exponent histogram (SplitZip "Abstract": exponent values are highly
 * redundant, so count them).  d_src: n elements (BF16 as 16-bit words,
 * E5M2 as bytes).  d_hist: 256 u64 counters, overwritten; for E5M2 only
 * bins 0..31 can be non-zero. */
sz_status sz_histogram(const void* d_src, uint64_t n, sz_dtype dtype,
                       uint64_t* d_hist, hipStream_t stream);

/* Histogram of a block sample -- an extension; the pages define no
 * sampling.  Only the 4096-element format blocks b with b % block_stride
 * == 0 are counted (block_stride >= 1; 1 gives sz_histogram's result).  The
 * premise is the "Abstract"'s observation that KV exponents are highly
 * repetitive, so a sample ranks them like the whole tensor; a codebook
 * built from it still yields a valid lossless stream (sz_encode accepts any
 * codebook), and encode then reads the input about once instead of twice.
 * d_hist: 256 u64, overwritten. */
sz_status sz_histogram_sampled(const void* d_src, uint64_t n, sz_dtype dtype, uint32_t block_stride,
                               uint64_t* d_hist, hipStream_t stream);

/* Codebook from a histogram ("Abstract": the most frequent exponent values
 * get the 4-bit codes).  d_hist: 256 u64 (device).  d_codebook: 16
 * bytes written as cb[0..14] = exponents of rank 0..14 (count descending,
 * then exponent ascending), cb[15] = 0. */
sz_status sz_build_codebook(const uint64_t* d_hist, sz_dtype dtype,
                            uint8_t* d_codebook, hipStream_t stream);

/* Encode one tensor ("Abstract"; FAQ "Is SplitZip lossy?").  d_codebook:
 * 16 device bytes, any values (a value listed twice takes its lowest code;
 * cb[15] is ignored and stored as 0).  d_dst receives the whole stream;
 * dst_capacity must be >= sz_max_compressed_bytes(n, dtype), else
 * SZ_ERR_BUFFER_TOO_SMALL.  d_out_bytes (u64 in device memory or in
 * device-accessible pinned host memory, may be NULL) receives C.
 * d_workspace: >= sz_encode_workspace_bytes(n, dtype) bytes (may be NULL
 * when n = 0), contents need not be initialised, clobbered. */
sz_status sz_encode(const void* d_src, uint64_t n, sz_dtype dtype,
                    const uint8_t* d_codebook, void* d_dst, uint64_t dst_capacity,
                    uint64_t* d_out_bytes, void* d_workspace, uint64_t workspace_bytes,
                    hipStream_t stream);

/* Decode one stream (FAQ "Is SplitZip lossy?": bit-exact output).
 * d_src: src_bytes readable bytes holding the stream (C <= src_bytes).
 * d_dst: n elements.  The stream is validated on the device against n,
 * dtype, src_bytes and its own header and offsets; if it does not match,
 * *d_status (device int32, may be NULL) is set to SZ_ERR_CORRUPT_STREAM,
 * the output is unspecified, and no access leaves [d_src, d_src+src_bytes)
 * or [d_dst, d_dst + n elements).  Otherwise *d_status is set to SZ_OK.
 * Returns SZ_ERR_CORRUPT_STREAM without launching if src_bytes is smaller
 * than any stream of n elements can be. */
sz_status sz_decode(const void* d_src, uint64_t src_bytes, uint64_t n, sz_dtype dtype,
                    void* d_dst, int32_t* d_status, hipStream_t stream);

/* ---- Batched forms: T tensors of the same n and dtype in one launch per
 * phase (one codebook per tensor, as for a KV cache's layer tensors).  The
 * d_*s pointer tables are device arrays of T device pointers, each pointing
 * to a 16-byte aligned buffer.  Results are byte-identical to T
 * single-tensor calls.  T * ceil(n / 4096) must stay below 2^31, else
 * SZ_ERR_INVALID_ARGUMENT. ---- */

/* 0 for count = 0 or a batch the calls reject for its size, as for a bad
 * dtype or n (the same holds for sz_compress_workspace_bytes_batched). */
uint64_t sz_encode_workspace_bytes_batched(uint32_t count, uint64_t n, sz_dtype dtype);

/* d_hists: count x 256 u64 */
sz_status sz_histogram_batched(const void* const* d_srcs, uint32_t count, uint64_t n,
                               sz_dtype dtype, uint64_t* d_hists, hipStream_t stream);

/* d_hists: count x 256 u64 */
sz_status sz_histogram_sampled_batched(const void* const* d_srcs, uint32_t count, uint64_t n,
                                       sz_dtype dtype, uint32_t block_stride, uint64_t* d_hists,
                                       hipStream_t stream);

/* d_hists: count x 256 u64; d_codebooks: count x 16 bytes */
sz_status sz_build_codebook_batched(const uint64_t* d_hists, uint32_t count, sz_dtype dtype,
                                    uint8_t* d_codebooks, hipStream_t stream);

/* d_codebooks: count x 16 bytes; every d_dsts[t] holds dst_capacity bytes;
 * d_out_bytes: count u64 (may be NULL). */
sz_status sz_encode_batched(const void* const* d_srcs, uint32_t count, uint64_t n,
                            sz_dtype dtype, const uint8_t* d_codebooks,
                            void* const* d_dsts, uint64_t dst_capacity, uint64_t* d_out_bytes,
                            void* d_workspace, uint64_t workspace_bytes, hipStream_t stream);

/* d_src_bytes: count u64 (device), readable bytes of each stream, e.g. the
 * d_out_bytes array an encode wrote.  d_status: count int32 (may be NULL). */
sz_status sz_decode_batched(const void* const* d_srcs, const uint64_t* d_src_bytes,
                            uint32_t count, uint64_t n, sz_dtype dtype,
                            void* const* d_dsts, int32_t* d_status, hipStream_t stream);

/* ---- One launch: histogram, codebook and encode together.  Computes
 * exactly what sz_histogram + sz_build_codebook + sz_encode compute (the
 * same histogram, codebook and stream bytes), for one tensor or, batched,
 * for T tensors of the same n and dtype.
 *
 * The codebook of a tensor needs all of its exponents ("Abstract": the
 * most frequent exponent values get the codes), so the separate calls read
 * every input twice: a histogram pass, then the encode.  This call reads
 * it once.  One kernel counts a 1/16 sample of each tensor (every 16th
 * 128 KB chunk) and ranks it into a provisional codebook; then it encodes
 * every full 4096-element block with that codebook while counting the
 * block into the tensor's full histogram; then it ranks the full histogram
 * into the final codebook.  The sample nearly always ranks the same values
 * in the same order.  Where it does not (12 of the 64 tensors of the
 * Llama-shaped BF16 cache), a short second kernel recodes that tensor's
 * code nibbles and staged escapes for the final codebook from what was
 * written, without reading the input again; the partial last block is
 * encoded with the final codebook afterwards.  A tensor of which more than
 * a quarter of the sample escapes under its own provisional codebook (an
 * escape-heavy tensor, where the final codebook nearly always differs and a
 * recode would rewrite most of the stream) is only counted in the first
 * kernel and encoded from its input by the second, with the final codebook,
 * its escapes written straight to their place (from per-item histograms the
 * first kernel keeps in the workspace).  The bytes written are the same as
 * the separate calls'.  Tensors below
 * the options' fused_min_elements run the separate calls' kernels, with the
 * same results; by default that is BF16 tensors under 2^21 elements, and
 * E5M2 tensors under 2^22 elements or in calls of fewer than 2^28 elements
 * in all (measured faster with the separate kernels).
 *
 * Work inside the kernel waits only for work of lower workgroup ids, which
 * the dispatcher starts first on each XCD, so a call makes progress
 * whatever else shares the GPU.  Waits are
 * bounded nonetheless: a workgroup that has polled the options' spin_limit
 * times without progress (about a second) gives up, and so does every
 * workgroup after it; each tensor they belong to gets SZ_ERR_TIMEOUT in
 * d_status, unspecified histogram and codebook, and a stream that stays
 * inside dst_capacity and starts with a zero magic, so that sz_decode
 * reports it as SZ_ERR_CORRUPT_STREAM even when d_status is NULL.
 *
 * d_hist(s): 256 (count x 256) u64, written.  d_codebook(s): 16 (count x
 * 16) bytes, written.  d_dst(s), dst_capacity, d_out_bytes: as sz_encode.
 * d_status: 1 (count) int32, SZ_OK or SZ_ERR_TIMEOUT, may be NULL.
 * Batched: T x (ceil(ceil(n / K) / 16) + ceil(ceil(n / 4096) / M) + 2),
 * the kernel's work items (K = 65536 and M = 16 for BF16, K = 131072 and
 * M = 32 for E5M2: one 128 KB sample chunk, one 128 KB main item), must
 * stay below 2^31 as well, else SZ_ERR_INVALID_ARGUMENT.
 * d_workspace: >= sz_compress_workspace_bytes[_batched] bytes, contents
 * need not be initialised, clobbered (the encode workspace followed by a
 * synchronisation area: 256 bytes plus 2048 x (R + 1) + 320 bytes per
 * tensor, with R = 16, 8, 4, 2 or 1 copies of each tensor's histogram for
 * calls of 1, 2-3, 4-7, 8-15 or more tensors).  Calls
 * sharing a workspace must not overlap in time.
 * options: per-call settings (host memory, read when the call is enqueued),
 * or NULL for the defaults; an options struct with a non-zero reserved
 * field is SZ_ERR_INVALID_ARGUMENT. ---- */

typedef struct {
    /* Smallest tensor (in elements) run through the one-launch kernel;
     * smaller ones take the separate calls' kernels (same results).  0 means
     * the defaults: 2^21 for BF16 (4 MiB tensors measured 15% faster fused,
     * 2 MiB ones 10% slower), and for E5M2 2^22 in calls of at least 2^28
     * elements (smaller calls measured as fast or faster separately); 1
     * sends every tensor of either type through the one-launch kernel. */
    uint64_t fused_min_elements;
    /* Polls a waiting workgroup makes before it gives up; 0 means the
     * default, 2^20 (about a second).  A small value reaches the give-up
     * path. */
    uint32_t spin_limit;
    uint32_t reserved;   /* must be 0 */
} sz_compress_options;

uint64_t sz_compress_workspace_bytes(uint64_t n, sz_dtype dtype);
uint64_t sz_compress_workspace_bytes_batched(uint32_t count, uint64_t n, sz_dtype dtype);

sz_status sz_compress(const void* d_src, uint64_t n, sz_dtype dtype, uint64_t* d_hist,
                      uint8_t* d_codebook, void* d_dst, uint64_t dst_capacity, uint64_t* d_out_bytes,
                      int32_t* d_status, void* d_workspace, uint64_t workspace_bytes,
                      const sz_compress_options* options, hipStream_t stream);

sz_status sz_compress_batched(const void* const* d_srcs, uint32_t count, uint64_t n, sz_dtype dtype,
                              uint64_t* d_hists, uint8_t* d_codebooks, void* const* d_dsts,
                              uint64_t dst_capacity, uint64_t* d_out_bytes, int32_t* d_status,
                              void* d_workspace, uint64_t workspace_bytes,
                              const sz_compress_options* options, hipStream_t stream);

/* ---- sz_compress without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It computes exactly what sz_compress
 * computes (same histogram, codebook, stream and status), for one tensor of
 * n <= SZ_NOALLOC_MAX_ELEMENTS elements (else SZ_ERR_BUFFER_TOO_SMALL,
 * before anything is enqueued), with its workspace in a scratch array of
 * SZ_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends.  The current device's array is used, so `stream`
 * must belong to the current device.  No call allocates or frees anything.
 * Every call on one device shares that device's array and leaves its own
 * contents there (the call clears what must start at zero), so calls that
 * overlap in time on one device race: issue them on one stream, or order
 * them.  Other arguments as sz_compress. ---- */
#define SZ_NOALLOC_MAX_ELEMENTS (1ull << 24)
#define SZ_NOALLOC_SCRATCH_BYTES ((16ull << 20) + (64ull << 10))

sz_status sz_compress_noalloc(const void* d_src, uint64_t n, sz_dtype dtype, uint64_t* d_hist,
                              uint8_t* d_codebook, void* d_dst, uint64_t dst_capacity, uint64_t* d_out_bytes,
                              int32_t* d_status, const sz_compress_options* options, hipStream_t stream);

/* Static description of a status code. */
const char* sz_status_string(sz_status status);

/* ---- ABI version of the library: SZ_ABI_VERSION as it was compiled.  A
 * binding built against one revision of this header checks it at load and
 * refuses a library from another revision, whose signatures or size rules
 * may differ (calling through mismatched signatures passes garbage
 * pointers).  Bumped whenever a signature, a struct or a size rule here
 * changes. ---- */
#define SZ_ABI_VERSION 4u
uint32_t sz_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPLITZIP_H */
