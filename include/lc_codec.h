/*
 * lc_codec.h -- C ABI of the LC-style comparison codec on MI355X (gfx950):
 * a generic lossless byte-transform chain, TUPL8_1 -> BIT_8 -> RZE_2, run
 * on the same KV-cache tensors as the exponent codec so that the two can
 * be compared on equal terms.
 *
 * Source: FastKVComp companion page, "Inside an LC-style pipeline": a chain
 * of TUPL8_1 and BIT_8, two stages that permute bits without changing the
 * size, feeding RZE_2, which shrinks the data by leaving out zero words (the
 * page sets this chain against nvCOMP).
 * The page gives no stage internals; the readings taken are:
 *
 *   L1 the input (n bytes, n < 2^31) is cut into chunks of 16384 bytes, the
 *      last one shorter; every chunk is coded on its own.
 *   L2 TUPL8_1: with q = floor(L/8), byte 8i+j moves to j*q+i (i < q,
 *      j < 8) -- eight byte streams; the last L mod 8 bytes stay.
 *   L3 BIT_8: with W = floor(L/8) little-endian 64-bit words and
 *      G = floor(W/8), plane b (b < 64) is G bytes; bit a of plane byte s is
 *      bit b of word 8s+a (bit b of a word = bit b%8 of its byte b/8).
 *      Bytes from 64G on stay.
 *   L4 RZE_2: with V = floor(L/2) little-endian 16-bit words: a bitmap of
 *      ceil(V/8) bytes (bit m%8 of byte m/8 set iff word m is non-zero),
 *      the non-zero words in order, then the last byte if L is odd.
 *   L5 a chunk whose RZE_2 output is not shorter than the chunk is stored
 *      raw; a chunk's stored size equals its length exactly when it is raw.
 *   L6 stream, little-endian (A16 / A256 = round up to 16 / 256):
 *        0  u8[4] 'L','C','K','V'      8  u64 n (input bytes)
 *        4  u8    version = 1          16 u64 C = ceil(n / 16384) chunks
 *        5  u8    pipeline = 1         24 u64 total stream bytes
 *        6  u8    log2 chunk = 14      32 u8[32] zero
 *        7  u8    zero
 *        64 C x (u32 offset, u32 size); zeros up to D = A256(64 + 8C)
 *        D  payloads: chunk c at D + offset_c, zero-padded to A16(size_c);
 *           offset_0 = 0, offset_{c+1} = offset_c + A16(size_c);
 *           total = D + sum of A16(size_c).
 *
 * Conventions are those of splitzip.h: d_* pointers are caller-owned HIP
 * device memory, 16-byte aligned; calls are asynchronous on `stream`; the
 * library never allocates, frees or synchronises; host-detectable errors
 * return before anything is enqueued; a failed launch returns SZ_ERR_HIP.
 */
#ifndef LC_CODEC_H
#define LC_CODEC_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "splitzip.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest stream for n input bytes (every chunk raw):
 * A256(64 + 8C) + sum of A16(chunk lengths).  Pure host function; 0 when
 * n >= 2^31. */
uint64_t lc_max_compressed_bytes(uint64_t n);

/* Workspace of an encode: one u32 coded size per chunk, rounded up to 256
 * bytes (count tensors for the batched form).  Pure host function; 0 for
 * n = 0, n >= 2^31, count = 0, or a batch of 2^31 chunks or more (which
 * the batched calls reject). */
uint64_t lc_encode_workspace_bytes(uint64_t n);
uint64_t lc_encode_workspace_bytes_batched(uint32_t count, uint64_t n);

/* Encode n bytes (readings L1..L6).  dst_capacity must be at least
 * lc_max_compressed_bytes(n), else SZ_ERR_BUFFER_TOO_SMALL; d_out_bytes
 * (device or device-accessible pinned host u64, may be NULL) receives the
 * total.  d_workspace: >= lc_encode_workspace_bytes(n) bytes, clobbered
 * (may be NULL when n = 0). */
sz_status lc_encode(const void* d_src, uint64_t n, void* d_dst, uint64_t dst_capacity,
                    uint64_t* d_out_bytes, void* d_workspace, uint64_t workspace_bytes,
                    hipStream_t stream);

/* Decode a stream of n input bytes.  The header, every table entry (offsets
 * chained as in L6, size <= chunk length) and every coded chunk's size
 * against its bitmap are checked on the device; on a mismatch *d_status
 * (device int32, may be NULL) is set to SZ_ERR_CORRUPT_STREAM and the output
 * is unspecified, and no access leaves [d_src, d_src + src_bytes) or
 * [d_dst, d_dst + n).  Otherwise *d_status is SZ_OK.  Returns
 * SZ_ERR_CORRUPT_STREAM without launching when src_bytes < A256(64 + 8C). */
sz_status lc_decode(const void* d_src, uint64_t src_bytes, uint64_t n, void* d_dst, int32_t* d_status,
                    hipStream_t stream);

/* Batched forms: count tensors of n bytes each, one launch per phase; the
 * d_*s tables are device arrays of count device pointers; results equal
 * count single calls.  d_out_bytes: count u64 (may be NULL); d_src_bytes:
 * count u64 (device), the readable bytes of each stream; d_status: count
 * int32 (may be NULL). */
sz_status lc_encode_batched(const void* const* d_srcs, uint32_t count, uint64_t n, void* const* d_dsts,
                            uint64_t dst_capacity, uint64_t* d_out_bytes, void* d_workspace,
                            uint64_t workspace_bytes, hipStream_t stream);

sz_status lc_decode_batched(const void* const* d_srcs, const uint64_t* d_src_bytes, uint32_t count,
                            uint64_t n, void* const* d_dsts, int32_t* d_status, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LC_CODEC_H */
