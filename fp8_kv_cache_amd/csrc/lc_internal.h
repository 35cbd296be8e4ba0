// lc_internal.h -- layout arithmetic and launch interfaces of the LC-style
// comparison codec; the stream format is documented in include/lc_codec.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sz_internal.h"

namespace lc {

using sz::DstRef;
using sz::SrcRef;

constexpr uint32_t kChunk = 16384;            // bytes per chunk
constexpr uint32_t kLog2Chunk = 14;
constexpr uint32_t kMagic = 0x564B434Cu;      // bytes 'L','C','K','V'
constexpr uint32_t kVersion = 1;
constexpr uint32_t kPipeline = 1;             // TUPL8_1 -> BIT_8 -> RZE_2
constexpr uint64_t kMaxInput = uint64_t(1) << 31;

__host__ __device__ inline uint64_t chunks_of(uint64_t n) { return (n + kChunk - 1) / kChunk; }
__host__ __device__ inline uint64_t align16(uint64_t x) { return (x + 15) & ~uint64_t(15); }
// start of the payload region, D = A256(64 + 8C)
__host__ __device__ inline uint64_t data_at(uint64_t n) { return sz::align256(64 + 8 * chunks_of(n)); }
__host__ __device__ inline uint32_t chunk_len(uint64_t n, uint64_t c) {
    return static_cast<uint32_t>(c + 1 < chunks_of(n) ? kChunk : n - c * kChunk);
}
__host__ __device__ inline uint64_t max_bytes(uint64_t n) {
    const uint64_t C = chunks_of(n);
    return C ? data_at(n) + (C - 1) * kChunk + align16(chunk_len(n, C - 1)) : data_at(n);
}
__host__ __device__ inline uint64_t workspace_bytes(uint32_t count, uint64_t n) {
    return sz::align256(4 * static_cast<uint64_t>(count) * chunks_of(n));
}

struct EncodeArgs {
    SrcRef src;
    DstRef dst;
    uint64_t* out_bytes;      // count u64, may be null
    uint32_t* sizes;          // workspace: count x C stored chunk sizes
    uint32_t count;
    uint64_t n;
};

struct DecodeArgs {
    SrcRef src;
    const uint64_t* src_bytes_table;   // per tensor (batched), else src_bytes
    uint64_t src_bytes;
    DstRef dst;
    int32_t* status;                   // count int32, may be null
    uint32_t count;
    uint64_t n;
};

hipError_t launch_encode(const EncodeArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

}  // namespace lc
