// sz_internal.h -- shared by the host entry points and the gfx950 kernels of
// the exponent codec library.  Stream layout arithmetic and kernel launch
// interfaces; the byte format itself is documented in include/splitzip.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sz {

constexpr uint32_t kBlockElems = 4096;      // elements per format block
constexpr uint32_t kLog2Block = 12;
constexpr uint32_t kCodes = 15;             // coded exponents; code 15 = escape
constexpr uint32_t kEscape = 15;
constexpr uint32_t kVersion = 1;
constexpr uint32_t kMagic = 0x564B5A53u;    // bytes 'S','Z','K','V'
constexpr uint32_t kWaveSize = 64;
constexpr uint32_t kThreads = 256;          // 4 waves per workgroup
constexpr uint32_t kWavesPerGroup = kThreads / kWaveSize;
constexpr uint32_t kDtypeBF16 = 1;
constexpr uint32_t kDtypeE5M2 = 2;

// Region sizes of one stream.  A(x) rounds x up to a multiple of 256.
struct Layout {
    uint64_t n;
    uint64_t blocks;       // B = ceil(n / 4096)
    uint64_t header;       // H = A(64 + 4B)
    uint64_t sm_bytes;     // S
    uint64_t sm_region;    // A(S)
    uint64_t code_bytes;   // ceil(n / 2)
    uint64_t code_region;  // A(ceil(n / 2))
    uint64_t sm_at, code_at, esc_at;
};

__host__ __device__ inline uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }

__host__ __device__ inline Layout layout_of(uint64_t n, uint32_t dtype) {
    Layout L;
    L.n = n;
    L.blocks = (n + kBlockElems - 1) / kBlockElems;
    L.header = align256(64 + 4 * L.blocks);
    L.sm_bytes = dtype == kDtypeBF16 ? n : (3 * n + 7) / 8;
    L.sm_region = align256(L.sm_bytes);
    L.code_bytes = (n + 1) / 2;
    L.code_region = align256(L.code_bytes);
    L.sm_at = L.header;
    L.code_at = L.sm_at + L.sm_region;
    L.esc_at = L.code_at + L.code_region;
    return L;
}

// Encode workspace: block escape counts (u32 per block), then 4096 staging
// bytes per block (at most every element of a block escapes).
__host__ __device__ inline uint64_t workspace_counts_bytes(uint32_t count, uint64_t blocks) {
    return align256(4 * static_cast<uint64_t>(count) * blocks);
}
__host__ __device__ inline uint64_t workspace_bytes_for(uint32_t count, uint64_t n) {
    const uint64_t blocks = (n + kBlockElems - 1) / kBlockElems;
    return workspace_counts_bytes(count, blocks) + static_cast<uint64_t>(count) * blocks * kBlockElems;
}

// A tensor is addressed either through a device table of pointers (batched
// calls) or directly (single-tensor calls).
struct SrcRef {
    const void* const* table;
    const void* single;
};
struct DstRef {
    void* const* table;
    void* single;
};

struct HistArgs {
    SrcRef src;
    uint64_t* hists;          // count x 256
    uint32_t count;
    uint32_t groups;          // workgroups per tensor, set by the launcher
    uint64_t n;
    uint64_t chunk;           // elements per workgroup (full histogram), set by the launcher
    uint32_t stride;          // count format blocks b with b % stride == 0 (1 = all)
    uint32_t per_group;       // sampled blocks per workgroup, set by the launcher
};

struct CodebookArgs {
    const uint64_t* hists;    // count x 256
    uint8_t* codebooks;       // count x 16
    uint32_t count;
};

struct EncodeArgs {
    SrcRef src;
    DstRef dst;
    const uint8_t* codebooks; // count x 16
    uint64_t* out_bytes;      // count, may be null
    uint32_t* counts;         // count x blocks escape counts (workspace)
    uint8_t* staging;         // count x blocks x 4096 staged escape bytes (workspace)
    uint32_t count;
    uint64_t n;
};

// One-launch compress (histogram, codebook and encode).  Its workspace is
// the encode workspace followed by a synchronisation area that a fill
// kernel zeroes before every launch:
//   u64 hist[count][256]   exponent counts accumulated by all workgroups
//   u32 ticket, u32 abort  (padded to 256 bytes)
//   per tensor t a 128-byte record: u32 at byte 0, 1 once t's codebook is
//   published
constexpr uint32_t kPassWaves = 16;                         // blocks per encode item, one per wave
constexpr uint32_t kPassThreads = kPassWaves * kWaveSize;   // 1024
constexpr uint64_t kPassLagBytes = 48ull << 20;             // input counted between a tensor's counting and its
                                                            // re-read: the lag in stages is this over the tensor size
constexpr uint32_t kCountIters = 1;                         // 128 KB input iterations per counting item
constexpr uint32_t kDefaultSpinLimit = 1u << 20;            // polls before a waiting workgroup gives up
constexpr uint64_t kDefaultFusedMin = 1ull << 21;           // smallest BF16 tensor (elements) the fused kernel takes

__host__ __device__ inline uint64_t sync_area_bytes(uint32_t count) {
    return 2048ull * count + 256 + 128ull * count;
}

struct CompressArgs {
    EncodeArgs enc;           // enc.codebooks is written by the compress kernel
    uint64_t* hists;          // count x 256, written
    uint8_t* codebooks;       // count x 16, written (same memory as enc.codebooks)
    uint8_t* sync;            // the synchronisation area
    int32_t* status;          // count, may be null
    uint32_t count_items;     // per tensor: ceil(n / elements per counting item)
    uint32_t encode_items;    // per tensor: ceil(full blocks / kPassWaves); plus one codebook item
    uint32_t lag;             // stages between counting and encoding a tensor, 1..count (see kPassLagBytes)
    uint32_t spin_limit;
};

// Work items of the one-launch compress, in ticket order (see k_compress).
enum : uint32_t { kItemCount = 0, kItemCodebook = 1, kItemEncode = 2, kItemNone = 3 };

struct PassItem {
    uint32_t kind;
    uint32_t t;
    uint32_t idx;
};

// Ticket k -> item, for T tensors, H counting and E encode items per
// tensor and 1 <= lag <= T.  Stage s holds, in this order: the H counting
// items of tensor s (s < T), the codebook item of tensor s - 1
// (1 <= s <= T), the E encode items of tensor s - lag (lag <= s < T + lag).
// Stage sizes are constant between the boundaries 0, 1, lag, T, T + 1,
// T + lag, so the ticket is located region by region.
__host__ __device__ inline PassItem pass_item(uint64_t k, uint32_t T, uint32_t H, uint32_t E, uint32_t lag) {
    const uint32_t edge[6] = {0, 1, lag, T, T + 1, T + lag};
    for (uint32_t r = 0; r < 5; ++r) {
        const uint32_t lo = edge[r], hi = edge[r + 1];
        if (hi <= lo) continue;
        const uint64_t size = (lo < T ? H : 0u) + (lo >= 1 && lo <= T ? 1u : 0u) + (lo >= lag ? E : 0u);
        const uint64_t span = static_cast<uint64_t>(hi - lo) * size;
        if (k >= span) {
            k -= span;
            continue;
        }
        const uint32_t s = lo + static_cast<uint32_t>(k / size);
        uint64_t q = k % size;
        if (s < T) {
            if (q < H) return {kItemCount, s, static_cast<uint32_t>(q)};
            q -= H;
        }
        if (s >= 1 && s <= T) {
            if (q == 0) return {kItemCodebook, s - 1, 0};
            q -= 1;
        }
        return {kItemEncode, s - lag, static_cast<uint32_t>(q)};
    }
    return {kItemNone, 0, 0};
}

struct DecodeArgs {
    SrcRef src;
    const uint64_t* src_bytes_table;  // count, or null
    uint64_t src_bytes;               // used when the table is null
    DstRef dst;
    int32_t* status;                  // count, may be null
    uint32_t count;
    uint64_t n;
};

hipError_t launch_fill_u64(uint64_t* p, uint64_t words, uint64_t value, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, uint64_t words, int32_t value, hipStream_t s);
hipError_t launch_histogram(const HistArgs& a, uint32_t dtype, hipStream_t s);
hipError_t launch_codebook(const CodebookArgs& a, uint32_t dtype, hipStream_t s);
// encode = three kernels: planes + staged escapes, offsets + header, escape scatter
hipError_t launch_encode(const EncodeArgs& a, uint32_t dtype, hipStream_t s);
hipError_t launch_encode_empty(const EncodeArgs& a, uint32_t dtype, hipStream_t s);
// compress (BF16) = one clear of the synchronisation area and the status
// words, the counting/encoding kernel, the partial-block encode, then the
// same offsets and escape scatter as encode
hipError_t launch_compress(const CompressArgs& a, uint32_t dtype, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, uint32_t dtype, hipStream_t s);
hipError_t launch_decode_empty(const DecodeArgs& a, uint32_t dtype, hipStream_t s);

}  // namespace sz
