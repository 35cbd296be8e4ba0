// sz_internal.h -- shared by the host entry points and the gfx950 kernels of
// the exponent codec library.  Stream layout arithmetic and kernel launch
// interfaces; the byte format itself is documented in include/splitzip.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Full unrolling of the fixed-size loops below keeps their arrays in
// registers on the GPU; other host compilers (the g++ schedule check) just
// run the loops.
#if defined(__clang__)
#define SZ_UNROLL _Pragma("unroll")
#else
#define SZ_UNROLL
#endif

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
    const uint32_t* records;  // the one-launch compress's per-tensor records (null for the separate calls):
                              // a tensor whose record shows no verdict or a give-up gets a header that
                              // does not decode
    uint32_t count;
    uint64_t n;
};

// One-launch compress (histogram, codebook and encode).  Its workspace is
// the encode workspace followed by a synchronisation area that a fill
// kernel zeroes before every launch:
//   u64 hist[count][R][256]  exponent counts of the whole tensor, in R =
//                            hist_replicas(count) copies
//   u64 sample[count][256]   exponent counts of the sampled chunks
//   u32 abort, u32 listed[3]   (padded to 256 bytes)
//   per tensor t a 128-byte record of u32 words: [0..3] the provisional
//   codebook (published once its bytes 0..14 are distinct; byte 15 is 1
//   when the tensor is escape-heavy, see kProvisionalCountOnly), [8] the
//   verdict on it once the final codebook is known (kProvisional*; 0 if
//   the tensor gave up), [9] 1 once any of its work gave up
//   list[3][count]           64-byte entries; the first listed[k] of list k
//                            describe the tensors whose provisional
//                            codebook was not used as the final one, [0]
//                            kProvisionalReordered, [1] kProvisionalDiffers,
//                            [2] kProvisionalCountOnly, in no set order
constexpr uint32_t kPassWaves = 16;                         // waves per workgroup
constexpr uint32_t kPassThreads = kPassWaves * kWaveSize;   // 1024
// Blocks per main item: one per wave for BF16, two for E5M2 (a block of
// half the bytes), so that every item moves the same bytes.
__host__ __device__ constexpr uint32_t item_blocks(uint32_t dtype) {
    return dtype == kDtypeBF16 ? kPassWaves : 2 * kPassWaves;
}
constexpr uint32_t kSampleStride = 16;                      // one counting chunk in 16 feeds the provisional codebook
constexpr uint32_t kPassLag = 4;                            // fewest stages between a tensor's sample and its main items
constexpr uint64_t kPassLagBytes = 128ull << 20;            // input bytes those stages span at least
constexpr uint32_t kDefaultSpinLimit = 1u << 20;            // polls before a waiting workgroup gives up
constexpr uint64_t kDefaultFusedMin = 1ull << 21;           // smallest BF16 tensor (elements) the fused kernel takes
constexpr uint64_t kDefaultFusedMinE5m2 = 1ull << 22;       // smallest E5M2 tensor it takes,
constexpr uint64_t kDefaultFusedCallE5m2 = 1ull << 28;      // in calls of at least this many elements
constexpr uint32_t kProvisionalSame = 1;       // no recoding
constexpr uint32_t kProvisionalReordered = 2;  // same 15 values, other codes: code nibbles recoded
constexpr uint32_t kProvisionalDiffers = 3;    // other values: code nibbles and escapes recoded
// Escape-heavy tensors: when more than 1/kCountOnlyRatio of the sample
// escapes under its own provisional codebook, the final codebook would
// nearly always differ and a recode would rewrite most of the stream, so
// the main items only count such a tensor and the recode launch encodes it
// from the input with the final codebook.
constexpr uint32_t kProvisionalCountOnly = 4;
constexpr uint32_t kCountOnlyRatio = 4;
constexpr uint32_t kLists = 3;
constexpr uint32_t kTranscodeGroups = 2048;                 // workgroups of the transcode kernel, at most

// Elements one sample item counts: 8 passes of a 16-byte vector per lane
// of the 1024-thread workgroup (128 KB of input).
__host__ __device__ inline uint64_t sample_chunk_elems(uint32_t dtype) {
    return 8ull * kPassThreads * (dtype == kDtypeBF16 ? 8 : 16);
}

// Copies of each tensor's whole-tensor histogram in the synchronisation
// area: main item i of a tensor adds its counts to copy i % R, and the
// final item sums the copies.  With few tensors in a call every main item
// would otherwise add to the same 256 counters, and their atomics queue on
// those few addresses; R x count >= 16 below 16 tensors.
__host__ __device__ inline uint32_t hist_replicas(uint32_t count) {
    return count >= 16 ? 1u : count >= 8 ? 2u : count >= 4 ? 4u : count >= 2 ? 8u : 16u;
}

__host__ __device__ inline uint64_t sync_hist_bytes(uint32_t count) {
    return 2048ull * count * (hist_replicas(count) + 1);   // the copies, then the sample histograms
}

__host__ __device__ inline uint64_t sync_area_bytes(uint32_t count) {
    return sync_hist_bytes(count) + 256 + 128ull * count + 64ull * kLists * count;
}

// The per-tensor records inside the synchronisation area (32 u32 words each).
__host__ __device__ inline uint64_t sync_records_offset(uint32_t count) { return sync_hist_bytes(count) + 256; }

struct CompressArgs {
    EncodeArgs enc;           // enc.codebooks (count x 16) is written by the compress kernel
    uint64_t* hists;          // count x 256, written
    uint8_t* sync;            // the synchronisation area
    int32_t* status;          // count, may be null
    uint32_t sample_items;    // per tensor: ceil(chunks / kSampleStride), chunks = ceil(n / sample chunk)
    uint32_t main_items;      // per tensor: ceil(blocks / item_blocks(dtype))
    uint32_t lag;             // stage of a tensor's main items after its sample items, >= 1
    uint32_t spin_limit;
    uint32_t sample_total;    // elements the sample items of one tensor count (n < 2^32)
};

// Work items of the one-launch compress, in schedule order: workgroup i
// runs item i (see k_compress).
enum : uint32_t { kItemSample = 0, kItemProvisional = 1, kItemMain = 2, kItemFinal = 3, kItemNone = 4 };
constexpr uint32_t kItemKinds = 4;

struct PassItem {
    uint32_t kind;
    uint32_t t;
    uint32_t idx;
};

// The schedule: T tensors; in stage s, kind j (in kind order) has per[j]
// items for tensor s - delay[j] when delay[j] <= s < delay[j] + T.
struct PassPlan {
    uint32_t T;
    uint32_t per[kItemKinds];
    uint32_t delay[kItemKinds];
};

__host__ __device__ inline PassPlan pass_plan(const CompressArgs& a) {
    PassPlan p;
    p.T = a.enc.count;
    p.per[kItemSample] = a.sample_items;
    p.per[kItemProvisional] = 1;
    p.per[kItemMain] = a.main_items;
    p.per[kItemFinal] = 1;
    p.delay[kItemSample] = 0;
    p.delay[kItemProvisional] = 1;
    p.delay[kItemMain] = a.lag;
    p.delay[kItemFinal] = a.lag + 1;
    return p;
}

// Item k of the schedule.  Stage sizes are constant between consecutive
// values of {delay[j], delay[j] + T}, so k is located region by region
// (fixed-size loops: no dynamically indexed arrays in device code).
__host__ __device__ inline PassItem pass_item(uint64_t k, const PassPlan& p) {
    constexpr uint32_t kEdges = 2 * kItemKinds;
    uint32_t edge[kEdges];
SZ_UNROLL
    for (uint32_t j = 0; j < kItemKinds; ++j) {
        edge[2 * j] = p.delay[j];
        edge[2 * j + 1] = p.delay[j] + p.T;
    }
SZ_UNROLL
    for (uint32_t i = 0; i + 1 < kEdges; ++i)
SZ_UNROLL
        for (uint32_t j = 0; j + 1 < kEdges - i; ++j) {
            const uint32_t x = edge[j], y = edge[j + 1];
            edge[j] = x < y ? x : y;
            edge[j + 1] = x < y ? y : x;
        }
SZ_UNROLL
    for (uint32_t r = 0; r + 1 < kEdges; ++r) {
        const uint32_t lo = edge[r], hi = edge[r + 1];
        if (hi <= lo) continue;
        uint64_t size = 0;
SZ_UNROLL
        for (uint32_t j = 0; j < kItemKinds; ++j)
            if (p.delay[j] <= lo && lo < p.delay[j] + p.T) size += p.per[j];
        if (size == 0) continue;
        const uint64_t span = static_cast<uint64_t>(hi - lo) * size;
        if (k >= span) {
            k -= span;
            continue;
        }
        const uint32_t s = lo + static_cast<uint32_t>(k / size);
        uint64_t q = k % size;
SZ_UNROLL
        for (uint32_t j = 0; j < kItemKinds; ++j) {
            if (!(p.delay[j] <= s && s < p.delay[j] + p.T)) continue;
            if (q < p.per[j]) return {j, s - p.delay[j], static_cast<uint32_t>(q)};
            q -= p.per[j];
        }
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
// encode = planes and staged escapes (full blocks, then a partial last
// block), then offsets, header and escape scatter (one kernel, or two for
// tensors of more than 2^16 blocks)
hipError_t launch_encode(const EncodeArgs& a, uint32_t dtype, hipStream_t s);
hipError_t launch_encode_empty(const EncodeArgs& a, uint32_t dtype, hipStream_t s);
// compress = one clear of the synchronisation area and the status words,
// the counting/encoding kernel, the partial-block encode, the transcode of
// tensors whose provisional codebook was not the final one, then the same
// offsets and escape scatter as encode
hipError_t launch_compress(const CompressArgs& a, uint32_t dtype, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, uint32_t dtype, hipStream_t s);
hipError_t launch_decode_empty(const DecodeArgs& a, uint32_t dtype, hipStream_t s);

}  // namespace sz
