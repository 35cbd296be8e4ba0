// kernels.hip -- gfx950 kernels of the lossless exponent codec.
//
// Method: SplitZip project page, "Abstract" (frequent exponents -> constant-width
// 4-bit codes, sign and mantissa kept as they are, rare exponents -> a
// separate escape stream) and FAQ "Is SplitZip lossy?" (bit-exact decode),
// FAQ "Does it work with an FP8 KV cache?" (E5M2 variant).  The byte layout
// is stream format v1, documented in include/splitzip.h.
//
// Work decomposition: one 64-lane wave owns one 4096-element format block.
// Lane l of a wave handles a contiguous run of 16 (BF16) or 32 (E5M2)
// elements in each 1024/2048-element sub-chunk, so every global access of a
// wave is one contiguous, 16-byte-per-lane transfer.  All arithmetic is
// integer bit manipulation; there is no matrix-core work anywhere.
#include "device_common.h"

namespace sz {
namespace {

// ---------------------------------------------------------------- helpers

// bit k*4 set iff nibble k of w equals 15 (the escape code)
__device__ inline uint32_t escape_nibbles(uint32_t w) {
    return w & (w >> 1) & (w >> 2) & (w >> 3) & 0x11111111u;
}

// nibble-granular mask of the first `valid` nibbles (0..8) of a code word
__device__ inline uint32_t valid_nibbles(int32_t valid) {
    return valid >= 8 ? 0xFFFFFFFFu : (valid <= 0 ? 0u : ((1u << (4 * valid)) - 1u));
}

// four code nibbles (one per byte of x) -> the four codebook bytes; the
// codebook is held in four registers cbw[0..3]
__device__ inline uint32_t lookup4(uint32_t x, const uint32_t (&cbw)[4]) {
    const uint32_t sel = x & 0x07070707u;
    const uint32_t lo = perm(cbw[1], cbw[0], sel);
    const uint32_t hi = perm(cbw[3], cbw[2], sel);
    const uint32_t m = ((x >> 3) & 0x01010101u) * 0xFFu;
    return (hi & m) | (lo & ~m);
}

template <uint32_t DT>
struct Geometry;
template <>
struct Geometry<kDtypeBF16> {
    static constexpr uint32_t kElemBytes = 2;
    static constexpr uint32_t kLaneElems = 8;    // elements per lane per sub-chunk
    static constexpr uint32_t kSubs = 8;          // sub-chunks per block
    static constexpr uint32_t kInWords = 4;       // input dwords per lane per sub-chunk
    static constexpr uint32_t kCodeWords = 1;     // code dwords per lane per sub-chunk
    static constexpr uint32_t kSmWords = 2;       // sign|mantissa dwords per lane per sub-chunk
    static constexpr uint32_t kDomain = 256;
};
template <>
struct Geometry<kDtypeE5M2> {
    static constexpr uint32_t kElemBytes = 1;
    static constexpr uint32_t kLaneElems = 32;
    static constexpr uint32_t kSubs = 2;
    static constexpr uint32_t kInWords = 8;
    static constexpr uint32_t kCodeWords = 4;
    static constexpr uint32_t kSmWords = 3;
    static constexpr uint32_t kDomain = 32;
};

// Input of one lane: elements [elem0, elem0 + kLaneElems) as kInWords
// dwords; those at or beyond n read as zero and no byte at or beyond n is
// touched.
template <uint32_t DT>
__device__ inline void load_lane(const SZ_GLOBAL uint8_t* src, uint64_t elem0, uint64_t n,
                                 uint32_t (&d)[Geometry<DT>::kInWords]) {
    using G = Geometry<DT>;
    if (elem0 + G::kLaneElems <= n) {
        const SZ_GLOBAL u32x4* p = (const SZ_GLOBAL u32x4*)(src + elem0 * G::kElemBytes);
#pragma unroll
        for (uint32_t v = 0; v < G::kInWords / 4; ++v) {
            const u32x4 x = p[v];
            d[4 * v] = x.x; d[4 * v + 1] = x.y; d[4 * v + 2] = x.z; d[4 * v + 3] = x.w;
        }
        return;
    }
#pragma unroll
    for (uint32_t i = 0; i < G::kInWords; ++i) d[i] = 0;
#pragma unroll
    for (uint32_t k = 0; k < G::kLaneElems; ++k) {
        if (elem0 + k < n) {
            uint32_t v;
            if (DT == kDtypeBF16)
                v = ((const SZ_GLOBAL uint16_t*)src)[elem0 + k];
            else
                v = src[elem0 + k];
            const uint32_t bit = (k * G::kElemBytes * 8) & 31;
            d[(k * G::kElemBytes) / 4] |= v << bit;
        }
    }
}

// ------------------------------------------------------------ fill kernels

__global__ void k_fill_u64(uint64_t* p, uint64_t words, uint64_t value) {
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < words;
         i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

// Zero two ranges in one launch (u64 words of a, i32 words of b; b may be
// null): the fused compress clears its synchronisation area and its status
// words (SZ_OK is 0) with one kernel instead of two.
__global__ void k_zero_two(uint64_t* a, uint64_t na, int32_t* b, uint64_t nb) {
    const uint64_t first = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = first; i < na; i += stride) a[i] = 0;
    if (b)
        for (uint64_t i = first; i < nb; i += stride) b[i] = 0;
}

__global__ void k_fill_i32(int32_t* p, uint64_t words, int32_t value) {
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < words;
         i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

// -------------------------------------------------------------- histogram
//
// Each workgroup counts one contiguous chunk of one tensor into
// lane-striped copies of the histogram in LDS.
//   BF16: 256 bins x 32 lane-striped copies, laid out [bin][copy]; lane l
//         adds into copy l & 31, so the 32 lanes of a half-wave hit 32
//         different banks whatever their exponents.  The byte address of
//         (bin e, copy c) is e*128 + 4c, and e*128 is simply u & 0x7F80.
//   E5M2: a byte per element makes the LDS atomics, not the reads, the
//         limit, so the two exponents of each element pair (bytes 0,1 and
//         2,3 of a dword) are counted together: 1024 pair bins as 16-bit
//         counters, two to a dword, in 16 lane-striped copies, laid out
//         [pair/2][copy] (32 KB).  An element without a partner (a ragged
//         end) is counted as the pair (e, 0), and the fold, which splits each
//         pair count back onto both of its exponents, takes those partners
//         off bin 0 again.  A 16-bit counter takes at most
//         16 * (chunk/512 + 128) increments (16 lanes per copy, one pair per
//         two elements, fewer than 128 unpaired elements per lane), so E5M2
//         chunks are capped at 2^20 elements.
template <uint32_t DT>
struct HistLds;
template <>
struct HistLds<kDtypeBF16> {
    static constexpr uint32_t kWords = 256 * 32;
};
template <>
struct HistLds<kDtypeE5M2> {
    static constexpr uint32_t kWords = 512 * 16;
};
constexpr uint64_t kE5m2MaxChunk = 1ull << 20;

template <uint32_t DT>
__device__ inline uint32_t hist_lane_bytes(uint32_t tid) {
    return DT == kDtypeBF16 ? (tid & 31u) << 2 : (tid & 15u) << 2;
}

template <uint32_t DT>
__device__ inline void count_dword(char* lds, uint32_t w, uint32_t lane_bytes) {
    if (DT == kDtypeBF16) {
        atomicAdd(reinterpret_cast<uint32_t*>(lds + ((w & 0x7F80u) | lane_bytes)), 1u);
        atomicAdd(reinterpret_cast<uint32_t*>(lds + (((w >> 16) & 0x7F80u) | lane_bytes)), 1u);
    } else {
        // pair index e_first | e_second << 5 of bytes (0,1) in the low half and (2,3) in the high half
        const uint32_t pk = ((w >> 2) & 0x001F001Fu) | ((w >> 5) & 0x03E003E0u);
        const uint32_t p0 = pk & 0xFFFFu, p1 = pk >> 16;
        atomicAdd(reinterpret_cast<uint32_t*>(lds + (((p0 >> 1) << 6) | lane_bytes)), (p0 & 1u) ? 0x10000u : 1u);
        atomicAdd(reinterpret_cast<uint32_t*>(lds + (((p1 >> 1) << 6) | lane_bytes)), (p1 & 1u) ? 0x10000u : 1u);
    }
}

// one element, raw bits u (E5M2: as the pair (e, 0))
template <uint32_t DT>
__device__ inline void count_one(char* lds, uint32_t u, uint32_t lane_bytes) {
    if constexpr (DT == kDtypeBF16) {
        atomicAdd(reinterpret_cast<uint32_t*>(lds + ((((u >> 7) & 0xFFu) << 7) | lane_bytes)), 1u);
    } else {
        const uint32_t p = (u >> 2) & 0x1Fu;
        atomicAdd(reinterpret_cast<uint32_t*>(lds + (((p >> 1) << 6) | lane_bytes)), (p & 1u) ? 0x10000u : 1u);
    }
}

template <uint32_t DT, uint32_t NT = kThreads>
__device__ inline void hist_clear(uint32_t* bins, uint32_t tid) {
    constexpr uint32_t kWords = HistLds<DT>::kWords;
    static_assert(kWords % (4 * NT) == 0, "cleared in 16-byte stores");
#pragma unroll
    for (uint32_t i = tid * 4; i < kWords; i += NT * 4)
        *reinterpret_cast<uint4*>(bins + i) = make_uint4(0, 0, 0, 0);
}

// Fold the copies and add the sums to the tensor's u64 histogram.  Every
// thread of the NT-thread workgroup calls it, after a barrier; the first
// 256 do the folding.  `unpaired` is the number of phantom zero exponents
// the workgroup counted (E5M2: elements counted one at a time as the pair
// (e, 0); both types: zero padding counted past the end of a tensor); they
// are taken off bin 0.  Rotating the start keeps the lanes of a wave on
// distinct banks.
template <uint32_t DT, uint32_t NT = kThreads>
__device__ inline void hist_flush(uint32_t* bins, uint32_t tid, SZ_GLOBAL uint64_t* hist, uint32_t unpaired) {
    static_assert(NT >= 256, "one folding thread per bin");
    const bool folds = NT == 256 || tid < 256;
    if constexpr (DT == kDtypeBF16) {
        if (!folds) return;
        uint32_t sum = tid == 0 ? 0u - unpaired : 0u;
#pragma unroll 8
        for (uint32_t j = 0; j < 32; ++j) sum += bins[tid * 32 + ((j + tid) & 31u)];
        if (sum) __hip_atomic_fetch_add(hist + tid, static_cast<uint64_t>(sum), __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    } else {
        // thread t folds pairs 4t..4t+3 (dwords 2t, 2t+1): their first exponents
        // are (4t + k) & 31, their second exponent is t >> 3
        uint32_t c[4] = {0, 0, 0, 0};
#pragma unroll
        for (uint32_t k = 0; k < 2; ++k) {
#pragma unroll 8
            for (uint32_t j = 0; j < 16; ++j) {
                const uint32_t w = folds ? bins[(2 * tid + k) * 16 + ((j + tid) & 15u)] : 0u;
                c[2 * k] += w & 0xFFFFu;
                c[2 * k + 1] += w >> 16;
            }
        }
        // the first 32 words, read by now, become the 32 exponent bins
        __syncthreads();
        if (tid < 32) bins[tid] = 0;
        __syncthreads();
        const uint32_t both = c[0] + c[1] + c[2] + c[3];
        if (both) atomicAdd(bins + (tid >> 3), both);
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k)
            if (c[k]) atomicAdd(bins + ((4 * tid + k) & 31u), c[k]);   // c[k] = 0 when !folds
        __syncthreads();
        const uint32_t sum = tid < 32 ? bins[tid] - (tid == 0 ? unpaired : 0u) : 0u;
        if (sum)
            __hip_atomic_fetch_add(hist + tid, static_cast<uint64_t>(sum), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Count elements [begin, end) one at a time (a ragged end; NT threads).
// Returns the phantom zero exponents to take off bin 0: E5M2 counts each
// element as the pair (e, 0); BF16 counts exactly.
template <uint32_t DT, uint32_t NT>
__device__ inline uint32_t count_ragged(char* lds, const SZ_GLOBAL uint8_t* src, uint64_t begin, uint64_t end,
                                        uint32_t tid) {
    const uint32_t copy4 = hist_lane_bytes<DT>(tid);
    for (uint64_t i = begin + tid; i < end; i += NT)
        count_one<DT>(lds, DT == kDtypeBF16 ? ((const SZ_GLOBAL uint16_t*)src)[i] : src[i], copy4);
    return DT == kDtypeE5M2 ? static_cast<uint32_t>(end - begin) : 0u;
}

// Count elements [begin, end) of src into the workgroup's LDS copies (NT
// threads).  Every pass a lane reads one 16-byte vector (a wave one
// contiguous kilobyte); eight passes are in flight per iteration.  Returns
// the number of phantom zero exponents to take off bin 0 (E5M2 counts the
// ragged end as pairs (e, 0); BF16 counts it exactly).  kStream selects
// non-temporal loads, for data read once; the one-launch compress's sample
// reads pass false so that the chunks they read may still be in the
// last-level cache when the main items read them again.
template <uint32_t DT, uint32_t NT, bool kStream = true>
__device__ inline uint32_t count_range(char* lds, const SZ_GLOBAL uint8_t* src, uint64_t begin, uint64_t end,
                                       uint32_t tid) {
    using G = Geometry<DT>;
    constexpr uint32_t kVecElems = 16 / G::kElemBytes;       // elements per 16-byte vector
    constexpr uint32_t kTile = NT * kVecElems;                // elements per pass
    constexpr uint32_t kPasses = 8;
    const uint32_t copy4 = hist_lane_bytes<DT>(tid);
    uint64_t base = begin;
    for (; base + kPasses * kTile <= end; base += kPasses * kTile) {
        const SZ_GLOBAL u32x4* q = (const SZ_GLOBAL u32x4*)(src + base * G::kElemBytes);
        u32x4 v[kPasses];
#pragma unroll
        for (uint32_t p = 0; p < kPasses; ++p)
            v[p] = kStream ? __builtin_nontemporal_load(q + p * NT + tid) : q[p * NT + tid];
#pragma unroll
        for (uint32_t p = 0; p < kPasses; ++p) {
            count_dword<DT>(lds, v[p].x, copy4);
            count_dword<DT>(lds, v[p].y, copy4);
            count_dword<DT>(lds, v[p].z, copy4);
            count_dword<DT>(lds, v[p].w, copy4);
        }
    }
    return count_ragged<DT, NT>(lds, src, base, end, tid);
}

// Each workgroup counts one contiguous chunk of one tensor.  The grid
// oversubscribes the GPU, so one workgroup's fold-and-flush tail overlaps
// other workgroups' streaming.
template <uint32_t DT>
__global__ __launch_bounds__(kThreads) void k_histogram(HistArgs a) {
    __shared__ uint32_t bins[HistLds<DT>::kWords];
    const uint32_t tid = threadIdx.x;
    const uint32_t t = blockIdx.x / a.groups;
    const uint32_t g = blockIdx.x - t * a.groups;
    hist_clear<DT>(bins, tid);
    __syncthreads();
    const uint64_t begin = static_cast<uint64_t>(g) * a.chunk;
    const uint64_t end = begin + a.chunk < a.n ? begin + a.chunk : a.n;
    const uint32_t phantom = count_range<DT, kThreads>(reinterpret_cast<char*>(bins), src_of(a.src, t), begin, end, tid);
    __syncthreads();
    hist_flush<DT>(bins, tid, gptr(a.hists) + 256ull * t, phantom);
}

// Histogram of a block sample: only format blocks b with b % stride == 0
// are counted.  Workgroup (t, g) takes sampled blocks [g*per_group,
// (g+1)*per_group) of tensor t; per block every lane reads 4096 / 256
// elements as 16-byte vectors.
template <uint32_t DT>
__global__ __launch_bounds__(kThreads) void k_histogram_sampled(HistArgs a) {
    using G = Geometry<DT>;
    constexpr uint32_t kVecElems = 16 / G::kElemBytes;
    constexpr uint32_t kVecs = kBlockElems / (kThreads * kVecElems);   // per lane per block
    __shared__ uint32_t bins[HistLds<DT>::kWords];
    const uint32_t tid = threadIdx.x;
    const uint32_t t = blockIdx.x / a.groups;
    const uint32_t g = blockIdx.x - t * a.groups;
    char* lds = reinterpret_cast<char*>(bins);
    hist_clear<DT>(bins, tid);
    __syncthreads();

    const SZ_GLOBAL uint8_t* src = src_of(a.src, t);
    const uint64_t blocks = (a.n + kBlockElems - 1) / kBlockElems;
    const uint64_t sampled = (blocks + a.stride - 1) / a.stride;
    const uint64_t k0 = static_cast<uint64_t>(g) * a.per_group;
    const uint64_t k1 = k0 + a.per_group < sampled ? k0 + a.per_group : sampled;
    const uint32_t copy4 = hist_lane_bytes<DT>(tid);
    uint32_t unpaired = 0;   // elements of a partial last block, counted one at a time
    for (uint64_t k = k0; k < k1; ++k) {
        const uint64_t begin = k * a.stride * kBlockElems;
        if (begin + kBlockElems <= a.n) {
            const SZ_GLOBAL u32x4* q = (const SZ_GLOBAL u32x4*)(src + begin * G::kElemBytes);
            u32x4 v[kVecs];
#pragma unroll
            for (uint32_t p = 0; p < kVecs; ++p) v[p] = q[p * kThreads + tid];
#pragma unroll
            for (uint32_t p = 0; p < kVecs; ++p) {
                count_dword<DT>(lds, v[p].x, copy4);
                count_dword<DT>(lds, v[p].y, copy4);
                count_dword<DT>(lds, v[p].z, copy4);
                count_dword<DT>(lds, v[p].w, copy4);
            }
        } else {
            unpaired += static_cast<uint32_t>(a.n - begin);
            for (uint64_t i = begin + tid; i < a.n; i += kThreads)
                count_one<DT>(lds, DT == kDtypeBF16 ? ((const SZ_GLOBAL uint16_t*)src)[i] : src[i], copy4);
        }
    }
    __syncthreads();
    hist_flush<DT>(bins, tid, gptr(a.hists) + 256ull * t, DT == kDtypeE5M2 ? unpaired : 0u);
}

// --------------------------------------------------------------- codebook
//
// Rank every exponent value of the type by (count descending, value
// ascending): value v's rank is the number of values that order before it.
// The values of rank 0..14 are the codebook.

template <uint32_t DT>
__global__ __launch_bounds__(256) void k_codebook(CodebookArgs a) {
    constexpr uint32_t D = Geometry<DT>::kDomain;
    __shared__ uint64_t counts[256];
    const uint32_t t = blockIdx.x, v = threadIdx.x;
    counts[v] = gptr(a.hists)[256ull * t + v];
    __syncthreads();
    if (v < D) {
        const uint64_t mine = counts[v];
        uint32_t rank = 0;
        for (uint32_t u = 0; u < D; ++u) {
            const uint64_t c = counts[u];
            rank += (c > mine) | ((c == mine) & (u < v));
        }
        if (rank < kCodes) gptr(a.codebooks)[16ull * t + rank] = static_cast<uint8_t>(v);
    }
    if (v == kEscape) gptr(a.codebooks)[16ull * t + kEscape] = 0;
}

// ----------------------------------------------------------------- encode
//
// Launches of which none waits on another workgroup (so block ids come
// straight from blockIdx and no ordering tickets are needed):
//   k_encode   one wave per 4096-element block: sign|mantissa and code
//              planes, the block's escape count, and its escape bytes
//              staged at block-local ranks in the workspace;
//   k_offsets_scatter  one thread per block: its offset (the counts of all
//              earlier blocks), the offset table, the escape bytes copied to
//              their place in the stream's escape region, and the header --
//              for tensors of up to 2^16 blocks; beyond that
//   k_offsets  one workgroup per tensor scans the counts into the offset
//              table and writes the header, and
//   k_scatter  copies each block's staged escapes.

// Inputs, planes and outputs are each read or written once per call, so
// the bulk loads and stores are non-temporal (streaming past the caches):
// on the Llama-shaped cache the stores made compress 5% and decode 4%
// faster, and the loads a further 3.5% and 3%.

// Header (64 bytes), the zero padding after the offset table and the
// stream size; `lane` is the calling thread's index (0..63 used).
__device__ inline void write_header(SZ_GLOBAL uint8_t* dst, const Layout& L, uint32_t dtype,
                                    const SZ_GLOBAL uint8_t* cb, uint64_t escapes, SZ_GLOBAL uint64_t* out_bytes,
                                    uint32_t lane) {
    const uint64_t total = L.esc_at + escapes;
    const SZ_GLOBAL uint32_t* cbw = (const SZ_GLOBAL uint32_t*)cb;
    uint32_t v = 0;
    switch (lane) {
        case 0: v = kMagic; break;
        case 1: v = kVersion | (dtype << 8) | (kLog2Block << 16) | (kCodes << 24); break;
        case 2: v = static_cast<uint32_t>(L.n); break;
        case 3: v = static_cast<uint32_t>(L.n >> 32); break;
        case 4: v = static_cast<uint32_t>(escapes); break;
        case 5: v = static_cast<uint32_t>(escapes >> 32); break;
        case 6: v = cbw[0]; break;
        case 7: v = cbw[1]; break;
        case 8: v = cbw[2]; break;
        case 9: v = cbw[3] & 0x00FFFFFFu; break;  // cb[15] is stored as 0
        case 10: v = static_cast<uint32_t>(total); break;
        case 11: v = static_cast<uint32_t>(total >> 32); break;
        default: v = 0; break;
    }
    SZ_GLOBAL uint32_t* h = (SZ_GLOBAL uint32_t*)dst;
    if (lane < 16) h[lane] = v;
    const uint64_t pad_from = (64 + 4 * L.blocks) / 4;
    const uint64_t pad_words = L.header / 4 - pad_from;
    if (lane < pad_words) h[pad_from + lane] = 0;
    if (out_bytes && lane == 0) *out_bytes = total;
}

// BF16: eight elements d[0..3] -> 8 sign|mantissa bytes and 8 code
// nibbles; elements at index >= valid get code 0 and zero bytes (they are
// zero in d already).  Returns the escape nibble mask in esc[0].
__device__ inline void encode_lane_bf16(const uint32_t (&d)[4], uint32_t valid, const uint8_t* tbl,
                                        uint32_t (&sm)[2], uint32_t (&cw)[1], uint32_t (&esc)[1]) {
    uint32_t c[8];
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) {
        c[2 * k] = tbl[(d[k] >> 7) & 0xFFu];
        c[2 * k + 1] = tbl[(d[k] >> 23) & 0xFFu];
    }
    if (valid < 8) {
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k)
            if (k >= valid) c[k] = 0;
    }
    uint32_t w = 0;
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) w |= c[k] << (4 * k);
    cw[0] = w;
    esc[0] = escape_nibbles(w);
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
        // low bytes (exponent lsb | mantissa) and high bytes (sign | exponent msbs)
        const uint32_t lo = perm(d[2 * q + 1], d[2 * q], 0x06040200u);
        const uint32_t hi = perm(d[2 * q + 1], d[2 * q], 0x07050301u);
        sm[q] = (hi & 0x80808080u) | (lo & 0x7F7F7F7Fu);
    }
}

// E5M2: 32 elements (4 per dword) -> 96 bits of 3-bit sign|mantissa
// fields (LSB-first) and 32 code nibbles.
__device__ inline void encode_lane_e5m2(const uint32_t (&d)[8], uint32_t valid, const uint8_t* tbl,
                                        uint32_t (&sm)[3], uint32_t (&cw)[4], uint32_t (&esc)[4]) {
    uint32_t c[32];
    uint32_t f[8];
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
        const uint32_t e4 = (d[k] >> 2) & 0x1F1F1F1Fu;
        c[4 * k + 0] = tbl[e4 & 0xFFu];
        c[4 * k + 1] = tbl[(e4 >> 8) & 0xFFu];
        c[4 * k + 2] = tbl[(e4 >> 16) & 0xFFu];
        c[4 * k + 3] = tbl[e4 >> 24];
        const uint32_t s = ((d[k] >> 5) & 0x04040404u) | (d[k] & 0x03030303u);
        f[k] = (s & 0x7u) | ((s >> 5) & 0x38u) | ((s >> 10) & 0x1C0u) | ((s >> 15) & 0xE00u);
    }
    if (valid < 32) {
#pragma unroll
        for (uint32_t k = 0; k < 32; ++k)
            if (k >= valid) c[k] = 0;
    }
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        uint32_t w = 0;
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k) w |= c[8 * q + k] << (4 * k);
        cw[q] = w;
        esc[q] = escape_nibbles(w);
    }
    sm[0] = f[0] | (f[1] << 12) | (f[2] << 24);
    sm[1] = (f[2] >> 8) | (f[3] << 4) | (f[4] << 16) | (f[5] << 28);
    sm[2] = (f[5] >> 4) | (f[6] << 8) | (f[7] << 20);
}

// A wave's share of block b: sub-chunk j, lane l holds elements
// [4096b + j * 64 * kLaneElems + l * kLaneElems, ... + kLaneElems).
template <uint32_t DT>
using BlockRegs = uint32_t[Geometry<DT>::kSubs][Geometry<DT>::kInWords];

// Load block b into registers.  kFull: the block holds 4096 elements, so
// the loads need no per-lane guards; otherwise elements at or beyond n
// read as zero.
template <uint32_t DT, bool kFull>
__device__ inline void load_block(const SZ_GLOBAL uint8_t* src, uint64_t n, uint64_t b, uint32_t lane,
                                  BlockRegs<DT>& d) {
    using G = Geometry<DT>;
    constexpr uint32_t kSubElems = kWaveSize * G::kLaneElems;
    const uint64_t blk0 = b * kBlockElems;
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; ++j) {
        const uint64_t elem0 = blk0 + j * kSubElems + lane * G::kLaneElems;
        if (kFull) {
            const SZ_GLOBAL u32x4* p = (const SZ_GLOBAL u32x4*)(src + elem0 * G::kElemBytes);
#pragma unroll
            for (uint32_t v = 0; v < G::kInWords / 4; ++v) {
                const u32x4 x = __builtin_nontemporal_load(p + v);
                d[j][4 * v] = x.x; d[j][4 * v + 1] = x.y; d[j][4 * v + 2] = x.z; d[j][4 * v + 3] = x.w;
            }
        } else {
            load_lane<DT>(src, elem0, n, d[j]);
        }
    }
}

// The wave's table of codes (256 bytes in tbl_words): the code of value v
// is the lowest c with cb[c] == v, else 15.  `mine` is cb[lane] for lanes
// below 15 (any value above 255 elsewhere).
__device__ inline const uint8_t* build_code_table(uint32_t* tbl_words, uint32_t lane, uint32_t mine) {
    uint8_t* tbl = reinterpret_cast<uint8_t*>(tbl_words);
    tbl_words[lane] = 0x0F0F0F0Fu;
    bool lowest = lane < kCodes;
#pragma unroll
    for (uint32_t c = 0; c + 1 < kCodes; ++c) {
        const uint32_t other = __builtin_amdgcn_readlane(mine, c);
        if (c < lane && other == mine) lowest = false;
    }
    if (lowest) tbl[mine] = static_cast<uint8_t>(lane);
    __builtin_amdgcn_wave_barrier();
    return tbl;
}

// Encode block b from its registers into stream dst with the code table
// tbl: planes, the block's escape count and its staged escape bytes (flat
// = the block's index over all tensors).
template <uint32_t DT, bool kFull>
__device__ inline void encode_loaded(const EncodeArgs& a, const Layout& L, SZ_GLOBAL uint8_t* dst, uint64_t b,
                                     uint64_t flat, uint32_t lane, const uint8_t* tbl, const BlockRegs<DT>& d) {
    using G = Geometry<DT>;
    constexpr uint32_t kSubElems = kWaveSize * G::kLaneElems;
    constexpr uint32_t kSmWords = G::kSmWords;
    const uint64_t blk0 = b * kBlockElems;

    uint32_t sm[G::kSubs][kSmWords];
    uint32_t cw[G::kSubs][G::kCodeWords];
    uint32_t esc[G::kSubs][G::kCodeWords];
    uint32_t cnt[G::kSubs];
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; ++j) {
        const uint64_t elem0 = blk0 + j * kSubElems + lane * G::kLaneElems;
        const uint32_t valid = kFull ? G::kLaneElems
                               : elem0 >= a.n ? 0u
                               : (a.n - elem0 >= G::kLaneElems ? G::kLaneElems
                                                                 : static_cast<uint32_t>(a.n - elem0));
        if constexpr (DT == kDtypeBF16)
            encode_lane_bf16(d[j], valid, tbl, sm[j], cw[j], esc[j]);
        else
            encode_lane_e5m2(d[j], valid, tbl, sm[j], cw[j], esc[j]);
        cnt[j] = 0;
#pragma unroll
        for (uint32_t q = 0; q < G::kCodeWords; ++q) cnt[j] += __builtin_popcount(esc[j][q]);
    }

    // planes; vectors at or beyond the padded plane end are not stored
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; ++j) {
        const uint64_t elem0 = blk0 + j * kSubElems + lane * G::kLaneElems;
        const uint64_t code_off = elem0 / 2;
        if constexpr (DT == kDtypeBF16) {
            if (kFull || elem0 < L.sm_region)
                __builtin_nontemporal_store(u32x2{sm[j][0], sm[j][1]}, (SZ_GLOBAL u32x2*)(dst + L.sm_at + elem0));
            if (kFull || code_off < L.code_region)
                __builtin_nontemporal_store(cw[j][0], (SZ_GLOBAL uint32_t*)(dst + L.code_at + code_off));
        } else {
            const uint64_t sm_off = elem0 / 32 * 12;
            SZ_GLOBAL uint32_t* smp = (SZ_GLOBAL uint32_t*)(dst + L.sm_at + sm_off);
#pragma unroll
            for (uint32_t i = 0; i < 3; ++i)
                if (kFull || sm_off + 4 * i < L.sm_region) __builtin_nontemporal_store(sm[j][i], smp + i);
            if (kFull || code_off < L.code_region)
                __builtin_nontemporal_store(u32x4{cw[j][0], cw[j][1], cw[j][2], cw[j][3]},
                                            (SZ_GLOBAL u32x4*)(dst + L.code_at + code_off));
        }
    }

    // Escape ranks inside the block: element order is (sub-chunk, lane,
    // element), so lane l's first escape in sub-chunk j has rank
    // (escapes of earlier sub-chunks) + (escapes of lanes < l in j).
    uint32_t base[G::kSubs];
    uint32_t block_total = 0;
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; j += 2) {
        const uint32_t packed = cnt[j] | (cnt[j + 1] << 16);
        const uint32_t incl = wave_scan_incl(packed);
        const uint32_t excl = incl - packed;
        const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
        base[j] = block_total + (excl & 0xFFFFu);
        block_total += tot & 0xFFFFu;
        base[j + 1] = block_total + (excl >> 16);
        block_total += tot >> 16;
    }
    if (lane == 0) gptr(a.counts)[flat] = uniform(block_total);

    // escape bytes, in element order, staged at their rank inside the block
    SZ_GLOBAL uint8_t* esc_out = gptr(a.staging) + flat * kBlockElems;
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; ++j) {
        if (cnt[j] == 0) continue;
        uint32_t rank = base[j];
#pragma unroll
        for (uint32_t q = 0; q < G::kCodeWords; ++q) {
            uint32_t m = esc[j][q];
            while (m) {
                const uint32_t k = 8 * q + (__builtin_ctz(m) >> 2);   // element within the lane
                uint32_t e;
                if constexpr (DT == kDtypeBF16) {
                    uint32_t word = 0;
#pragma unroll
                    for (uint32_t i = 0; i < G::kInWords; ++i)
                        if (i == (k >> 1)) word = d[j][i];
                    e = (k & 1) ? (word >> 23) & 0xFFu : (word >> 7) & 0xFFu;
                } else {
                    uint32_t word = 0;
#pragma unroll
                    for (uint32_t i = 0; i < 8; ++i)
                        if (i == (k >> 2)) word = d[j][i];
                    e = (word >> (8 * (k & 3) + 2)) & 0x1Fu;
                }
                esc_out[rank++] = static_cast<uint8_t>(e);
                m &= m - 1;
            }
        }
    }
}

// One block with the codebook given in memory: the lane's codebook entry
// first, then the block's input, then the encode.
template <uint32_t DT, bool kFull>
__device__ inline void encode_block(const EncodeArgs& a, const Layout& L, uint32_t t, uint64_t b,
                                    uint64_t flat, uint32_t lane, uint32_t* tbl_words) {
    const SZ_GLOBAL uint8_t* cb = gptr(a.codebooks) + 16ull * t;
    const uint32_t mine = lane < kCodes ? cb[lane] : 0xFFFFu;
    const SZ_GLOBAL uint8_t* src = src_of(a.src, t);
    SZ_GLOBAL uint8_t* dst = dst_of(a.dst, t);
    BlockRegs<DT> d;
    load_block<DT, kFull>(src, a.n, b, lane, d);
    __builtin_amdgcn_sched_barrier(0);
    encode_loaded<DT, kFull>(a, L, dst, b, flat, lane, build_code_table(tbl_words, lane, mine), d);
}

// Full blocks only: wave i of the grid takes the i-th full block in
// (tensor, block) order.  A partial last block goes to k_encode_tail, so
// this kernel is compiled without per-lane guards.
template <uint32_t DT>
__global__ __launch_bounds__(kThreads) void k_encode(EncodeArgs a) {
    __shared__ uint32_t s_tbl[kWavesPerGroup][64];   // 256 one-byte codes per wave
    const uint32_t wave = uniform(threadIdx.x / kWaveSize);
    const Layout L = layout_of(a.n, DT);
    const uint64_t full = a.n / kBlockElems;          // full blocks per tensor
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * kWavesPerGroup + wave;
    if (i >= static_cast<uint64_t>(a.count) * full) return;
    const uint32_t t = static_cast<uint32_t>(i / full);
    const uint64_t b = i - static_cast<uint64_t>(t) * full;
    encode_block<DT, true>(a, L, t, b, static_cast<uint64_t>(t) * L.blocks + b, lane_id(), s_tbl[wave]);
}

// The partial last block of every tensor, one wave each.
template <uint32_t DT>
__global__ __launch_bounds__(kWaveSize) void k_encode_tail(EncodeArgs a) {
    __shared__ uint32_t s_tbl[64];
    const Layout L = layout_of(a.n, DT);
    const uint32_t t = blockIdx.x;
    const uint64_t b = L.blocks - 1;
    encode_block<DT, false>(a, L, t, b, static_cast<uint64_t>(t) * L.blocks + b, lane_id(), s_tbl);
}

// One workgroup per tensor: off[b] = escapes in blocks [0, b), then the
// header.  Thread i scans a contiguous run of ceil(B / 256) block counts.
template <uint32_t DT>
__global__ __launch_bounds__(256) void k_offsets(EncodeArgs a) {
    __shared__ uint32_t s_wave_total[kWavesPerGroup];
    const uint32_t t = blockIdx.x, tid = threadIdx.x;
    const uint32_t lane = lane_id(), wave = uniform(tid / kWaveSize);
    const Layout L = layout_of(a.n, DT);
    const SZ_GLOBAL uint32_t* counts = gptr(a.counts) + static_cast<uint64_t>(t) * L.blocks;
    SZ_GLOBAL uint8_t* dst = dst_of(a.dst, t);
    SZ_GLOBAL uint32_t* offs = (SZ_GLOBAL uint32_t*)(dst + 64);
    const uint64_t per = (L.blocks + 255) / 256;
    const uint64_t lo = tid * per < L.blocks ? tid * per : L.blocks;
    const uint64_t hi = lo + per < L.blocks ? lo + per : L.blocks;
    uint32_t sum = 0;
    for (uint64_t b = lo; b < hi; ++b) sum += counts[b];
    const uint32_t incl = wave_scan_incl(sum);
    if (lane == 63) s_wave_total[wave] = incl;
    __syncthreads();
    uint32_t run = incl - sum;
    for (uint32_t w = 0; w < wave; ++w) run += s_wave_total[w];
    const uint32_t escapes = s_wave_total[0] + s_wave_total[1] + s_wave_total[2] + s_wave_total[3];
    for (uint64_t b = lo; b < hi; ++b) {
        offs[b] = run;
        run += counts[b];
    }
    write_header(dst, L, DT, gptr(a.codebooks) + 16ull * t, escapes,
                 a.out_bytes ? gptr(a.out_bytes) + t : nullptr, tid);
}

// Staged escapes -> the stream's escape region; one thread per block,
// reading the staged bytes 16 at a time (a block's staging slot is
// 4096-byte aligned) and writing them to their unaligned destination.
template <uint32_t DT>
__global__ __launch_bounds__(kThreads) void k_scatter(EncodeArgs a) {
    const Layout L = layout_of(a.n, DT);
    const uint64_t flat = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (flat >= static_cast<uint64_t>(a.count) * L.blocks) return;
    const uint32_t t = static_cast<uint32_t>(flat / L.blocks);
    const uint64_t b = flat - static_cast<uint64_t>(t) * L.blocks;
    SZ_GLOBAL uint8_t* dst = dst_of(a.dst, t);
    const uint32_t cnt = gptr(a.counts)[flat];
    const uint32_t off = ((const SZ_GLOBAL uint32_t*)(dst + 64))[b];
    const SZ_GLOBAL u32x4* from = (const SZ_GLOBAL u32x4*)(gptr(a.staging) + flat * kBlockElems);
    SZ_GLOBAL uint8_t* to = dst + L.esc_at + off;
    for (uint32_t i = 0; i < cnt; i += 16) {
        const u32x4 v = from[i / 16];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (uint32_t k = 0; k < 16; ++k)
            if (i + k < cnt) to[i + k] = static_cast<uint8_t>(w[k / 4] >> (8 * (k & 3)));
    }
}

// k_offsets and k_scatter in one launch, for tensors of at most
// kFusedGroups x 256 blocks.  Workgroup g of tensor t takes blocks
// [256g, 256g + 256): its base offset is the sum of the counts of every
// earlier block, read directly (fewer than 256 x 256 reads, from L2), so no
// workgroup waits for another; an in-group scan gives each block its offset,
// which it writes to the table before copying its staged escapes.  The last
// workgroup of a tensor writes the header.
constexpr uint64_t kFusedGroups = 256;

template <uint32_t DT>
__global__ __launch_bounds__(kThreads) void k_offsets_scatter(EncodeArgs a) {
    __shared__ uint32_t s_sums[kWavesPerGroup];
    const Layout L = layout_of(a.n, DT);
    const uint32_t groups = static_cast<uint32_t>((L.blocks + kThreads - 1) / kThreads);
    const uint32_t t = blockIdx.x / groups, g = blockIdx.x - t * groups, tid = threadIdx.x;
    const SZ_GLOBAL uint32_t* counts = gptr(a.counts) + static_cast<uint64_t>(t) * L.blocks;
    uint32_t before = 0;
    for (uint32_t k = tid; k < g * kThreads; k += kThreads) before += counts[k];
    uint32_t base;
    block_scan_excl(before, tid, s_sums, base);
    __syncthreads();
    const uint64_t b = static_cast<uint64_t>(g) * kThreads + tid;
    const uint32_t cnt = b < L.blocks ? counts[b] : 0u;
    uint32_t in_group;
    const uint32_t off = base + block_scan_excl(cnt, tid, s_sums, in_group);
    SZ_GLOBAL uint8_t* dst = dst_of(a.dst, t);
    if (b < L.blocks) {
        ((SZ_GLOBAL uint32_t*)(dst + 64))[b] = off;
        const SZ_GLOBAL u32x4* from =
            (const SZ_GLOBAL u32x4*)(gptr(a.staging) + (static_cast<uint64_t>(t) * L.blocks + b) * kBlockElems);
        SZ_GLOBAL uint8_t* to = dst + L.esc_at + off;
        for (uint32_t i = 0; i < cnt; i += 16) {
            const u32x4 v = from[i / 16];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (uint32_t k = 0; k < 16; ++k)
                if (i + k < cnt) to[i + k] = static_cast<uint8_t>(w[k / 4] >> (8 * (k & 3)));
        }
    }
    if (g == groups - 1)
        write_header(dst, L, DT, gptr(a.codebooks) + 16ull * t, base + in_group,
                     a.out_bytes ? gptr(a.out_bytes) + t : nullptr, tid);
}

// n == 0: a header-only stream per tensor
template <uint32_t DT>
__global__ void k_encode_empty(EncodeArgs a) {
    const uint32_t t = blockIdx.x;
    const Layout L = layout_of(0, DT);
    SZ_GLOBAL uint8_t* dst = dst_of(a.dst, t);
    write_header(dst, L, DT, gptr(a.codebooks) + 16ull * t, 0, a.out_bytes ? gptr(a.out_bytes) + t : nullptr, lane_id());
}

// ---------------------------------------------------- one-launch compress
//
// Histogram, codebook and encode of every tensor in one launch that reads
// the input once.  A tensor's codebook depends on all of its exponents, but
// a sample of them nearly always ranks the same values first, so each
// tensor is coded with a provisional codebook built from a sample and
// checked against the final codebook afterwards.  Work items:
//   sample item (every kSampleStride-th 128 KB chunk of the tensor): counts
//     its chunk into the tensor's sample histogram.  It never waits.
//   provisional item: polls the sample histogram until it is complete (its
//     bins sum to the sampled element count; counts only grow), ranks the
//     values (count descending, then value ascending) and publishes the
//     first 15 as the provisional codebook.
//   main item (16 blocks, one per wave): loads its blocks and the
//     provisional codebook (waiting for it if it is not complete yet), counts
//     the blocks into the tensor's full histogram (the item that holds a
//     partial last block counts that block too) and encodes its full blocks
//     with the provisional codebook exactly as k_encode does.
//   final item: polls the full histogram until it is complete, writes the
//     histogram and codebook outputs and records whether the provisional
//     codebook is the final one.
// Where it is not, k_transcode rewrites the tensor's code nibbles and
// staged escapes for the final codebook from what the main items wrote,
// without reading the input again.  It is a separate launch, so what this
// kernel wrote is visible to it without cache maintenance.  The partial
// last block of a tensor is left to k_encode_tail, which runs with the
// final codebook.
//
// Work items are handed out by a ticket counter in the order workgroups
// start, in stages (pass_plan): stage s holds the sample items of tensor s,
// the provisional item of tensor s - 1, the main items of tensor s - lag
// and the final item of tensor s - lag - 1.  Every wait is for items with
// earlier tickets (a provisional item for sample items, a main item for
// the provisional item, a final item for main items and the provisional
// item), and sample items never wait, so every awaited workgroup is already
// running or done: the launch always makes progress, whatever else shares
// the GPU.  The waits are still bounded: after spin_limit polls, or once
// any workgroup has given up, a workgroup sets its tensor's status, zeroes
// its blocks' escape counts and leaves.
//
// Signalling between workgroups uses no cache-wide maintenance.  Everything
// one workgroup tells another inside the kernel travels through relaxed
// agent-scope atomics, which are coherent across the XCDs' L2 caches:
// read-modify-writes (histogram counts, tickets, the list) or sc1 loads and
// stores (the abort word, the provisional codebook).  The provisional
// codebook needs no separate flag and no store order: a reading of its
// four words is complete exactly when its 15 bytes differ (see
// codebook_complete).  Agent-scope acquire/release orderings would instead
// write back or invalidate a whole L2 at every publication and at every
// poll of every waiting workgroup.

struct SyncView {
    SZ_GLOBAL uint64_t* hist;     // count x 256, whole tensors
    SZ_GLOBAL uint64_t* sample;   // count x 256, sampled chunks
    SZ_GLOBAL uint32_t* ticket;
    SZ_GLOBAL uint32_t* abort;
    SZ_GLOBAL uint32_t* listed;   // [2]: entries in use of the two lists
    SZ_GLOBAL uint32_t* records;  // per tensor 32 words, see kRec*
    SZ_GLOBAL uint32_t* list;     // [2][count] entries of kEntryWords: tensors to recode, reordered ones, then the others
};

// A list entry: everything the recode of one tensor needs, in one 64-byte
// line: [0] tensor, [1..2] its stream's address, [4..7] the provisional
// codebook P, [8..11] the final codebook F, [12..15] map[c] = the code F
// gives the value P[c] (15 when F does not hold it; 15 -> 15).
constexpr uint32_t kEntryWords = 16;

constexpr uint32_t kRecProvisional = 0;  // 4 words: the provisional codebook (complete once 15 bytes differ)
constexpr uint32_t kRecVerdict = 8;      // kProvisionalSame / Reordered / Differs

__device__ inline SyncView sync_view(uint8_t* base, uint32_t count) {
    SyncView v;
    v.hist = gptr(reinterpret_cast<uint64_t*>(base));
    v.sample = v.hist + 256ull * count;
    SZ_GLOBAL uint32_t* w = gptr(reinterpret_cast<uint32_t*>(base + 4096ull * count));
    v.ticket = w;
    v.abort = w + 1;
    v.listed = w + 2;
    v.records = w + 64;
    v.list = v.records + 32ull * count;   // 2 x count entries
    return v;
}

__device__ inline uint32_t load_agent(const SZ_GLOBAL uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t load_agent(const SZ_GLOBAL uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void store_agent(SZ_GLOBAL uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int32_t kStatusGaveUp = 5;   // SZ_ERR_TIMEOUT

// A reading of a tensor's provisional codebook (lanes 0..3 of a wave each
// hold one of its words) is complete when bytes 0..14 are 15 distinct
// values: the record starts zeroed and every published codebook lists 15
// distinct values, so a reading that mixes published and still-zero words
// repeats a byte.  No flag, and no order among the four word stores, is
// needed.  Every lane of the wave calls it and gets the same result; lane c
// below 15 also gets byte c in `mine`.
__device__ inline bool codebook_complete(uint32_t word, uint32_t lane, uint32_t& mine) {
    const uint32_t w0 = __builtin_amdgcn_readlane(word, 0), w1 = __builtin_amdgcn_readlane(word, 1);
    const uint32_t w2 = __builtin_amdgcn_readlane(word, 2), w3 = __builtin_amdgcn_readlane(word, 3);
    const uint32_t c = lane < kCodes ? lane : 0u;
    const uint32_t w = c < 4 ? w0 : (c < 8 ? w1 : (c < 12 ? w2 : w3));
    mine = (w >> (8 * (c & 3u))) & 0xFFu;
    bool dup = false;
#pragma unroll
    for (uint32_t k = 0; k + 1 < kCodes; ++k) {
        const uint32_t other = __builtin_amdgcn_readlane(mine, k);
        if (k < c && other == mine) dup = true;
    }
    return __ballot(dup) == 0;
}

// One wave waits for a complete reading of the provisional codebook at
// `words`, starting from the reading it holds (`word`, lanes 0..3; updated
// by every poll).  Returns true with lane c's byte in `mine` (c < 15),
// false after spin_limit polls (raising the abort word) or once the abort
// word is up.  Every lane of the wave calls it and gets the same result.
__device__ inline bool wait_codebook(const SZ_GLOBAL uint32_t* words, uint32_t& word, const SyncView& sv,
                                     uint32_t spin_limit, uint32_t lane, uint32_t& mine) {
    for (uint32_t polls = 0;; ++polls) {
        if (codebook_complete(word, lane, mine)) return true;
        if (polls >= spin_limit) {
            if (lane == 0) store_agent(sv.abort, 1u);
            return false;
        }
        if (uniform(load_agent(sv.abort))) return false;
        __builtin_amdgcn_s_sleep(8);
        if (lane < 4) word = load_agent(words + lane);
    }
}

// Every thread of the workgroup polls a tensor's histogram until its bins
// sum to `total` (counts only grow, so that reading is final).  Returns 1
// with c = this thread's bin (0 for threads past the domain), or 2 after
// giving up.  Uses s_word[8..12].
template <uint32_t DT>
__device__ inline uint32_t wait_histogram(const SZ_GLOBAL uint64_t* hist, uint64_t total, const SyncView& sv,
                                          uint32_t spin_limit, uint32_t* s_word, uint32_t tid, uint32_t lane,
                                          uint32_t wave, uint64_t& c) {
    constexpr uint32_t D = Geometry<DT>::kDomain;
    for (uint32_t polls = 0;; ++polls) {
        c = tid < D ? load_agent(hist + tid) : 0;
        const uint32_t sum = __builtin_amdgcn_readlane(wave_scan_incl(static_cast<uint32_t>(c)), 63);
        if (lane == 0 && wave < 4) s_word[8 + wave] = sum;   // counts are at most n < 2^32
        __syncthreads();
        if (tid == 0) {
            const uint64_t got = static_cast<uint64_t>(s_word[8]) + s_word[9] + s_word[10] + s_word[11];
            uint32_t st = got == total ? 1u : 0u;
            if (!st && polls >= spin_limit) {
                store_agent(sv.abort, 1u);
                st = 2;
            }
            if (!st && load_agent(sv.abort)) st = 2;
            s_word[12] = st;
        }
        __syncthreads();
        const uint32_t state = s_word[12];
        if (state) return state;
        __syncthreads();   // every thread has read this round's words before the next round rewrites them
        __builtin_amdgcn_s_sleep(8);
    }
}

// Rank the values of the domain by (count descending, value ascending);
// the values of rank 0..14 become the codebook, left in s_word[2..5] (byte
// 15 zero).  c: this thread's bin.  The workgroup's kParts groups of 256
// threads each compare against a share of the keys; bins holds the keys
// and the partial ranks.  Ends with a barrier.
template <uint32_t DT>
__device__ inline void rank_codebook(uint64_t c, uint32_t* bins, uint32_t* s_word, uint32_t tid) {
    constexpr uint32_t D = Geometry<DT>::kDomain;
    constexpr uint32_t kParts = kPassThreads / 256;
    uint64_t* keys = reinterpret_cast<uint64_t*>(bins);
    uint32_t* parts = bins + 2 * 256;   // [kParts][256] partial ranks, after the keys
    if (tid < D) keys[tid] = (c << 8) | (255u - tid);
    if (tid < 4) s_word[2 + tid] = 0;
    __syncthreads();
    const uint32_t v = tid & 255u, q = tid >> 8;
    if (v < D) {
        const uint64_t key = keys[v];
        uint32_t part = 0;
        for (uint32_t u = q * (D / kParts); u < (q + 1) * (D / kParts); ++u) part += keys[u] > key ? 1u : 0u;
        parts[q * 256 + v] = part;
    }
    __syncthreads();
    if (q == 0 && v < D) {
        uint32_t rank = 0;
#pragma unroll
        for (uint32_t k = 0; k < kParts; ++k) rank += parts[k * 256 + v];
        if (rank < kCodes) reinterpret_cast<uint8_t*>(s_word + 2)[rank] = static_cast<uint8_t>(v);
    }
    __syncthreads();
}

// One work item; every thread of the workgroup calls it and every return
// is taken by all of them.  LDS: bins (counting and ranking), s_tbl (the
// code table, 256 bytes), s_word ([2..5] codebook, [6] the final item's
// "other values" flag, [8..13] poll words, [16..19] the provisional
// codebook in the final item; [0], [14], [15] hold the item and are not
// written).
template <uint32_t DT>
__device__ inline void run_item(const CompressArgs& a, const SyncView& sv, const PassItem& it, uint32_t* bins,
                                uint32_t* s_tbl, uint32_t* s_word, uint32_t tid, uint32_t lane, uint32_t wave) {
    const uint32_t t = it.t;
    const uint64_t n = a.enc.n;
    const SZ_GLOBAL uint8_t* src = src_of(a.enc.src, t);
    char* lds = reinterpret_cast<char*>(bins);
    SZ_GLOBAL uint32_t* rec = sv.records + 32ull * t;

    if (it.kind == kItemSample) {
        // ---- sample item: chunk idx * kSampleStride
        hist_clear<DT, kPassThreads>(bins, tid);
        __syncthreads();
        const uint64_t chunk = sample_chunk_elems(DT);
        const uint64_t begin = static_cast<uint64_t>(it.idx) * kSampleStride * chunk;
        const uint64_t end = n - begin < chunk ? n : begin + chunk;
        const uint32_t phantom = count_range<DT, kPassThreads, false>(lds, src, begin, end, tid);
        __syncthreads();
        hist_flush<DT, kPassThreads>(bins, tid, sv.sample + 256ull * t, phantom);
        return;
    }

    if (it.kind == kItemProvisional) {
        // ---- provisional item: rank the sample, publish the codebook
        uint64_t c = 0;
        if (wait_histogram<DT>(sv.sample + 256ull * t, a.sample_total, sv, a.spin_limit, s_word, tid, lane, wave,
                               c) != 1) {
            if (tid == 0 && a.status) gptr(a.status)[t] = kStatusGaveUp;
            return;
        }
        rank_codebook<DT>(c, bins, s_word, tid);
        if (tid < 4) store_agent(rec + kRecProvisional + tid, s_word[2 + tid]);   // the publication itself
        return;
    }

    if (it.kind == kItemFinal) {
        // ---- final item: rank the whole histogram, compare with the provisional codebook
        uint64_t c = 0;
        uint32_t ok = wait_histogram<DT>(sv.hist + 256ull * t, n, sv, a.spin_limit, s_word, tid, lane, wave, c) == 1;
        if (ok) {
            if (wave == 0) {
                uint32_t word = lane < 4 ? load_agent(rec + kRecProvisional + lane) : 0u, mine;
                const bool got = wait_codebook(rec + kRecProvisional, word, sv, a.spin_limit, lane, mine);
                if (got && lane < 4) s_word[16 + lane] = word;
                if (lane == 0) s_word[13] = got ? 1u : 0u;
            }
            __syncthreads();
            ok = s_word[13];
        }
        if (!ok) {
            if (tid == 0 && a.status) gptr(a.status)[t] = kStatusGaveUp;
            return;
        }
        if (tid < 256) gptr(a.hists)[256ull * t + tid] = c;
        rank_codebook<DT>(c, bins, s_word, tid);
        if (tid < 4) gptr(reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(a.enc.codebooks) + 16ull * t))[tid] =
            s_word[2 + tid];
        // same values in the same order, the same values in another order
        // (thread v < D: is v in both codebooks or in neither?), or others;
        // threads c < 16 also find the code F gives P[c] (the recode map)
        if (tid == 0) s_word[6] = 0;
        __syncthreads();
        if (tid < 16) {
            const uint8_t* pb = reinterpret_cast<const uint8_t*>(s_word + 16);
            const uint8_t* fb = reinterpret_cast<const uint8_t*>(s_word + 2);
            uint32_t m = kEscape;
            if (tid < kCodes) {
#pragma unroll
                for (uint32_t k = kCodes; k-- > 0;)
                    if (fb[k] == pb[tid]) m = k;
            }
            reinterpret_cast<uint8_t*>(s_word + 8)[tid] = static_cast<uint8_t>(m);
        }
        if (tid < Geometry<DT>::kDomain) {
            const uint8_t* pb = reinterpret_cast<const uint8_t*>(s_word + 16);
            const uint8_t* fb = reinterpret_cast<const uint8_t*>(s_word + 2);
            bool in_p = false, in_f = false;
#pragma unroll
            for (uint32_t k = 0; k < kCodes; ++k) {
                in_p |= pb[k] == tid;
                in_f |= fb[k] == tid;
            }
            if (in_p != in_f) s_word[6] = 1;   // benign race: every writer stores 1
        }
        __syncthreads();
        if (tid == 0) {
            bool same = true;
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) same &= s_word[16 + k] == s_word[2 + k];
            store_agent(rec + kRecVerdict,
                        same ? kProvisionalSame : (s_word[6] ? kProvisionalDiffers : kProvisionalReordered));
            uint32_t slot = ~0u;
            if (!same) {
                const uint32_t k = s_word[6] ? 1u : 0u;   // list 0: reordered, 1: other values
                slot = k * a.enc.count +
                       __hip_atomic_fetch_add(sv.listed + k, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            s_word[7] = slot;   // a tensor is listed at most once, so a slot stays below 2 x count
        }
        __syncthreads();
        const uint32_t slot = s_word[7];
        if (slot != ~0u && tid < kEntryWords) {   // the entry, read by the next launch
            const uint64_t d = reinterpret_cast<uint64_t>(dst_of(a.enc.dst, t));
            const uint32_t word = tid == 0   ? t
                                  : tid == 1 ? static_cast<uint32_t>(d)
                                  : tid == 2 ? static_cast<uint32_t>(d >> 32)
                                  : tid < 4  ? 0u
                                  : tid < 8  ? s_word[16 + tid - 4]
                                  : tid < 12 ? s_word[2 + tid - 8]
                                             : s_word[8 + tid - 12];
            sv.list[static_cast<uint64_t>(slot) * kEntryWords + tid] = word;
        }
        return;
    }
    if (it.kind != kItemMain) return;

    // ---- main item: blocks 16 * idx + wave of tensor t.  Block loads and
    // the provisional codebook first (it is normally complete long before);
    // wave 0 checks the codebook and builds the one code table all 16 waves
    // share, while the LDS histogram is cleared; then every wave encodes its
    // block and counts its exponents in the same pass, and the item adds
    // its counts to the tensor's histogram.
    const Layout L = layout_of(n, DT);
    const uint64_t full_blocks = n / kBlockElems;
    const uint64_t b = static_cast<uint64_t>(it.idx) * kPassWaves + wave;
    const bool mine_full = b < full_blocks;
    const uint64_t flat = static_cast<uint64_t>(t) * L.blocks + b;
    uint32_t word = wave == 0 && lane < 4 ? load_agent(rec + kRecProvisional + lane) : 0u;
    BlockRegs<DT> d;
    if (mine_full) load_block<DT, true>(src, n, b, lane, d);
    hist_clear<DT, kPassThreads>(bins, tid);
    if (wave == 0) {
        uint32_t mine;
        const bool got = wait_codebook(rec + kRecProvisional, word, sv, a.spin_limit, lane, mine);
        if (got) build_code_table(s_tbl, lane, lane < kCodes ? mine : 0xFFFFu);
        if (lane == 0) s_word[12] = got ? 1u : 0u;
    }
    __syncthreads();
    if (mine_full) {
        const uint32_t copy4 = hist_lane_bytes<DT>(tid);
#pragma unroll
        for (uint32_t j = 0; j < Geometry<DT>::kSubs; ++j)
#pragma unroll
            for (uint32_t i = 0; i < Geometry<DT>::kInWords; ++i) count_dword<DT>(lds, d[j][i], copy4);
    }
    if (s_word[12]) {
        if (mine_full)
            encode_loaded<DT, true>(a.enc, L, dst_of(a.enc.dst, t), b, flat, lane,
                                    reinterpret_cast<const uint8_t*>(s_tbl), d);
    } else {
        // gave up: no escapes for this block (so the scatter that follows
        // stays inside the stream) and an error for the tensor
        if (mine_full && lane == 0) gptr(a.enc.counts)[flat] = 0;
        if (tid == 0 && a.status) gptr(a.status)[t] = kStatusGaveUp;
    }
    uint32_t phantom = 0;
    if (n % kBlockElems && full_blocks / kPassWaves == it.idx)   // the partial last block is in this item
        phantom = count_ragged<DT, kPassThreads>(lds, src, full_blocks * kBlockElems, n, tid);
    __syncthreads();
    hist_flush<DT, kPassThreads>(bins, tid, sv.hist + 256ull * t, phantom);
}

// One workgroup per item: the ticket taken at the start fixes the item.
template <uint32_t DT>
__global__ __launch_bounds__(kPassThreads, 8) void k_compress(CompressArgs a) {
    static_assert(kPassThreads % 256 == 0 && Geometry<DT>::kDomain % (kPassThreads / 256) == 0, "rank split");
    __shared__ uint32_t bins[HistLds<DT>::kWords];
    __shared__ uint32_t s_tbl[64];    // the code table of a main item, shared by its waves
    __shared__ uint32_t s_word[20];   // [0], [14], [15] the item
    const uint32_t tid = threadIdx.x, lane = lane_id();
    const uint32_t wave = uniform(tid / kWaveSize);
    const SyncView sv = sync_view(a.sync, a.enc.count);
    if (tid == 0) {
        // one thread locates the item (the schedule arithmetic stays out of
        // the scalar registers the rest of the kernel needs)
        const uint32_t ticket = __hip_atomic_fetch_add(sv.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const PassItem it = pass_item(ticket, pass_plan(a));
        s_word[0] = it.kind;
        s_word[14] = it.t;
        s_word[15] = it.idx;
    }
    __syncthreads();
    const PassItem it{uniform(s_word[0]), uniform(s_word[14]), uniform(s_word[15])};
    run_item<DT>(a, sv, it, bins, s_tbl, s_word, tid, lane, wave);
}

// Byte c (0..15) of a 16-byte table held in four registers; c may differ
// between lanes (a byte permute, not an indexed register array).
__device__ inline uint32_t table_byte(const uint32_t (&w)[4], uint32_t c) {
    return lookup4(c & 0xFu, w) & 0xFFu;
}

// What a wave reads of block b before recoding it: the code words, the
// escape count and the first 256 staged escape bytes (16 bytes in each of
// lanes 0..15; most blocks have fewer escapes, and the rest, if any, is
// read when the block is recoded).  None of it depends on the count, so
// the reads of the next block are in flight while this one is recoded.
template <uint32_t DT>
struct TranscodeIn {
    uint32_t cw[Geometry<DT>::kSubs][Geometry<DT>::kCodeWords];
    uint32_t count;
    u32x4 head;
};

template <uint32_t DT>
__device__ inline void transcode_read(const EncodeArgs& a, const Layout& L, const SZ_GLOBAL uint8_t* dst, uint64_t b,
                                      uint64_t flat, uint32_t lane, bool codes_only, TranscodeIn<DT>& in) {
    using G = Geometry<DT>;
    constexpr uint32_t kSubBytes = kWaveSize * G::kLaneElems / 2;   // code bytes per sub-chunk
    const SZ_GLOBAL uint8_t* codes = dst + L.code_at + b * (kBlockElems / 2) + lane * (G::kLaneElems / 2);
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; ++j) {
        if constexpr (G::kCodeWords == 1) {
            in.cw[j][0] = __builtin_nontemporal_load((const SZ_GLOBAL uint32_t*)(codes + j * kSubBytes));
        } else {
            const u32x4 v = __builtin_nontemporal_load((const SZ_GLOBAL u32x4*)(codes + j * kSubBytes));
            in.cw[j][0] = v.x; in.cw[j][1] = v.y; in.cw[j][2] = v.z; in.cw[j][3] = v.w;
        }
    }
    in.count = 0;
    in.head = u32x4{0, 0, 0, 0};
    if (codes_only) return;
    in.count = gptr(a.counts)[flat];
    if (lane < 16) in.head = *(const SZ_GLOBAL u32x4*)(gptr(a.staging) + flat * kBlockElems + 16 * lane);
}

// A block of a reordered tensor: only its code nibbles change (escapes
// keep their codes, values and places).
template <uint32_t DT>
__device__ inline void transcode_codes(const Layout& L, SZ_GLOBAL uint8_t* dst, uint64_t b, uint32_t lane,
                                       const uint32_t (&map)[4], const TranscodeIn<DT>& in) {
    using G = Geometry<DT>;
    constexpr uint32_t kSubBytes = kWaveSize * G::kLaneElems / 2;
    SZ_GLOBAL uint8_t* codes = dst + L.code_at + b * (kBlockElems / 2) + lane * (G::kLaneElems / 2);
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; ++j) {
        uint32_t x[G::kCodeWords];
#pragma unroll
        for (uint32_t q = 0; q < G::kCodeWords; ++q) {
            const uint32_t w = in.cw[j][q];
            x[q] = lookup4(w & 0x0F0F0F0Fu, map) | (lookup4((w >> 4) & 0x0F0F0F0Fu, map) << 4);
        }
        if constexpr (G::kCodeWords == 1)
            __builtin_nontemporal_store(x[0], (SZ_GLOBAL uint32_t*)(codes + j * kSubBytes));
        else
            __builtin_nontemporal_store(u32x4{x[0], x[1], x[2], x[3]}, (SZ_GLOBAL u32x4*)(codes + j * kSubBytes));
    }
}

// Block b, coded with codebook P (bytes pw), recoded for the codebook whose
// code table is tbl.  map: P's code c -> the new code of value P[c] (15 ->
// 15).  The block's P escapes are copied to LDS (esc) first, so the new
// escapes can be staged in their place.  An escape count or code plane that
// was never written (a tensor that gave up) is harmless: every rank stays
// below 4096, inside the block's LDS copy and staging slot.
template <uint32_t DT>
__device__ inline void transcode_block(const EncodeArgs& a, const Layout& L, SZ_GLOBAL uint8_t* dst, uint64_t b,
                                       uint64_t flat, uint32_t lane, const uint8_t* tbl, const uint32_t (&map)[4],
                                       const uint32_t (&pw)[4], uint32_t* esc_words, const TranscodeIn<DT>& in) {
    using G = Geometry<DT>;
    constexpr uint32_t kCW = G::kCodeWords;
    SZ_GLOBAL uint8_t* stage = gptr(a.staging) + flat * kBlockElems;
    uint32_t old_total = uniform(in.count);
    old_total = old_total < kBlockElems ? old_total : kBlockElems;
    if (lane < 16) {
        esc_words[4 * lane] = in.head.x; esc_words[4 * lane + 1] = in.head.y;
        esc_words[4 * lane + 2] = in.head.z; esc_words[4 * lane + 3] = in.head.w;
    }
    for (uint32_t i = 256 + lane * 16; i < old_total; i += kWaveSize * 16) {
        const u32x4 v = *(const SZ_GLOBAL u32x4*)(stage + i);
        esc_words[i / 4] = v.x; esc_words[i / 4 + 1] = v.y; esc_words[i / 4 + 2] = v.z; esc_words[i / 4 + 3] = v.w;
    }
    __builtin_amdgcn_wave_barrier();
    const uint8_t* esc = reinterpret_cast<const uint8_t*>(esc_words);

    // Element order is (sub-chunk, lane, element), so sub-chunks are taken
    // in order, two at a time, with running old and new escape ranks.
    constexpr uint32_t kSubBytes = kWaveSize * G::kLaneElems / 2;
    SZ_GLOBAL uint8_t* codes = dst + L.code_at + b * (kBlockElems / 2) + lane * (G::kLaneElems / 2);
    uint32_t orun = 0, nrun = 0;
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; j += 2) {
        // old ranks of this lane's first escape in sub-chunks j and j + 1
        uint32_t c0 = 0, c1 = 0;
#pragma unroll
        for (uint32_t q = 0; q < kCW; ++q) {
            c0 += __builtin_popcount(escape_nibbles(in.cw[j][q]));
            c1 += __builtin_popcount(escape_nibbles(in.cw[j + 1][q]));
        }
        uint32_t packed = c0 | (c1 << 16);
        uint32_t incl = wave_scan_incl(packed);
        uint32_t excl = incl - packed;
        uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
        const uint32_t ob[2] = {orun + (excl & 0xFFFFu), orun + (tot & 0xFFFFu) + (excl >> 16)};
        orun += (tot & 0xFFFFu) + (tot >> 16);
        // new code words: P codes through the map, P escapes through the table
        uint32_t nw[2][kCW];
        c0 = 0;
        c1 = 0;
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            uint32_t r = ob[h];
#pragma unroll
            for (uint32_t q = 0; q < kCW; ++q) {
                const uint32_t w = in.cw[j + h][q];
                uint32_t x = lookup4(w & 0x0F0F0F0Fu, map) | (lookup4((w >> 4) & 0x0F0F0F0Fu, map) << 4);
                uint32_t m = escape_nibbles(w);
                while (m) {
                    const uint32_t sh = __builtin_ctz(m);   // 4 * nibble index
                    const uint32_t v = esc[r < kBlockElems ? r : kBlockElems - 1];
                    ++r;
                    x = (x & ~(0xFu << sh)) | (static_cast<uint32_t>(tbl[v]) << sh);
                    m &= m - 1;
                }
                nw[h][q] = x;
                (h ? c1 : c0) += __builtin_popcount(escape_nibbles(x));
            }
            if constexpr (kCW == 1)
                __builtin_nontemporal_store(nw[h][0], (SZ_GLOBAL uint32_t*)(codes + (j + h) * kSubBytes));
            else
                __builtin_nontemporal_store(u32x4{nw[h][0], nw[h][1], nw[h][2], nw[h][3]},
                                            (SZ_GLOBAL u32x4*)(codes + (j + h) * kSubBytes));
        }
        // new ranks, then the new escape bytes: a P code that lost its place
        // escapes with its value P[c]; a P escape that stays one keeps its byte
        packed = c0 | (c1 << 16);
        incl = wave_scan_incl(packed);
        excl = incl - packed;
        tot = __builtin_amdgcn_readlane(incl, 63);
        const uint32_t nb[2] = {nrun + (excl & 0xFFFFu), nrun + (tot & 0xFFFFu) + (excl >> 16)};
        nrun += (tot & 0xFFFFu) + (tot >> 16);
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            uint32_t rank = nb[h];
            uint32_t before = ob[h];   // P escapes of this lane in the sub-chunk ahead of word q
#pragma unroll
            for (uint32_t q = 0; q < kCW; ++q) {
                const uint32_t w = in.cw[j + h][q];
                const uint32_t oe = escape_nibbles(w);
                uint32_t m = escape_nibbles(nw[h][q]);
                while (m) {
                    const uint32_t sh = __builtin_ctz(m);
                    const uint32_t c = (w >> sh) & 0xFu;
                    uint32_t v;
                    if (c < kEscape) {
                        v = table_byte(pw, c);
                    } else {
                        const uint32_t r = before + __builtin_popcount(oe & ((1u << sh) - 1u));
                        v = esc[r < kBlockElems ? r : kBlockElems - 1];
                    }
                    stage[rank < kBlockElems ? rank : kBlockElems - 1] = static_cast<uint8_t>(v);
                    ++rank;
                    m &= m - 1;
                }
                before += __builtin_popcount(oe);
            }
        }
    }
    if (lane == 0) gptr(a.counts)[flat] = uniform(nrun);
}

// A listed tensor's tables, from its list entry (one 64-byte load): its
// index, stream, provisional codebook P and recode map.  The wave's LDS
// table tbl_words receives the code of every value under the final
// codebook F.
struct TranscodeTables {
    uint32_t t;
    SZ_GLOBAL uint8_t* dst;
    uint32_t pw[4];
    uint32_t map[4];
};

__device__ inline TranscodeTables transcode_tables(const SZ_GLOBAL uint32_t* list, uint64_t entry,
                                                   uint32_t* tbl_words, uint32_t lane) {
    const uint32_t word = lane < kEntryWords ? list[entry * kEntryWords + lane] : 0u;
    TranscodeTables r;
    // (readlane returns a signed int: each word is taken as unsigned before
    // it is widened, or a set bit 31 would fill the high half)
    r.t = static_cast<uint32_t>(__builtin_amdgcn_readlane(word, 0));
    const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(word, 1));
    const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(word, 2));
    r.dst = reinterpret_cast<SZ_GLOBAL uint8_t*>(lo | (hi << 32));
    uint32_t fw[4];
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) {
        r.pw[k] = __builtin_amdgcn_readlane(word, 4 + k);
        fw[k] = __builtin_amdgcn_readlane(word, 8 + k);
        r.map[k] = __builtin_amdgcn_readlane(word, 12 + k);
    }
    build_code_table(tbl_words, lane, lane < kCodes ? table_byte(fw, lane) : 0xFFFFu);
    return r;
}

// The full blocks of the `listed` tensors of one list, split into equal
// contiguous runs, one per wave of the grid (wave w of `waves`).  A wave
// reads its next block while it recodes the current one.  kCodesOnly: the
// list of reordered tensors, whose escapes stay as they are.
template <uint32_t DT, bool kCodesOnly>
__device__ inline void transcode_list(const CompressArgs& a, const SyncView& sv, const SZ_GLOBAL uint32_t* list,
                                      uint32_t listed, uint64_t w, uint64_t waves, uint32_t* tbl_words,
                                      uint32_t* esc_words, uint32_t lane) {
    const uint64_t full_blocks = a.enc.n / kBlockElems;
    const uint64_t total = static_cast<uint64_t>(listed < a.enc.count ? listed : a.enc.count) * full_blocks;
    const uint64_t per = (total + waves - 1) / waves;
    const uint64_t first = w * per;
    const uint64_t last = first + per < total ? first + per : total;
    if (first >= last) return;
    const Layout L = layout_of(a.enc.n, DT);
    const uint8_t* tbl = reinterpret_cast<const uint8_t*>(tbl_words);
    __builtin_amdgcn_wave_barrier();   // a table of an earlier list is no longer read
    TranscodeTables tt = transcode_tables(list, first / full_blocks, tbl_words, lane);
    TranscodeIn<DT> cur, next;
    transcode_read<DT>(a.enc, L, tt.dst, first % full_blocks,
                       static_cast<uint64_t>(tt.t) * L.blocks + first % full_blocks, lane, kCodesOnly, cur);
    for (uint64_t i = first; i < last; ++i) {
        const uint64_t b = i % full_blocks;
        const bool ahead = i + 1 < last && (i + 1) / full_blocks == i / full_blocks;   // same tensor
        if (ahead)
            transcode_read<DT>(a.enc, L, tt.dst, b + 1, static_cast<uint64_t>(tt.t) * L.blocks + b + 1, lane,
                               kCodesOnly, next);
        if (kCodesOnly)
            transcode_codes<DT>(L, tt.dst, b, lane, tt.map, cur);
        else
            transcode_block<DT>(a.enc, L, tt.dst, b, static_cast<uint64_t>(tt.t) * L.blocks + b, lane, tbl, tt.map,
                                tt.pw, esc_words, cur);
        if (i + 1 < last) {
            if (!ahead) {
                __builtin_amdgcn_wave_barrier();   // the previous tensor's table is no longer read
                tt = transcode_tables(list, (i + 1) / full_blocks, tbl_words, lane);
                transcode_read<DT>(a.enc, L, tt.dst, 0, static_cast<uint64_t>(tt.t) * L.blocks, lane, kCodesOnly,
                                   next);
            }
            cur = next;
        }
    }
}

// Tensors whose provisional codebook was not the final one (the final
// items list them): every full block of a listed tensor is recoded for the
// final codebook, first the reordered tensors' code nibbles, then the other
// tensors' codes and escapes, each list spread over every wave of the grid
// so a short list still covers the whole GPU; with empty lists every
// workgroup leaves at once.
template <uint32_t DT>
__global__ __launch_bounds__(kThreads, 8) void k_transcode(CompressArgs a) {
    __shared__ uint32_t s_tbl[kWavesPerGroup][64];
    __shared__ uint32_t s_esc[kWavesPerGroup][kBlockElems / 4];
    const uint32_t lane = lane_id(), wave = uniform(threadIdx.x / kWaveSize);
    const SyncView sv = sync_view(a.sync, a.enc.count);
    const uint64_t waves = static_cast<uint64_t>(gridDim.x) * kWavesPerGroup;
    const uint64_t w = static_cast<uint64_t>(blockIdx.x) * kWavesPerGroup + wave;
    transcode_list<DT, true>(a, sv, sv.list, uniform(sv.listed[0]), w, waves, s_tbl[wave], s_esc[wave], lane);
    transcode_list<DT, false>(a, sv, sv.list + static_cast<uint64_t>(a.enc.count) * kEntryWords,
                              uniform(sv.listed[1]), w, waves, s_tbl[wave], s_esc[wave], lane);
}

// ----------------------------------------------------------------- decode

// The 16 header dwords of a stream (caller guarantees src_bytes >= 64).
__device__ inline void load_header(const SZ_GLOBAL uint8_t* src, uint32_t (&w)[16]) {
    const SZ_GLOBAL uint32_t* h = (const SZ_GLOBAL uint32_t*)src;
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i) w[i] = h[i];
}

// Header check shared by all waves of a stream.  Returns the escape count
// or -1 when the stream does not match (n, dtype, src_bytes) or itself;
// fills the codebook registers.
template <uint32_t DT>
__device__ inline int64_t check_header(const uint32_t (&h)[16], uint64_t src_bytes, const Layout& L,
                                       uint32_t (&cbw)[4]) {
    uint32_t w[16];
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i) w[i] = uniform(h[i]);
    const uint64_t n = w[2] | (static_cast<uint64_t>(w[3]) << 32);
    const uint64_t escapes = w[4] | (static_cast<uint64_t>(w[5]) << 32);
    const uint64_t total = w[10] | (static_cast<uint64_t>(w[11]) << 32);
    bool ok = w[0] == kMagic;
    ok &= w[1] == (kVersion | (DT << 8) | (kLog2Block << 16) | (kCodes << 24));
    ok &= n == L.n;
    ok &= (w[9] >> 24) == 0;
    ok &= (w[12] | w[13] | w[14] | w[15]) == 0;
    ok &= escapes <= L.n;
    ok &= total == L.esc_at + escapes;
    ok &= total <= src_bytes;
    cbw[0] = w[6]; cbw[1] = w[7]; cbw[2] = w[8]; cbw[3] = w[9];
    return ok ? static_cast<int64_t>(escapes) : -1;
}

__device__ inline void mark_corrupt(SZ_GLOBAL int32_t* status, uint32_t lane) {
    if (status && lane == 0) *status = 3;  // SZ_ERR_CORRUPT_STREAM
}

__device__ inline void put_byte(uint32_t& w0, uint32_t& w1, uint32_t k, uint32_t e) {
    const uint32_t shift = 8 * (k & 3);
    const uint32_t clear = ~(0xFFu << shift);
    if (k < 4)
        w0 = (w0 & clear) | (e << shift);
    else
        w1 = (w1 & clear) | (e << shift);
}

// Decode work split.  BF16: lane l of sub-chunk j owns 8 elements, so per
// lane one code dword, two sign|mantissa dwords and four output dwords.
// E5M2: 16 elements per lane, so per lane two code dwords, the lane's 48
// bits of 3-bit fields (inside one aligned dword pair) and four output
// dwords.  Either way every code load and output store of the wave is one
// contiguous run.
template <uint32_t DT>
struct DecodeGeometry;
template <>
struct DecodeGeometry<kDtypeBF16> {
    static constexpr uint32_t kLaneElems = 8;
    static constexpr uint32_t kSubs = 8;
    static constexpr uint32_t kCodeWords = 1;
    static constexpr uint32_t kSmWords = 2;
    static constexpr uint32_t kOutWords = 4;
};
template <>
struct DecodeGeometry<kDtypeE5M2> {
    static constexpr uint32_t kLaneElems = 16;
    static constexpr uint32_t kSubs = 4;
    static constexpr uint32_t kCodeWords = 2;
    static constexpr uint32_t kSmWords = 2;
    static constexpr uint32_t kOutWords = 4;
};

constexpr uint32_t kPrefetch = 2 * kWaveSize;   // escape bytes staged in LDS per block

// Replace the exponent bytes of this lane's escaped elements (escape nibble
// mask m over the 8 elements held in e0/e1) with the next escape bytes.
// `near` is wave-uniform: when every escape of the block sits in the LDS
// copy, the loop touches no global memory, so it never waits on the
// block's outstanding stores.
__device__ inline void patch_escapes(uint32_t& e0, uint32_t& e1, uint32_t m, uint32_t& rank, bool near,
                                     const uint8_t* esc_near, const SZ_GLOBAL uint8_t* esc_in) {
    if (near) {
        while (m) {
            put_byte(e0, e1, __builtin_ctz(m) >> 2, esc_near[rank++]);
            m &= m - 1;
        }
    } else {
        while (m) {
            put_byte(e0, e1, __builtin_ctz(m) >> 2, esc_in[rank++]);
            m &= m - 1;
        }
    }
}

// One block.  kFull: the block holds 4096 elements (every lane's elements
// exist), so the loads and stores need no per-lane guards.
template <uint32_t DT, bool kFull>
__device__ inline void decode_block(const DecodeArgs& a, const Layout& L, uint32_t t, uint64_t b,
                                    uint32_t lane, uint8_t* esc_near) {
    using G = DecodeGeometry<DT>;
    constexpr uint32_t kSubElems = kWaveSize * G::kLaneElems;
    const SZ_GLOBAL uint8_t* src = src_of(a.src, t);
    const uint64_t src_bytes = a.src_bytes_table ? gptr(a.src_bytes_table)[t] : a.src_bytes;
    SZ_GLOBAL int32_t* status = a.status ? gptr(a.status) + t : nullptr;
    // Every read below lies in [0, esc_at) -- header, offsets, both planes
    // (an E5M2 lane's 8-byte field load may run past the plane into its padding
    // or the code region) --
    // or, for escape bytes, below src_bytes.  With that range readable, all
    // loads are issued at once and the stream is validated afterwards.
    if (src_bytes < L.esc_at) {
        mark_corrupt(status, lane);
        return;
    }
    // one load: header dwords (lanes 0..15) and offsets b, b+1 (lanes 16, 17;
    // the offset table starts at dword 16); other lanes re-read dword 0
    const uint64_t meta_at = lane < 16 ? lane
                             : lane == 16 ? 16 + b
                             : (lane == 17 && b + 1 < L.blocks) ? 17 + b : 0;
    const uint32_t meta = ((const SZ_GLOBAL uint32_t*)src)[meta_at];

    const uint64_t blk0 = b * kBlockElems;
    uint32_t cw[G::kSubs][G::kCodeWords];
    uint32_t sm[G::kSubs][G::kSmWords];
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; ++j) {
        const uint64_t elem0 = blk0 + j * kSubElems + lane * G::kLaneElems;
        if (kFull || elem0 < L.n) {
            if constexpr (DT == kDtypeBF16) {
                cw[j][0] = __builtin_nontemporal_load((const SZ_GLOBAL uint32_t*)(src + L.code_at + elem0 / 2));
                const u32x2 v = __builtin_nontemporal_load((const SZ_GLOBAL u32x2*)(src + L.sm_at + elem0));
                sm[j][0] = v.x; sm[j][1] = v.y;
            } else {
                const u32x2 c = __builtin_nontemporal_load((const SZ_GLOBAL u32x2*)(src + L.code_at + elem0 / 2));
                cw[j][0] = c.x; cw[j][1] = c.y;
                // the lane's 6 field bytes start 0 or 2 bytes into this dword pair
                const uint64_t sm_off = elem0 / 16 * 6;
                const u32x2 v = __builtin_nontemporal_load((const SZ_GLOBAL u32x2*)(src + L.sm_at + (sm_off & ~3ull)));
                sm[j][0] = v.x; sm[j][1] = v.y;
            }
        } else {
#pragma unroll
            for (uint32_t q = 0; q < G::kCodeWords; ++q) cw[j][q] = 0;
#pragma unroll
            for (uint32_t q = 0; q < G::kSmWords; ++q) sm[j][q] = 0;
        }
    }

    // keep every plane load ahead of the wait for the offset below
    __builtin_amdgcn_sched_barrier(0);

    // The block's first escape bytes, fetched as soon as its offset is known
    // (addresses clamped into the buffer; bytes past the block are unused).
    const uint32_t first = __builtin_amdgcn_readlane(meta, 16);
    const uint64_t esc_first = L.esc_at + first;
    const uint64_t last = src_bytes - 1;
    const uint64_t p0 = esc_first + lane, p1 = esc_first + kWaveSize + lane;
    const uint32_t pre0 = src[p0 < last ? p0 : last];
    const uint32_t pre1 = src[p1 < last ? p1 : last];

    uint32_t hdr[16], cbw[4];
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i) hdr[i] = __builtin_amdgcn_readlane(meta, i);
    const int64_t escapes = check_header<DT>(hdr, src_bytes, L, cbw);
    // (offsets are unsigned 32-bit: readlane's signed result is taken as
    // unsigned before widening, so offsets from 2^31 on stay what they are)
    const uint32_t next_word = static_cast<uint32_t>(__builtin_amdgcn_readlane(meta, 17));
    const uint64_t next = b + 1 < L.blocks ? static_cast<uint64_t>(next_word) : static_cast<uint64_t>(escapes);
    if (escapes < 0 || (b == 0 && first != 0) || next < first || next > static_cast<uint64_t>(escapes)) {
        mark_corrupt(status, lane);
        return;
    }

    uint32_t esc[G::kSubs][G::kCodeWords];
    uint32_t cnt[G::kSubs];
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; ++j) {
        cnt[j] = 0;
        const uint64_t elem0 = blk0 + j * kSubElems + lane * G::kLaneElems;
        const int64_t valid = static_cast<int64_t>(L.n) - static_cast<int64_t>(elem0);
#pragma unroll
        for (uint32_t q = 0; q < G::kCodeWords; ++q) {
            esc[j][q] = escape_nibbles(cw[j][q]);
            if (!kFull)
                esc[j][q] &= valid_nibbles(static_cast<int32_t>(valid > 64 ? 64 : valid) - 8 * static_cast<int32_t>(q));
            cnt[j] += __builtin_popcount(esc[j][q]);
        }
    }

    // Escape ranks inside the block (element order = sub-chunk, lane,
    // element); sub-chunk counts are scanned two at a time in 16-bit halves.
    uint32_t base[G::kSubs];
    uint32_t block_total = 0;
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; j += 2) {
        const uint32_t packed = cnt[j] | (cnt[j + 1] << 16);
        const uint32_t incl = wave_scan_incl(packed);
        const uint32_t excl = incl - packed;
        const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
        base[j] = block_total + (excl & 0xFFFFu);
        block_total += tot & 0xFFFFu;
        base[j + 1] = block_total + (excl >> 16);
        block_total += tot >> 16;
    }
    block_total = uniform(block_total);
    if (block_total != next - first) {
        mark_corrupt(status, lane);
        return;
    }
    esc_near[lane] = static_cast<uint8_t>(pre0);
    esc_near[kWaveSize + lane] = static_cast<uint8_t>(pre1);
    __builtin_amdgcn_wave_barrier();

    const SZ_GLOBAL uint8_t* esc_in = src + esc_first;
    const bool near = block_total <= kPrefetch;   // all escapes of the block are in LDS
    SZ_GLOBAL uint8_t* dst = dst_of(a.dst, t);
#pragma unroll
    for (uint32_t j = 0; j < G::kSubs; ++j) {
        const uint64_t elem0 = blk0 + j * kSubElems + lane * G::kLaneElems;
        if (!kFull && elem0 >= L.n) continue;
        uint32_t rank = base[j];
        uint32_t out[G::kOutWords];
        if constexpr (DT == kDtypeBF16) {
            const uint32_t c = cw[j][0];
            const uint32_t ev = lookup4(c & 0x0F0F0F0Fu, cbw);         // elements 0,2,4,6
            const uint32_t od = lookup4((c >> 4) & 0x0F0F0F0Fu, cbw);  // elements 1,3,5,7
            uint32_t e0 = perm(od, ev, 0x05010400u);                    // elements 0..3
            uint32_t e1 = perm(od, ev, 0x07030602u);                    // elements 4..7
            patch_escapes(e0, e1, esc[j][0], rank, near, esc_near, esc_in);
            // (sign|mantissa byte s, exponent byte e) pairs -> BF16 words
#pragma unroll
            for (uint32_t h = 0; h < 4; ++h) {
                const uint32_t ew = h < 2 ? e0 : e1;
                const uint32_t v = perm(ew, sm[j][h >> 1], (h & 1) ? 0x07030602u : 0x05010400u);
                out[h] = ((v >> 1) & 0x7F807F80u) | ((v << 8) & 0x80008000u) | (v & 0x007F007Fu);
            }
        } else {
            // 48 field bits: four 12-bit groups of four elements each
            const uint32_t shift = (static_cast<uint32_t>(elem0 / 16 * 6) & 3u) * 8u;   // 0 or 16
            const uint32_t lo = __builtin_amdgcn_alignbit(sm[j][1], sm[j][0], shift);
            const uint32_t hi = sm[j][1] >> shift;
            uint32_t f[4];
            f[0] = lo & 0xFFFu;
            f[1] = (lo >> 12) & 0xFFFu;
            f[2] = (lo >> 24) | ((hi & 0xFu) << 8);
            f[3] = (hi >> 4) & 0xFFFu;
#pragma unroll
            for (uint32_t q = 0; q < 2; ++q) {
                const uint32_t c = cw[j][q];
                const uint32_t ev = lookup4(c & 0x0F0F0F0Fu, cbw);
                const uint32_t od = lookup4((c >> 4) & 0x0F0F0F0Fu, cbw);
                uint32_t e0 = perm(od, ev, 0x05010400u);
                uint32_t e1 = perm(od, ev, 0x07030602u);
                patch_escapes(e0, e1, esc[j][q], rank, near, esc_near, esc_in);
#pragma unroll
                for (uint32_t h = 0; h < 2; ++h) {
                    const uint32_t v = f[2 * q + h];
                    const uint32_t sf = (v & 0x7u) | ((v & 0x38u) << 5) | ((v & 0x1C0u) << 10) | ((v & 0xE00u) << 15);
                    const uint32_t e = h ? e1 : e0;
                    out[2 * q + h] = ((sf & 0x04040404u) << 5) | ((e & 0x1F1F1F1Fu) << 2) | (sf & 0x03030303u);
                }
            }
        }
        SZ_GLOBAL uint8_t* p = dst + elem0 * (DT == kDtypeBF16 ? 2 : 1);
        if (kFull || elem0 + G::kLaneElems <= L.n) {
            __builtin_nontemporal_store(u32x4{out[0], out[1], out[2], out[3]}, (SZ_GLOBAL u32x4*)p);
        } else {
            const uint32_t valid = static_cast<uint32_t>(L.n - elem0);
#pragma unroll
            for (uint32_t k = 0; k < G::kLaneElems; ++k) {
                if (k < valid) {
                    if constexpr (DT == kDtypeBF16)
                        ((SZ_GLOBAL uint16_t*)p)[k] = static_cast<uint16_t>(out[k / 2] >> (16 * (k & 1)));
                    else
                        p[k] = static_cast<uint8_t>(out[k / 4] >> (8 * (k & 3)));
                }
            }
        }
    }
}

// Full blocks only (as k_encode); partial last blocks go to k_decode_tail.
// Bounded to 6 waves per SIMD (at most 80 VGPRs): measured 1.3% faster than
// the 5 waves the unbounded BF16 instance fits; 8 waves would spill.
template <uint32_t DT>
__global__ __launch_bounds__(kThreads, 6) void k_decode(DecodeArgs a) {
    __shared__ uint8_t s_esc[kWavesPerGroup][kPrefetch];
    const uint32_t wave = uniform(threadIdx.x / kWaveSize);
    const Layout L = layout_of(a.n, DT);
    const uint64_t full = a.n / kBlockElems;
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * kWavesPerGroup + wave;
    if (i >= static_cast<uint64_t>(a.count) * full) return;
    const uint32_t t = static_cast<uint32_t>(i / full);
    const uint64_t b = i - static_cast<uint64_t>(t) * full;
    decode_block<DT, true>(a, L, t, b, lane_id(), s_esc[wave]);
}

template <uint32_t DT>
__global__ __launch_bounds__(kWaveSize) void k_decode_tail(DecodeArgs a) {
    __shared__ uint8_t s_esc[kPrefetch];
    const Layout L = layout_of(a.n, DT);
    decode_block<DT, false>(a, L, blockIdx.x, L.blocks - 1, lane_id(), s_esc);
}

// n == 0: only the header can be checked
template <uint32_t DT>
__global__ void k_decode_empty(DecodeArgs a) {
    const uint32_t t = blockIdx.x;
    const Layout L = layout_of(0, DT);
    const SZ_GLOBAL uint8_t* src = src_of(a.src, t);
    const uint64_t src_bytes = a.src_bytes_table ? gptr(a.src_bytes_table)[t] : a.src_bytes;
    SZ_GLOBAL int32_t* status = a.status ? gptr(a.status) + t : nullptr;
    if (src_bytes < L.esc_at) {
        mark_corrupt(status, lane_id());
        return;
    }
    uint32_t hdr[16], cbw[4];
    load_header(src, hdr);
    if (check_header<DT>(hdr, src_bytes, L, cbw) < 0) mark_corrupt(status, lane_id());
}

uint32_t grid_for(uint64_t items, uint32_t per_group) {
    return static_cast<uint32_t>((items + per_group - 1) / per_group);
}

}  // namespace

// --------------------------------------------------------------- launchers

hipError_t launch_fill_u64(uint64_t* p, uint64_t words, uint64_t value, hipStream_t s) {
    if (!words) return hipSuccess;
    uint64_t groups = (words + 255) / 256;
    if (groups > 4096) groups = 4096;
    hipLaunchKernelGGL(k_fill_u64, dim3(static_cast<uint32_t>(groups)), dim3(256), 0, s, p, words, value);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, uint64_t words, int32_t value, hipStream_t s) {
    if (!words) return hipSuccess;
    uint64_t groups = (words + 255) / 256;
    if (groups > 4096) groups = 4096;
    hipLaunchKernelGGL(k_fill_i32, dim3(static_cast<uint32_t>(groups)), dim3(256), 0, s, p, words, value);
    return hipGetLastError();
}

// Histogram grid: about kHistGroups workgroups in total, each counting a
// contiguous multiple of one iteration's elements (8 passes x 256 lanes x
// one 16-byte vector) of one tensor.
constexpr uint64_t kHistGroups = 2048;

template <uint32_t DT>
void enqueue_histogram(HistArgs a, hipStream_t s) {
    constexpr uint64_t kQuantum = 8ull * kThreads * (16 / Geometry<DT>::kElemBytes);
    uint64_t want = kHistGroups / a.count;
    if (want < 1) want = 1;
    const uint64_t units = (a.n + kQuantum - 1) / kQuantum;
    if (want > units) want = units;
    a.chunk = (units + want - 1) / want * kQuantum;
    if (DT == kDtypeE5M2 && a.chunk > kE5m2MaxChunk) a.chunk = kE5m2MaxChunk;   // 16-bit pair counters
    a.groups = static_cast<uint32_t>((a.n + a.chunk - 1) / a.chunk);
    hipLaunchKernelGGL(k_histogram<DT>, dim3(a.count * a.groups), dim3(kThreads), 0, s, a);
}

template <uint32_t DT>
void enqueue_histogram_sampled(HistArgs a, hipStream_t s) {
    const uint64_t blocks = (a.n + kBlockElems - 1) / kBlockElems;
    const uint64_t sampled = (blocks + a.stride - 1) / a.stride;
    a.per_group = 4;
    a.groups = static_cast<uint32_t>((sampled + a.per_group - 1) / a.per_group);
    hipLaunchKernelGGL(k_histogram_sampled<DT>, dim3(a.count * a.groups), dim3(kThreads), 0, s, a);
}

hipError_t launch_histogram(const HistArgs& a, uint32_t dtype, hipStream_t s) {
    if (a.stride > 1) {
        if (dtype == kDtypeBF16)
            enqueue_histogram_sampled<kDtypeBF16>(a, s);
        else
            enqueue_histogram_sampled<kDtypeE5M2>(a, s);
    } else if (dtype == kDtypeBF16) {
        enqueue_histogram<kDtypeBF16>(a, s);
    } else {
        enqueue_histogram<kDtypeE5M2>(a, s);
    }
    return hipGetLastError();
}

hipError_t launch_codebook(const CodebookArgs& a, uint32_t dtype, hipStream_t s) {
    if (dtype == kDtypeBF16)
        hipLaunchKernelGGL(k_codebook<kDtypeBF16>, dim3(a.count), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_codebook<kDtypeE5M2>, dim3(a.count), dim3(256), 0, s, a);
    return hipGetLastError();
}

// offsets, header and escape scatter, after the planes and staged escapes
template <uint32_t DT>
void enqueue_encode_finish(const EncodeArgs& a, hipStream_t s) {
    const Layout L = layout_of(a.n, DT);
    const uint64_t blocks = static_cast<uint64_t>(a.count) * L.blocks;
    const uint32_t scatter_groups = grid_for(blocks, kThreads);
    const uint64_t groups = (L.blocks + kThreads - 1) / kThreads;     // 256-block groups per tensor
    if (groups <= kFusedGroups) {
        hipLaunchKernelGGL(k_offsets_scatter<DT>, dim3(static_cast<uint32_t>(a.count * groups)), dim3(kThreads), 0,
                           s, a);
    } else {
        hipLaunchKernelGGL(k_offsets<DT>, dim3(a.count), dim3(256), 0, s, a);
        hipLaunchKernelGGL(k_scatter<DT>, dim3(scatter_groups), dim3(kThreads), 0, s, a);
    }
}

template <uint32_t DT>
void enqueue_encode(const EncodeArgs& a, hipStream_t s) {
    const uint64_t full = static_cast<uint64_t>(a.count) * (a.n / kBlockElems);
    if (full) hipLaunchKernelGGL(k_encode<DT>, dim3(grid_for(full, kWavesPerGroup)), dim3(kThreads), 0, s, a);
    if (a.n % kBlockElems) hipLaunchKernelGGL(k_encode_tail<DT>, dim3(a.count), dim3(kWaveSize), 0, s, a);
    enqueue_encode_finish<DT>(a, s);
}

hipError_t launch_encode(const EncodeArgs& a, uint32_t dtype, hipStream_t s) {
    if (dtype == kDtypeBF16)
        enqueue_encode<kDtypeBF16>(a, s);
    else
        enqueue_encode<kDtypeE5M2>(a, s);
    return hipGetLastError();
}

hipError_t launch_encode_empty(const EncodeArgs& a, uint32_t dtype, hipStream_t s) {
    if (dtype == kDtypeBF16)
        hipLaunchKernelGGL(k_encode_empty<kDtypeBF16>, dim3(a.count), dim3(kWaveSize), 0, s, a);
    else
        hipLaunchKernelGGL(k_encode_empty<kDtypeE5M2>, dim3(a.count), dim3(kWaveSize), 0, s, a);
    return hipGetLastError();
}

template <uint32_t DT>
void enqueue_compress(const CompressArgs& a, hipStream_t s) {
    const uint32_t grid = a.enc.count * (a.sample_items + 1 + a.main_items + 1);   // one workgroup per item
    hipLaunchKernelGGL(k_compress<DT>, dim3(grid), dim3(kPassThreads), 0, s, a);
    if (a.enc.n % kBlockElems) hipLaunchKernelGGL(k_encode_tail<DT>, dim3(a.enc.count), dim3(kWaveSize), 0, s, a.enc);
    const uint64_t full_blocks = a.enc.n / kBlockElems;
    if (full_blocks) {
        // about one block per wave when every tensor is listed, capped
        const uint64_t blocks = static_cast<uint64_t>(a.enc.count) * full_blocks;
        const uint64_t groups = (blocks + kWavesPerGroup - 1) / kWavesPerGroup;
        const uint32_t grid = static_cast<uint32_t>(groups < kTranscodeGroups ? groups : kTranscodeGroups);
        hipLaunchKernelGGL(k_transcode<DT>, dim3(grid), dim3(kThreads), 0, s, a);
    }
    enqueue_encode_finish<DT>(a.enc, s);
}

hipError_t launch_compress(const CompressArgs& a, uint32_t dtype, hipStream_t s) {
    if (dtype != kDtypeBF16) return hipErrorInvalidValue;   // E5M2 takes the separate kernels
    const uint64_t words = sync_area_bytes(a.enc.count) / 8;
    const uint64_t most = words > a.enc.count ? words : a.enc.count;
    const uint32_t groups = grid_for(most < 4096ull * 256 ? most : 4096ull * 256, 256);
    hipLaunchKernelGGL(k_zero_two, dim3(groups), dim3(256), 0, s, reinterpret_cast<uint64_t*>(a.sync), words, a.status,
                       static_cast<uint64_t>(a.enc.count));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    enqueue_compress<kDtypeBF16>(a, s);
    return hipGetLastError();
}

template <uint32_t DT>
void enqueue_decode(const DecodeArgs& a, hipStream_t s) {
    const uint64_t full = static_cast<uint64_t>(a.count) * (a.n / kBlockElems);
    if (full) hipLaunchKernelGGL(k_decode<DT>, dim3(grid_for(full, kWavesPerGroup)), dim3(kThreads), 0, s, a);
    if (a.n % kBlockElems) hipLaunchKernelGGL(k_decode_tail<DT>, dim3(a.count), dim3(kWaveSize), 0, s, a);
}

hipError_t launch_decode(const DecodeArgs& a, uint32_t dtype, hipStream_t s) {
    if (dtype == kDtypeBF16)
        enqueue_decode<kDtypeBF16>(a, s);
    else
        enqueue_decode<kDtypeE5M2>(a, s);
    return hipGetLastError();
}

hipError_t launch_decode_empty(const DecodeArgs& a, uint32_t dtype, hipStream_t s) {
    if (dtype == kDtypeBF16)
        hipLaunchKernelGGL(k_decode_empty<kDtypeBF16>, dim3(a.count), dim3(kWaveSize), 0, s, a);
    else
        hipLaunchKernelGGL(k_decode_empty<kDtypeE5M2>, dim3(a.count), dim3(kWaveSize), 0, s, a);
    return hipGetLastError();
}

}  // namespace sz
