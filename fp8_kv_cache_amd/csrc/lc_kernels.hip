// lc_kernels.hip -- gfx950 kernels of the LC-style comparison codec
// (TUPL8_1 -> BIT_8 -> RZE_2 on 16 KB chunks; FastKVComp companion page,
// "Inside an LC-style pipeline"; stage readings in include/lc_codec.h).
//
// One 256-thread workgroup codes or decodes one chunk.  For a full chunk
// the two rearranging stages compose into one bit permutation: bit k of
// input byte 512I + 64a + 8c + j (I < 32, a, c, j, k < 8) lands on bit a of
// plane byte (8c + k)*256 + 32j + I.  Thread (I, c) therefore gathers the
// eight 8-byte words a = 0..7 of its (I, c) slot, transposes the 8x8 bit
// matrix of every byte lane in registers (three swap rounds), and a 4x4
// byte transpose across each quad of lanes (two DPP exchanges) turns its
// columns into 4-byte pieces of plane rows, which land in LDS as dwords.
// Decoding runs the same two transposes backwards (both are involutions).
// The last, shorter chunk of a tensor takes a plain by-definition path.
// All arithmetic is integer; there is no matrix-core work.
#include "device_common.h"
#include "lc_internal.h"

namespace lc {
namespace {

using sz::DstRef;
using sz::SrcRef;
using sz::gptr;
using sz::lane_id;
using sz::perm;
using sz::u32x2;
using sz::u32x4;
using sz::uniform;
using sz::wave_scan_incl;

constexpr auto block_scan = sz::block_scan_excl;

constexpr uint32_t kThreads = 256;
constexpr uint32_t kRowStride = 520;            // LDS stride of a 512-byte input row: 8 spare bytes
constexpr uint32_t kBitmap = kChunk / 16;       // RZE_2 bitmap bytes of a full chunk (8192 words)
// A full chunk's RZE_2 words sit in LDS after the bitmap with 4 spare bytes
// after every 64: thread t's run of non-zero words starts where the counts
// of the threads before it end, so when every thread holds the same count
// (a plane of all-zero or all-non-zero words, as 4-bit codes give) the runs
// are a fixed number of dwords apart, and a 16-dword stride would put 16
// lanes on one bank; with the spare dword the stride is odd.
__device__ inline uint32_t word_at(uint32_t w) { return kBitmap + 2 * w + 4 * (w >> 5); }
constexpr uint32_t kPaddedPayload = kBitmap + (kChunk - kBitmap) / 64 * 68;   // 17344 bytes
// A full chunk's plane image z sits in LDS with 16 spare bytes after every
// 256: then neither the transposes (lane (I, c) of a wave takes dword
// 64(8c + k) + 8(4g + q) + p, the two halves c apart by 8 plane rows) nor a
// thread's 64-byte read of its own plane words (lanes 64 bytes apart) put
// two lanes of a wave on one of the 64 banks; without them the first
// doubles and the second quadruples the cycles of each access.
__device__ inline uint32_t plane_at(uint32_t z) { return z + 16 * (z >> 8); }
constexpr uint32_t kPaddedPlane = kChunk / 256 * 272;   // 17408 bytes
constexpr uint32_t kLds = kPaddedPlane;                  // also holds the padded payload and the 32 input rows
static_assert(kLds >= kPaddedPayload && kLds >= 32 * kRowStride, "LDS buffer");
// Payload vector v of a full chunk (16 bytes at 16 v) in LDS: 4 dwords at
// byte `payload_at(v)` on, contiguous, 4-byte aligned.
__device__ inline uint32_t payload_at(uint32_t v) {
    return 16 * v < kBitmap ? 16 * v : word_at((16 * v - kBitmap) / 2);
}

struct Lds {
    alignas(16) uint8_t buf[kLds];
    uint32_t sums[kThreads / 64];
};

// ---------------------------------------------------------------- helpers

// Transposes the 8x8 bit matrix of every byte lane of L: afterwards bit a of
// byte j of L[k] is what bit k of byte j of L[a] was.
template <uint32_t S>
__device__ inline void swap_round(uint64_t (&L)[8], uint64_t mask) {
#pragma unroll
    for (uint32_t a = 0; a < 8; ++a) {
        if (a & S) continue;
        const uint64_t t = ((L[a] >> S) ^ L[a + S]) & mask;
        L[a + S] ^= t;
        L[a] ^= t << S;
    }
}
__device__ inline void transpose_bits(uint64_t (&L)[8]) {
    swap_round<4>(L, 0x0F0F0F0F0F0F0F0Full);
    swap_round<2>(L, 0x3333333333333333ull);
    swap_round<1>(L, 0x5555555555555555ull);
}

// 4x4 byte transpose across the lanes of a quad (q = lane & 3): byte j of
// lane q's value ends up as byte q of lane j's result.
__device__ inline uint32_t quad_transpose(uint32_t v, uint32_t q) {
    const uint32_t x2 = __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    const uint32_t h = perm(x2, v, q < 2 ? 0x05040100u : 0x03020706u);
    const uint32_t x1 = __builtin_amdgcn_update_dpp(0u, h, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    return perm(x1, h, (q & 1) ? 0x03070105u : 0x06020400u);
}

// Header, table entries c and c+1, and the checks every workgroup makes
// before touching chunk c's payload.  Returns false if the stream does not
// match n or itself.  On success *off / *size hold chunk c's entry.
__device__ inline bool check_entry(const SZ_GLOBAL uint8_t* src, uint64_t src_bytes, uint64_t n, uint64_t c,
                                   uint32_t lane, uint32_t* off, uint32_t* size) {
    const uint64_t C = chunks_of(n), D = data_at(n);
    if (src_bytes < D) return false;
    // one load: header dwords (lanes 0..15), entry c (16, 17), entry c+1 (18, 19)
    const uint64_t at = lane < 16 ? lane
                        : lane < 18 ? 16 + 2 * c + (lane - 16)
                        : (lane < 20 && c + 1 < C) ? 16 + 2 * (c + 1) + (lane - 18) : 0;
    const uint32_t v = ((const SZ_GLOBAL uint32_t*)src)[at];
    uint32_t h[20];
#pragma unroll
    for (uint32_t i = 0; i < 20; ++i) h[i] = __builtin_amdgcn_readlane(v, i);
    const uint64_t hn = h[2] | (static_cast<uint64_t>(h[3]) << 32);
    const uint64_t hc = h[4] | (static_cast<uint64_t>(h[5]) << 32);
    const uint64_t total = h[6] | (static_cast<uint64_t>(h[7]) << 32);
    bool ok = h[0] == kMagic && h[1] == (kVersion | (kPipeline << 8) | (kLog2Chunk << 16));
    ok &= hn == n && hc == C && total <= src_bytes && total >= D;
    ok &= (h[8] | h[9] | h[10] | h[11] | h[12] | h[13] | h[14] | h[15]) == 0;
    const uint64_t o = h[16], s = h[17];
    const uint64_t end = o + align16(s);
    ok &= (o & 15) == 0 && s <= chunk_len(n, c) && (c != 0 || o == 0) && D + end <= total;
    ok &= c + 1 < C ? h[18] == end : total == D + end;
    *off = static_cast<uint32_t>(o);
    *size = static_cast<uint32_t>(s);
    return ok;
}

__device__ inline void mark_corrupt(int32_t* status, uint32_t t, uint32_t tid) {
    if (status && tid == 0) gptr(status)[t] = 3;   // SZ_ERR_CORRUPT_STREAM
}

// ------------------------------------------------------------- full chunk

// Chunk inputs, payloads and decoded chunks are each read or written once
// per call, so their bulk accesses are non-temporal, as in the exponent
// codec's kernels (so that the two codecs are compared on equal terms).

// x (16384 bytes, global) -> LDS rows of 512 bytes at stride kRowStride.
// `keep` receives the thread's four 16-byte vectors.
__device__ inline void stage_input(const SZ_GLOBAL uint8_t* x, Lds& s, uint32_t tid, u32x4 (&keep)[4]) {
#pragma unroll
    for (uint32_t v = 0; v < 4; ++v) {
        const uint32_t o = 16 * (tid + kThreads * v);
        keep[v] = __builtin_nontemporal_load((const SZ_GLOBAL u32x4*)(x + o));
        uint8_t* d = s.buf + (o / 512) * kRowStride + (o % 512);
        *reinterpret_cast<u32x2*>(d) = u32x2{keep[v].x, keep[v].y};
        *reinterpret_cast<u32x2*>(d + 8) = u32x2{keep[v].z, keep[v].w};
    }
}

// Padded input rows in LDS -> plane image z = BIT_8(TUPL8_1(x)) in buf
// (byte z at plane_at(z)).  Barriers inside; every thread calls it.
__device__ inline void forward_full(Lds& s, uint32_t tid) {
    const uint32_t I = tid & 31, c = tid >> 5, q = I & 3, p = I >> 2;
    uint64_t L[8];
#pragma unroll
    for (uint32_t a = 0; a < 8; ++a)
        L[a] = *reinterpret_cast<const uint64_t*>(s.buf + I * kRowStride + 64 * a + 8 * c);
    __syncthreads();
    transpose_bits(L);
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
#pragma unroll
        for (uint32_t g = 0; g < 2; ++g) {
            const uint32_t v = quad_transpose(static_cast<uint32_t>(L[k] >> (32 * g)), q);
            *reinterpret_cast<uint32_t*>(s.buf + plane_at((8 * c + k) * 256 + 32 * (4 * g + q) + 4 * p)) = v;
        }
    }
    __syncthreads();
}

// Plane image in buf (byte z at plane_at(z)) -> input bytes, written to
// out (global).
__device__ inline void inverse_full(Lds& s, uint32_t tid, SZ_GLOBAL uint8_t* out) {
    const uint32_t I = tid & 31, c = tid >> 5, q = I & 3, p = I >> 2;
    uint64_t L[8];
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
        uint64_t w = 0;
#pragma unroll
        for (uint32_t g = 0; g < 2; ++g) {
            const uint32_t v = *reinterpret_cast<const uint32_t*>(s.buf + plane_at((8 * c + k) * 256 + 32 * (4 * g + q) + 4 * p));
            w |= static_cast<uint64_t>(quad_transpose(v, q)) << (32 * g);
        }
        L[k] = w;
    }
    __syncthreads();
    transpose_bits(L);
#pragma unroll
    for (uint32_t a = 0; a < 8; ++a)
        *reinterpret_cast<uint64_t*>(s.buf + I * kRowStride + 64 * a + 8 * c) = L[a];
    __syncthreads();
#pragma unroll
    for (uint32_t v = 0; v < 4; ++v) {
        const uint32_t o = 16 * (tid + kThreads * v);
        const uint8_t* d = s.buf + (o / 512) * kRowStride + (o % 512);
        const u32x2 lo = *reinterpret_cast<const u32x2*>(d);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(d + 8);
        __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y}, (SZ_GLOBAL u32x4*)(out + o));
    }
}

// The thread's 32 plane words (bytes 64t .. 64t+63 of z) and their
// non-zero flags (bit i for word 32t + i).
__device__ inline uint32_t read_words(const Lds& s, uint32_t tid, uint32_t (&w)[16]) {
    uint32_t flags = 0;
#pragma unroll
    for (uint32_t v = 0; v < 4; ++v) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(s.buf + plane_at(16 * (4 * tid + v)));
        w[4 * v] = x.x; w[4 * v + 1] = x.y; w[4 * v + 2] = x.z; w[4 * v + 3] = x.w;
    }
#pragma unroll
    for (uint32_t d = 0; d < 16; ++d) {
        flags |= static_cast<uint32_t>((w[d] & 0xFFFFu) != 0) << (2 * d);
        flags |= static_cast<uint32_t>((w[d] >> 16) != 0) << (2 * d + 1);
    }
    return flags;
}

// Coded size of a full chunk whose plane image is in LDS (kChunk if raw).
// With kWrite the RZE_2 payload is assembled in buf[0, A16(size)).
template <bool kWrite>
__device__ inline uint32_t rze_full(Lds& s, uint32_t tid) {
    uint32_t w[16];
    const uint32_t flags = read_words(s, tid, w);
    uint32_t nonzero;
    const uint32_t base = block_scan(__builtin_popcount(flags), tid, s.sums, nonzero);
    const uint32_t size = kBitmap + 2 * nonzero;
    if (!kWrite || size >= kChunk) return size < kChunk ? size : kChunk;
    __syncthreads();                                   // every plane word is in registers
    reinterpret_cast<uint32_t*>(s.buf)[tid] = flags;   // bitmap dword t covers words 32t..32t+31
    // word i's slot: the non-zero words before it, counted with a masked popcount
#pragma unroll
    for (uint32_t i = 0; i < 32; ++i) {
        if (flags & (1u << i))
            *reinterpret_cast<uint16_t*>(s.buf + word_at(base + __builtin_popcount(flags & ((1u << i) - 1u)))) =
                static_cast<uint16_t>(w[i / 2] >> (16 * (i & 1)));
    }
    const uint32_t padded = static_cast<uint32_t>(align16(size));
    if (tid < 8 && size + 2 * tid < padded) *reinterpret_cast<uint16_t*>(s.buf + word_at((size - kBitmap) / 2 + tid)) = 0;
    __syncthreads();
    return size;
}

// ---------------------------------------------------------- partial chunk

// Position of bit k of input byte p in the plane image of an L-byte chunk
// (readings L2 and L3, by definition): returns z byte * 8 + bit.
__device__ inline uint32_t plane_bit(uint32_t p, uint32_t k, uint32_t L) {
    const uint32_t q = L / 8, G = q / 8;
    const uint32_t y = p < 8 * q ? (p % 8) * q + p / 8 : p;
    if (y >= 64 * G) return 8 * y + k;
    const uint32_t w = y / 8;
    return 8 * ((8 * (y % 8) + k) * G + w / 8) + w % 8;
}

// Plane image of a short chunk (L < kChunk) built in buf[0, L) by scattering
// input bits with LDS atomics.
__device__ inline void forward_partial(const SZ_GLOBAL uint8_t* x, uint32_t L, Lds& s, uint32_t tid) {
    uint32_t* z = reinterpret_cast<uint32_t*>(s.buf);
    for (uint32_t i = tid; i < (L + 3) / 4; i += kThreads) z[i] = 0;
    __syncthreads();
    for (uint32_t p = tid; p < L; p += kThreads) {
        const uint32_t v = x[p];
        for (uint32_t k = 0; k < 8; ++k) {
            if (!((v >> k) & 1u)) continue;
            const uint32_t b = plane_bit(p, k, L);
            atomicOr(z + b / 32, 1u << (b % 32));
        }
    }
    __syncthreads();
}

// RZE_2 of a short chunk's plane image in buf[0, L): coded size (L if raw);
// with kWrite the payload is assembled in buf[0, A16(size)).
template <bool kWrite>
__device__ inline uint32_t rze_partial(Lds& s, uint32_t L, uint32_t tid) {
    const uint32_t V = L / 2, nb = (V + 7) / 8;
    uint32_t w[32];
    uint32_t flags = 0;
#pragma unroll
    for (uint32_t i = 0; i < 32; ++i) {
        const uint32_t m = 32 * tid + i;
        w[i] = m < V ? s.buf[2 * m] | (static_cast<uint32_t>(s.buf[2 * m + 1]) << 8) : 0u;
        flags |= static_cast<uint32_t>(w[i] != 0) << i;
    }
    const uint32_t odd = (L & 1) ? s.buf[L - 1] : 0u;
    uint32_t nonzero;
    const uint32_t base = block_scan(__builtin_popcount(flags), tid, s.sums, nonzero);
    const uint32_t size = nb + 2 * nonzero + (L & 1);
    if (!kWrite || size >= L) return size < L ? size : L;
    __syncthreads();
    for (uint32_t b = 0; b < 4; ++b)
        if (4 * tid + b < nb) s.buf[4 * tid + b] = static_cast<uint8_t>(flags >> (8 * b));
    uint32_t at = nb + 2 * base;
#pragma unroll
    for (uint32_t i = 0; i < 32; ++i) {
        if (flags & (1u << i)) {
            s.buf[at] = static_cast<uint8_t>(w[i]);
            s.buf[at + 1] = static_cast<uint8_t>(w[i] >> 8);
            at += 2;
        }
    }
    if (tid == 0 && (L & 1)) s.buf[size - 1] = static_cast<uint8_t>(odd);
    if (tid < 16 && size + tid < align16(size)) s.buf[size + tid] = 0;
    __syncthreads();
    return size;
}

// ----------------------------------------------------------------- encode

// Stored size of every chunk (pass 1): grid = count x C workgroups.
__global__ __launch_bounds__(kThreads) void k_lc_size(EncodeArgs a) {
    __shared__ Lds s;
    const uint32_t tid = threadIdx.x;
    const uint64_t C = chunks_of(a.n);
    const uint32_t t = static_cast<uint32_t>(blockIdx.x / C);
    const uint64_t c = blockIdx.x - static_cast<uint64_t>(t) * C;
    const uint32_t L = chunk_len(a.n, c);
    const SZ_GLOBAL uint8_t* x = sz::src_of(a.src, t) + c * kChunk;
    uint32_t size;
    if (L == kChunk) {
        u32x4 keep[4];
        stage_input(x, s, tid, keep);
        __syncthreads();
        forward_full(s, tid);
        size = rze_full<false>(s, tid);
    } else {
        forward_partial(x, L, s, tid);
        size = rze_partial<false>(s, L, tid);
    }
    if (tid == 0) gptr(a.sizes)[static_cast<uint64_t>(t) * C + c] = size;
}

// One workgroup per tensor: offsets (exclusive scan of the padded sizes),
// the table, the header and the zero padding up to D; the total to
// out_bytes.  Thread i takes a contiguous run of ceil(C / 256) chunks.
__global__ __launch_bounds__(kThreads) void k_lc_table(EncodeArgs a) {
    __shared__ uint32_t sums[kThreads / 64];
    const uint32_t t = blockIdx.x, tid = threadIdx.x;
    const uint64_t C = chunks_of(a.n), D = data_at(a.n);
    const SZ_GLOBAL uint32_t* sizes = gptr(a.sizes) + static_cast<uint64_t>(t) * C;
    SZ_GLOBAL uint8_t* dst = sz::dst_of(a.dst, t);
    const uint64_t per = (C + kThreads - 1) / kThreads;
    const uint64_t lo = tid * per < C ? tid * per : C;
    const uint64_t hi = lo + per < C ? lo + per : C;
    uint32_t mine = 0;
    for (uint64_t c = lo; c < hi; ++c) mine += static_cast<uint32_t>(align16(sizes[c]));
    uint32_t all;
    uint32_t off = block_scan(mine, tid, sums, all);
    SZ_GLOBAL u32x2* table = (SZ_GLOBAL u32x2*)(dst + 64);
    for (uint64_t c = lo; c < hi; ++c) {
        const uint32_t size = sizes[c];
        table[c] = u32x2{off, size};
        off += static_cast<uint32_t>(align16(size));
    }
    const uint64_t total = D + all;
    SZ_GLOBAL uint32_t* h = (SZ_GLOBAL uint32_t*)dst;
    uint32_t v = 0;
    switch (tid) {
        case 0: v = kMagic; break;
        case 1: v = kVersion | (kPipeline << 8) | (kLog2Chunk << 16); break;
        case 2: v = static_cast<uint32_t>(a.n); break;
        case 3: v = static_cast<uint32_t>(a.n >> 32); break;
        case 4: v = static_cast<uint32_t>(C); break;
        case 5: v = static_cast<uint32_t>(C >> 32); break;
        case 6: v = static_cast<uint32_t>(total); break;
        case 7: v = static_cast<uint32_t>(total >> 32); break;
        default: v = 0; break;
    }
    if (tid < 16) h[tid] = v;
    const uint64_t pad_from = (64 + 8 * C) / 4;
    if (tid < D / 4 - pad_from) h[pad_from + tid] = 0;
    if (a.out_bytes && tid == 0) gptr(a.out_bytes)[t] = total;
}

// Payloads (pass 2): raw chunks are copied, coded chunks are transformed
// again and their RZE_2 payload written, each with its zero padding.
__global__ __launch_bounds__(kThreads) void k_lc_write(EncodeArgs a) {
    __shared__ Lds s;
    const uint32_t tid = threadIdx.x;
    const uint64_t C = chunks_of(a.n);
    const uint32_t t = static_cast<uint32_t>(blockIdx.x / C);
    const uint64_t c = blockIdx.x - static_cast<uint64_t>(t) * C;
    const uint32_t L = chunk_len(a.n, c);
    const SZ_GLOBAL uint8_t* x = sz::src_of(a.src, t) + c * kChunk;
    SZ_GLOBAL uint8_t* dst = sz::dst_of(a.dst, t);
    const uint32_t size = uniform(gptr(a.sizes)[static_cast<uint64_t>(t) * C + c]);
    const uint32_t off = uniform(((const SZ_GLOBAL uint32_t*)(dst + 64))[2 * c]);
    SZ_GLOBAL uint8_t* out = dst + data_at(a.n) + off;
    if (L == kChunk) {
        if (size == kChunk) {
#pragma unroll
            for (uint32_t v = 0; v < 4; ++v) {
                const uint32_t o = 16 * (tid + kThreads * v);
                __builtin_nontemporal_store(__builtin_nontemporal_load((const SZ_GLOBAL u32x4*)(x + o)),
                                            (SZ_GLOBAL u32x4*)(out + o));
            }
            return;
        }
        u32x4 keep[4];
        stage_input(x, s, tid, keep);
        __syncthreads();
        forward_full(s, tid);
        rze_full<true>(s, tid);
    } else if (size == L) {
        for (uint32_t p = tid; p < align16(L); p += kThreads) out[p] = p < L ? x[p] : 0;
        return;
    } else {
        forward_partial(x, L, s, tid);
        rze_partial<true>(s, L, tid);
    }
    // the payload and its padding: buf[0, A16(size)), a full chunk's words
    // with their spare bytes
    for (uint32_t v = tid; v < align16(size) / 16; v += kThreads) {
        u32x4 x;
        if (L == kChunk) {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(s.buf + payload_at(v));
            x = u32x4{p[0], p[1], p[2], p[3]};
        } else {
            x = reinterpret_cast<const u32x4*>(s.buf)[v];
        }
        __builtin_nontemporal_store(x, (SZ_GLOBAL u32x4*)(out + 16 * v));
    }
}

// ----------------------------------------------------------------- decode

// 8 waves per SIMD (at most 64 VGPRs): a coded chunk's decode is a chain of
// dependent steps, so more resident workgroups hide more of it.
__global__ __launch_bounds__(kThreads, 8) void k_lc_decode(DecodeArgs a) {
    __shared__ Lds s;
    const uint32_t tid = threadIdx.x;
    const uint64_t C = chunks_of(a.n);
    const uint32_t t = static_cast<uint32_t>(blockIdx.x / C);
    const uint64_t c = blockIdx.x - static_cast<uint64_t>(t) * C;
    const uint32_t L = chunk_len(a.n, c);
    const SZ_GLOBAL uint8_t* src = sz::src_of(a.src, t);
    const uint64_t src_bytes = a.src_bytes_table ? gptr(a.src_bytes_table)[t] : a.src_bytes;
    SZ_GLOBAL uint8_t* out = sz::dst_of(a.dst, t) + c * kChunk;
    uint32_t off, size;
    if (!check_entry(src, src_bytes, a.n, c, lane_id(), &off, &size)) {
        mark_corrupt(a.status, t, tid);
        return;
    }
    off = uniform(off);
    size = uniform(size);
    const SZ_GLOBAL uint8_t* in = src + data_at(a.n) + off;   // A16(size) readable bytes
    if (size == L) {                                         // raw
        if (L == kChunk) {
#pragma unroll
            for (uint32_t v = 0; v < 4; ++v) {
                const uint32_t o = 16 * (tid + kThreads * v);
                __builtin_nontemporal_store(__builtin_nontemporal_load((const SZ_GLOBAL u32x4*)(in + o)),
                                            (SZ_GLOBAL u32x4*)(out + o));
            }
        } else {
            for (uint32_t p = tid; p < L; p += kThreads) out[p] = in[p];
        }
        return;
    }
    for (uint32_t v = tid; v < align16(size) / 16; v += kThreads) {
        const u32x4 x = __builtin_nontemporal_load((const SZ_GLOBAL u32x4*)(in + 16 * v));
        if (L == kChunk) {
            uint32_t* p = reinterpret_cast<uint32_t*>(s.buf + payload_at(v));
            p[0] = x.x; p[1] = x.y; p[2] = x.z; p[3] = x.w;
        } else {
            reinterpret_cast<u32x4*>(s.buf)[v] = x;
        }
    }
    __syncthreads();
    const uint32_t V = L / 2, nb = (V + 7) / 8;
    // this thread's 32 words m = 32t + i: flags from the bitmap (bits m >= V cleared)
    uint32_t flags = 0;
#pragma unroll
    for (uint32_t b = 0; b < 4; ++b)
        if (4 * tid + b < nb) flags |= static_cast<uint32_t>(s.buf[4 * tid + b]) << (8 * b);
    if (32 * tid + 32 > V) flags &= 32 * tid >= V ? 0u : (1u << (V - 32 * tid)) - 1u;
    uint32_t nonzero;
    const uint32_t base = block_scan(__builtin_popcount(flags), tid, s.sums, nonzero);
    if (nb + 2 * nonzero + (L & 1) != size) {
        mark_corrupt(a.status, t, tid);
        return;
    }
    // read phase: the thread's words from the payload; word i's slot is the
    // number of non-zero words before it (a masked popcount)
    uint32_t w[16];
    if (L == kChunk) {                                  // words after the 1024-byte bitmap, spare bytes between
#pragma unroll
        for (uint32_t d = 0; d < 16; ++d) {
            uint32_t v = 0;
#pragma unroll
            for (uint32_t h = 0; h < 2; ++h) {
                const uint32_t i = 2 * d + h;
                if (flags & (1u << i))
                    v |= static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(
                             s.buf + word_at(base + __builtin_popcount(flags & ((1u << i) - 1u)))))
                         << (16 * h);
            }
            w[d] = v;
        }
    } else {                                            // bitmap of any length: byte reads
#pragma unroll
        for (uint32_t d = 0; d < 16; ++d) {
            uint32_t v = 0;
#pragma unroll
            for (uint32_t h = 0; h < 2; ++h) {
                const uint32_t i = 2 * d + h;
                if (flags & (1u << i)) {
                    const uint32_t at = nb + 2 * (base + __builtin_popcount(flags & ((1u << i) - 1u)));
                    v |= (s.buf[at] | (static_cast<uint32_t>(s.buf[at + 1]) << 8)) << (16 * h);
                }
            }
            w[d] = v;
        }
    }
    const uint32_t odd = (L & 1) ? s.buf[size - 1] : 0u;
    __syncthreads();
    if (L == kChunk) {
#pragma unroll
        for (uint32_t v = 0; v < 4; ++v)
            *reinterpret_cast<u32x4*>(s.buf + plane_at(16 * (4 * tid + v))) =
                u32x4{w[4 * v], w[4 * v + 1], w[4 * v + 2], w[4 * v + 3]};
        __syncthreads();
        inverse_full(s, tid, out);
        return;
    }
    // short chunk: plane image in buf[0, L), then every input byte gathered
    for (uint32_t i = 0; i < 32; ++i) {
        const uint32_t m = 32 * tid + i;
        if (m < V) {
            s.buf[2 * m] = static_cast<uint8_t>(w[i / 2] >> (16 * (i & 1)));
            s.buf[2 * m + 1] = static_cast<uint8_t>(w[i / 2] >> (16 * (i & 1) + 8));
        }
    }
    if (tid == 0 && (L & 1)) s.buf[L - 1] = static_cast<uint8_t>(odd);
    __syncthreads();
    for (uint32_t p = tid; p < L; p += kThreads) {
        uint32_t v = 0;
        for (uint32_t k = 0; k < 8; ++k) {
            const uint32_t b = plane_bit(p, k, L);
            v |= ((s.buf[b / 8] >> (b % 8)) & 1u) << k;
        }
        out[p] = static_cast<uint8_t>(v);
    }
}

// n == 0: a header-only stream; only the header can be checked
__global__ void k_lc_decode_empty(DecodeArgs a) {
    const uint32_t t = blockIdx.x;
    const SZ_GLOBAL uint8_t* src = sz::src_of(a.src, t);
    const uint64_t src_bytes = a.src_bytes_table ? gptr(a.src_bytes_table)[t] : a.src_bytes;
    bool ok = src_bytes >= data_at(0);
    if (ok) {
        const SZ_GLOBAL uint32_t* h = (const SZ_GLOBAL uint32_t*)src;
        ok = h[0] == kMagic && h[1] == (kVersion | (kPipeline << 8) | (kLog2Chunk << 16));
        for (uint32_t i = 2; i < 16; ++i) ok &= i == 6 ? h[i] == data_at(0) : h[i] == 0;
    }
    if (!ok) mark_corrupt(a.status, t, threadIdx.x);
}

}  // namespace

hipError_t launch_encode(const EncodeArgs& a, hipStream_t s) {
    const uint64_t blocks = static_cast<uint64_t>(a.count) * chunks_of(a.n);
    if (blocks) hipLaunchKernelGGL(k_lc_size, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(k_lc_table, dim3(a.count), dim3(kThreads), 0, s, a);
    if (blocks) hipLaunchKernelGGL(k_lc_write, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    const uint64_t blocks = static_cast<uint64_t>(a.count) * chunks_of(a.n);
    if (blocks)
        hipLaunchKernelGGL(k_lc_decode, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(k_lc_decode_empty, dim3(a.count), dim3(1), 0, s, a);
    return hipGetLastError();
}

}  // namespace lc
