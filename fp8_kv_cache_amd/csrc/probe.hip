// probe.hip -- HBM streaming-rate probes for gfx950 (libszprobe.so).  The
// benchmark uses them to measure, on the same GPU and in the same run, the
// ceilings the codec's kernels are compared with: a read-only pass, a copy,
// and the one-launch compress's mix of traffic (read every 16-byte vector,
// write three of every four back), each with plain or with non-temporal
// accesses.  Measurement infrastructure only: not part of the codec's C ABI
// and not called by it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kThreads = 256;
constexpr uint32_t kInFlight = 8;   // 16-byte loads in flight per lane

// Grid-stride pass over n vectors of src.  MIX = vectors written per 4 read:
// 4 copies, 3 writes vector i to (i / 4) * 3 + i % 4 when i % 4 < 3 (a
// packed destination three quarters the size), 0 only reads (the XOR of
// the loads is stored to dst[thread] under a condition the benchmark's
// input never meets, so the loads cannot be dropped).
template <bool kNT, uint32_t MIX>
__global__ __launch_bounds__(kThreads) void k_stream(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     uint64_t n) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads * kInFlight;
    u32x4 acc = u32x4{0, 0, 0, 0};
    for (uint64_t first = static_cast<uint64_t>(blockIdx.x) * kThreads * kInFlight + threadIdx.x; first < n;
         first += stride) {
        u32x4 v[kInFlight];
#pragma unroll
        for (uint32_t p = 0; p < kInFlight; ++p) {
            const uint64_t i = first + p * kThreads;
            v[p] = i < n ? (kNT ? __builtin_nontemporal_load(src + i) : src[i]) : u32x4{0, 0, 0, 0};
        }
        if constexpr (MIX == 0) {
#pragma unroll
            for (uint32_t p = 0; p < kInFlight; ++p) acc ^= v[p];
        } else {
#pragma unroll
            for (uint32_t p = 0; p < kInFlight; ++p) {
                const uint64_t i = first + p * kThreads;
                if (i < n && (i & 3) < MIX) {
                    const uint64_t j = (i >> 2) * MIX + (i & 3);
                    if (kNT)
                        __builtin_nontemporal_store(v[p], dst + j);
                    else
                        dst[j] = v[p];
                }
            }
        }
    }
    if constexpr (MIX == 0) {
        if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u && acc.z == 0x2545F491u && acc.w == 0x4F6CDD1Du)
            dst[static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
    }
}

template <bool kNT>
void launch(uint32_t mix, const u32x4* src, u32x4* dst, uint64_t n, uint32_t groups, hipStream_t s) {
    if (mix == 0)
        hipLaunchKernelGGL((k_stream<kNT, 0>), dim3(groups), dim3(kThreads), 0, s, src, dst, n);
    else if (mix == 3)
        hipLaunchKernelGGL((k_stream<kNT, 3>), dim3(groups), dim3(kThreads), 0, s, src, dst, n);
    else
        hipLaunchKernelGGL((k_stream<kNT, 4>), dim3(groups), dim3(kThreads), 0, s, src, dst, n);
}

}  // namespace

// One pass over src_bytes of src (a multiple of 64; src and dst 16-byte
// aligned device memory).  mix: 0 read only, 3 the compress mix, 4 copy.
// dst must hold groups * 4096 bytes (mix 0), src_bytes * 3 / 4 (mix 3) or
// src_bytes (mix 4).  groups: workgroups of 256 threads, 1..65535.
// Asynchronous on stream.  Returns 0, -1 for invalid arguments (nothing
// enqueued) or -2 if the launch failed.
extern "C" __attribute__((visibility("default"))) int szp_stream(const void* src, void* dst, uint64_t src_bytes,
                                                                 uint64_t dst_bytes, uint32_t mix,
                                                                 uint32_t nontemporal, uint32_t groups,
                                                                 hipStream_t stream) {
    if (!src || !dst || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
        return -1;
    if (src_bytes == 0 || src_bytes % 64 || groups == 0 || groups > 65535) return -1;
    if (mix != 0 && mix != 3 && mix != 4) return -1;
    const uint64_t need = mix == 0 ? static_cast<uint64_t>(groups) * kThreads * 16
                                   : (mix == 3 ? src_bytes / 4 * 3 : src_bytes);
    if (dst_bytes < need) return -1;
    const uint64_t n = src_bytes / 16;
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    if (nontemporal)
        launch<true>(mix, s, d, n, groups, stream);
    else
        launch<false>(mix, s, d, n, groups, stream);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
