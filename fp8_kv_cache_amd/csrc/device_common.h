// device_common.h -- small gfx950 device helpers shared by the kernel files
// of the library (lane arithmetic, wave scans, global-address casts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sz_internal.h"

namespace sz {

__device__ inline uint32_t lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ inline uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// All tensors, streams and tables live in device global memory.  Casting
// to address space 1 lets the compiler emit global_* instead of flat_*
// memory instructions for pointers that were loaded from tables.
#define SZ_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ inline SZ_GLOBAL T* gptr(T* p) {
    return (SZ_GLOBAL T*)(p);
}

__device__ inline const SZ_GLOBAL uint8_t* src_of(const SrcRef& r, uint32_t t) {
    return gptr(static_cast<const uint8_t*>(r.table ? gptr(r.table)[t] : r.single));
}
__device__ inline SZ_GLOBAL uint8_t* dst_of(const DstRef& r, uint32_t t) {
    return gptr(static_cast<uint8_t*>(r.table ? gptr(r.table)[t] : r.single));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: four row
// shifts build scans inside each 16-lane row, then two row broadcasts carry
// row totals across the wave.
__device__ inline uint32_t wave_scan_incl(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Exclusive prefix of x over a 256-thread (4-wave) workgroup; `total` gets
// the sum.  `sums` is 4 words of LDS.  Contains a barrier; callers barrier
// again before reusing `sums`.
__device__ inline uint32_t block_scan_excl(uint32_t x, uint32_t tid, uint32_t* sums, uint32_t& total) {
    const uint32_t incl = wave_scan_incl(x);
    const uint32_t w = tid / 64;
    if ((tid & 63) == 63) sums[w] = incl;
    __syncthreads();
    uint32_t base = 0;
    for (uint32_t k = 0; k < w; ++k) base += sums[k];
    total = sums[0] + sums[1] + sums[2] + sums[3];
    return base + incl - x;
}

// byte select from the pair (hi, lo): selector bytes 0..3 pick lo's bytes,
// 4..7 hi's, 0x0C gives zero
__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

}  // namespace sz
