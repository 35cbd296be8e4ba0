// lc_api.cpp -- C ABI entry points of the LC-style comparison codec
// (declared and documented in include/lc_codec.h).  Host-side argument
// checks, then kernel launches on the caller's stream; nothing is
// allocated, freed or synchronised.
#include "lc_codec.h"

#include "lc_internal.h"

#define LC_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned(const void* p, uintptr_t to) { return (reinterpret_cast<uintptr_t>(p) & (to - 1)) == 0; }
bool usable(const void* p) { return p != nullptr && aligned(p, 16); }
sz_status from_hip(hipError_t e) { return e == hipSuccess ? SZ_OK : SZ_ERR_HIP; }

// workgroups per launch stay below 2^31
bool grid_ok(uint32_t count, uint64_t n) { return static_cast<uint64_t>(count) * lc::chunks_of(n) < (1ull << 31); }

sz_status encode_impl(sz::SrcRef src, uint32_t count, uint64_t n, sz::DstRef dst, uint64_t* d_out_bytes,
                      void* d_workspace, hipStream_t s) {
    lc::EncodeArgs a{};
    a.src = src;
    a.dst = dst;
    a.out_bytes = d_out_bytes;
    a.sizes = static_cast<uint32_t*>(d_workspace);
    a.count = count;
    a.n = n;
    return from_hip(lc::launch_encode(a, s));
}

sz_status decode_impl(sz::SrcRef src, const uint64_t* d_src_bytes, uint64_t src_bytes, uint32_t count, uint64_t n,
                      sz::DstRef dst, int32_t* d_status, hipStream_t s) {
    if (d_status) {
        hipError_t e = sz::launch_fill_i32(d_status, count, SZ_OK, s);
        if (e != hipSuccess) return SZ_ERR_HIP;
    }
    lc::DecodeArgs a{};
    a.src = src;
    a.src_bytes_table = d_src_bytes;
    a.src_bytes = src_bytes;
    a.dst = dst;
    a.status = d_status;
    a.count = count;
    a.n = n;
    return from_hip(lc::launch_decode(a, s));
}

}  // namespace

LC_EXPORT uint64_t lc_max_compressed_bytes(uint64_t n) { return n < lc::kMaxInput ? lc::max_bytes(n) : 0; }

LC_EXPORT uint64_t lc_encode_workspace_bytes_batched(uint32_t count, uint64_t n) {
    if (count == 0 || n == 0 || n >= lc::kMaxInput || !grid_ok(count, n)) return 0;
    return lc::workspace_bytes(count, n);
}

LC_EXPORT uint64_t lc_encode_workspace_bytes(uint64_t n) { return lc_encode_workspace_bytes_batched(1, n); }

LC_EXPORT sz_status lc_encode(const void* d_src, uint64_t n, void* d_dst, uint64_t dst_capacity,
                              uint64_t* d_out_bytes, void* d_workspace, uint64_t workspace_bytes,
                              hipStream_t stream) {
    if (n >= lc::kMaxInput || !usable(d_dst) || (n && !usable(d_src)) || (d_out_bytes && !aligned(d_out_bytes, 8)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (dst_capacity < lc::max_bytes(n)) return SZ_ERR_BUFFER_TOO_SMALL;
    if (n) {
        if (!usable(d_workspace)) return SZ_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < lc::workspace_bytes(1, n)) return SZ_ERR_BUFFER_TOO_SMALL;
    }
    return encode_impl(sz::SrcRef{nullptr, d_src}, 1, n, sz::DstRef{nullptr, d_dst}, d_out_bytes, d_workspace,
                       stream);
}

LC_EXPORT sz_status lc_encode_batched(const void* const* d_srcs, uint32_t count, uint64_t n, void* const* d_dsts,
                                      uint64_t dst_capacity, uint64_t* d_out_bytes, void* d_workspace,
                                      uint64_t workspace_bytes, hipStream_t stream) {
    if (n >= lc::kMaxInput || count == 0 || !grid_ok(count, n) || !usable(d_srcs) || !usable(d_dsts) ||
        (d_out_bytes && !aligned(d_out_bytes, 8)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (dst_capacity < lc::max_bytes(n)) return SZ_ERR_BUFFER_TOO_SMALL;
    if (n) {
        if (!usable(d_workspace)) return SZ_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < lc::workspace_bytes(count, n)) return SZ_ERR_BUFFER_TOO_SMALL;
    }
    return encode_impl(sz::SrcRef{d_srcs, nullptr}, count, n, sz::DstRef{d_dsts, nullptr}, d_out_bytes,
                       d_workspace, stream);
}

LC_EXPORT sz_status lc_decode(const void* d_src, uint64_t src_bytes, uint64_t n, void* d_dst, int32_t* d_status,
                              hipStream_t stream) {
    if (n >= lc::kMaxInput || !usable(d_src) || (n && !usable(d_dst)) || (d_status && !aligned(d_status, 4)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (src_bytes < lc::data_at(n)) return SZ_ERR_CORRUPT_STREAM;
    return decode_impl(sz::SrcRef{nullptr, d_src}, nullptr, src_bytes, 1, n, sz::DstRef{nullptr, d_dst}, d_status,
                       stream);
}

LC_EXPORT sz_status lc_decode_batched(const void* const* d_srcs, const uint64_t* d_src_bytes, uint32_t count,
                                      uint64_t n, void* const* d_dsts, int32_t* d_status, hipStream_t stream) {
    if (n >= lc::kMaxInput || count == 0 || !grid_ok(count, n) || !usable(d_srcs) || !usable(d_src_bytes) ||
        !usable(d_dsts) || (d_status && !aligned(d_status, 4)))
        return SZ_ERR_INVALID_ARGUMENT;
    return decode_impl(sz::SrcRef{d_srcs, nullptr}, d_src_bytes, 0, count, n, sz::DstRef{d_dsts, nullptr},
                       d_status, stream);
}
