// api.cpp -- C ABI entry points of the exponent codec (declared and
// documented in include/splitzip.h).  Every entry point validates its
// arguments on the host, then enqueues kernels on the caller's stream; it
// never allocates, frees or synchronises.
#include "splitzip.h"

#include <cstring>
#include <mutex>

#include "sz_internal.h"

#define SZ_EXPORT extern "C" __attribute__((visibility("default")))

// The workspace of sz_compress_noalloc: one array per device, held by the
// library for the life of the process.  Host code never uses its name as an
// address: the device address comes from hipGetSymbolAddress, once per
// device (scratch_on_current_device).
static __device__ __align__(256) uint8_t scratch[SZ_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace sz;

constexpr uint64_t kMaxElems = uint64_t(1) << 32;   // offsets are u32

// A C caller may pass any int as an enum argument, and a value outside the
// enumerators' range must not be read as a C++ enum: the enum arguments are
// checked through their bytes, and forwarded only once they are valid.
template <typename E>
int raw_value(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

bool dtype_ok(const sz_dtype& dt) {
    const int v = raw_value(dt);
    return v == SZ_DTYPE_BF16 || v == SZ_DTYPE_FP8_E5M2;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool usable(const void* p) { return p != nullptr && aligned16(p); }

sz_status from_hip(hipError_t e) { return e == hipSuccess ? SZ_OK : SZ_ERR_HIP; }

// every launch's workgroup count (at most one per format block) stays below 2^31
bool grid_ok(uint32_t count, uint64_t n) {
    return static_cast<uint64_t>(count) * ((n + kBlockElems - 1) / kBlockElems) < (uint64_t(1) << 31);
}

uint64_t workspace_bytes(uint32_t count, uint64_t n) { return workspace_bytes_for(count, n); }

// The fused compress kernel's sample items per tensor: every
// kSampleStride-th counting chunk.
uint64_t sample_items(uint64_t n, sz_dtype dt) {
    const uint64_t chunk = sample_chunk_elems(dt);
    const uint64_t chunks = (n + chunk - 1) / chunk;
    return (chunks + kSampleStride - 1) / kSampleStride;
}

// Its work items per tensor: sample items, the provisional codebook item,
// main items (item_blocks blocks each, the partial block included), the
// final codebook item.
uint64_t main_items(uint64_t n, sz_dtype dt) {
    const uint64_t per = item_blocks(dt == SZ_DTYPE_BF16 ? kDtypeBF16 : kDtypeE5M2);
    return ((n + kBlockElems - 1) / kBlockElems + per - 1) / per;
}

uint64_t compress_items(uint64_t n, sz_dtype dt) {
    return sample_items(n, dt) + 1 + main_items(n, dt) + 1;
}

uint64_t compress_workspace_bytes(uint32_t count, uint64_t n) {
    return workspace_bytes_for(count, n) + sync_area_bytes(count);
}

// Per-call settings of the one-launch compress, defaults filled in.  By
// default E5M2 tensors take the one-launch kernel only in large calls: with
// one byte per element, the second read it saves is small beside its fixed
// start (sample, provisional codebook) and the recodes, so the default
// asks for tensors of at least 2^22 elements and at least 2^28 elements in
// the call (measured: 2^28 and 2^29 elements in the call took 0.80-0.99 of
// the separate kernels' time, 2^27 about the same time, one 2^27-element
// tensor 1.04).  A caller's fused_min_elements applies to both types, with
// no call-size condition.
struct CompressSettings {
    uint64_t fused_min_bf16, fused_min_e5m2, call_min_e5m2;
    uint32_t spin_limit;
    bool fuses(sz_dtype dt, uint32_t count, uint64_t n) const {
        if (dt == SZ_DTYPE_BF16) return n >= fused_min_bf16;
        return n >= fused_min_e5m2 && static_cast<uint64_t>(count) * n >= call_min_e5m2;
    }
};

bool settings_of(const sz_compress_options* o, CompressSettings& c) {
    const bool given = o && o->fused_min_elements;
    c.fused_min_bf16 = given ? o->fused_min_elements : kDefaultFusedMin;
    c.fused_min_e5m2 = given ? o->fused_min_elements : kDefaultFusedMinE5m2;
    c.call_min_e5m2 = given ? 0 : kDefaultFusedCallE5m2;
    c.spin_limit = o && o->spin_limit ? o->spin_limit : kDefaultSpinLimit;
    return !o || o->reserved == 0;
}

sz_status histogram_impl(SrcRef src, uint32_t count, uint64_t n, sz_dtype dt, uint32_t stride,
                         uint64_t* d_hists, hipStream_t s) {
    hipError_t e = launch_fill_u64(d_hists, 256ull * count, 0, s);
    if (e != hipSuccess || n == 0) return from_hip(e);
    HistArgs a{};
    a.src = src;
    a.hists = d_hists;
    a.count = count;
    a.n = n;
    a.stride = stride;
    return from_hip(launch_histogram(a, dt, s));
}

sz_status encode_impl(SrcRef src, uint32_t count, uint64_t n, sz_dtype dt, const uint8_t* d_codebooks,
                      DstRef dst, uint64_t* d_out_bytes, void* d_workspace, hipStream_t s) {
    EncodeArgs a{};
    a.src = src;
    a.dst = dst;
    a.codebooks = d_codebooks;
    a.out_bytes = d_out_bytes;
    a.count = count;
    a.n = n;
    if (n == 0) return from_hip(launch_encode_empty(a, dt, s));
    a.counts = static_cast<uint32_t*>(d_workspace);
    a.staging = static_cast<uint8_t*>(d_workspace) + workspace_counts_bytes(count, layout_of(n, dt).blocks);
    return from_hip(launch_encode(a, dt, s));
}

// Histogram, codebook and encode in one launch that reads the input once
// (plus the short transcode, offset and scatter launches) for the tensors
// cs.fuses picks; the others take the separate kernels, as does n = 0.  The
// results are the same either way.
sz_status compress_impl(SrcRef src, uint32_t count, uint64_t n, sz_dtype dt, uint64_t* d_hists,
                        uint8_t* d_codebooks, DstRef dst, uint64_t* d_out_bytes, int32_t* d_status,
                        void* d_workspace, const CompressSettings& cs, hipStream_t s) {
    if (n == 0 || !cs.fuses(dt, count, n)) {
        if (d_status && launch_fill_i32(d_status, count, SZ_OK, s) != hipSuccess) return SZ_ERR_HIP;
        sz_status st = histogram_impl(src, count, n, dt, 1, d_hists, s);
        if (st != SZ_OK) return st;
        CodebookArgs c{d_hists, d_codebooks, count};
        if (launch_codebook(c, dt, s) != hipSuccess) return SZ_ERR_HIP;
        return encode_impl(src, count, n, dt, d_codebooks, dst, d_out_bytes, d_workspace, s);
    }
    CompressArgs a{};
    a.enc.src = src;
    a.enc.dst = dst;
    a.enc.codebooks = d_codebooks;
    a.enc.out_bytes = d_out_bytes;
    a.enc.count = count;
    a.enc.n = n;
    a.enc.counts = static_cast<uint32_t*>(d_workspace);
    a.enc.staging = static_cast<uint8_t*>(d_workspace) + workspace_counts_bytes(count, layout_of(n, dt).blocks);
    a.hists = d_hists;
    a.sync = static_cast<uint8_t*>(d_workspace) + workspace_bytes_for(count, n);
    a.enc.records = reinterpret_cast<const uint32_t*>(a.sync + sync_records_offset(count));
    a.status = d_status;
    const uint64_t chunk = sample_chunk_elems(dt);
    a.sample_items = static_cast<uint32_t>(sample_items(n, dt));
    a.sample_total = 0;
    for (uint64_t i = 0; i < a.sample_items; ++i) {
        const uint64_t begin = i * kSampleStride * chunk;
        a.sample_total += static_cast<uint32_t>(n - begin < chunk ? n - begin : chunk);
    }
    a.main_items = static_cast<uint32_t>(main_items(n, dt));
    // (compress_items(n, dt) is the item count per tensor; the entry points
    // keep count * that below 2^31, the launch's workgroup count)
    // Main items of a tensor come lag stages after its sample items: long
    // enough for the sample items to finish and the provisional codebook to
    // be ranked before the main items start (a main item that has to wait
    // holds its CU slot idle).  That takes about the same time whatever the
    // tensor size, and a stage's time is proportional to it, so the lag
    // spans kPassLagBytes of input (measured on 1 GB caches: 2^21-element
    // tensors need 16 stages or more, 2^23-element ones 8; 4 stages cost
    // them 70% and 3%), and is never below kPassLag.
    const uint64_t tensor_bytes = static_cast<uint64_t>(n) * (dt == SZ_DTYPE_BF16 ? 2 : 1);
    const uint64_t lag = (kPassLagBytes + tensor_bytes - 1) / tensor_bytes;
    a.lag = static_cast<uint32_t>(lag < kPassLag ? kPassLag : (lag > count + 1u ? count + 1u : lag));
    a.spin_limit = cs.spin_limit;
    return from_hip(launch_compress(a, dt, s));
}

// Device address of `scratch` on the current device, looked up with the
// device current the first time the device is seen; null on a HIP error.
constexpr int kScratchDevices = 1024;
std::mutex g_scratch_lock;
void* g_scratch_ptr[kScratchDevices];

void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
    std::lock_guard<std::mutex> hold(g_scratch_lock);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

sz_status decode_impl(SrcRef src, const uint64_t* d_src_bytes, uint64_t src_bytes, uint32_t count,
                      uint64_t n, sz_dtype dt, DstRef dst, int32_t* d_status, hipStream_t s) {
    if (d_status) {
        hipError_t e = launch_fill_i32(d_status, count, SZ_OK, s);
        if (e != hipSuccess) return SZ_ERR_HIP;
    }
    DecodeArgs a{};
    a.src = src;
    a.src_bytes_table = d_src_bytes;
    a.src_bytes = src_bytes;
    a.dst = dst;
    a.status = d_status;
    a.count = count;
    a.n = n;
    if (n == 0) return from_hip(launch_decode_empty(a, dt, s));
    return from_hip(launch_decode(a, dt, s));
}

}  // namespace

SZ_EXPORT uint64_t sz_max_compressed_bytes(uint64_t n, sz_dtype dtype) {
    if (!dtype_ok(dtype) || n >= kMaxElems) return 0;
    return layout_of(n, dtype).esc_at + n;
}

// The size queries answer 0 for a batch the calls would reject for its
// size (so no product here can wrap around 2^64 either).
SZ_EXPORT uint64_t sz_encode_workspace_bytes_batched(uint32_t count, uint64_t n, sz_dtype dtype) {
    if (!dtype_ok(dtype) || n >= kMaxElems || count == 0 || !grid_ok(count, n)) return 0;
    return workspace_bytes(count, n);
}

SZ_EXPORT uint64_t sz_encode_workspace_bytes(uint64_t n, sz_dtype dtype) {
    if (!dtype_ok(dtype)) return 0;
    return sz_encode_workspace_bytes_batched(1, n, dtype);
}

SZ_EXPORT sz_status sz_histogram(const void* d_src, uint64_t n, sz_dtype dtype, uint64_t* d_hist,
                                 hipStream_t stream) {
    if (!dtype_ok(dtype) || n >= kMaxElems || !usable(d_hist) || (n && !usable(d_src)))
        return SZ_ERR_INVALID_ARGUMENT;
    return histogram_impl(SrcRef{nullptr, d_src}, 1, n, dtype, 1, d_hist, stream);
}

SZ_EXPORT sz_status sz_histogram_batched(const void* const* d_srcs, uint32_t count, uint64_t n,
                                         sz_dtype dtype, uint64_t* d_hists, hipStream_t stream) {
    if (!dtype_ok(dtype) || n >= kMaxElems || count == 0 || !grid_ok(count, n) || !usable(d_hists) || !usable(d_srcs))
        return SZ_ERR_INVALID_ARGUMENT;
    return histogram_impl(SrcRef{d_srcs, nullptr}, count, n, dtype, 1, d_hists, stream);
}

SZ_EXPORT sz_status sz_histogram_sampled(const void* d_src, uint64_t n, sz_dtype dtype, uint32_t block_stride,
                                         uint64_t* d_hist, hipStream_t stream) {
    if (!dtype_ok(dtype) || n >= kMaxElems || block_stride == 0 || !usable(d_hist) || (n && !usable(d_src)))
        return SZ_ERR_INVALID_ARGUMENT;
    return histogram_impl(SrcRef{nullptr, d_src}, 1, n, dtype, block_stride, d_hist, stream);
}

SZ_EXPORT sz_status sz_histogram_sampled_batched(const void* const* d_srcs, uint32_t count, uint64_t n,
                                                 sz_dtype dtype, uint32_t block_stride, uint64_t* d_hists,
                                                 hipStream_t stream) {
    if (!dtype_ok(dtype) || n >= kMaxElems || count == 0 || !grid_ok(count, n) || block_stride == 0 || !usable(d_hists) ||
        !usable(d_srcs))
        return SZ_ERR_INVALID_ARGUMENT;
    return histogram_impl(SrcRef{d_srcs, nullptr}, count, n, dtype, block_stride, d_hists, stream);
}

SZ_EXPORT sz_status sz_build_codebook_batched(const uint64_t* d_hists, uint32_t count, sz_dtype dtype,
                                              uint8_t* d_codebooks, hipStream_t stream) {
    if (!dtype_ok(dtype) || count == 0 || !usable(d_hists) || !usable(d_codebooks))
        return SZ_ERR_INVALID_ARGUMENT;
    CodebookArgs a{d_hists, d_codebooks, count};
    return from_hip(launch_codebook(a, dtype, stream));
}

SZ_EXPORT sz_status sz_build_codebook(const uint64_t* d_hist, sz_dtype dtype, uint8_t* d_codebook,
                                      hipStream_t stream) {
    if (!dtype_ok(dtype)) return SZ_ERR_INVALID_ARGUMENT;
    return sz_build_codebook_batched(d_hist, 1, dtype, d_codebook, stream);
}

SZ_EXPORT sz_status sz_encode(const void* d_src, uint64_t n, sz_dtype dtype, const uint8_t* d_codebook,
                              void* d_dst, uint64_t dst_capacity, uint64_t* d_out_bytes,
                              void* d_workspace, uint64_t workspace_bytes_given, hipStream_t stream) {
    if (!dtype_ok(dtype) || n >= kMaxElems || !usable(d_codebook) || !usable(d_dst) ||
        (n && !usable(d_src)) || (d_out_bytes && (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (dst_capacity < sz_max_compressed_bytes(n, dtype)) return SZ_ERR_BUFFER_TOO_SMALL;
    if (n) {
        if (!usable(d_workspace)) return SZ_ERR_INVALID_ARGUMENT;
        if (workspace_bytes_given < workspace_bytes(1, n)) return SZ_ERR_BUFFER_TOO_SMALL;
    }
    return encode_impl(SrcRef{nullptr, d_src}, 1, n, dtype, d_codebook, DstRef{nullptr, d_dst},
                       d_out_bytes, d_workspace, stream);
}

SZ_EXPORT sz_status sz_encode_batched(const void* const* d_srcs, uint32_t count, uint64_t n,
                                      sz_dtype dtype, const uint8_t* d_codebooks, void* const* d_dsts,
                                      uint64_t dst_capacity, uint64_t* d_out_bytes, void* d_workspace,
                                      uint64_t workspace_bytes_given, hipStream_t stream) {
    if (!dtype_ok(dtype) || n >= kMaxElems || count == 0 || !grid_ok(count, n) || !usable(d_srcs) || !usable(d_codebooks) ||
        !usable(d_dsts) || (d_out_bytes && (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (dst_capacity < sz_max_compressed_bytes(n, dtype)) return SZ_ERR_BUFFER_TOO_SMALL;
    if (n) {
        if (!usable(d_workspace)) return SZ_ERR_INVALID_ARGUMENT;
        if (workspace_bytes_given < workspace_bytes(count, n)) return SZ_ERR_BUFFER_TOO_SMALL;
    }
    return encode_impl(SrcRef{d_srcs, nullptr}, count, n, dtype, d_codebooks, DstRef{d_dsts, nullptr},
                       d_out_bytes, d_workspace, stream);
}

SZ_EXPORT uint64_t sz_compress_workspace_bytes_batched(uint32_t count, uint64_t n, sz_dtype dtype) {
    if (!dtype_ok(dtype) || n >= kMaxElems || count == 0 || !grid_ok(count, n) ||
        static_cast<uint64_t>(count) * compress_items(n, dtype) >= (uint64_t(1) << 31))
        return 0;
    return compress_workspace_bytes(count, n);
}

SZ_EXPORT uint64_t sz_compress_workspace_bytes(uint64_t n, sz_dtype dtype) {
    if (!dtype_ok(dtype)) return 0;
    return sz_compress_workspace_bytes_batched(1, n, dtype);
}

SZ_EXPORT sz_status sz_compress(const void* d_src, uint64_t n, sz_dtype dtype, uint64_t* d_hist,
                                uint8_t* d_codebook, void* d_dst, uint64_t dst_capacity, uint64_t* d_out_bytes,
                                int32_t* d_status, void* d_workspace, uint64_t workspace_bytes_given,
                                const sz_compress_options* options, hipStream_t stream) {
    CompressSettings cs;
    if (!settings_of(options, cs) || !dtype_ok(dtype) || n >= kMaxElems || !usable(d_hist) || !usable(d_codebook) ||
        !usable(d_dst) || !usable(d_workspace) || (n && !usable(d_src)) ||
        (d_out_bytes && (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u)) ||
        (d_status && (reinterpret_cast<uintptr_t>(d_status) & 3u)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (dst_capacity < sz_max_compressed_bytes(n, dtype)) return SZ_ERR_BUFFER_TOO_SMALL;
    if (workspace_bytes_given < compress_workspace_bytes(1, n)) return SZ_ERR_BUFFER_TOO_SMALL;
    return compress_impl(SrcRef{nullptr, d_src}, 1, n, dtype, d_hist, d_codebook, DstRef{nullptr, d_dst},
                         d_out_bytes, d_status, d_workspace, cs, stream);
}

SZ_EXPORT sz_status sz_compress_noalloc(const void* d_src, uint64_t n, sz_dtype dtype, uint64_t* d_hist,
                                        uint8_t* d_codebook, void* d_dst, uint64_t dst_capacity,
                                        uint64_t* d_out_bytes, int32_t* d_status,
                                        const sz_compress_options* options, hipStream_t stream) {
    static_assert(SZ_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch keeps the workspace alignment");
    CompressSettings cs;
    if (!settings_of(options, cs) || !dtype_ok(dtype) || n >= kMaxElems || !usable(d_hist) || !usable(d_codebook) ||
        !usable(d_dst) || (n && !usable(d_src)) || (d_out_bytes && (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u)) ||
        (d_status && (reinterpret_cast<uintptr_t>(d_status) & 3u)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (dst_capacity < sz_max_compressed_bytes(n, dtype)) return SZ_ERR_BUFFER_TOO_SMALL;
    if (n > SZ_NOALLOC_MAX_ELEMENTS || compress_workspace_bytes(1, n) > SZ_NOALLOC_SCRATCH_BYTES)
        return SZ_ERR_BUFFER_TOO_SMALL;
    void* ws = scratch_on_current_device();
    if (!ws) return SZ_ERR_HIP;
    return compress_impl(SrcRef{nullptr, d_src}, 1, n, dtype, d_hist, d_codebook, DstRef{nullptr, d_dst},
                         d_out_bytes, d_status, ws, cs, stream);
}

SZ_EXPORT sz_status sz_compress_batched(const void* const* d_srcs, uint32_t count, uint64_t n, sz_dtype dtype,
                                        uint64_t* d_hists, uint8_t* d_codebooks, void* const* d_dsts,
                                        uint64_t dst_capacity, uint64_t* d_out_bytes, int32_t* d_status,
                                        void* d_workspace, uint64_t workspace_bytes_given,
                                        const sz_compress_options* options, hipStream_t stream) {
    CompressSettings cs;
    if (!settings_of(options, cs) || !dtype_ok(dtype) || n >= kMaxElems || count == 0 || !grid_ok(count, n) ||
        static_cast<uint64_t>(count) * compress_items(n, dtype) >= (uint64_t(1) << 31) || !usable(d_srcs) ||
        !usable(d_hists) || !usable(d_codebooks) || !usable(d_dsts) || !usable(d_workspace) ||
        (d_out_bytes && (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u)) ||
        (d_status && (reinterpret_cast<uintptr_t>(d_status) & 3u)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (dst_capacity < sz_max_compressed_bytes(n, dtype)) return SZ_ERR_BUFFER_TOO_SMALL;
    if (workspace_bytes_given < compress_workspace_bytes(count, n)) return SZ_ERR_BUFFER_TOO_SMALL;
    return compress_impl(SrcRef{d_srcs, nullptr}, count, n, dtype, d_hists, d_codebooks, DstRef{d_dsts, nullptr},
                         d_out_bytes, d_status, d_workspace, cs, stream);
}

SZ_EXPORT sz_status sz_decode(const void* d_src, uint64_t src_bytes, uint64_t n, sz_dtype dtype,
                              void* d_dst, int32_t* d_status, hipStream_t stream) {
    if (!dtype_ok(dtype) || n >= kMaxElems || !usable(d_src) || (n && !usable(d_dst)) ||
        (d_status && (reinterpret_cast<uintptr_t>(d_status) & 3u)))
        return SZ_ERR_INVALID_ARGUMENT;
    if (src_bytes < layout_of(n, dtype).esc_at) return SZ_ERR_CORRUPT_STREAM;
    return decode_impl(SrcRef{nullptr, d_src}, nullptr, src_bytes, 1, n, dtype, DstRef{nullptr, d_dst},
                       d_status, stream);
}

SZ_EXPORT sz_status sz_decode_batched(const void* const* d_srcs, const uint64_t* d_src_bytes,
                                      uint32_t count, uint64_t n, sz_dtype dtype, void* const* d_dsts,
                                      int32_t* d_status, hipStream_t stream) {
    if (!dtype_ok(dtype) || n >= kMaxElems || count == 0 || !grid_ok(count, n) || !usable(d_srcs) || !usable(d_src_bytes) ||
        !usable(d_dsts) || (d_status && (reinterpret_cast<uintptr_t>(d_status) & 3u)))
        return SZ_ERR_INVALID_ARGUMENT;
    return decode_impl(SrcRef{d_srcs, nullptr}, d_src_bytes, 0, count, n, dtype, DstRef{d_dsts, nullptr},
                       d_status, stream);
}

SZ_EXPORT uint32_t sz_abi_version(void) { return SZ_ABI_VERSION; }

SZ_EXPORT const char* sz_status_string(sz_status status) {
    switch (raw_value(status)) {
        case SZ_OK: return "ok";
        case SZ_ERR_INVALID_ARGUMENT: return "invalid argument";
        case SZ_ERR_BUFFER_TOO_SMALL: return "buffer too small";
        case SZ_ERR_CORRUPT_STREAM: return "corrupt stream";
        case SZ_ERR_HIP: return "HIP launch failure";
        case SZ_ERR_TIMEOUT: return "gave up waiting for the codebook";
    }
    return "unknown status";
}
