"""Allocation helpers over the C ABI: torch allocates the device buffers, the
library's kernels do all the work (histogram -> codebook -> encode, and
decode).  Raw elements are passed as torch tensors of 16-bit words (BF16 bit
patterns, dtype int16/bfloat16) or bytes (E5M2, dtype uint8/float8_e5m2).
"""
import torch

from . import (SZ_DTYPE_BF16, SZ_DTYPE_FP8_E5M2, SZ_ERR_TIMEOUT, SZ_OK, check, pointer_table, sz_build_codebook, sz_histogram_sampled,
               sz_histogram_sampled_batched, sz_compress, sz_compress_batched, sz_compress_workspace_bytes,
               sz_compress_workspace_bytes_batched,
               sz_build_codebook_batched, sz_decode, sz_decode_batched, sz_encode, sz_encode_batched,
               sz_encode_workspace_bytes, sz_encode_workspace_bytes_batched, sz_histogram,
               sz_histogram_batched, sz_max_compressed_bytes)

ELEMENT_BYTES = {SZ_DTYPE_BF16: 2, SZ_DTYPE_FP8_E5M2: 1}


def _raw_dtype(dtype):
    return torch.int16 if dtype == SZ_DTYPE_BF16 else torch.uint8


def compress(x, dtype, codebook=None, stream=None, block_stride=1):
    """Encode one tensor.  Returns (stream bytes as a uint8 tensor of exactly
    C bytes, histogram int64[256] or None, codebook uint8[16]).  With
    block_stride > 1 the codebook comes from a histogram of every
    block_stride-th 4096-element block."""
    dev = x.device
    n = x.numel()
    hist = None
    if codebook is None:
        hist = torch.empty(256, dtype=torch.int64, device=dev)
        codebook = torch.empty(16, dtype=torch.uint8, device=dev)
        if block_stride == 1:
            check(sz_histogram(x, n, dtype, hist, stream), "sz_histogram")
        else:
            check(sz_histogram_sampled(x if n else None, n, dtype, block_stride, hist, stream),
                  "sz_histogram_sampled")
        check(sz_build_codebook(hist, dtype, codebook, stream), "sz_build_codebook")
    cap = sz_max_compressed_bytes(n, dtype)
    dst = torch.empty(cap, dtype=torch.uint8, device=dev)
    out_bytes = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_bytes = sz_encode_workspace_bytes(n, dtype)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    check(sz_encode(x if n else None, n, dtype, codebook, dst, cap, out_bytes, ws, ws_bytes, stream),
          "sz_encode")
    size = int(out_bytes.item())
    return dst[:size], hist, codebook


def compress_fused(x, dtype, stream=None, options=None, retry=True):
    """Histogram, codebook and encode of one tensor in one launch
    (sz_compress).  Returns (stream bytes, histogram int64[256], codebook
    uint8[16], device status); the results equal compress()'s.  options: an
    SzCompressOptions (compress_options()) or None for the defaults.  If the
    kernel gave up (SZ_ERR_TIMEOUT) and `retry`, the tensor is encoded again
    with the separate calls and their results are returned with SZ_OK."""
    dev = x.device
    n = x.numel()
    hist = torch.empty(256, dtype=torch.int64, device=dev)
    codebook = torch.empty(16, dtype=torch.uint8, device=dev)
    cap = sz_max_compressed_bytes(n, dtype)
    dst = torch.empty(cap, dtype=torch.uint8, device=dev)
    out_bytes = torch.zeros(1, dtype=torch.int64, device=dev)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    ws_bytes = sz_compress_workspace_bytes(n, dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    check(sz_compress(x if n else None, n, dtype, hist, codebook, dst, cap, out_bytes, status, ws, ws_bytes,
                      options, stream), "sz_compress")
    st = int(status.item())
    if st == SZ_ERR_TIMEOUT and retry:
        # the one-launch kernel gave up waiting (its stream does not decode):
        # the separate calls' kernels compute the same results without waits
        stream_bytes, hist, codebook = compress(x, dtype, stream=stream)
        return stream_bytes, hist, codebook, SZ_OK
    size = int(out_bytes.item())
    return dst[:size], hist, codebook, st


def decompress(stream_bytes, n, dtype, src_bytes=None, stream=None):
    """Decode one stream.  Returns (raw elements tensor, device status)."""
    dev = stream_bytes.device
    out = torch.empty(max(n, 1), dtype=_raw_dtype(dtype), device=dev)[:n]
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    nbytes = stream_bytes.numel() if src_bytes is None else src_bytes
    check(sz_decode(stream_bytes, nbytes, n, dtype, out if n else None, status, stream), "sz_decode")
    return out, int(status.item())


class BatchCodec:
    """Device buffers for `count` tensors of n elements each: histograms,
    codebooks, streams (each sz_max_compressed_bytes long), sizes,
    workspace, decode outputs and statuses, plus their pointer tables."""

    def __init__(self, count, n, dtype, device="cuda"):
        self.count, self.n, self.dtype = count, n, dtype
        self.capacity = sz_max_compressed_bytes(n, dtype)
        cap = -(-self.capacity // 256) * 256
        self.hists = torch.zeros(count, 256, dtype=torch.int64, device=device)
        self.codebooks = torch.zeros(count, 16, dtype=torch.uint8, device=device)
        self.streams = torch.empty(count, cap, dtype=torch.uint8, device=device)
        self.sizes = torch.zeros(count, dtype=torch.int64, device=device)
        # the fused call's workspace holds the encode workspace at its start
        self.ws_bytes = sz_encode_workspace_bytes_batched(count, n, dtype)
        self.fused_ws_bytes = sz_compress_workspace_bytes_batched(count, n, dtype)
        self.workspace = torch.empty(max(self.fused_ws_bytes, 16), dtype=torch.uint8, device=device)
        self.fused_status = torch.full((count,), -1, dtype=torch.int32, device=device)
        # rows start 16-byte aligned, as the C ABI requires of every output
        row = -(-max(n, 1) * ELEMENT_BYTES[dtype] // 16) * 16
        self.outputs = torch.empty(count, row, dtype=torch.uint8, device=device)
        self.status = torch.full((count,), -1, dtype=torch.int32, device=device)
        self.stream_ptrs = pointer_table([self.streams[i] for i in range(count)])
        self.output_ptrs = pointer_table([self.outputs[i] for i in range(count)])
        self.src_ptrs = None

    def set_inputs(self, tensors):
        assert len(tensors) == self.count
        self._inputs = list(tensors)  # keep alive
        self.src_ptrs = pointer_table(self._inputs)

    def histogram(self, stream=None, block_stride=1):
        if block_stride == 1:
            check(sz_histogram_batched(self.src_ptrs, self.count, self.n, self.dtype, self.hists, stream),
                  "sz_histogram_batched")
        else:
            check(sz_histogram_sampled_batched(self.src_ptrs, self.count, self.n, self.dtype, block_stride,
                                               self.hists, stream), "sz_histogram_sampled_batched")

    def build_codebooks(self, stream=None):
        check(sz_build_codebook_batched(self.hists, self.count, self.dtype, self.codebooks, stream),
              "sz_build_codebook_batched")

    def encode(self, stream=None):
        check(sz_encode_batched(self.src_ptrs, self.count, self.n, self.dtype, self.codebooks,
                                self.stream_ptrs, self.capacity, self.sizes, self.workspace,
                                self.ws_bytes, stream), "sz_encode_batched")

    def compress(self, stream=None):
        self.histogram(stream)
        self.build_codebooks(stream)
        self.encode(stream)

    def compress_fused(self, stream=None, options=None):
        """Same histograms, codebooks and streams as compress(), in one
        launch (sz_compress_batched); per-tensor status in fused_status
        (asynchronous: see settle()).  options: an SzCompressOptions or None
        for the defaults."""
        check(sz_compress_batched(self.src_ptrs, self.count, self.n, self.dtype, self.hists, self.codebooks,
                                  self.stream_ptrs, self.capacity, self.sizes, self.fused_status, self.workspace,
                                  self.fused_ws_bytes, options, stream), "sz_compress_batched")

    def settle(self, stream=None):
        """After compress_fused(): waits for it, and if any tensor gave up
        (SZ_ERR_TIMEOUT; its stream does not decode) encodes the whole batch
        again with the separate calls, which compute the same results
        without waits.  Returns the number of tensors that had given up."""
        torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
        gave_up = int((self.fused_status == SZ_ERR_TIMEOUT).sum().item())
        if gave_up:
            self.compress(stream)
            self.fused_status.fill_(SZ_OK)
        return gave_up

    def decompress(self, stream=None):
        check(sz_decode_batched(self.stream_ptrs, self.sizes, self.count, self.n, self.dtype,
                                self.output_ptrs, self.status, stream), "sz_decode_batched")

    def stream(self, i):
        return self.streams[i, :int(self.sizes[i].item())]

    def output(self, i):
        return self.outputs[i, :self.n * ELEMENT_BYTES[self.dtype]].view(_raw_dtype(self.dtype))
