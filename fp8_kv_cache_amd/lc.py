"""Allocation helpers for the LC-style comparison codec (TUPL8_1 -> BIT_8 ->
RZE_2 on 16 KB chunks; FastKVComp companion page, "Inside an LC-style
pipeline").  torch allocates device buffers; the library's kernels do the
work.  Inputs are any contiguous tensors, coded as their raw bytes.
"""
import torch

from . import (check, lc_decode, lc_decode_batched, lc_encode, lc_encode_batched, lc_encode_workspace_bytes,
               lc_encode_workspace_bytes_batched, lc_max_compressed_bytes, pointer_table)


def _nbytes(x):
    return x.numel() * x.element_size()


def compress(x, stream=None):
    """Stream of x's bytes as a uint8 tensor of exactly its total length."""
    n = _nbytes(x)
    cap = lc_max_compressed_bytes(n)
    dst = torch.empty(cap, dtype=torch.uint8, device=x.device)
    out_bytes = torch.zeros(1, dtype=torch.int64, device=x.device)
    ws_bytes = lc_encode_workspace_bytes(n)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
    check(lc_encode(x if n else None, n, dst, cap, out_bytes, ws, ws_bytes, stream), "lc_encode")
    return dst[:int(out_bytes.item())]


def decompress(stream_bytes, n, src_bytes=None, stream=None):
    """(n decoded bytes as a uint8 tensor, device status)."""
    dev = stream_bytes.device
    out = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)[:n]
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    nbytes = stream_bytes.numel() if src_bytes is None else src_bytes
    check(lc_decode(stream_bytes, nbytes, n, out if n else None, status, stream), "lc_decode")
    return out, int(status.item())


class LcBatch:
    """Device buffers for `count` tensors of n bytes each: streams (each
    lc_max_compressed_bytes long), sizes, workspace, outputs and statuses."""

    def __init__(self, count, n, device="cuda"):
        self.count, self.n = count, n
        self.capacity = lc_max_compressed_bytes(n)
        cap = -(-self.capacity // 256) * 256
        self.streams = torch.zeros(count, cap, dtype=torch.uint8, device=device)
        self.sizes = torch.zeros(count, dtype=torch.int64, device=device)
        self.ws_bytes = lc_encode_workspace_bytes_batched(count, n)
        self.workspace = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=device)
        # rows start 16-byte aligned, as the C ABI requires of every output
        self.outputs = torch.empty(count, -(-max(n, 1) // 16) * 16, dtype=torch.uint8, device=device)
        self.status = torch.full((count,), -1, dtype=torch.int32, device=device)
        self.stream_ptrs = pointer_table([self.streams[i] for i in range(count)])
        self.output_ptrs = pointer_table([self.outputs[i] for i in range(count)])
        self.src_ptrs = None

    def set_inputs(self, tensors):
        assert len(tensors) == self.count and all(_nbytes(t) == self.n for t in tensors)
        self._inputs = list(tensors)
        self.src_ptrs = pointer_table(self._inputs)

    def encode(self, stream=None):
        check(lc_encode_batched(self.src_ptrs, self.count, self.n, self.stream_ptrs, self.capacity, self.sizes,
                                self.workspace, self.ws_bytes, stream), "lc_encode_batched")

    def decode(self, stream=None):
        check(lc_decode_batched(self.stream_ptrs, self.sizes, self.count, self.n, self.output_ptrs, self.status,
                                stream), "lc_decode_batched")

    def stream(self, i):
        return self.streams[i, :int(self.sizes[i].item())]

    def output(self, i):
        return self.outputs[i, :self.n]
