"""Layer-pipelined KV transfer over a copy link, with and without the codec.

What the codec is for (SplitZip project page, FAQ "How can I reduce KV cache
transfer time between prefill and decode nodes?"): compress each KV layer on
the sending GPU, move fewer bytes over the link, decompress on the receiving
GPU, with the codec running much faster than the link.  The FastKVComp page
("Equation 1: does it pay?") states the condition: compression pays when
encode + decode time is below the link time it saves.

On one GPU the link is emulated by the PCIe path: every layer crosses
device -> pinned host memory (the sending side) and pinned host memory ->
device (the receiving side) through the copy engines, the way a prefill
GPU's tensor leaves through one NIC and lands through another on a decode
GPU.  The two sides have copy streams of their own, so while layer i is
received, layer i+1 is already being sent (PCIe carries both directions at
once, as two machines' NICs would).

  ship_raw         copies the raw layers over the link;
  ship_compressed  compresses a group of layers with one batched
                   histogram + codebook + encode call (sz_compress_batched)
                   while the previous group's exact-size streams cross the
                   link, and decodes each layer as it lands.

Both return the received tensors, so callers can check bit-exactness.
Streams run at the default priority.
"""
import torch

from . import SZ_DTYPE_BF16, check, pointer_table, sz_compress_batched, sz_compress_workspace_bytes_batched, \
    sz_decode, sz_max_compressed_bytes
from .codec import ELEMENT_BYTES


class _Layer:
    """Device and pinned-host buffers for one layer tensor of n elements."""

    def __init__(self, n, dtype, device):
        self.n, self.dtype = n, dtype
        self.capacity = sz_max_compressed_bytes(n, dtype)
        self.stream = torch.empty(-(-self.capacity // 256) * 256, dtype=torch.uint8, device=device)
        self.host = torch.empty(self.capacity, dtype=torch.uint8, pin_memory=True)
        self.landed = torch.empty(self.capacity, dtype=torch.uint8, device=device)
        self.output = torch.empty(n * ELEMENT_BYTES[dtype], dtype=torch.uint8, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)


class Link:
    """Buffers for shipping `count` layer tensors of n elements each, in
    groups of up to `group` layers per compress call."""

    def __init__(self, count, n, dtype=SZ_DTYPE_BF16, device="cuda", group=8):
        self.count, self.n, self.dtype, self.group = count, n, dtype, group
        self.layers = [_Layer(n, dtype, device) for _ in range(count)]
        raw = n * ELEMENT_BYTES[dtype]
        self.raw_host = [torch.empty(raw, dtype=torch.uint8, pin_memory=True) for _ in range(count)]
        self.raw_landed = [torch.empty(raw, dtype=torch.uint8, device=device) for _ in range(count)]
        self.hists = torch.empty(count, 256, dtype=torch.int64, device=device)
        self.codebooks = torch.empty(count, 16, dtype=torch.uint8, device=device)
        self.fused_status = torch.zeros(count, dtype=torch.int32, device=device)
        # each layer's stream size goes straight to pinned host memory: no
        # copy-engine transfer that could queue behind earlier layers' copies
        self.sizes_host = torch.zeros(count, dtype=torch.int64, pin_memory=True)
        self.ws_bytes = sz_compress_workspace_bytes_batched(min(group, count), n, dtype)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        # one device pointer table per group (the batched call wants each
        # table 16-byte aligned)
        self.bounds = [(lo, min(lo + group, count)) for lo in range(0, count, group)]
        self.dst_tables = [pointer_table([L.stream for L in self.layers[lo:hi]]) for lo, hi in self.bounds]
        self._src = (None, None)
        self.codec_stream = torch.cuda.Stream()
        self.send_stream = torch.cuda.Stream()      # device -> pinned host
        self.recv_stream = torch.cuda.Stream()      # pinned host -> device

    def _src_tables(self, tensors):
        key = tuple(t.data_ptr() for t in tensors)
        if self._src[0] != key:
            self._src = (key, [pointer_table(list(tensors[lo:hi])) for lo, hi in self.bounds])
        return self._src[1]

    def _cross(self, src, host, landed):
        """Queue one crossing: send src into host memory, then receive it
        into `landed` once sent.  Returns the event marking its arrival."""
        with torch.cuda.stream(self.send_stream):
            host.copy_(src, non_blocking=True)
            sent = torch.cuda.Event()
            sent.record(self.send_stream)
        self.recv_stream.wait_event(sent)
        with torch.cuda.stream(self.recv_stream):
            landed.copy_(host, non_blocking=True)
            done = torch.cuda.Event()
            done.record(self.recv_stream)
        return done

    def ship_raw(self, tensors):
        """Raw layers over the link; returns the landed copies (uint8 views)."""
        cur = torch.cuda.current_stream()
        self.send_stream.wait_stream(cur)
        for t, host, landed in zip(tensors, self.raw_host, self.raw_landed):
            self._cross(t.view(torch.uint8).reshape(-1), host, landed)
        cur.wait_stream(self.recv_stream)
        return self.raw_landed

    def ship_compressed(self, tensors):
        """Compress -> link -> decode, pipelined across groups of layers.
        Group g is compressed by one sz_compress_batched call on the codec
        stream; then the host waits for group g-1's call (its stream sizes
        land in pinned host memory) and queues its exact-size copies behind
        one wait on the send stream, so the link starts after the first
        group and the GPU keeps compressing later groups meanwhile.  Each
        layer is decoded as it lands."""
        cur = torch.cuda.current_stream()
        cs = self.codec_stream
        cs.wait_stream(cur)
        self.send_stream.wait_stream(cur)
        srcs = self._src_tables(tensors)
        encoded, landed_events = [], []

        def queue_compress(g, lo, hi):
            s = cs.cuda_stream
            check(sz_compress_batched(srcs[g], hi - lo, self.n, self.dtype, self.hists[lo], self.codebooks[lo],
                                      self.dst_tables[g], self.layers[0].capacity,
                                      self.sizes_host.data_ptr() + 8 * lo, self.fused_status[lo], self.workspace,
                                      self.ws_bytes, None, s), "sz_compress_batched")
            ev = torch.cuda.Event()
            ev.record(cs)
            encoded.append(ev)

        def queue_copies(g, lo, hi):
            encoded[g].synchronize()
            self.send_stream.wait_event(encoded[g])
            for i in range(lo, hi):
                L = self.layers[i]
                nbytes = int(self.sizes_host[i])
                # copy-engine friendly length: a 4 KiB multiple (the stream buffer
                # holds at least that much; the bytes past the stream are unused)
                span = min(-(-nbytes // 4096) * 4096, L.capacity)
                landed_events.append((self._cross(L.stream[:span], L.host[:span], L.landed[:span]), nbytes))

        bounds = self.bounds
        for g, (lo, hi) in enumerate(bounds):
            queue_compress(g, lo, hi)
            if g:
                queue_copies(g - 1, *bounds[g - 1])
        queue_copies(len(bounds) - 1, *bounds[-1])
        for (done, nbytes), L in zip(landed_events, self.layers):
            cs.wait_event(done)
            check(sz_decode(L.landed, nbytes, self.n, self.dtype, L.output, L.status, cs.cuda_stream),
                  "sz_decode")
        cur.wait_stream(cs)
        return [L.output for L in self.layers]

    def compressed_bytes(self):
        return int(self.sizes_host.sum())

    def statuses(self):
        return [int(L.status[0]) for L in self.layers]

    def compress_statuses(self):
        return self.fused_status.cpu().tolist()
