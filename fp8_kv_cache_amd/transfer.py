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
  ship_compressed  encodes layer i+1 while layer i's exact-size stream
                   crosses the link, and decodes each layer as it lands.

Both return the received tensors, so callers can check bit-exactness.
Streams run at the default priority.
"""
import torch

from . import SZ_DTYPE_BF16, check, sz_build_codebook, sz_decode, sz_encode, sz_encode_workspace_bytes, \
    sz_histogram, sz_max_compressed_bytes
from .codec import ELEMENT_BYTES


class _Layer:
    """Device and pinned-host buffers for one layer tensor of n elements."""

    def __init__(self, n, dtype, device):
        self.n, self.dtype = n, dtype
        self.capacity = sz_max_compressed_bytes(n, dtype)
        self.hist = torch.empty(256, dtype=torch.int64, device=device)
        self.codebook = torch.empty(16, dtype=torch.uint8, device=device)
        self.stream = torch.empty(self.capacity, dtype=torch.uint8, device=device)
        self.ws_bytes = sz_encode_workspace_bytes(n, dtype)
        self.workspace = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=device)
        self.host = torch.empty(self.capacity, dtype=torch.uint8, pin_memory=True)
        self.size_host = torch.zeros(1, dtype=torch.int64, pin_memory=True)
        self.landed = torch.empty(self.capacity, dtype=torch.uint8, device=device)
        self.output = torch.empty(n * ELEMENT_BYTES[dtype], dtype=torch.uint8, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)


class Link:
    """Buffers for shipping `count` layer tensors of n elements each."""

    def __init__(self, count, n, dtype=SZ_DTYPE_BF16, device="cuda"):
        self.count, self.n, self.dtype = count, n, dtype
        self.layers = [_Layer(n, dtype, device) for _ in range(count)]
        raw = n * ELEMENT_BYTES[dtype]
        self.raw_host = [torch.empty(raw, dtype=torch.uint8, pin_memory=True) for _ in range(count)]
        self.raw_landed = [torch.empty(raw, dtype=torch.uint8, device=device) for _ in range(count)]
        self.codec_stream = torch.cuda.Stream()
        self.send_stream = torch.cuda.Stream()      # device -> pinned host
        self.recv_stream = torch.cuda.Stream()      # pinned host -> device

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

    def ship_compressed(self, tensors, group=8):
        """Encode -> link -> decode, pipelined across layers.  Layers go to
        the link in groups of `group`: the host waits for a group's encodes
        (each stream size lands in pinned host memory), then queues the
        group's exact-size copies behind one wait on the send stream; the GPU
        keeps encoding later layers meanwhile.  One wait per group instead of per
        layer measured ≈4% faster with groups of 8 on 64 layers of 16 MiB."""
        cur = torch.cuda.current_stream()
        cs = self.codec_stream
        cs.wait_stream(cur)
        self.send_stream.wait_stream(cur)
        encoded, landed_events = [], []

        def queue_encode(t, L):
            s = cs.cuda_stream
            check(sz_histogram(t, self.n, self.dtype, L.hist, s), "sz_histogram")
            check(sz_build_codebook(L.hist, self.dtype, L.codebook, s), "sz_build_codebook")
            # the stream size goes straight to pinned host memory: no copy-engine
            # transfer that could queue behind earlier layers' big copies
            check(sz_encode(t, self.n, self.dtype, L.codebook, L.stream, L.capacity, L.size_host,
                            L.workspace, L.ws_bytes, s), "sz_encode")
            ev = torch.cuda.Event()
            ev.record(cs)
            encoded.append(ev)

        def queue_copies(lo, hi):
            encoded[hi - 1].synchronize()
            self.send_stream.wait_event(encoded[hi - 1])
            for i in range(lo, hi):
                L = self.layers[i]
                nbytes = int(L.size_host[0])
                # copy-engine friendly length: a 4 KiB multiple (the stream buffer
                # holds at least that much; the bytes past the stream are unused)
                span = min(-(-nbytes // 4096) * 4096, L.capacity)
                landed_events.append((self._cross(L.stream[:span], L.host[:span], L.landed[:span]), nbytes))

        # encode group g, then put group g-1 on the link, so the link starts
        # right after the first group instead of after every encode is queued
        count = len(self.layers)
        bounds = [(lo, min(lo + group, count)) for lo in range(0, count, group)]
        for g, (lo, hi) in enumerate(bounds):
            for i in range(lo, hi):
                queue_encode(tensors[i], self.layers[i])
            if g:
                queue_copies(*bounds[g - 1])
        queue_copies(*bounds[-1])
        for (done, nbytes), L in zip(landed_events, self.layers):
            cs.wait_event(done)
            check(sz_decode(L.landed, nbytes, self.n, self.dtype, L.output, L.status, cs.cuda_stream),
                  "sz_decode")
        cur.wait_stream(cs)
        return [L.output for L in self.layers]

    def compressed_bytes(self):
        return sum(int(L.size_host[0]) for L in self.layers)

    def statuses(self):
        return [int(L.status[0]) for L in self.layers]
