"""sz_compress_noalloc: sz_compress with its workspace in the library's own
scratch array, for callers that cannot allocate.  Called through the C ABI
and compared with sz_compress (its own workspace) to the same bar: bit-exact
histogram, codebook, stream, size and status, on two calls in a row whose
second input is smaller (the scratch keeps the first call's contents), on
both the one-launch kernel and the separate kernels, and against the
oracle."""
import sys

import numpy as np
import pytest
import torch

import kvsynth
import oracle

pytestmark = pytest.mark.gpu

BF16, E5M2 = 1, 2


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sz():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp8_kv_cache_amd
    return fp8_kv_cache_amd


def _outputs(sz, n, dt, dev):
    return dict(hist=torch.full((256,), -1, dtype=torch.int64, device=dev),
                codebook=torch.full((16,), 0xAB, dtype=torch.uint8, device=dev),
                dst=torch.full((sz.sz_max_compressed_bytes(n, dt),), 0xCD, dtype=torch.uint8, device=dev),
                out_bytes=torch.zeros(1, dtype=torch.int64, device=dev),
                status=torch.full((1,), -1, dtype=torch.int32, device=dev))


def _run_both(sz, x, dt, options):
    n, dev = x.numel(), x.device
    a, b = _outputs(sz, n, dt, dev), _outputs(sz, n, dt, dev)
    ws_bytes = sz.sz_compress_workspace_bytes(n, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    sz.check(sz.sz_compress(x, n, dt, a["hist"], a["codebook"], a["dst"], a["dst"].numel(), a["out_bytes"],
                            a["status"], ws, ws_bytes, options), "sz_compress")
    sz.check(sz.sz_compress_noalloc(x, n, dt, b["hist"], b["codebook"], b["dst"], b["dst"].numel(), b["out_bytes"],
                                    b["status"], options), "sz_compress_noalloc")
    torch.cuda.synchronize()
    return a, b


def _same(sz, x, dt, a, b):
    assert int(a["status"]) == 0 and int(b["status"]) == 0
    assert torch.equal(a["hist"], b["hist"]) and torch.equal(a["codebook"], b["codebook"])
    size = int(a["out_bytes"])
    assert int(b["out_bytes"]) == size
    assert torch.equal(a["dst"][:size], b["dst"][:size])
    host = x.cpu().numpy()
    assert np.array_equal(b["dst"][:size].cpu().numpy(), oracle.encode(host.view(np.uint16) if dt == BF16 else host, dt))


@pytest.mark.parametrize("dt,fused_min", [(BF16, 0), (BF16, 1), (E5M2, 0)])
def test_noalloc_matches_sz_compress_on_two_calls(sz, dt, fused_min):
    """Two calls in a row, the second on a smaller tensor: the one-launch
    kernel (BF16 from 2^21 elements, or every size with fused_min = 1) and
    the separate kernels (E5M2, small BF16) both reuse the scratch left by
    the previous call."""
    options = sz.compress_options(fused_min_elements=fused_min)
    sizes = [(1 << 22) + 777, (1 << 21) + 5] if dt == BF16 else [(1 << 22) + 777, 100003]
    for k, n in enumerate(sizes):
        bits = kvsynth.stress(n, seed=900 + k) if k else kvsynth.single_tensor(n, seed=900)
        host = bits if dt == BF16 else kvsynth.e5m2_of(bits)
        x = torch.from_numpy(host.view(np.int16) if dt == BF16 else host).to("cuda")
        say("noalloc", dt, fused_min, n)
        a, b = _run_both(sz, x, dt, options)
        _same(sz, x, dt, a, b)


def test_noalloc_limit_and_largest_size(sz):
    """The largest tensor the scratch holds compresses like sz_compress; one
    element more is rejected on the host before anything is enqueued."""
    n = sz.SZ_NOALLOC_MAX_ELEMENTS
    x = torch.from_numpy(kvsynth.single_tensor(n, seed=910).view(np.int16)).to("cuda")
    say("noalloc largest", n)
    a, b = _run_both(sz, x, BF16, None)
    _same(sz, x, BF16, a, b)
    big = n + 1
    xb = torch.zeros(big, dtype=torch.int16, device="cuda")   # a valid input of that size
    out = _outputs(sz, big, BF16, "cuda")
    rc = sz.sz_compress_noalloc(xb, big, BF16, out["hist"], out["codebook"], out["dst"], out["dst"].numel(),
                                out["out_bytes"], out["status"])
    assert rc == sz.SZ_ERR_BUFFER_TOO_SMALL
    torch.cuda.synchronize()
    assert int(out["status"]) == -1   # nothing ran
