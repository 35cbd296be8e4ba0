"""The HBM probe kernels the benchmark measures its ceilings with
(libszprobe.so): the copy and the compress-mix pass write exactly what
they read, and the read-only pass writes nothing."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "fp8_kv_cache_amd", "libszprobe.so"))
    lib.szp_stream.restype = ctypes.c_int
    lib.szp_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                               ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("nt", [0, 1])
def test_probe_passes_write_what_they_read(nt):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    print("[gpu-case] probe nt", nt, flush=True)
    lib = _lib()
    stream = torch.cuda.current_stream()
    n = (1 << 20) + 3 * 64                      # bytes; several grid strides and a ragged last stride
    g = torch.Generator().manual_seed(31 + nt)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).cuda()
    copy = torch.zeros(n, dtype=torch.uint8, device="cuda")
    assert lib.szp_stream(src.data_ptr(), copy.data_ptr(), n, n, 4, nt, 64, stream.cuda_stream) == 0
    mix = torch.zeros(n // 4 * 3, dtype=torch.uint8, device="cuda")
    assert lib.szp_stream(src.data_ptr(), mix.data_ptr(), n, mix.numel(), 3, nt, 64, stream.cuda_stream) == 0
    sink = torch.zeros(64 * 256 * 16, dtype=torch.uint8, device="cuda")
    assert lib.szp_stream(src.data_ptr(), sink.data_ptr(), n, sink.numel(), 0, nt, 64, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(copy, src)
    assert torch.equal(mix, src.view(-1, 4, 16)[:, :3, :].reshape(-1))
    assert not sink.any()
