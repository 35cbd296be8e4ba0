"""Python binding of libsplitzip.so, the gfx950 lossless exponent codec for
BF16 and FP8-E5M2 KV-cache tensors (SplitZip project page, "Abstract"), and
of the LC-style comparison codec in the same library (FastKVComp companion
page, "Inside an LC-style pipeline").

Thin ctypes marshalling over the C ABI declared in include/splitzip.h and
include/lc_codec.h: the functions below carry the C names and arguments.  Pointer arguments accept
a torch tensor (its data_ptr()), a plain integer address or None; `stream`
defaults to torch's current stream.  torch provides device memory and
streams only -- every step of the codec runs in the library's HIP kernels.

The library must be built (python fp8_kv_cache_amd/build.py); importing this
package without it raises ImportError, there is no fallback path.
"""
import ctypes
import os

import torch  # load torch's HIP runtime first; the library binds to it

__all__ = [
    "SZ_DTYPE_BF16", "SZ_DTYPE_FP8_E5M2", "SZ_OK", "SZ_ERR_INVALID_ARGUMENT",
    "SZ_ERR_BUFFER_TOO_SMALL", "SZ_ERR_CORRUPT_STREAM", "SZ_ERR_HIP", "SZ_ERR_TIMEOUT", "SzError",
    "sz_max_compressed_bytes", "sz_encode_workspace_bytes", "sz_encode_workspace_bytes_batched",
    "sz_histogram", "sz_histogram_sampled", "sz_build_codebook", "sz_encode", "sz_decode",
    "sz_histogram_sampled_batched",
    "sz_histogram_batched", "sz_build_codebook_batched", "sz_encode_batched", "sz_decode_batched",
    "sz_compress_workspace_bytes", "sz_compress_workspace_bytes_batched", "sz_compress",
    "sz_compress_batched", "SzCompressOptions", "compress_options", "sz_compress_noalloc",
    "SZ_NOALLOC_MAX_ELEMENTS", "SZ_NOALLOC_SCRATCH_BYTES",
    "sz_status_string", "check", "pointer_table", "library_path",
    "lc_max_compressed_bytes", "lc_encode_workspace_bytes", "lc_encode_workspace_bytes_batched",
    "lc_encode", "lc_decode", "lc_encode_batched", "lc_decode_batched",
]

SZ_DTYPE_BF16 = 1
SZ_DTYPE_FP8_E5M2 = 2
SZ_OK = 0
SZ_ERR_INVALID_ARGUMENT = 1
SZ_ERR_BUFFER_TOO_SMALL = 2
SZ_ERR_CORRUPT_STREAM = 3
SZ_ERR_HIP = 4
SZ_ERR_TIMEOUT = 5
SZ_NOALLOC_MAX_ELEMENTS = 1 << 24                  # include/splitzip.h
SZ_NOALLOC_SCRATCH_BYTES = (16 << 20) + (64 << 10)
SZ_ABI_VERSION = 4                                 # include/splitzip.h: the signatures below are for it

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsplitzip.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run `python fp8_kv_cache_amd/build.py`")

_lib = ctypes.CDLL(_LIB_PATH)
_u64, _u32, _i32, _vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p

_SIGNATURES = {
    "sz_max_compressed_bytes": (_u64, [_u64, _i32]),
    "sz_encode_workspace_bytes": (_u64, [_u64, _i32]),
    "sz_encode_workspace_bytes_batched": (_u64, [_u32, _u64, _i32]),
    "sz_histogram": (_i32, [_vp, _u64, _i32, _vp, _vp]),
    "sz_histogram_sampled": (_i32, [_vp, _u64, _i32, _u32, _vp, _vp]),
    "sz_histogram_sampled_batched": (_i32, [_vp, _u32, _u64, _i32, _u32, _vp, _vp]),
    "sz_build_codebook": (_i32, [_vp, _i32, _vp, _vp]),
    "sz_encode": (_i32, [_vp, _u64, _i32, _vp, _vp, _u64, _vp, _vp, _u64, _vp]),
    "sz_decode": (_i32, [_vp, _u64, _u64, _i32, _vp, _vp, _vp]),
    "sz_histogram_batched": (_i32, [_vp, _u32, _u64, _i32, _vp, _vp]),
    "sz_build_codebook_batched": (_i32, [_vp, _u32, _i32, _vp, _vp]),
    "sz_encode_batched": (_i32, [_vp, _u32, _u64, _i32, _vp, _vp, _u64, _vp, _vp, _u64, _vp]),
    "sz_decode_batched": (_i32, [_vp, _vp, _u32, _u64, _i32, _vp, _vp, _vp]),
    "sz_compress_workspace_bytes": (_u64, [_u64, _i32]),
    "sz_compress_workspace_bytes_batched": (_u64, [_u32, _u64, _i32]),
    "sz_compress": (_i32, [_vp, _u64, _i32, _vp, _vp, _vp, _u64, _vp, _vp, _vp, _u64, _vp, _vp]),
    "sz_compress_batched": (_i32, [_vp, _u32, _u64, _i32, _vp, _vp, _vp, _u64, _vp, _vp, _vp, _u64, _vp, _vp]),
    "sz_compress_noalloc": (_i32, [_vp, _u64, _i32, _vp, _vp, _vp, _u64, _vp, _vp, _vp, _vp]),
    "sz_status_string": (ctypes.c_char_p, [_i32]),
    "sz_abi_version": (_u32, []),
    "lc_max_compressed_bytes": (_u64, [_u64]),
    "lc_encode_workspace_bytes": (_u64, [_u64]),
    "lc_encode_workspace_bytes_batched": (_u64, [_u32, _u64]),
    "lc_encode": (_i32, [_vp, _u64, _vp, _u64, _vp, _vp, _u64, _vp]),
    "lc_decode": (_i32, [_vp, _u64, _u64, _vp, _vp, _vp]),
    "lc_encode_batched": (_i32, [_vp, _u32, _u64, _vp, _u64, _vp, _vp, _u64, _vp]),
    "lc_decode_batched": (_i32, [_vp, _vp, _u32, _u64, _vp, _vp, _vp]),
}
if not hasattr(_lib, "sz_abi_version"):
    raise ImportError(f"{_LIB_PATH} predates the ABI version check; rebuild it")
_lib.sz_abi_version.restype = _u32
if _lib.sz_abi_version() != SZ_ABI_VERSION:
    # a library from another revision: its signatures may not be the ones below
    raise ImportError(f"{_LIB_PATH} has ABI version {_lib.sz_abi_version()}, this binding wants "
                      f"{SZ_ABI_VERSION}; rebuild it")
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class SzError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {sz_status_string(status)} ({status})" if what else sz_status_string(status))


def library_path():
    return _LIB_PATH


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def check(status, what=""):
    """Raise SzError unless status is SZ_OK; returns status."""
    if status != SZ_OK:
        raise SzError(status, what)
    return status


def pointer_table(tensors, device=None):
    """Device int64 tensor holding the data pointers of `tensors`, for the
    batched calls' pointer-table arguments."""
    device = device or tensors[0].device
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=device)


def sz_status_string(status):
    return _lib.sz_status_string(status).decode()


def sz_max_compressed_bytes(n, dtype):
    return _lib.sz_max_compressed_bytes(n, dtype)


def sz_encode_workspace_bytes(n, dtype):
    return _lib.sz_encode_workspace_bytes(n, dtype)


def sz_encode_workspace_bytes_batched(count, n, dtype):
    return _lib.sz_encode_workspace_bytes_batched(count, n, dtype)


def sz_histogram(src, n, dtype, hist, stream=None):
    return _lib.sz_histogram(_ptr(src), n, dtype, _ptr(hist), _stream(stream))


def sz_histogram_sampled(src, n, dtype, block_stride, hist, stream=None):
    return _lib.sz_histogram_sampled(_ptr(src), n, dtype, block_stride, _ptr(hist), _stream(stream))


def sz_histogram_sampled_batched(srcs, count, n, dtype, block_stride, hists, stream=None):
    return _lib.sz_histogram_sampled_batched(_ptr(srcs), count, n, dtype, block_stride, _ptr(hists),
                                             _stream(stream))


def sz_build_codebook(hist, dtype, codebook, stream=None):
    return _lib.sz_build_codebook(_ptr(hist), dtype, _ptr(codebook), _stream(stream))


def sz_encode(src, n, dtype, codebook, dst, dst_capacity, out_bytes, workspace, workspace_bytes,
              stream=None):
    return _lib.sz_encode(_ptr(src), n, dtype, _ptr(codebook), _ptr(dst), dst_capacity,
                          _ptr(out_bytes), _ptr(workspace), workspace_bytes, _stream(stream))


def sz_decode(src, src_bytes, n, dtype, dst, status=None, stream=None):
    return _lib.sz_decode(_ptr(src), src_bytes, n, dtype, _ptr(dst), _ptr(status), _stream(stream))


def sz_histogram_batched(srcs, count, n, dtype, hists, stream=None):
    return _lib.sz_histogram_batched(_ptr(srcs), count, n, dtype, _ptr(hists), _stream(stream))


def sz_build_codebook_batched(hists, count, dtype, codebooks, stream=None):
    return _lib.sz_build_codebook_batched(_ptr(hists), count, dtype, _ptr(codebooks), _stream(stream))


def sz_encode_batched(srcs, count, n, dtype, codebooks, dsts, dst_capacity, out_bytes, workspace,
                      workspace_bytes, stream=None):
    return _lib.sz_encode_batched(_ptr(srcs), count, n, dtype, _ptr(codebooks), _ptr(dsts),
                                  dst_capacity, _ptr(out_bytes), _ptr(workspace), workspace_bytes,
                                  _stream(stream))


def sz_decode_batched(srcs, src_bytes, count, n, dtype, dsts, status=None, stream=None):
    return _lib.sz_decode_batched(_ptr(srcs), _ptr(src_bytes), count, n, dtype, _ptr(dsts),
                                  _ptr(status), _stream(stream))


def sz_compress_workspace_bytes(n, dtype):
    return _lib.sz_compress_workspace_bytes(n, dtype)


def sz_compress_workspace_bytes_batched(count, n, dtype):
    return _lib.sz_compress_workspace_bytes_batched(count, n, dtype)


class SzCompressOptions(ctypes.Structure):
    """sz_compress_options: per-call settings of sz_compress[_batched]
    (0 in a field means its default)."""
    _fields_ = [("fused_min_elements", ctypes.c_uint64), ("spin_limit", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


def compress_options(fused_min_elements=0, spin_limit=0):
    """An SzCompressOptions, or None (the defaults) when every field is 0."""
    if not fused_min_elements and not spin_limit:
        return None
    return SzCompressOptions(fused_min_elements, spin_limit, 0)


def _opts(o):
    return None if o is None else ctypes.addressof(o)


def sz_compress(src, n, dtype, hist, codebook, dst, dst_capacity, out_bytes, status, workspace,
                workspace_bytes, options=None, stream=None):
    return _lib.sz_compress(_ptr(src), n, dtype, _ptr(hist), _ptr(codebook), _ptr(dst), dst_capacity,
                            _ptr(out_bytes), _ptr(status), _ptr(workspace), workspace_bytes, _opts(options),
                            _stream(stream))


def sz_compress_noalloc(src, n, dtype, hist, codebook, dst, dst_capacity, out_bytes, status, options=None,
                        stream=None):
    return _lib.sz_compress_noalloc(_ptr(src), n, dtype, _ptr(hist), _ptr(codebook), _ptr(dst), dst_capacity,
                                    _ptr(out_bytes), _ptr(status), _opts(options), _stream(stream))


def sz_compress_batched(srcs, count, n, dtype, hists, codebooks, dsts, dst_capacity, out_bytes, status,
                        workspace, workspace_bytes, options=None, stream=None):
    return _lib.sz_compress_batched(_ptr(srcs), count, n, dtype, _ptr(hists), _ptr(codebooks), _ptr(dsts),
                                    dst_capacity, _ptr(out_bytes), _ptr(status), _ptr(workspace),
                                    workspace_bytes, _opts(options), _stream(stream))


def lc_max_compressed_bytes(n):
    return _lib.lc_max_compressed_bytes(n)


def lc_encode_workspace_bytes(n):
    return _lib.lc_encode_workspace_bytes(n)


def lc_encode_workspace_bytes_batched(count, n):
    return _lib.lc_encode_workspace_bytes_batched(count, n)


def lc_encode(src, n, dst, dst_capacity, out_bytes, workspace, workspace_bytes, stream=None):
    return _lib.lc_encode(_ptr(src), n, _ptr(dst), dst_capacity, _ptr(out_bytes), _ptr(workspace),
                          workspace_bytes, _stream(stream))


def lc_decode(src, src_bytes, n, dst, status=None, stream=None):
    return _lib.lc_decode(_ptr(src), src_bytes, n, _ptr(dst), _ptr(status), _stream(stream))


def lc_encode_batched(srcs, count, n, dsts, dst_capacity, out_bytes, workspace, workspace_bytes, stream=None):
    return _lib.lc_encode_batched(_ptr(srcs), count, n, _ptr(dsts), dst_capacity, _ptr(out_bytes),
                                  _ptr(workspace), workspace_bytes, _stream(stream))


def lc_decode_batched(srcs, src_bytes, count, n, dsts, status=None, stream=None):
    return _lib.lc_decode_batched(_ptr(srcs), _ptr(src_bytes), count, n, _ptr(dsts), _ptr(status),
                                  _stream(stream))
