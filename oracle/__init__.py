"""CPU oracle of the SplitZip-style exponent codec (format v1).

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
CPU-baseline leg of `bench.py` may import this package.  The GPU library and
its Python binding never import it, and it imports nothing from them.

Two independent implementations of the same stream format live here:
  * `sz_oracle.c` -- plain scalar C, loaded through ctypes (`encode`,
    `decode`, `histogram`, `codebook`, `max_bytes`, `exact_bytes` below);
  * `sz_ref.py`   -- pure Python, for tiny inputs and cross-checks.
The format and every reading taken where the SplitZip project page is silent
are written out in the header comment of `sz_oracle.c`.
"""
import ctypes
import os
import subprocess

import numpy as np

BF16 = 1
E5M2 = 2
OK, INVALID_ARGUMENT, BUFFER_TOO_SMALL, CORRUPT_STREAM = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sz_oracle.c")
_LIB = os.path.join(_HERE, "libszoracle.so")
_lib = None
_LC_SRC = os.path.join(_HERE, "lc_oracle.c")
_LC_LIB = os.path.join(_HERE, "liblcoracle.so")
_lc = None


def _compile(src, lib):
    tmp = lib + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                           "-o", tmp, src])
    os.replace(tmp, lib)


def build():
    """Compile the C oracles with gcc -O2 (plain scalar code, no intrinsics)."""
    _compile(_SRC, _LIB)
    _compile(_LC_SRC, _LC_LIB)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        _compile(_SRC, _LIB)
    lib = ctypes.CDLL(_LIB)
    u64, i32, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
    lib.szo_max_bytes.argtypes = [u64, i32]
    lib.szo_max_bytes.restype = u64
    lib.szo_exact_bytes.argtypes = [u64, i32, u64]
    lib.szo_exact_bytes.restype = u64
    lib.szo_histogram.argtypes = [vp, u64, i32, vp]
    lib.szo_histogram.restype = i32
    lib.szo_histogram_sampled.argtypes = [vp, u64, i32, u64, vp]
    lib.szo_histogram_sampled.restype = i32
    lib.szo_codebook.argtypes = [vp, i32, vp]
    lib.szo_codebook.restype = i32
    lib.szo_encode.argtypes = [vp, u64, i32, vp, vp, u64, vp]
    lib.szo_encode.restype = i32
    lib.szo_decode.argtypes = [vp, u64, u64, i32, vp]
    lib.szo_decode.restype = i32
    _lib = lib
    return lib


def _raw(values, dt):
    a = np.ascontiguousarray(values)
    want = np.uint16 if dt == BF16 else np.uint8
    if a.dtype != want:
        a = a.view(want) if a.dtype.itemsize == np.dtype(want).itemsize else a.astype(want)
    return np.ascontiguousarray(a.reshape(-1))


def max_bytes(n, dt):
    return int(_load().szo_max_bytes(n, dt))


def exact_bytes(n, dt, escapes):
    return int(_load().szo_exact_bytes(n, dt, escapes))


def histogram(values, dt):
    a = _raw(values, dt)
    h = np.zeros(256, np.uint64)
    rc = _load().szo_histogram(a.ctypes.data, a.size, dt, h.ctypes.data)
    if rc:
        raise ValueError(f"szo_histogram failed: {rc}")
    return h


def histogram_sampled(values, dt, stride):
    """Histogram of the 4096-element blocks b with b % stride == 0."""
    a = _raw(values, dt)
    h = np.zeros(256, np.uint64)
    rc = _load().szo_histogram_sampled(a.ctypes.data if a.size else None, a.size, dt, stride, h.ctypes.data)
    if rc:
        raise ValueError(f"szo_histogram_sampled failed: {rc}")
    return h


def codebook(hist, dt):
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    cb = np.zeros(16, np.uint8)
    rc = _load().szo_codebook(h.ctypes.data, dt, cb.ctypes.data)
    if rc:
        raise ValueError(f"szo_codebook failed: {rc}")
    return cb


def encode(values, dt, cb=None):
    """Encode raw elements (uint16 BF16 bit patterns or uint8 E5M2 bytes);
    returns the stream as a numpy uint8 array of exactly C bytes."""
    a = _raw(values, dt)
    cap = max_bytes(a.size, dt)
    out = np.zeros(max(cap, 1), np.uint8)
    nbytes = ctypes.c_uint64(0)
    cbp = None
    if cb is not None:
        if isinstance(cb, (bytes, bytearray)):
            cb = np.frombuffer(bytes(cb), np.uint8)
        cbv = np.ascontiguousarray(cb, dtype=np.uint8)
        assert cbv.size == 16
        cbp = cbv.ctypes.data
    rc = _load().szo_encode(a.ctypes.data if a.size else None, a.size, dt, cbp,
                            out.ctypes.data, cap, ctypes.byref(nbytes))
    if rc:
        raise ValueError(f"szo_encode failed: {rc}")
    return out[:nbytes.value].copy()


def decode(stream, n, dt):
    """Returns (status, raw elements or None)."""
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    out = np.zeros(max(n, 1), np.uint16 if dt == BF16 else np.uint8)
    rc = _load().szo_decode(s.ctypes.data if s.size else None, s.size, n, dt, out.ctypes.data)
    if rc != OK:
        return rc, None
    return OK, out[:n]


def stream_fields(stream):
    """Header fields of a stream (for tests and reports)."""
    s = bytes(np.ascontiguousarray(stream, dtype=np.uint8)[:64])
    return {
        "magic": s[0:4], "version": s[4], "dtype": s[5], "log2_block": s[6], "ncodes": s[7],
        "n": int.from_bytes(s[8:16], "little"), "escapes": int.from_bytes(s[16:24], "little"),
        "codebook": list(s[24:40]), "bytes": int.from_bytes(s[40:48], "little"),
    }


# ---- LC-style comparison codec (lc_oracle.c) -------------------------------

def _load_lc():
    global _lc
    if _lc is not None:
        return _lc
    if not os.path.exists(_LC_LIB) or os.path.getmtime(_LC_LIB) < os.path.getmtime(_LC_SRC):
        _compile(_LC_SRC, _LC_LIB)
    lib = ctypes.CDLL(_LC_LIB)
    u64, i32, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
    for name in ("lco_tupl8_1", "lco_untupl8_1", "lco_bit8", "lco_unbit8"):
        getattr(lib, name).argtypes = [vp, u64, vp]
        getattr(lib, name).restype = None
    lib.lco_rze2.argtypes = [vp, u64, vp]
    lib.lco_rze2.restype = u64
    lib.lco_unrze2.argtypes = [vp, u64, u64, vp]
    lib.lco_unrze2.restype = i32
    lib.lco_max_bytes.argtypes = [u64]
    lib.lco_max_bytes.restype = u64
    lib.lco_encode.argtypes = [vp, u64, vp, u64, vp]
    lib.lco_encode.restype = i32
    lib.lco_decode.argtypes = [vp, u64, u64, vp]
    lib.lco_decode.restype = i32
    _lc = lib
    return lib


def _bytes_of(values):
    a = np.ascontiguousarray(values)
    return np.ascontiguousarray(a.reshape(-1).view(np.uint8))


def _stage(name, data):
    a = _bytes_of(data)
    out = np.zeros(max(a.size, 1), np.uint8)
    getattr(_load_lc(), name)(a.ctypes.data if a.size else None, a.size, out.ctypes.data)
    return out[:a.size]


def lc_tupl8_1(data):
    return _stage("lco_tupl8_1", data)


def lc_untupl8_1(data):
    return _stage("lco_untupl8_1", data)


def lc_bit8(data):
    return _stage("lco_bit8", data)


def lc_unbit8(data):
    return _stage("lco_unbit8", data)


def lc_rze2(data):
    a = _bytes_of(data)
    out = np.zeros(a.size + a.size // 16 + 16, np.uint8)
    k = _load_lc().lco_rze2(a.ctypes.data if a.size else None, a.size, out.ctypes.data)
    return out[:k].copy()


def lc_unrze2(payload, length):
    """Inverse of lc_rze2 for a chunk of `length` bytes; None if the payload
    size does not match its bitmap."""
    p = _bytes_of(payload)
    out = np.zeros(max(length, 1), np.uint8)
    rc = _load_lc().lco_unrze2(p.ctypes.data if p.size else None, p.size, length, out.ctypes.data)
    return None if rc else out[:length]


def lc_max_bytes(n):
    return int(_load_lc().lco_max_bytes(n))


def lc_encode(data):
    """LC-style stream of the raw bytes of `data` (any dtype, C order)."""
    a = _bytes_of(data)
    cap = lc_max_bytes(a.size)
    out = np.zeros(max(cap, 1), np.uint8)
    nbytes = ctypes.c_uint64(0)
    rc = _load_lc().lco_encode(a.ctypes.data if a.size else None, a.size, out.ctypes.data, cap,
                               ctypes.byref(nbytes))
    if rc:
        raise ValueError(f"lco_encode failed: {rc}")
    return out[:nbytes.value].copy()


def lc_decode(stream, n):
    """Returns (status, n raw bytes or None)."""
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    out = np.zeros(max(n, 1), np.uint8)
    rc = _load_lc().lco_decode(s.ctypes.data if s.size else None, s.size, n, out.ctypes.data)
    if rc != OK:
        return rc, None
    return OK, out[:n]
