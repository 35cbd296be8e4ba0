"""The C-ABI library loads and exports every symbol that include/*.h
declares; host-side argument checks and size functions (no GPU needed: none
of these calls reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


@pytest.fixture(scope="module")
def sz():
    import fp8_kv_cache_amd
    return fp8_kv_cache_amd


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:sz|lc)_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_codec_calls():
    names = declared_functions()
    for want in ("sz_histogram", "sz_build_codebook", "sz_encode", "sz_decode",
                 "sz_max_compressed_bytes", "lc_encode", "lc_decode", "lc_encode_batched",
                 "lc_decode_batched", "lc_max_compressed_bytes"):
        assert want in names


def test_library_exports_every_declared_symbol(sz):
    lib = ctypes.CDLL(sz.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", sz.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared_functions()) <= exported
    # nothing else of ours leaks out of the library
    assert all(not s.startswith(("sz_", "lc_")) or s in declared_functions() for s in exported)


def test_abi_version_matches_header_and_binding(sz):
    """The library reports the header's SZ_ABI_VERSION and the binding was
    written for that version (it refuses to load any other)."""
    text = open(os.path.join(ROOT, "include", "splitzip.h")).read()
    want = int(re.search(r"#define SZ_ABI_VERSION (\d+)u", text).group(1))
    lib = ctypes.CDLL(sz.library_path())
    lib.sz_abi_version.restype = ctypes.c_uint32
    assert lib.sz_abi_version() == want == sz.SZ_ABI_VERSION


def test_library_contains_no_cpu_codec_path(sz):
    """The product library links neither the oracle nor any CPU codec."""
    out = subprocess.run(["nm", "-D", sz.library_path()], capture_output=True, text=True).stdout
    assert "szo_" not in out and "lco_" not in out


@pytest.mark.parametrize("dt", [1, 2])
@pytest.mark.parametrize("n", [0, 1, 2, 3, 511, 4095, 4096, 4097, 1 << 20, (1 << 23) + 17, (1 << 32) - 1])
def test_max_bytes_matches_oracle(sz, dt, n):
    assert sz.sz_max_compressed_bytes(n, dt) == oracle.max_bytes(n, dt)


def test_max_bytes_rejects_bad_input(sz):
    assert sz.sz_max_compressed_bytes(1 << 32, 1) == 0
    assert sz.sz_max_compressed_bytes(10, 0) == 0
    assert sz.sz_max_compressed_bytes(10, 3) == 0


def test_workspace_bytes(sz):
    # a u32 count per 4096-element block, padded to 256 bytes, then 4096 staging bytes per block
    assert sz.sz_encode_workspace_bytes(0, 1) == 0
    assert sz.sz_encode_workspace_bytes(4096, 1) == 256 + 4096
    assert sz.sz_encode_workspace_bytes(4097, 2) == 256 + 2 * 4096
    assert sz.sz_encode_workspace_bytes_batched(64, 1 << 23, 1) == 4 * 64 * 2048 + 64 * 2048 * 4096
    assert sz.sz_encode_workspace_bytes_batched(0, 100, 1) == 0
    assert sz.sz_encode_workspace_bytes(1 << 32, 1) == 0
    # a batch the calls would reject for its size gets 0, not a wrapped size
    assert sz.sz_encode_workspace_bytes_batched(1 << 31, 4096, 1) == 0
    assert sz.sz_encode_workspace_bytes_batched(0xFFFFFFFF, (1 << 32) - 1, 1) == 0
    assert sz.sz_compress_workspace_bytes_batched(0xFFFFFFFF, (1 << 32) - 1, 1) == 0
    assert sz.lc_encode_workspace_bytes_batched(0xFFFFFFFF, (1 << 31) - 1) == 0


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced: every call below fails its host check


def test_host_argument_errors_return_before_launch(sz):
    E_ARG, E_SMALL, E_CORRUPT = sz.SZ_ERR_INVALID_ARGUMENT, sz.SZ_ERR_BUFFER_TOO_SMALL, sz.SZ_ERR_CORRUPT_STREAM
    # histogram: null / misaligned / bad dtype / too many elements
    assert sz.sz_histogram(None, 10, 1, FAKE, stream=0) == E_ARG
    assert sz.sz_histogram(FAKE, 10, 1, None, stream=0) == E_ARG
    assert sz.sz_histogram(FAKE + 1, 10, 1, FAKE, stream=0) == E_ARG
    assert sz.sz_histogram(FAKE, 10, 7, FAKE, stream=0) == E_ARG
    assert sz.sz_histogram(FAKE, 1 << 32, 1, FAKE, stream=0) == E_ARG
    assert sz.sz_histogram_sampled(FAKE, 10, 1, 0, FAKE, stream=0) == E_ARG      # stride 0
    assert sz.sz_histogram_sampled(FAKE, 10, 3, 4, FAKE, stream=0) == E_ARG
    assert sz.sz_histogram_sampled_batched(FAKE, 2, 10, 1, 0, FAKE, stream=0) == E_ARG
    assert sz.sz_build_codebook(None, 1, FAKE, stream=0) == E_ARG
    assert sz.sz_build_codebook(FAKE, 5, FAKE, stream=0) == E_ARG
    # encode: capacity and workspace below the bound
    cap = sz.sz_max_compressed_bytes(5000, 1)
    ws = sz.sz_encode_workspace_bytes(5000, 1)
    assert sz.sz_encode(FAKE, 5000, 1, FAKE, FAKE, cap - 1, None, FAKE, ws, stream=0) == E_SMALL
    assert sz.sz_encode(FAKE, 5000, 1, FAKE, FAKE, cap, None, FAKE, ws - 1, stream=0) == E_SMALL
    assert sz.sz_encode(FAKE, 5000, 1, FAKE, FAKE, cap, None, None, ws, stream=0) == E_ARG
    assert sz.sz_encode(FAKE, 5000, 1, None, FAKE, cap, None, FAKE, ws, stream=0) == E_ARG
    assert sz.sz_encode(FAKE, 5000, 1, FAKE, FAKE, cap, FAKE + 4, FAKE, ws, stream=0) == E_ARG
    # decode: a buffer smaller than any stream of n elements
    assert sz.sz_decode(FAKE, 100, 5000, 1, FAKE, None, stream=0) == E_CORRUPT
    assert sz.sz_decode(None, 100000, 5000, 1, FAKE, None, stream=0) == E_ARG
    assert sz.sz_decode(FAKE, 100000, 5000, 1, FAKE, FAKE + 2, stream=0) == E_ARG
    # batched forms
    assert sz.sz_histogram_batched(FAKE, 0, 10, 1, FAKE, stream=0) == E_ARG
    assert sz.sz_encode_batched(FAKE, 2, 5000, 1, FAKE, FAKE, cap, None, FAKE,
                                sz.sz_encode_workspace_bytes(5000, 1), stream=0) == E_SMALL
    assert sz.sz_decode_batched(FAKE, None, 2, 5000, 1, FAKE, None, stream=0) == E_ARG


def test_compress_sizes_and_host_errors(sz):
    """Single-pass calls: workspace = the encode workspace plus, per tensor,
    R copies of a 2048-byte whole-tensor histogram (R = 16, 8, 4, 2, 1 for
    1, 2-3, 4-7, 8-15, 16+ tensors) and a 2048-byte sample histogram, then
    256 bytes of counters, a 128-byte record per tensor and three 64-byte
    list entries per tensor; argument errors return before any launch."""
    for count, n in [(1, 0), (1, 4097), (64, 1 << 23), (3, 100), (2, 5000), (7, 5000), (8, 5000), (15, 5000),
                     (16, 5000)]:
        copies = 1 if count >= 16 else 2 if count >= 8 else 4 if count >= 4 else 8 if count >= 2 else 16
        sync = 2048 * count * (copies + 1) + 256 + 128 * count + 3 * 64 * count
        assert sz.sz_compress_workspace_bytes_batched(count, n, 1) == \
            sz.sz_encode_workspace_bytes_batched(count, n, 1) + sync
    assert sz.sz_compress_workspace_bytes(1 << 32, 1) == 0
    assert sz.sz_compress_workspace_bytes_batched(0, 10, 1) == 0
    E_ARG, E_SMALL = sz.SZ_ERR_INVALID_ARGUMENT, sz.SZ_ERR_BUFFER_TOO_SMALL
    n = 5000
    cap = sz.sz_max_compressed_bytes(n, 2)
    ws = sz.sz_compress_workspace_bytes(n, 2)
    ok = dict(src=FAKE, n=n, dtype=2, hist=FAKE, codebook=FAKE, dst=FAKE, dst_capacity=cap, out_bytes=None,
              status=None, workspace=FAKE, workspace_bytes=ws)

    def call(**kw):
        args = dict(ok, **kw)
        return sz.sz_compress(*args.values(), stream=0)
    assert call(dtype=3) == E_ARG
    assert call(n=1 << 32) == E_ARG
    assert call(src=None) == E_ARG
    assert call(hist=None) == E_ARG
    assert call(codebook=FAKE + 8) == E_ARG
    assert call(workspace=None) == E_ARG
    assert call(out_bytes=FAKE + 4) == E_ARG
    assert call(status=FAKE + 2) == E_ARG
    assert call(dst_capacity=cap - 1) == E_SMALL
    assert call(workspace_bytes=ws - 1) == E_SMALL
    assert sz.sz_compress_batched(FAKE, 0, n, 2, FAKE, FAKE, FAKE, cap, None, None, FAKE, ws, stream=0) == E_ARG
    assert sz.sz_compress_batched(FAKE, 2, n, 2, FAKE, FAKE, FAKE, cap, None, None, FAKE, ws, stream=0) == E_SMALL
    assert sz.sz_compress_batched(FAKE, 2048, (1 << 32) - 1, 1, FAKE, FAKE, FAKE, 1 << 40, None, None, FAKE,
                                  1 << 62, stream=0) == E_ARG
    # tiny tensors: four work items each (sample, provisional codebook, main,
    # final codebook) -- 2^30 of them would overflow the grid
    cap1 = sz.sz_max_compressed_bytes(1, 1)
    assert sz.sz_compress_batched(FAKE, 1 << 30, 1, 1, FAKE, FAKE, FAKE, cap1, None, None, FAKE, 1 << 62,
                                  stream=0) == E_ARG


def test_compress_options_are_per_call(sz):
    """The one-launch compress takes its settings per call: NULL or zero
    fields mean the defaults, a non-zero reserved field is an argument error
    returned before any launch, and the library keeps no process-wide
    setting (the old setters are not exported)."""
    n = 5000
    cap = sz.sz_max_compressed_bytes(n, 1)
    ws = sz.sz_compress_workspace_bytes(n, 1)
    bad = sz.SzCompressOptions(1, 1, 7)
    args = (FAKE, n, 1, FAKE, FAKE, FAKE, cap, None, None, FAKE, ws)
    assert sz.sz_compress(*args, options=bad, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.sz_compress_batched(FAKE, 2, n, 1, FAKE, FAKE, FAKE, cap, None, None, FAKE,
                                  sz.sz_compress_workspace_bytes_batched(2, n, 1), options=bad,
                                  stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.compress_options() is None
    o = sz.compress_options(fused_min_elements=1, spin_limit=3)
    assert (o.fused_min_elements, o.spin_limit, o.reserved) == (1, 3, 0)
    lib = ctypes.CDLL(sz.library_path())
    for gone in ("sz_compress_spin_limit", "sz_compress_fused_min_elements"):
        assert not hasattr(lib, gone), gone


def test_status_strings(sz):
    assert sz.sz_status_string(0) == "ok"
    assert sz.sz_status_string(3) == "corrupt stream"
    assert sz.sz_status_string(5) == "gave up waiting for the codebook"
    assert sz.sz_status_string(99) == "unknown status"


@pytest.mark.parametrize("n", [0, 1, 15, 16, 16383, 16384, 16385, 100000, (1 << 31) - 1])
def test_lc_max_bytes_matches_oracle(sz, n):
    assert sz.lc_max_compressed_bytes(n) == oracle.lc_max_bytes(n)


def test_lc_sizes_and_host_errors(sz):
    assert sz.lc_max_compressed_bytes(1 << 31) == 0
    assert sz.lc_encode_workspace_bytes(0) == 0
    assert sz.lc_encode_workspace_bytes(16385) == 256
    assert sz.lc_encode_workspace_bytes_batched(64, 1 << 24) == 64 * 1024 * 4
    fake = 1 << 20                     # aligned, never dereferenced: every call fails on the host
    n = 40000
    cap = sz.lc_max_compressed_bytes(n)
    ws = sz.lc_encode_workspace_bytes(n)
    assert sz.lc_encode(fake, 1 << 31, fake, cap, None, fake, ws, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.lc_encode(fake + 8, n, fake, cap, None, fake, ws, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.lc_encode(fake, n, fake, cap - 1, None, fake, ws, stream=0) == sz.SZ_ERR_BUFFER_TOO_SMALL
    assert sz.lc_encode(fake, n, fake, cap, None, fake, ws - 1, stream=0) == sz.SZ_ERR_BUFFER_TOO_SMALL
    assert sz.lc_encode(fake, n, fake, cap, None, None, ws, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.lc_encode(fake, n, fake, cap, fake + 4, fake, ws, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.lc_decode(fake, 255, n, fake, stream=0) == sz.SZ_ERR_CORRUPT_STREAM
    assert sz.lc_decode(None, cap, n, fake, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.lc_decode(fake, cap, n, fake, fake + 2, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.lc_encode_batched(fake, 0, n, fake, cap, None, fake, ws, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.lc_encode_batched(fake, 100, n, fake, cap, None, fake, ws, stream=0) == sz.SZ_ERR_BUFFER_TOO_SMALL
    assert sz.lc_decode_batched(fake, fake, 0, n, fake, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.lc_decode_batched(fake, None, 1, n, fake, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT


def test_batched_grid_limit(sz):
    """count x ceil(n/4096) must stay below 2^31 (one workgroup per block at most)."""
    n = (1 << 32) - 1                       # 2^20 blocks per tensor
    assert sz.sz_histogram_batched(FAKE, 2048, n, 1, FAKE, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
    assert sz.sz_decode_batched(FAKE, FAKE, 2048, n, 1, FAKE, stream=0) == sz.SZ_ERR_INVALID_ARGUMENT
