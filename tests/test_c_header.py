"""The public headers are plain C: a C99 program that includes both, links
libsplitzip.so and calls the host-side functions (sizes, argument errors,
status strings) builds with gcc and runs without a GPU.  No call here
reaches a kernel launch."""
import os
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "fp8_kv_cache_amd")

PROGRAM = r"""
#include <stdio.h>
#include "splitzip.h"
#include "lc_codec.h"

int main(void) {
    /* exponent codec: worst-case sizes and workspace */
    printf("%llu\n", (unsigned long long)sz_max_compressed_bytes(1u << 20, SZ_DTYPE_BF16));
    printf("%llu\n", (unsigned long long)sz_max_compressed_bytes(4097, SZ_DTYPE_FP8_E5M2));
    printf("%llu\n", (unsigned long long)sz_encode_workspace_bytes(1u << 20, SZ_DTYPE_BF16));
    /* argument errors are returned before any launch */
    printf("%d\n", (int)sz_histogram(NULL, 10, SZ_DTYPE_BF16, NULL, NULL));
    printf("%d\n", (int)sz_encode((const void*)0x100000, 10, (sz_dtype)7, (const uint8_t*)0x100000,
                                  (void*)0x100000, 1u << 20, NULL, (void*)0x100000, 1u << 20, NULL));
    printf("%s\n", sz_status_string(SZ_ERR_CORRUPT_STREAM));
    /* comparison codec */
    printf("%llu\n", (unsigned long long)lc_max_compressed_bytes(100000));
    printf("%d\n", (int)lc_decode((const void*)0x100000, 10, 100000, (void*)0x100000, NULL, NULL));
    return 0;
}
"""


def test_headers_compile_as_c99_and_link(tmp_path):
    import fp8_kv_cache_amd  # noqa: F401  (the library is built)
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    # outside hipcc, ROCm's runtime header needs the platform named on the command line
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", str(src), "-o", str(exe), "-L", LIBDIR, "-lsplitzip",
           f"-Wl,-rpath,{LIBDIR}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode and "hip_runtime_api.h" in r.stderr:
        pytest.skip("HIP headers not usable from plain C here: " + r.stderr[:200])
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines()
    assert int(out[0]) == oracle.max_bytes(1 << 20, 1)
    assert int(out[1]) == oracle.max_bytes(4097, 2)
    assert int(out[2]) > 0
    assert int(out[3]) == 1 and int(out[4]) == 1            # SZ_ERR_INVALID_ARGUMENT
    assert out[5] == "corrupt stream"
    assert int(out[6]) == oracle.lc_max_bytes(100000)
    assert int(out[7]) == 3                                 # too short for any stream of n bytes
