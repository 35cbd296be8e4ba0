"""The library's host entry points (api.cpp, lc_api.cpp) built with
AddressSanitizer, UBSan and the unsigned-overflow check on the host side
only, driven by tests/api_sanitize.cpp with stub kernel launchers: every
argument error of every entry point returns its documented status before
any launch, valid calls reach a launcher, the size queries hold over the
edges of their domains, and enum arguments outside the enumerators (any int
a C caller passes) are rejected without being read as enums.  No GPU is
used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_kv_cache_amd", "csrc")


def test_host_entry_points_under_asan_and_ubsan(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = tmp_path / "api_sanitize"
    # host-only instrumentation: every sanitizer flag goes to the host compile
    host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fsanitize=unsigned-integer-overflow", "-Xarch_host", "-fno-sanitize-recover=all"]
    cmd = [hipcc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", *host, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "lc_api.cpp"),
           os.path.join(ROOT, "tests", "api_sanitize.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if build.returncode and "asan" in build.stderr.lower() and "not found" in build.stderr.lower():
        pytest.skip("sanitizer runtime unavailable: " + build.stderr[:200])
    assert build.returncode == 0, build.stderr[-4000:]
    # the HIP runtime's own allocations outlive main, so leak reports are off;
    # ASan only relaxes its check that its runtime comes first among libraries
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout[-3000:] + run.stderr[-4000:]
