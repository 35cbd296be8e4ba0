"""Both CPU oracles built with AddressSanitizer and UBSan (gcc, host code
only) and driven by tests/oracle_sanitize.c: round trips over many lengths,
and decodes of streams with a flipped byte or cut short, touch nothing
outside their buffers and hit no undefined behaviour."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracles_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "oracle_sanitize"
    srcs = [os.path.join(ROOT, "tests", "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "sz_oracle.c"),
            os.path.join(ROOT, "oracle", "lc_oracle.c")]
    sanitize = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    build = subprocess.run(["gcc", "-O1", "-g", "-std=c11", *sanitize, *srcs, "-o", str(exe)],
                           capture_output=True, text=True)
    if build.returncode and "asan" in build.stderr.lower():
        pytest.skip("sanitizer runtime unavailable: " + build.stderr[:200])
    assert build.returncode == 0, build.stderr
    # the environment is passed on unchanged; ASan only relaxes its own
    # check that its runtime comes first among loaded libraries
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout[-2000:] + run.stderr[-4000:]
