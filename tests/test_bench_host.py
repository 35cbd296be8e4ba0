"""Host-side parts of bench.py, on the CPU: the one-GPU guard, the
counter-derived traffic lookup (profiles/traffic.json), which is tied to a
hash of the kernel sources so that counters taken on other kernels are
never reported, and the probe library's argument checks."""
import ctypes
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

ROOFLINE_KERNELS = ["k_zero_two", "k_compress<bf16>", "k_transcode<bf16>", "k_offsets_scatter<bf16>"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_step_counts_are_checked_before_anything_runs():
    for flags in (["--steps", "0"], ["--warmup", "-1"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *flags],
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 2, flags
        assert "--steps >= 1" in r.stderr and r.stdout == ""


def _traffic_file(tmp_path, sha, kernels):
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"kernel_sources_sha256": sha,
                             "kernels": {k: {"hbm_bytes_per_launch": v} for k, v in kernels.items()}}))
    return str(p)


def test_traffic_is_summed_over_the_call_kernels(tmp_path, monkeypatch):
    path = _traffic_file(tmp_path, bench.kernel_source_hash(), {"a": 10.0, "b": 32.5, "c": 1.0})
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    assert bench.traffic_for(["a", "b"]) == 42.5


def test_traffic_is_null_for_other_sources_a_missing_kernel_or_no_file(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _traffic_file(tmp_path, "0" * 64, {"a": 10.0}))
    assert bench.traffic_for(["a"]) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _traffic_file(tmp_path, bench.kernel_source_hash(), {"a": 10.0}))
    assert bench.traffic_for(["a", "b"]) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.traffic_for(["a"]) is None


def test_source_hash_changes_with_every_kernel_source(tmp_path, monkeypatch):
    copies = []
    for src in bench.KERNEL_SOURCES:
        dst = tmp_path / os.path.basename(src)
        shutil.copyfile(src, dst)
        copies.append(str(dst))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", copies)
    base = bench.kernel_source_hash()
    assert base == bench.kernel_source_hash()
    for path in copies:
        with open(path, "a") as f:   # a comment and blank lines leave the code, and the hash, as they were
            f.write("\n// a comment\n/* another */\n\n")
        assert bench.kernel_source_hash() == base
        with open(path, "a") as f:
            f.write("int one_more_declaration;\n")
        changed = bench.kernel_source_hash()
        assert changed != base
        base = changed


def test_code_only_strips_comments_but_not_literals():
    src = 'int a = 1; // c\n/* b\n c */ const char* s = "x // y /* z"; char q = \'"\';\n   int   b;'
    assert bench.code_only(src) == 'int a = 1; const char* s = "x // y /* z"; char q = \'"\'; int b;'


def test_committed_traffic_covers_the_roofline_kernels():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert len(rec["kernel_sources_sha256"]) == 64
    for k in ROOFLINE_KERNELS:
        assert rec["kernels"][k]["hbm_bytes_per_launch"] > 0, k


def test_probe_rejects_invalid_arguments_before_any_launch():
    """libszprobe.so's argument checks run on the host, so every call below
    returns -1 without touching a GPU."""
    lib = ctypes.CDLL(bench.PROBE_LIB)
    lib.szp_stream.restype = ctypes.c_int
    lib.szp_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                               ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    a, b = 1 << 20, 2 << 20          # aligned stand-in addresses, never dereferenced
    bad = [
        (None, b, 4096, 4096, 4, 0, 8),        # null source
        (a + 8, b, 4096, 4096, 4, 0, 8),       # misaligned source
        (a, b + 4, 4096, 4096, 4, 0, 8),       # misaligned destination
        (a, b, 4096 + 16, 8192, 4, 0, 8),      # size not a multiple of 64
        (a, b, 0, 4096, 4, 0, 8),              # empty
        (a, b, 4096, 4096, 2, 0, 8),           # unknown mix
        (a, b, 4096, 4096, 4, 0, 0),           # no workgroups
        (a, b, 4096, 4096, 4, 0, 65536),       # too many workgroups
        (a, b, 4096, 4095, 4, 0, 8),           # copy into a smaller buffer
        (a, b, 4096, 3071, 3, 1, 8),           # mix into less than 3/4 of the size
        (a, b, 4096, 8 * 4096 - 1, 0, 0, 8),   # read-only sink below 4 KB per workgroup
    ]
    for args in bad:
        assert lib.szp_stream(*args, None) == -1, args
