"""Build libsplitzip.so (gfx950) in-tree with hipcc, and libszprobe.so, the
HBM streaming-rate probes the benchmark measures its ceilings with.

    python fp8_kv_cache_amd/build.py

(run as a file: importing the package would load the library being rebuilt)
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsplitzip.so")
SOURCES = [os.path.join(CSRC, f) for f in ("kernels.hip", "api.cpp", "lc_kernels.hip", "lc_api.cpp")]
PROBE_LIB = os.path.join(HERE, "libszprobe.so")
PROBE_SOURCES = [os.path.join(CSRC, "probe.hip")]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return [
        "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        f"--offload-arch={ARCH}",
        # packed FP32 instructions are disabled for every device compile
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def build(verbose=False):
    """Compile every source (device code for gfx950 only) and link both
    shared libraries next to this file.  Returns the codec library's path."""
    _link(SOURCES, LIB, verbose)
    _link(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def _link(sources, lib, verbose):
    cc = hipcc()
    objs = []
    tmpdir = os.path.join(ROOT, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    for src in sources:
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc, *flags(), *lang, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
