"""The library's own gfx950 device code, compiled here to assembly with the
build's flags, holds no matrix-core (MFMA) instruction -- the codecs are
integer bandwidth work -- and no packed-FP32 instruction (they are disabled
on every compile).  Only code built from this repository is inspected."""
import importlib.util
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _builder():
    """fp8_kv_cache_amd/build.py, loaded by path: the flags the library is built with."""
    spec = importlib.util.spec_from_file_location("_splitzip_build_flags",
                                                  os.path.join(ROOT, "fp8_kv_cache_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _device_asm(src):
    build = _builder()
    cmd = [build.hipcc(), *build.flags(), "--cuda-device-only", "-S", "-o", "-", src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


@pytest.mark.parametrize("name", ["kernels.hip", "lc_kernels.hip"])
def test_no_mfma_and_no_packed_fp32(name):
    asm = _device_asm(os.path.join(ROOT, "fp8_kv_cache_amd", "csrc", name))
    instructions = [ln.split()[0] for ln in asm.splitlines() if re.match(r"\s+[sv]_\w+", ln)]
    assert len(instructions) > 500                      # the kernels are really there
    assert not [i for i in instructions if i.startswith("v_mfma") or i.startswith("v_smfmac")]
    assert not [i for i in instructions if i in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")]
    # the kernels do use the vector integer and permute instructions they are built on
    assert "v_perm_b32" in instructions
