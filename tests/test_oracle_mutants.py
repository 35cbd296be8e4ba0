"""The oracle's pins catch plausible mistakes (mutation check, CPU only).

Each mutant below plants one mistake in a copy of an oracle source file --
a shifted or narrowed bit field, a flipped sort key, a reversed nibble or
bit order, a dropped term, an off-by-one -- and reruns the pin and property
tests against it in a fresh interpreter.  The C-versus-Python agreement test
is left out of those runs, so every mutant has to be caught by a pin that
does not come from the other oracle (float semantics, hand-derived streams,
brute force, closed forms, round trips, corruption cases).

Mistakes are planted in copies under a temporary folder; the oracle sources
themselves are never changed.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C_SRC = os.path.join(ROOT, "oracle", "sz_oracle.c")
PY_SRC = os.path.join(ROOT, "oracle", "sz_ref.py")
LC_SRC = os.path.join(ROOT, "oracle", "lc_oracle.c")
PIN_FILES = [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
             os.path.join(ROOT, "tests", "test_oracle_properties.py")]
LC_PIN_FILES = [os.path.join(ROOT, "tests", "test_lc_oracle_pins.py")]

# (name, text to replace -- must occur exactly once, replacement)
C_MUTANTS = [
    ("bf16 exponent field shifted", "return (u >> 7) & 0xFFu;", "return (u >> 8) & 0xFFu;"),
    ("e5m2 exponent mask narrowed", "return (u >> 2) & 0x1Fu;", "return (u >> 2) & 0x0Fu;"),
    ("bf16 sign dropped", "((u >> 8) & 0x80u) | (u & 0x7Fu)", "(u & 0x7Fu)"),
    ("e5m2 sign bit misplaced", "((u >> 5) & 0x4u)", "((u >> 4) & 0x4u)"),
    ("bf16 reassembly sign shift", "((sm & 0x80u) << 8)", "((sm & 0x80u) << 7)"),
    ("e5m2 reassembly exponent shift", "((e & 0x1Fu) << 2)", "((e & 0x1Fu) << 3)"),
    ("codebook ties by value descending", "return x->value < y->value ? -1 : 1;",
     "return x->value > y->value ? -1 : 1;"),
    ("codebook counts ascending", "return x->count > y->count ? -1 : 1;",
     "return x->count < y->count ? -1 : 1;"),
    ("e5m2 codebook domain halved", "return dt == SZO_BF16 ? 256u : 32u;",
     "return dt == SZO_BF16 ? 256u : 16u;"),
    ("repeated codebook value takes its last code",
     "if (code_of[cb[c]] == SZO_ESC) code_of[cb[c]] = c;", "code_of[cb[c]] = c;"),
    ("code nibbles high first", "(uint8_t)(code << (4 * (i % 2)))", "(uint8_t)(code << (4 * (1 - i % 2)))"),
    ("offsets taken after a block's first element", "if (i % SZO_BLOCK == 0) put_u32",
     "if (i % SZO_BLOCK == 1) put_u32"),
    ("offsets drift by one per block", "(i / SZO_BLOCK), (uint32_t)escapes);",
     "(i / SZO_BLOCK), (uint32_t)(escapes + i / SZO_BLOCK));"),
    ("format block of 2048 elements", "#define SZO_BLOCK 4096u", "#define SZO_BLOCK 2048u"),
    ("header region not padded", "return round256(64u + 4u * n_blocks(n));",
     "return 64u + 4u * n_blocks(n);"),
    ("e5m2 field bits most significant first", "if ((sm >> k) & 1u) dst[sm_at",
     "if ((sm >> (2u - k)) & 1u) dst[sm_at"),
    ("escape stream holds the raw element", "dst[esc_at + escapes] = (uint8_t)e;",
     "dst[esc_at + escapes] = (uint8_t)u;"),
    ("header escape count off by one", "put_u64(dst + 16, escapes);", "put_u64(dst + 16, escapes + (n > 0));"),
    ("decode escape cursor not advanced", "src[esc_at + j++]", "src[esc_at + j]"),
    ("decode codebook slot mirrored", ": cb[code];", ": cb[14 - code];"),
    ("decode skips the offset span check", "if (next < first || next - first != count) return",
     "if (next < first) return"),
    ("decode skips the reserved bytes", "if (src[k] != 0) return SZO_CORRUPT_STREAM;", "(void)0;"),
    ("decode accepts a wrong version", "if (src[4] != 1 || src[5]", "if (src[5]"),
    ("histogram drops the last element", "for (uint64_t i = 0; i < n; i++) hist[",
     "for (uint64_t i = 0; i + 1 < n; i++) hist["),
    ("sampled histogram strides elements", "if ((i / SZO_BLOCK) % stride == 0)", "if (i % stride == 0)"),
]

PY_MUTANTS = [
    ("bf16 exponent field shifted", "exponent = (u >> 7) & 0xFF", "exponent = (u >> 8) & 0xFF"),
    ("e5m2 mantissa narrowed", "mantissa = u & 0x3\n", "mantissa = u & 0x1\n"),
    ("codebook ties by value descending", "key=lambda v: (-counts[v], v)", "key=lambda v: (-counts[v], -v)"),
    ("repeated codebook value takes its last code", "lookup.setdefault(cb[c], c)", "lookup[cb[c]] = c"),
    ("code nibbles high first", "code << (4 if i % 2 else 0)", "code << (0 if i % 2 else 4)"),
    ("offsets taken after a block's first element", "if i % _BLOCK == 0:", "if i % _BLOCK == 1:"),
    ("ncodes header byte", "head[7] = 15", "head[7] = 16"),
    ("e5m2 field bits most significant first in a byte", "|= 1 << (bit % 8)", "|= 1 << (7 - bit % 8)"),
    ("decode codebook slot shifted", "e = s[24 + codes[i]]", "e = s[23 + codes[i]]"),
    ("bf16 reassembly sign shift", "((sm >> 7) & 1) << 15", "((sm >> 7) & 1) << 14"),
    ("decode skips the offset span check", "if span_end - offsets[b] != count:", "if span_end < offsets[b]:"),
]

LC_MUTANTS = [
    ("tuple split left as is", "y[j * q + i] = x[8 * i + j];", "y[8 * i + j] = x[8 * i + j];"),
    ("bit planes with the word order reversed", "(unsigned)(b % 8)) << a;", "(unsigned)(b % 8)) << (7u - a);"),
    ("bit planes read the wrong byte of a word", "8 * (8 * s + a) + b / 8, (unsigned)(b % 8)) << a;",
     "8 * (8 * s + a) + b % 8, (unsigned)(b / 8)) << a;"),
    ("zero test on the low byte only", "if (z[2 * m] | z[2 * m + 1]) {", "if (z[2 * m]) {"),
    ("bitmap bits most significant first", "out[m / 8] |= (uint8_t)(1u << (m % 8));",
     "out[m / 8] |= (uint8_t)(1u << (7u - m % 8));"),
    ("odd byte dropped", "if (L & 1u) out[at++] = z[L - 1];", "(void)0;"),
    ("coded chunk kept when as long as the chunk", "if (len < L) {", "if (len <= L) {"),
    ("payloads padded to 8 bytes", "return (x + 15u) / 16u * 16u;", "return (x + 7u) / 8u * 8u;"),
    ("data region not padded", "return up256(64u + 8u * chunks_of(n));", "return 64u + 8u * chunks_of(n);"),
    ("chunks of 8192 bytes", "#define LCO_CHUNK 16384u", "#define LCO_CHUNK 8192u"),
    ("header total without the data region", "put_u64(dst + 24, D + off);", "put_u64(dst + 24, off);"),
    ("decode accepts sizes over the chunk length", "if (o != off || size > L) return", "if (o != off) return"),
]

# run in the child: point the oracle package at the mutant, then the pins
_CHILD = r"""
import importlib.util, os, sys
root, kind, path = sys.argv[1:4]
sys.path.insert(0, root)
import oracle
if kind == "c":
    oracle._SRC, oracle._LIB = path, path[:-2] + ".so"
elif kind == "lc":
    oracle._LC_SRC, oracle._LC_LIB = path, path[:-2] + ".so"
else:
    spec = importlib.util.spec_from_file_location("oracle.sz_ref", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    sys.modules["oracle.sz_ref"] = mod
    oracle.sz_ref = mod
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", "-k", "not c_and_python_oracles_agree",
                      *sys.argv[4:]]))
"""


def _plant(src, old, new, dest):
    with open(src) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation anchor {old!r} occurs {text.count(old)} times in {src}"
    with open(dest, "w") as f:
        f.write(text.replace(old, new))


def _run(kind, path, workdir):
    if kind in ("c", "lc"):
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-w", "-shared", "-fPIC", "-o", path[:-2] + ".so", path])
    env = dict(os.environ, HYPOTHESIS_STORAGE_DIRECTORY=os.path.join(workdir, ".hypothesis"))
    pins = LC_PIN_FILES if kind == "lc" else PIN_FILES
    r = subprocess.run([sys.executable, "-c", _CHILD, ROOT, kind, path, *pins],
                       cwd=workdir, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_unmutated_copies_pass(tmp_path):
    """The harness itself: unchanged copies of both oracles pass every pin."""
    for kind, src in (("c", C_SRC), ("py", PY_SRC), ("lc", LC_SRC)):
        d = tmp_path / kind
        d.mkdir()
        dest = str(d / os.path.basename(src))
        with open(src) as f, open(dest, "w") as g:
            g.write(f.read())
        rc, out = _run(kind, dest, str(d))
        assert rc == 0, out


def test_every_mutant_is_caught(tmp_path):
    jobs = []
    for kind, src, mutants in (("c", C_SRC, C_MUTANTS), ("py", PY_SRC, PY_MUTANTS), ("lc", LC_SRC, LC_MUTANTS)):
        for i, (name, old, new) in enumerate(mutants):
            d = tmp_path / f"{kind}{i}"
            d.mkdir()
            dest = str(d / os.path.basename(src))
            _plant(src, old, new, dest)
            jobs.append((f"{kind}: {name}", kind, dest, str(d)))
    with cf.ThreadPoolExecutor(min(6, os.cpu_count() or 1)) as pool:
        results = list(pool.map(lambda j: (j[0], *_run(*j[1:])), jobs))
    survivors = [(name, rc, out) for name, rc, out in results if rc != 1]
    assert not survivors, "\n\n".join(f"{name}: exit {rc}\n{out}" for name, rc, out in survivors)
