"""Pins of the LC-style comparison codec's CPU oracle (oracle/lc_oracle.c).

FastKVComp companion page, "Inside an LC-style pipeline": TUPL8_1 then BIT_8
(size-preserving bit permutations) then RZE_2 (zero words left out).
The page prints no byte layout, so each stage is checked against its
plainest reading built from numpy primitives (reshape/transpose for the
tuple split, unpackbits/packbits for the bit planes, a boolean mask for the
zero elimination), against hand-derived streams under tests/golden/, and
against closed forms and invariants (the first two stages are bit
permutations, sizes follow from the bitmap, round trips are exact).
"""
import os

import numpy as np
import pytest

import kvsynth
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CHUNK = 16384
LENGTHS = [0, 1, 2, 7, 8, 9, 15, 63, 64, 65, 127, 128, 1000, 4097, 16383, 16384]


def _rng_bytes(n, seed):
    return np.random.default_rng(seed).integers(0, 256, n, dtype=np.uint8)


def np_tupl8_1(x):
    q = x.size // 8
    return np.concatenate([x[:8 * q].reshape(q, 8).T.ravel(), x[8 * q:]])


def np_bit8(y):
    g = (y.size // 8) // 8
    words = y[:64 * g].reshape(8 * g, 8)                                 # 8g words of 8 bytes
    bits = np.unpackbits(words, axis=1, bitorder="little")              # [word][bit b]
    planes = np.packbits(bits.T.reshape(64, 8 * g), axis=1, bitorder="little")  # [b][s], bit a = word 8s+a
    return np.concatenate([planes.ravel(), y[64 * g:]])


def np_rze2(z):
    v = z.size // 2
    words = z[:2 * v].reshape(v, 2)
    nz = (words != 0).any(axis=1)
    bitmap = np.packbits(nz, bitorder="little")
    return np.concatenate([bitmap, words[nz].ravel(), z[2 * v:]]).astype(np.uint8)


def _inputs(L):
    yield "random", _rng_bytes(L, L + 1)
    yield "zeros", np.zeros(L, np.uint8)
    yield "codes", _rng_bytes(L, L + 2) & 0x0F                # 4-bit codes, one per byte
    sparse = _rng_bytes(L, L + 3)
    sparse[np.random.default_rng(L).random(L) < 0.97] = 0
    yield "sparse", sparse


@pytest.mark.parametrize("L", LENGTHS)
def test_stages_match_numpy_readings(L):
    for name, x in _inputs(L):
        y = oracle.lc_tupl8_1(x)
        assert np.array_equal(y, np_tupl8_1(x)), name
        z = oracle.lc_bit8(y)
        assert np.array_equal(z, np_bit8(y)), name
        r = oracle.lc_rze2(z)
        assert np.array_equal(r, np_rze2(z)), name


@pytest.mark.parametrize("L", LENGTHS)
def test_stages_are_invertible_permutations(L):
    for name, x in _inputs(L):
        y = oracle.lc_tupl8_1(x)
        z = oracle.lc_bit8(y)
        # the first two stages move bits only: same length, same number of ones
        assert y.size == z.size == L
        ones = int(np.unpackbits(x).sum())
        assert int(np.unpackbits(y).sum()) == ones == int(np.unpackbits(z).sum()), name
        assert np.array_equal(oracle.lc_untupl8_1(y), x), name
        assert np.array_equal(oracle.lc_unbit8(z), y), name
        r = oracle.lc_rze2(z)
        v = L // 2
        nonzero = int(np.count_nonzero(z[:2 * v].reshape(v, 2).any(axis=1)))
        assert r.size == -(-v // 8) + 2 * nonzero + (L & 1), name
        assert np.array_equal(oracle.lc_unrze2(r, L), z), name
        assert oracle.lc_unrze2(np.concatenate([r, [0]]).astype(np.uint8), L) is None


def _load_golden(name):
    spec = {"chunks": [], "payloads": [], "raw": set(), "input": []}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "input_ramp":
            spec["input"].append(np.arange(int(rest[0]), dtype=np.uint8))
        elif key == "input_fill":
            spec["input"].append(np.full(int(rest[0]), int(rest[1], 16), np.uint8))
        elif key == "input_tail":
            t = np.zeros(int(rest[0]), np.uint8)
            for kv in rest[1:]:
                k, v = kv.split("=")
                t[int(k)] = int(v, 16)
            spec["input"].append(t)
        elif key == "total":
            spec["total"] = int(rest[0])
        elif key == "chunk":
            spec["chunks"].append((int(rest[0]), int(rest[1])))
        elif key == "payload_raw":
            spec["raw"].add(int(rest[0]))
        elif key == "payload":
            spec["payloads"].append(bytes.fromhex("".join(rest)))
    spec["input"] = np.concatenate(spec["input"])
    return spec


@pytest.mark.parametrize("name", ["lc_ramp64.txt", "lc_raw_then_coded.txt"])
def test_golden_streams(name):
    spec = _load_golden(name)
    x = spec["input"]
    n, C = x.size, len(spec["chunks"])
    data = -(-(64 + 8 * C) // 256) * 256
    expected = np.zeros(spec["total"], np.uint8)
    head = bytearray(64)
    head[0:8] = b"LCKV\x01\x01\x0e\x00"
    head[8:16] = n.to_bytes(8, "little")
    head[16:24] = C.to_bytes(8, "little")
    head[24:32] = spec["total"].to_bytes(8, "little")
    expected[:64] = np.frombuffer(bytes(head), np.uint8)
    coded = iter(spec["payloads"])
    for c, (off, size) in enumerate(spec["chunks"]):
        expected[64 + 8 * c: 72 + 8 * c] = np.frombuffer(off.to_bytes(4, "little") + size.to_bytes(4, "little"),
                                                       np.uint8)
        payload = x[c * CHUNK: c * CHUNK + size].tobytes() if c in spec["raw"] else next(coded)
        assert len(payload) == size
        expected[data + off: data + off + size] = np.frombuffer(payload, np.uint8)
    got = oracle.lc_encode(x)
    assert got.size == spec["total"]
    assert np.array_equal(got, expected)
    status, y = oracle.lc_decode(got, n)
    assert status == oracle.OK and np.array_equal(y, x)


def _table(stream):
    C = int.from_bytes(stream[16:24].tobytes(), "little")
    t = stream[64:64 + 8 * C].view(np.uint32).reshape(C, 2) if C else np.zeros((0, 2), np.uint32)
    return C, t


@pytest.mark.parametrize("n", [0, 1, 15, 16, 16383, 16384, 16385, 3 * 16384 + 5, 100000])
def test_container_closed_forms(n):
    C = -(-n // CHUNK)
    data = -(-(64 + 8 * C) // 256) * 256
    lengths = [min(CHUNK, n - c * CHUNK) for c in range(C)]
    assert oracle.lc_max_bytes(n) == data + sum(-(-L // 16) * 16 for L in lengths)
    for name, x in (("zeros", np.zeros(n, np.uint8)), ("random", _rng_bytes(n, n)),
                    ("codes", _rng_bytes(n, n + 9) & 0x0F)):
        s = oracle.lc_encode(x)
        count, table = _table(s)
        assert count == C
        off = 0
        for c, L in enumerate(lengths):
            assert table[c, 0] == off, (name, c)
            size = int(table[c, 1])
            if name == "zeros":
                # every word is zero: bitmap (all clear) plus the odd byte
                expect = -(-(L // 2) // 8) + (L & 1)
                assert size == (expect if expect < L else L), (name, c)
            elif name == "random":
                assert size == L, (name, c)              # random bytes are stored raw
            else:
                # bits 4..7 of every code byte are zero, so planes 8i+4..8i+7
                # (half of the 64 planes) vanish in a full chunk
                if L == CHUNK:
                    assert size <= 1024 + 8192, (name, c)
            off += -(-size // 16) * 16
        assert s.size == data + off == int.from_bytes(s[24:32].tobytes(), "little")
        assert s.size <= oracle.lc_max_bytes(n)
        status, y = oracle.lc_decode(s, n)
        assert status == oracle.OK and np.array_equal(y, x), name


def test_round_trip_on_kv_caches():
    for x in (kvsynth.llama_kv(2, 0, shape=(64, 8, 128)), kvsynth.e5m2_of(kvsynth.single_tensor(70001, seed=3)),
              kvsynth.stress(50001, seed=4)):
        s = oracle.lc_encode(x)
        status, y = oracle.lc_decode(s, x.nbytes)
        assert status == oracle.OK and np.array_equal(y, np.ascontiguousarray(x).view(np.uint8).ravel())


def test_corrupt_streams_are_rejected():
    x = np.concatenate([_rng_bytes(CHUNK, 1), _rng_bytes(CHUNK, 2) & 0x0F, np.zeros(1000, np.uint8)])
    s = oracle.lc_encode(x)
    n = x.size
    data = 256
    _, table = _table(s)
    coded = int(table[1, 0])

    def bad(edit):
        t = s.copy()
        edit(t)
        return t
    cases = {
        "magic": bad(lambda t: t.__setitem__(0, 0)),
        "version": bad(lambda t: t.__setitem__(4, 2)),
        "pipeline": bad(lambda t: t.__setitem__(5, 2)),
        "chunk_log2": bad(lambda t: t.__setitem__(6, 13)),
        "n": bad(lambda t: t.__setitem__(8, t[8] ^ 1)),
        "count": bad(lambda t: t.__setitem__(16, t[16] + 1)),
        "total": bad(lambda t: t.__setitem__(24, t[24] ^ 16)),
        "reserved": bad(lambda t: t.__setitem__(40, 1)),
        "offset": bad(lambda t: t.__setitem__(64 + 8, t[64 + 8] ^ 16)),
        "size_over_length": bad(lambda t: t[68:72].__setitem__(slice(None), np.frombuffer((CHUNK + 1).to_bytes(4, "little"), np.uint8))),
        "bitmap_bit": bad(lambda t: t.__setitem__(data + coded, t[data + coded] ^ 0x01)),
    }
    for name, t in cases.items():
        status, _ = oracle.lc_decode(t, n)
        assert status == oracle.CORRUPT_STREAM, name
    assert oracle.lc_decode(s[:-1], n)[0] == oracle.CORRUPT_STREAM
    assert oracle.lc_decode(s, n + 1)[0] == oracle.CORRUPT_STREAM


def test_size_over_length_is_rejected_even_with_a_matching_bitmap():
    """A raw last chunk of 1000 bytes relabelled with size 1001 keeps every
    offset and the total (both round to 1008), and its first bytes read as
    a bitmap with 469 of 500 words present: 63 + 2 * 469 = 1001, so only the
    check size <= chunk length rejects it."""
    rng = np.random.default_rng(5)
    last = rng.integers(0, 256, 1000, dtype=np.uint8)
    bits = np.zeros(504, np.uint8)
    bits[rng.choice(500, 469, replace=False)] = 1
    last[:63] = np.packbits(bits, bitorder="little")
    x = np.concatenate([rng.integers(0, 256, CHUNK, dtype=np.uint8), last])
    s = oracle.lc_encode(x)
    _, table = _table(s)
    assert int(table[1, 1]) == 1000                     # stored raw
    t = s.copy()
    t[64 + 12: 64 + 16] = np.frombuffer((1001).to_bytes(4, "little"), np.uint8)
    assert oracle.lc_decode(t, x.size)[0] == oracle.CORRUPT_STREAM


def test_coded_size_equal_to_chunk_length_is_stored_raw():
    """Reading L5 at its boundary: a 64-byte chunk whose plane image has 30
    of its 32 words non-zero codes to 4 + 60 = 64 bytes, no shorter than
    the chunk, so the chunk is stored raw.  The input is built from that
    image with numpy's inverses of the two rearranging stages."""
    rng = np.random.default_rng(11)
    z = rng.integers(1, 256, 64, dtype=np.uint8)
    z[[10, 11, 40, 41]] = 0                          # words 5 and 20 are zero
    planes = np.unpackbits(z.reshape(64, 1), axis=1, bitorder="little")   # [plane b][word a]
    words = np.packbits(planes.T, axis=1, bitorder="little")              # word a, bit b
    x = words.reshape(8, 8).T.ravel()                # undo the tuple split (q = 8)
    assert np.array_equal(np_bit8(np_tupl8_1(x)), z)
    assert oracle.lc_rze2(z).size == 64
    s = oracle.lc_encode(x)
    _, table = _table(s)
    assert int(table[0, 1]) == 64
    assert np.array_equal(s[256:320], x)
    status, y = oracle.lc_decode(s, 64)
    assert status == oracle.OK and np.array_equal(y, x)
