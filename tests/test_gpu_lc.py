"""GPU parity of the LC-style comparison codec (TUPL8_1 -> BIT_8 -> RZE_2;
FastKVComp companion page, "Inside an LC-style pipeline"): the HIP kernels,
called through the C ABI, against the CPU oracle byte for byte -- whole
streams (header, table, payloads, padding) and decoded bytes.  Byte codec:
the bar is bit-exact."""
import sys

import numpy as np
import pytest
import torch

import kvsynth
import oracle

pytestmark = pytest.mark.gpu

CHUNK = 16384


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sz():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp8_kv_cache_amd
    from fp8_kv_cache_amd import lc
    fp8_kv_cache_amd.lc = lc
    return fp8_kv_cache_amd


def content(kind, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "random":
        return rng.integers(0, 256, n, dtype=np.uint8)
    if kind == "zeros":
        return np.zeros(n, np.uint8)
    if kind == "codes":                                  # one 4-bit code per byte
        return rng.integers(0, 16, n, dtype=np.uint8)
    if kind == "sparse":
        x = rng.integers(0, 256, n, dtype=np.uint8)
        x[rng.random(n) < 0.98] = 0
        return x
    if kind == "mixed":                                  # alternate raw and coded chunks
        x = rng.integers(0, 256, n, dtype=np.uint8)
        for c in range(0, n, 2 * CHUNK):
            x[c:c + CHUNK] &= 0x0F
        return x
    if kind == "bf16_kv":
        return np.ascontiguousarray(kvsynth.stress(-(-n // 2), seed=seed)).view(np.uint8)[:n].copy()
    raise ValueError(kind)


LENGTHS = [1, 2, 15, 16, 63, 64, 65, 1000, 4097, 16383, 16384, 16385, 32768, 50001, 100000]
CASES = [(k, n) for n in LENGTHS for k in ("random", "zeros", "codes", "sparse")] + \
        [("mixed", 5 * CHUNK + 777), ("bf16_kv", 3 * CHUNK + 10)]


@pytest.mark.parametrize("kind,n", CASES)
def test_stream_parity(sz, kind, n):
    x = content(kind, n, seed=n)
    say("lc stream parity", kind, n)
    stream = sz.lc.compress(torch.from_numpy(x).to("cuda"))
    expected = oracle.lc_encode(x)
    got = stream.cpu().numpy()
    assert got.size == expected.size
    assert np.array_equal(got, expected)
    y, status = sz.lc.decompress(stream, n)
    assert status == 0
    assert np.array_equal(y.cpu().numpy(), x)


def test_empty_input(sz):
    say("lc empty")
    stream = sz.lc.compress(torch.zeros(0, dtype=torch.uint8, device="cuda"))
    assert np.array_equal(stream.cpu().numpy(), oracle.lc_encode(np.zeros(0, np.uint8)))
    _, status = sz.lc.decompress(stream, 0)
    assert status == 0
    bad = stream.clone()
    bad[0] = 0
    _, status = sz.lc.decompress(bad, 0)
    assert status == 3


def test_golden_inputs(sz):
    """The two hand-derived fixtures under tests/golden/, through the GPU."""
    from tests.test_lc_oracle_pins import _load_golden
    for name in ("lc_ramp64.txt", "lc_raw_then_coded.txt"):
        spec = _load_golden(name)
        x = spec["input"]
        say("lc golden", name)
        stream = sz.lc.compress(torch.from_numpy(x).to("cuda"))
        assert stream.numel() == spec["total"]
        assert np.array_equal(stream.cpu().numpy(), oracle.lc_encode(x))


def test_batched_equals_single_and_oracle(sz):
    n, kinds = 3 * CHUNK + 4321, ["random", "zeros", "codes", "sparse", "mixed", "bf16_kv"]
    xs = [content(k, n, seed=40 + i) for i, k in enumerate(kinds)]
    say("lc batched", len(xs), n)
    b = sz.lc.LcBatch(len(xs), n)
    dev = [torch.from_numpy(x).to("cuda") for x in xs]
    b.set_inputs(dev)
    b.encode()
    b.decode()
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        expected = oracle.lc_encode(x)
        assert np.array_equal(b.stream(i).cpu().numpy(), expected), kinds[i]
        assert np.array_equal(sz.lc.compress(dev[i]).cpu().numpy(), expected), kinds[i]
        assert int(b.status[i]) == 0
        assert np.array_equal(b.output(i).cpu().numpy(), x), kinds[i]


def _corruptions(stream, n):
    C = -(-n // CHUNK)
    D = -(-(64 + 8 * C) // 256) * 256
    table = stream[64:64 + 8 * C].view(np.uint32).reshape(C, 2)
    coded = [c for c in range(C) if table[c, 1] != min(CHUNK, n - c * CHUNK)]
    out = {}

    def edit(name, fn):
        t = stream.copy()
        fn(t)
        out[name] = t
    edit("magic", lambda t: t.__setitem__(0, 0))
    edit("version", lambda t: t.__setitem__(4, 2))
    edit("pipeline", lambda t: t.__setitem__(5, 0))
    edit("log2_chunk", lambda t: t.__setitem__(6, 15))
    edit("n", lambda t: t.__setitem__(8, t[8] ^ 1))
    edit("count", lambda t: t.__setitem__(16, t[16] + 1))
    edit("total_up", lambda t: t.__setitem__(24, t[24] ^ 32))
    edit("reserved", lambda t: t.__setitem__(63, 1))
    edit("first_offset", lambda t: t.__setitem__(64, 16))
    edit("offset_chain", lambda t: t.__setitem__(64 + 8 * (C - 1), t[64 + 8 * (C - 1)] ^ 16))
    edit("size_over_length", lambda t: t[68:72].__setitem__(slice(None), np.frombuffer(
        (CHUNK + 16).to_bytes(4, "little"), np.uint8)))
    if coded:
        at = D + int(table[coded[0], 0])
        edit("bitmap_bit", lambda t: t.__setitem__(at, t[at] ^ 0x01))
    return out


def test_corrupt_streams_flagged_on_device(sz):
    n = 2 * CHUNK + 999
    x = content("mixed", n, seed=9)
    stream = oracle.lc_encode(x)
    for name, bad in _corruptions(stream, n).items():
        say("lc corrupt", name)
        assert oracle.lc_decode(bad, n)[0] == oracle.CORRUPT_STREAM, name
        _, status = sz.lc.decompress(torch.from_numpy(bad).to("cuda"), n)
        assert status == 3, name
    say("lc truncated")
    _, status = sz.lc.decompress(torch.from_numpy(stream).to("cuda"), n, src_bytes=stream.size - 1)
    assert status == 3


def test_llama_kv_cache_full_size(sz):
    """The 64-tensor Llama-3-8B-shaped BF16 cache (16 MiB per tensor) through
    the batched calls: every tensor decodes bit-exactly; the first two
    streams equal the oracle's byte for byte."""
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(8) as pool:
        xs = list(pool.map(lambda i: kvsynth.llama_kv(i // 2, i % 2, (8192, 8, 128)), range(64)))
    n = xs[0].nbytes
    say("lc llama full size", len(xs), n)
    b = sz.lc.LcBatch(len(xs), n)
    b.set_inputs([torch.from_numpy(x.view(np.uint8).ravel()).to("cuda") for x in xs])
    b.encode()
    b.decode()
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        assert int(b.status[i]) == 0, i
        assert torch.equal(b.output(i), b._inputs[i]), i
    for i in range(2):
        assert np.array_equal(b.stream(i).cpu().numpy(), oracle.lc_encode(xs[i])), i


def test_codes_full_size(sz):
    """A 64 MiB tensor of 4-bit codes (one per byte), every chunk coded:
    bit-exact round trip and stream equal to the oracle's."""
    n = 64 << 20
    x = content("codes", n, seed=77)
    say("lc codes full size", n)
    stream = sz.lc.compress(torch.from_numpy(x).to("cuda"))
    assert np.array_equal(stream.cpu().numpy(), oracle.lc_encode(x))
    y, status = sz.lc.decompress(stream, n)
    assert status == 0 and np.array_equal(y.cpu().numpy(), x)


def test_graph_replay_matches_eager(sz):
    """The batched LC encode and decode captured in one HIP graph and replayed
    three times, with eager work and a synchronisation between replays:
    every replay reproduces the eager streams, sizes, statuses and outputs."""
    n = 2 * CHUNK + 555
    xs = [content(k, n, seed=60 + i) for i, k in enumerate(["mixed", "codes", "random"])]
    say("lc graph replay", n)
    b = sz.lc.LcBatch(len(xs), n)
    b.set_inputs([torch.from_numpy(x).to("cuda") for x in xs])
    b.encode()
    b.decode()
    torch.cuda.synchronize()
    ref_sizes = b.sizes.clone()
    ref = [b.stream(i).clone() for i in range(len(xs))]
    for i, x in enumerate(xs):
        assert np.array_equal(ref[i].cpu().numpy(), oracle.lc_encode(x)), i
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.encode()
        b.decode()
    for replay in range(3):
        b.streams.zero_()
        b.sizes.zero_()
        b.outputs.zero_()
        b.status.fill_(-1)
        noise = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        assert torch.equal(b.sizes, ref_sizes), replay
        for i, x in enumerate(xs):
            assert int(b.status[i]) == 0, (replay, i)
            assert torch.equal(b.stream(i), ref[i]), (replay, i)
            assert np.array_equal(b.output(i).cpu().numpy(), x), (replay, i)
