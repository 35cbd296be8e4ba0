"""GPU parity of the fused calls (sz_compress, sz_compress_batched):
histogram, codebook and stream of every tensor, computed in one launch,
against the CPU oracle byte for byte and against the three separate calls.
Integer codec: the bar is bit-exact."""
import concurrent.futures as cf
import sys

import numpy as np
import pytest
import torch

import kvsynth
import oracle
from tests.test_gpu_parity import CASES, to_dev, to_host

pytestmark = pytest.mark.gpu

BF16, E5M2 = 1, 2


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sz():
    """The library with every BF16 tensor sent through the fused kernel
    (by default tensors under 2^21 elements take the separate kernels), so
    the small cases below exercise it; restored afterwards."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp8_kv_cache_amd
    from fp8_kv_cache_amd import codec
    fp8_kv_cache_amd.codec = codec
    previous = fp8_kv_cache_amd.sz_compress_fused_min_elements(1)
    yield fp8_kv_cache_amd
    fp8_kv_cache_amd.sz_compress_fused_min_elements(previous)


def _check_against_oracle(x, dt, stream, hist, cb):
    h = oracle.histogram(x, dt)
    assert np.array_equal(hist.cpu().numpy().view(np.uint64), h)
    assert np.array_equal(cb.cpu().numpy(), oracle.codebook(h, dt))
    expected = oracle.encode(x, dt)
    got = stream.cpu().numpy()
    assert got.size == expected.size
    assert np.array_equal(got, expected)


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_parity(sz, name):
    make, dt = CASES[name]
    x = make()
    say("fused parity", name, "n", x.size, "dtype", dt)
    stream, hist, cb, status = sz.codec.compress_fused(to_dev(x), dt)
    torch.cuda.synchronize()
    assert status == 0
    _check_against_oracle(x, dt, stream, hist, cb)
    y, st = sz.codec.decompress(stream, x.size, dt)
    assert st == 0 and np.array_equal(to_host(y, dt), x)


@pytest.mark.parametrize("dt", [BF16, E5M2])
@pytest.mark.parametrize("n", [4096, 8 * 4096, 8 * 4096 + 1, 3 * 8 * 4096 + 4097, 25 * 4096 - 3])
def test_fused_batched(sz, dt, n):
    """Several tensors; whole and partial workgroup items, a partial last
    block: equal to the oracle and to the three separate calls."""
    xs = [kvsynth.stress(n, seed=400 + i) if i % 2 else kvsynth.single_tensor(n, seed=400 + i) for i in range(7)]
    if dt == E5M2:
        xs = [kvsynth.e5m2_of(x) for x in xs]
    say("fused batched", dt, n, len(xs))
    dev = [to_dev(x) for x in xs]
    one = sz.codec.BatchCodec(len(xs), n, dt)
    one.set_inputs(dev)
    one.compress_fused()
    three = sz.codec.BatchCodec(len(xs), n, dt)
    three.set_inputs(dev)
    three.compress()
    torch.cuda.synchronize()
    assert (one.fused_status.cpu().numpy() == 0).all()
    assert torch.equal(one.sizes, three.sizes)
    assert torch.equal(one.hists, three.hists)
    assert torch.equal(one.codebooks, three.codebooks)
    for i, x in enumerate(xs):
        assert torch.equal(one.stream(i), three.stream(i)), i
        _check_against_oracle(x, dt, one.stream(i), one.hists[i], one.codebooks[i])
    one.decompress()
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        assert int(one.status[i]) == 0
        assert np.array_equal(to_host(one.output(i), dt), x), i


@pytest.mark.parametrize("count,n", [(2, 16 * 4096 * 3 + 5), (5, 200705), (300, 3 * 16 * 4096 + 4097)])
def test_fused_schedule_shapes(sz, count, n):
    """Tensor counts below, at and far above the counting-to-encoding lag
    (so the stage schedule's first, middle and last regions all occur),
    with ragged counting items, ragged encode items and a partial last
    block: everything equal to the three separate calls, and a sample of
    tensors equal to the oracle."""
    rng = np.random.default_rng(count)
    xs = [kvsynth.stress(n, seed=int(s)) for s in rng.integers(0, 1 << 30, count)]
    say("fused schedule shapes", count, n)
    dev = [to_dev(x) for x in xs]
    one = sz.codec.BatchCodec(count, n, BF16)
    one.set_inputs(dev)
    one.compress_fused()
    three = sz.codec.BatchCodec(count, n, BF16)
    three.set_inputs(dev)
    three.compress()
    torch.cuda.synchronize()
    assert (one.fused_status.cpu().numpy() == 0).all()
    assert torch.equal(one.sizes, three.sizes)
    assert torch.equal(one.hists, three.hists)
    assert torch.equal(one.codebooks, three.codebooks)
    for i in range(count):
        assert torch.equal(one.stream(i), three.stream(i)), i
    for i in sorted({0, count // 2, count - 1}):
        _check_against_oracle(xs[i], BF16, one.stream(i), one.hists[i], one.codebooks[i])


@pytest.mark.parametrize("n", [(1 << 21) - 4096, 1 << 21])
def test_default_size_threshold(sz, n):
    """With the default threshold, a tensor just under 2^21 elements takes
    the separate kernels and one at 2^21 the fused kernel: both give the
    oracle's histogram, codebook and stream."""
    previous = sz.sz_compress_fused_min_elements(0)
    try:
        x = kvsynth.stress(n, seed=n)
        say("fused threshold", n)
        stream, hist, cb, status = sz.codec.compress_fused(to_dev(x), BF16)
        torch.cuda.synchronize()
        assert status == 0
        _check_against_oracle(x, BF16, stream, hist, cb)
    finally:
        sz.sz_compress_fused_min_elements(previous)


def test_fused_is_deterministic(sz):
    x = to_dev(kvsynth.stress(3 << 20, seed=19))
    say("fused determinism")
    first = None
    for _ in range(6):
        s, _, _, status = sz.codec.compress_fused(x, BF16)
        assert status == 0
        s = s.cpu().numpy()
        if first is None:
            first = s
        assert np.array_equal(s, first)


def test_llama_kv_cache_full_size_fused(sz):
    """The Llama-3-8B-shaped BF16 cache (64 x [8192, 8, 128]) in one batched
    fused call: every histogram, codebook and stream against the
    oracle, every decoded tensor against its input."""
    say("llama fused: generating")
    with cf.ThreadPoolExecutor(8) as pool:
        xs = list(pool.map(lambda i: kvsynth.llama_kv(i // 2, i % 2), range(64)))
    n = xs[0].size
    bc = sz.codec.BatchCodec(64, n, BF16)
    bc.set_inputs([to_dev(x) for x in xs])
    say("llama fused: encode+decode")
    bc.compress_fused()
    bc.decompress()
    torch.cuda.synchronize()
    assert (bc.fused_status.cpu().numpy() == 0).all()
    assert (bc.status.cpu().numpy() == 0).all()
    sizes = bc.sizes.cpu().numpy()
    hists = bc.hists.cpu().numpy().view(np.uint64)
    cbs = bc.codebooks.cpu().numpy()

    def check(i):
        h = oracle.histogram(xs[i], BF16)
        ok = np.array_equal(hists[i], h) and np.array_equal(cbs[i], oracle.codebook(h, BF16))
        expected = oracle.encode(xs[i], BF16)
        got = bc.streams[i, :sizes[i]].cpu().numpy()
        return i, ok and got.size == expected.size and np.array_equal(got, expected)

    say("llama fused: oracle")
    with cf.ThreadPoolExecutor(8) as pool:
        results = dict(pool.map(check, range(64)))
    assert all(results.values()), [i for i, ok in results.items() if not ok]
    for i in range(64):
        assert torch.equal(bc.output(i), bc._inputs[i]), i


@pytest.mark.parametrize("dt", [BF16, E5M2])
def test_fused_large_tensor(sz, dt):
    """One 2^26-element tensor (larger than the last-level cache): the same
    histogram, codebook and stream as the separate calls and the oracle."""
    n = 1 << 26
    x_dev = kvsynth.stress_device("cuda", n=n)
    if dt == E5M2:
        x_dev = to_dev(kvsynth.e5m2_of(x_dev.cpu().numpy().view(np.uint16)))
    say("fused large", dt, n)
    stream, hist, cb, status = sz.codec.compress_fused(x_dev, dt)
    ref, ref_hist, ref_cb = sz.codec.compress(x_dev, dt)
    torch.cuda.synchronize()
    assert status == 0
    assert torch.equal(hist, ref_hist) and torch.equal(cb, ref_cb) and torch.equal(stream, ref)
    x = to_host(x_dev, dt)
    _check_against_oracle(x, dt, stream, hist, cb)


@pytest.mark.parametrize("dt", [BF16, E5M2])
def test_fused_graph_replay(sz, dt):
    """Single-pass compress and decode captured in one HIP graph and replayed
    three times, with eager work between replays: every replay reproduces
    the eager results, which equal the oracle's."""
    n, count = 5 * 8 * 4096 + 777, 4
    xs = [kvsynth.stress(n, seed=500 + i) for i in range(count)]
    if dt == E5M2:
        xs = [kvsynth.e5m2_of(x) for x in xs]
    say("fused graph", dt, n, count)
    bc = sz.codec.BatchCodec(count, n, dt)
    bc.set_inputs([to_dev(x) for x in xs])
    bc.compress_fused()
    bc.decompress()
    torch.cuda.synchronize()
    ref_sizes = bc.sizes.clone()
    ref_streams = [bc.stream(i).clone() for i in range(count)]
    ref_hists = bc.hists.clone()
    for i, x in enumerate(xs):
        assert np.array_equal(ref_streams[i].cpu().numpy(), oracle.encode(x, dt)), i
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bc.compress_fused()
        bc.decompress()
    for replay in range(3):
        bc.outputs.zero_()
        bc.streams.zero_()
        bc.sizes.zero_()
        bc.hists.zero_()
        bc.codebooks.zero_()
        bc.status.fill_(-1)
        bc.fused_status.fill_(-1)
        noise = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        assert torch.equal(bc.sizes, ref_sizes), replay
        assert torch.equal(bc.hists, ref_hists), replay
        for i, x in enumerate(xs):
            assert int(bc.fused_status[i]) == 0 and int(bc.status[i]) == 0, (replay, i)
            assert torch.equal(bc.stream(i), ref_streams[i]), (replay, i)
            assert np.array_equal(to_host(bc.output(i), dt), x), (replay, i)


def test_two_fused_calls_on_two_streams(sz):
    """Two batched fused calls enqueued on two streams at once (each
    with its own workspace) share the GPU; both finish with the oracle's
    streams."""
    n = 1 << 20
    groups = []
    for k in range(2):
        xs = [kvsynth.llama_kv(k, i % 2, shape=(1024, 8, 128)) for i in range(8)]
        bc = sz.codec.BatchCodec(len(xs), n, BF16)
        bc.set_inputs([to_dev(x) for x in xs])
        groups.append((xs, bc))
    torch.cuda.synchronize()
    say("fused two streams")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for (xs, bc), s in zip(groups, streams):
        with torch.cuda.stream(s):
            bc.compress_fused()
    torch.cuda.synchronize()
    for xs, bc in groups:
        assert (bc.fused_status.cpu().numpy() == 0).all()
        for i, x in enumerate(xs):
            assert np.array_equal(bc.stream(i).cpu().numpy(), oracle.encode(x, BF16)), i


def test_give_up_path_is_reported_and_bounded(sz):
    """With the poll limit set to 1 from the host, workgroups that find
    their tensor not yet ready give up at once: every tensor ends with
    SZ_OK and the oracle's stream, or SZ_ERR_TIMEOUT and a stream size
    inside the capacity; the kernel always finishes.  Calls after the limit
    is restored are exact again."""
    n, count = 64 * 4096, 16
    xs = [kvsynth.stress(n, seed=600 + i) for i in range(count)]
    bc = sz.codec.BatchCodec(count, n, BF16)
    bc.set_inputs([to_dev(x) for x in xs])
    say("fused give-up")
    previous = sz.sz_compress_spin_limit(1)
    try:
        bc.compress_fused()
        torch.cuda.synchronize()
    finally:
        sz.sz_compress_spin_limit(previous)
    status = bc.fused_status.cpu().numpy()
    sizes = bc.sizes.cpu().numpy()
    assert set(status.tolist()) <= {0, sz.SZ_ERR_TIMEOUT}
    say("give-up statuses", status.tolist())
    for i, x in enumerate(xs):
        assert 0 < sizes[i] <= bc.capacity
        if status[i] == 0:
            assert np.array_equal(bc.stream(i).cpu().numpy(), oracle.encode(x, BF16)), i
    bc.compress_fused()
    torch.cuda.synchronize()
    assert (bc.fused_status.cpu().numpy() == 0).all()
    for i, x in enumerate(xs):
        assert np.array_equal(bc.stream(i).cpu().numpy(), oracle.encode(x, BF16)), i


# The fused kernel ranks a provisional codebook from a sample (every 16th
# chunk of 65536 BF16 elements) and recodes a tensor when the full
# histogram ranks differently.  These inputs are built so that the sample
# and the whole tensor rank differently in a known way (checked with the
# oracle on the CPU first), which drives the recoding path.
SAMPLE_CHUNK, SAMPLE_STRIDE = 1 << 16, 16


def _sample_mask(n):
    m = np.zeros(n, dtype=bool)
    for c in range(0, -(-n // SAMPLE_CHUNK), SAMPLE_STRIDE):
        m[c * SAMPLE_CHUNK:(c + 1) * SAMPLE_CHUNK] = True
    return m


def _set_exponent(bits, where, e):
    bits[where] = (bits[where] & 0x807F) | (e << 7)


def _skewed(n, seed, kind):
    """single_tensor(n) with its sampled chunks altered: 'order' swaps the
    sample's two most frequent exponents (same 15 values, other codes),
    'members' moves the sample's 15th exponent to a value outside the full
    top 15 (other values: codes and escapes both change)."""
    x = kvsynth.single_tensor(n, seed=seed).copy()
    s = _sample_mask(n)
    e = (x >> 7) & 0xFF
    top = oracle.codebook(oracle.histogram(x, BF16), BF16)[:15]
    if kind == "order":
        first, second = int(top[0]), int(top[1])
        idx = np.flatnonzero(s & (e == first))
        gap = int((e[s] == first).sum() - (e[s] == second).sum())
        _set_exponent(x, idx[:gap // 2 + gap // 8 + 1], second)
    else:
        out = int(top[14])
        unused = next(v for v in range(1, 255) if not (e == v).any())
        _set_exponent(x, s & (e == out), unused)
    return x


def _codebooks(x):
    full = oracle.codebook(oracle.histogram(x, BF16), BF16)[:15]
    part = oracle.codebook(oracle.histogram(x[_sample_mask(x.size)], BF16), BF16)[:15]
    return full, part


@pytest.mark.parametrize("kind", ["order", "members"])
@pytest.mark.parametrize("n", [1 << 21, (1 << 21) + 12345])
def test_fused_recodes_when_the_sample_ranks_differently(sz, kind, n):
    """Three tensors, the middle one skewed: its provisional codebook is not
    the final one (same values in another order, or other values), so its
    codes -- and for 'members' its escapes -- are recoded after the main
    pass.  Every stream equals the oracle's."""
    xs = [kvsynth.single_tensor(n, seed=703), _skewed(n, 701, kind), kvsynth.single_tensor(n, seed=702)]
    full, part = _codebooks(xs[1])
    assert not np.array_equal(full, part)
    assert (set(full.tolist()) == set(part.tolist())) == (kind == "order")
    for x in (xs[0], xs[2]):
        f, p = _codebooks(x)
        assert np.array_equal(f, p)   # these two need no recoding
    say("fused recode", kind, n)
    bc = sz.codec.BatchCodec(len(xs), n, BF16)
    bc.set_inputs([to_dev(x) for x in xs])
    bc.compress_fused()
    bc.decompress()
    torch.cuda.synchronize()
    assert (bc.fused_status.cpu().numpy() == 0).all()
    for i, x in enumerate(xs):
        _check_against_oracle(x, BF16, bc.stream(i), bc.hists[i], bc.codebooks[i])
        assert int(bc.status[i]) == 0 and np.array_equal(to_host(bc.output(i), BF16), x), i


def test_fused_recodes_escape_heavy_tensors(sz):
    """Heavy-tailed tensors (most elements escape, ~150 exponent values):
    samples and whole tensors rank differently, so recoding rewrites many
    staged escapes per block; a ragged last block too."""
    n = (1 << 22) + 777
    xs = [kvsynth.stress(n, seed=710 + i) for i in range(3)]
    assert any(not np.array_equal(*_codebooks(x)) for x in xs)
    say("fused recode escape-heavy", n)
    bc = sz.codec.BatchCodec(len(xs), n, BF16)
    bc.set_inputs([to_dev(x) for x in xs])
    bc.compress_fused()
    torch.cuda.synchronize()
    assert (bc.fused_status.cpu().numpy() == 0).all()
    for i, x in enumerate(xs):
        _check_against_oracle(x, BF16, bc.stream(i), bc.hists[i], bc.codebooks[i])


def _degenerate(n, kind):
    """'zeros' and 'ones': a single exponent value.  'unsampled': exponents
    127 and 126 everywhere, and 200 only in chunks the sample skips, so the
    provisional codebook lacks a value the final one ranks third: its
    elements are staged as escapes and recoded to code 2."""
    if kind == "zeros":
        return np.zeros(n, np.uint16)
    if kind == "ones":
        return np.full(n, 0x3F80, np.uint16)
    rng = np.random.default_rng(720)
    e = np.where(rng.random(n) < 0.7, 127, 126)
    e[~_sample_mask(n) & (rng.random(n) < 0.1)] = 200
    sign = rng.integers(0, 2, n)
    mant = rng.integers(0, 1 << 7, n)
    return ((sign << 15) | (e << 7) | mant).astype(np.uint16)


@pytest.mark.parametrize("kind", ["zeros", "ones", "unsampled"])
def test_fused_degenerate_alphabets(sz, kind):
    """Tensors with one to three exponent values over several items and a
    ragged end, between two ordinary tensors."""
    n = (1 << 21) + 777
    xs = [kvsynth.single_tensor(n, seed=721), _degenerate(n, kind), kvsynth.single_tensor(n, seed=722)]
    full, part = _codebooks(xs[1])
    if kind == "unsampled":
        assert 200 in full.tolist() and 200 not in part.tolist()
    else:
        assert np.array_equal(full, part)
    say("fused degenerate", kind, n)
    bc = sz.codec.BatchCodec(len(xs), n, BF16)
    bc.set_inputs([to_dev(x) for x in xs])
    bc.compress_fused()
    bc.decompress()
    torch.cuda.synchronize()
    assert (bc.fused_status.cpu().numpy() == 0).all()
    for i, x in enumerate(xs):
        _check_against_oracle(x, BF16, bc.stream(i), bc.hists[i], bc.codebooks[i])
        assert int(bc.status[i]) == 0 and np.array_equal(to_host(bc.output(i), BF16), x), i
