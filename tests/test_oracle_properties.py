"""Property and failure-handling tests of the CPU oracle (no GPU)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from oracle import sz_ref

BF16, E5M2 = oracle.BF16, oracle.E5M2


def _arrays(dt, max_n=9000):
    lo_exps = st.integers(0, 255) if dt == BF16 else st.integers(0, 31)

    @st.composite
    def build(draw):
        n = draw(st.integers(0, max_n))
        seed = draw(st.integers(0, 2**32 - 1))
        mode = draw(st.sampled_from(["raw", "few_exponents", "one_exponent"]))
        rng = np.random.default_rng(seed)
        if dt == BF16:
            x = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
            if mode != "raw":
                k = 1 if mode == "one_exponent" else draw(st.integers(2, 40))
                exps = rng.choice(256, k, replace=False)
                pick = exps[rng.integers(0, k, n)]
                x = (x & 0x807F) | (pick.astype(np.uint16) << 7)
        else:
            x = rng.integers(0, 256, n, dtype=np.uint16).astype(np.uint8)
            if mode != "raw":
                k = 1 if mode == "one_exponent" else draw(st.integers(2, 32))
                exps = rng.choice(32, k, replace=False)
                pick = exps[rng.integers(0, k, n)]
                x = ((x & 0x83) | (pick.astype(np.uint8) << 2)).astype(np.uint8)
        cb = None
        if draw(st.booleans()):
            cb = np.array(draw(st.lists(lo_exps, min_size=16, max_size=16)), np.uint8)
        return x, cb

    return build()


@pytest.mark.parametrize("dt", [BF16, E5M2])
def test_round_trip_and_size_properties(dt):
    @settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
    @given(_arrays(dt))
    def check(case):
        x, cb = case
        n = x.size
        stream = oracle.encode(x, dt, cb)
        f = oracle.stream_fields(stream)
        assert f["n"] == n and f["bytes"] == stream.size
        assert stream.size == oracle.exact_bytes(n, dt, f["escapes"])
        assert stream.size <= oracle.max_bytes(n, dt)
        if cb is None:
            h = oracle.histogram(x, dt)
            assert f["escapes"] == n - int(h[np.array(f["codebook"][:15])].sum())
            domain = 256 if dt == BF16 else 32
            if np.count_nonzero(h[:domain]) <= 15:
                assert f["escapes"] == 0
        status, y = oracle.decode(stream, n, dt)
        assert status == oracle.OK and np.array_equal(x, y)
    check()


def _valid_stream(dt=BF16, n=9000, seed=3):
    rng = np.random.default_rng(seed)
    if dt == BF16:
        x = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
        x = (x & 0x807F) | (rng.integers(100, 140, n).astype(np.uint16) << 7)  # 40 exponents
    else:
        x = rng.integers(0, 256, n, dtype=np.uint16).astype(np.uint8)
    return x, oracle.encode(x, dt)


def _corruptions(stream, n):
    s = stream.copy()
    nblocks = -(-n // 4096)
    out = {}

    def mutate(name, fn):
        t = s.copy()
        t = fn(t)
        out[name] = t

    mutate("magic", lambda t: (t.__setitem__(0, ord("X")), t)[1])
    mutate("version", lambda t: (t.__setitem__(4, 2), t)[1])
    mutate("dtype", lambda t: (t.__setitem__(5, 3 - t[5]), t)[1])
    mutate("block_log2", lambda t: (t.__setitem__(6, 11), t)[1])
    mutate("ncodes", lambda t: (t.__setitem__(7, 14), t)[1])
    mutate("n_field", lambda t: (t.__setitem__(8, t[8] ^ 1), t)[1])
    mutate("escape_slot", lambda t: (t.__setitem__(39, 5), t)[1])
    mutate("reserved", lambda t: (t.__setitem__(50, 1), t)[1])
    mutate("escape_count_up", lambda t: (t.__setitem__(16, t[16] + 1), t)[1])
    mutate("total_bytes", lambda t: (t.__setitem__(40, t[40] ^ 4), t)[1])
    mutate("truncated", lambda t: t[:-1])
    mutate("too_short", lambda t: t[:40])
    mutate("first_offset", lambda t: (t.__setitem__(64, 1), t)[1])
    if nblocks > 1:
        mutate("offset_swap", lambda t: (t.__setitem__(68, t[68] + 1), t)[1])
    # turn the first element's code into the escape code (or back): the
    # block's escape count no longer matches its offset span
    def align(v):
        return -(-v // 256) * 256
    sm_bytes = n if s[5] == BF16 else -(-3 * n // 8)
    code_at = align(64 + 4 * nblocks) + align(sm_bytes)

    def flip_code(t):
        t[code_at] = (t[code_at] | 0x0F) if (t[code_at] & 0x0F) != 0x0F else (t[code_at] & 0xF0)
        return t

    mutate("code_flip", flip_code)
    return out


@pytest.mark.parametrize("dt", [BF16, E5M2])
def test_corrupt_streams_are_rejected_by_both_oracles(dt):
    x, stream = _valid_stream(dt)
    n = x.size
    assert oracle.decode(stream, n, dt)[0] == oracle.OK
    for name, bad in _corruptions(stream, n).items():
        status, _ = oracle.decode(bad, n, dt)
        assert status == oracle.CORRUPT_STREAM, name
        assert sz_ref.decode(bytes(bad), n, dt)[0] == oracle.CORRUPT_STREAM, name
    # caller-side mismatches
    assert oracle.decode(stream, n + 1, dt)[0] == oracle.CORRUPT_STREAM
    assert oracle.decode(stream, n, 3 - dt)[0] == oracle.CORRUPT_STREAM
    # a longer buffer than the stream is fine
    padded = np.concatenate([stream, np.full(100, 7, np.uint8)])
    status, y = oracle.decode(padded, n, dt)
    assert status == oracle.OK and np.array_equal(x, y)


def test_encode_argument_errors():
    assert oracle._load().szo_encode(None, 5, BF16, None, None, 0, None) == oracle.INVALID_ARGUMENT
    x = np.zeros(100, np.uint16)
    out = np.zeros(10, np.uint8)
    rc = oracle._load().szo_encode(x.ctypes.data, 100, BF16, None, out.ctypes.data, 10, None)
    assert rc == oracle.BUFFER_TOO_SMALL
    rc = oracle._load().szo_encode(x.ctypes.data, 100, 9, None, out.ctypes.data, 10, None)
    assert rc == oracle.INVALID_ARGUMENT
    assert oracle.max_bytes(1 << 32, BF16) == 0
    assert oracle.max_bytes(5, 0) == 0
