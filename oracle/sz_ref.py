"""Pure-Python second oracle of the SplitZip-style exponent codec (format v1).

TEST INFRASTRUCTURE ONLY: used by the tests to cross-check the C oracle on
small inputs.  Written independently of the C oracle (no shared code or
tables) and of the GPU library.  Loops are element-by-element, so keep n
small (a few thousand).

Method, from the SplitZip project page:
  * Abstract -- the commonest exponent values get constant-width 4-bit
    codes, sign and mantissa bits are kept as they are, and rare exponents
    go to a separate escape stream;
  * FAQ "Is SplitZip lossy?" -- decoding is bit-exact;
  * FAQ "Does it work with an FP8 KV cache?" -- E5M2 variant, gaining at
    most 1.14x.
The byte layout is the reading documented in the C oracle's header comment
(readings R1..R8): codes 0..14 = top-15 exponents ranked by (count desc,
value asc), code 15 = escape; BF16 sign|mantissa byte; E5M2 3-bit LSB-first
field; nibbles low-first; escape bytes in element order; u32 offsets per
4096-element block; 64-byte header; regions padded to 256 bytes.
"""

BF16 = 1
E5M2 = 2
OK, INVALID_ARGUMENT, BUFFER_TOO_SMALL, CORRUPT_STREAM = 0, 1, 2, 3

_BLOCK = 4096
_ESCAPE_CODE = 15


def _align(x):
    return -(-x // 256) * 256


def _layout(n, dt):
    """(header region, sign|mantissa plane bytes, code plane bytes)."""
    nblocks = -(-n // _BLOCK)
    header = _align(64 + 4 * nblocks)
    sm = n if dt == BF16 else -(-3 * n // 8)
    codes = -(-n // 2)
    return header, sm, codes


def exact_bytes(n, dt, escapes):
    header, sm, codes = _layout(n, dt)
    return header + _align(sm) + _align(codes) + escapes


def max_bytes(n, dt):
    # a caller-given codebook may leave every element to the escape stream
    return exact_bytes(n, dt, n)


def _split(u, dt):
    """(sign|mantissa field, exponent field) of one raw element."""
    if dt == BF16:
        sign = (u >> 15) & 1
        exponent = (u >> 7) & 0xFF
        mantissa = u & 0x7F
        return (sign << 7) | mantissa, exponent
    sign = (u >> 7) & 1
    exponent = (u >> 2) & 0x1F
    mantissa = u & 0x3
    return (sign << 2) | mantissa, exponent


def _join(sm, exponent, dt):
    if dt == BF16:
        return ((sm >> 7) & 1) << 15 | (exponent & 0xFF) << 7 | (sm & 0x7F)
    return ((sm >> 2) & 1) << 7 | (exponent & 0x1F) << 2 | (sm & 0x3)


def histogram(values, dt):
    counts = [0] * 256
    for u in values:
        counts[_split(int(u), dt)[1]] += 1
    return counts


def codebook(counts, dt):
    domain = 256 if dt == BF16 else 32
    ranked = sorted(range(domain), key=lambda v: (-counts[v], v))
    return ranked[:15] + [0]


def encode(values, dt, cb=None):
    values = [int(u) for u in values]
    n = len(values)
    if cb is None:
        cb = codebook(histogram(values, dt), dt)
    cb = list(cb[:15]) + [0]
    lookup = {}
    for c in range(15):
        lookup.setdefault(cb[c], c)

    header, sm_len, code_len = _layout(n, dt)
    sm_plane = bytearray(_align(sm_len))
    code_plane = bytearray(_align(code_len))
    offsets = []
    escapes = bytearray()
    for i, u in enumerate(values):
        if i % _BLOCK == 0:
            offsets.append(len(escapes))
        sm, e = _split(u, dt)
        code = lookup.get(e, _ESCAPE_CODE)
        if code == _ESCAPE_CODE:
            escapes.append(e)
        if dt == BF16:
            sm_plane[i] = sm
        else:
            for k in range(3):
                if sm >> k & 1:
                    bit = 3 * i + k
                    sm_plane[bit // 8] |= 1 << (bit % 8)
        code_plane[i // 2] |= code << (4 if i % 2 else 0)

    total = header + len(sm_plane) + len(code_plane) + len(escapes)
    head = bytearray(header)
    head[0:4] = b"SZKV"
    head[4] = 1
    head[5] = dt
    head[6] = 12
    head[7] = 15
    head[8:16] = n.to_bytes(8, "little")
    head[16:24] = len(escapes).to_bytes(8, "little")
    head[24:40] = bytes(cb)
    head[40:48] = total.to_bytes(8, "little")
    for b, off in enumerate(offsets):
        head[64 + 4 * b: 68 + 4 * b] = off.to_bytes(4, "little")
    return bytes(head + sm_plane + code_plane + escapes)


def decode(stream, n, dt):
    """Return (status, list of raw elements or None)."""
    s = bytes(stream)
    if len(s) < 64:
        return CORRUPT_STREAM, None
    if s[0:4] != b"SZKV" or s[4] != 1 or s[5] != dt or s[6] != 12 or s[7] != 15:
        return CORRUPT_STREAM, None
    if int.from_bytes(s[8:16], "little") != n or s[39] != 0 or any(s[48:64]):
        return CORRUPT_STREAM, None
    escapes = int.from_bytes(s[16:24], "little")
    total = int.from_bytes(s[40:48], "little")
    if escapes > n or total != exact_bytes(n, dt, escapes) or total > len(s):
        return CORRUPT_STREAM, None
    header, sm_len, code_len = _layout(n, dt)
    sm_at = header
    code_at = sm_at + _align(sm_len)
    esc_at = code_at + _align(code_len)
    codes = [(s[code_at + i // 2] >> (4 if i % 2 else 0)) & 0xF for i in range(n)]
    nblocks = -(-n // _BLOCK)
    offsets = [int.from_bytes(s[64 + 4 * b: 68 + 4 * b], "little") for b in range(nblocks)]
    if nblocks and offsets[0] != 0:
        return CORRUPT_STREAM, None
    for b in range(nblocks):
        span_end = offsets[b + 1] if b + 1 < nblocks else escapes
        count = codes[b * _BLOCK:(b + 1) * _BLOCK].count(_ESCAPE_CODE)
        if span_end - offsets[b] != count:
            return CORRUPT_STREAM, None
    out = []
    j = 0
    for i in range(n):
        if codes[i] == _ESCAPE_CODE:
            e = s[esc_at + j]
            j += 1
        else:
            e = s[24 + codes[i]]
        if dt == BF16:
            sm = s[sm_at + i]
        else:
            sm = sum(((s[sm_at + (3 * i + k) // 8] >> ((3 * i + k) % 8)) & 1) << k for k in range(3))
        out.append(_join(sm, e, dt))
    return OK, out
