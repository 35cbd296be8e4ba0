"""Seeded synthetic KV-cache inputs for the codec's tests and benchmark.

This module only synthesises values.  It holds none of the codec's
arithmetic (no exponent split, no ranking, no packing), so the CPU oracle
and the GPU library can both be fed from it without sharing codec code.

Every tensor is returned as raw bit patterns: numpy ``uint16`` for BF16 and
``uint8`` for FP8 E5M2 (or torch ``int16`` / ``uint8`` on a device).

The SplitZip project page measured on real KV activations of Qwen3-32B,
Qwen3-30B-A3B, Llama-3-8B and Phi-2 (FAQ "Which models were tested?").
Those need trained weights, so these generators stand in for them with the
same KV shapes and heavy-tailed value mixes:

  single_tensor   n values N(0,1) -> BF16 (round to nearest even), then
                  round(0.001 n) distinct positions scaled exactly by
                  2^(+-k), k uniform in [16, 40]: forced rare exponents.
  llama_kv        one layer tensor [tokens, kv_heads, head_dim] of a
                  Llama-3-8B-shaped cache (8192 x 8 x 128): N(0,1) times a
                  per-(head, dim) lognormal(0, 1) scale; K tensors have 4
                  outlier dims per head scaled x20.
  long_kv_device  one layer of a Qwen3-32B-shaped long-context cache
                  (131072 x 8 x 128), single_tensor's value mix, drawn on a
                  torch device (Philox) because 128 such tensors (34 GB)
                  are too slow to draw on the host.
  e5m2_of         BF16 values -> FP8 E5M2, round to nearest even,
                  non-saturating (overflow gives +-Inf).
  stress          Cauchy(0,1) x 2^U(-60,60) -> BF16, plus 1% special bit
                  patterns (+-0, subnormals, +-Inf, NaN with random payload).
"""
import math

import numpy as np
import torch

LLAMA_KV_SHAPE = (8192, 8, 128)
LONG_KV_SHAPE = (131072, 8, 128)


def _bf16_bits(x_f32):
    """float32 numpy array -> BF16 bit patterns (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_to_f32(bits_u16):
    t = torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float32).numpy()


def single_tensor(n=1 << 20, seed=1, escape_fraction=0.001):
    """BF16 N(0,1) values with a fraction forced to rare exponents."""
    rng = np.random.default_rng(seed)
    bits = _bf16_bits(rng.standard_normal(n, dtype=np.float32))
    m = int(round(escape_fraction * n))
    if m:
        idx = rng.choice(n, m, replace=False)
        sign = rng.choice(np.array([-1, 1]), m)
        k = rng.integers(16, 41, m)
        vals = _bf16_to_f32(bits[idx])
        # power-of-two scaling is exact in float32 and stays in BF16 range
        bits[idx] = _bf16_bits(np.ldexp(vals, sign * k).astype(np.float32))
    return bits


def llama_kv(layer, kv, shape=LLAMA_KV_SHAPE, base_seed=2000):
    """One Llama-3-8B-shaped layer tensor; kv = 0 for K, 1 for V."""
    tokens, heads, dim = shape
    rng = np.random.default_rng(base_seed + 2 * layer + kv)
    z = rng.standard_normal(tokens * heads * dim, dtype=np.float32).reshape(tokens, heads, dim)
    scale = rng.lognormal(0.0, 1.0, size=(heads, dim)).astype(np.float32)
    if kv == 0:
        for h in range(heads):
            outliers = rng.choice(dim, 4, replace=False)
            scale[h, outliers] *= np.float32(20.0)
    return _bf16_bits((z * scale[None, :, :]).reshape(-1))


def llama_kv_cache(layers=32, shape=LLAMA_KV_SHAPE):
    """All 2 * layers tensors of the Llama-3-8B-shaped cache, order (l, K/V)."""
    return [llama_kv(layer, kv, shape) for layer in range(layers) for kv in (0, 1)]


def e5m2_of(bf16_bits):
    """BF16 bit patterns -> FP8 E5M2 bytes (RNE, overflow to +-Inf)."""
    t = torch.from_numpy(np.ascontiguousarray(bf16_bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float32).to(torch.float8_e5m2).view(torch.uint8).numpy().copy()


def stress(n=1 << 28, seed=5, special_fraction=0.01):
    """Escape-heavy BF16 stress input (host numpy draw)."""
    rng = np.random.default_rng(seed)
    c = rng.standard_cauchy(n) * np.exp2(rng.uniform(-60.0, 60.0, n))
    bits = _bf16_bits(c.astype(np.float32))
    m = int(round(special_fraction * n))
    if m:
        idx = rng.choice(n, m, replace=False)
        kind = rng.integers(0, 4, m)             # 0: +-0, 1: subnormal, 2: +-Inf, 3: NaN
        sign = rng.integers(0, 2, m).astype(np.uint16) << 15
        payload = rng.integers(1, 128, m).astype(np.uint16)
        pattern = np.where(kind == 0, 0,
                  np.where(kind == 1, payload,
                  np.where(kind == 2, 0x7F80, 0x7F80 | payload))).astype(np.uint16)
        bits[idx] = sign | pattern
    return bits


def long_kv_device(layer, kv, device, shape=LONG_KV_SHAPE, base_seed=30000,
                   escape_fraction=0.001):
    """One long-context layer tensor drawn on `device` with torch's Philox
    generator; returns an int16 tensor of BF16 bit patterns."""
    n = math.prod(shape)
    g = torch.Generator(device=device)
    g.manual_seed(base_seed + 2 * layer + kv)
    x = torch.randn(n, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    m = int(round(escape_fraction * n))
    idx = torch.randperm(n, generator=g, device=device)[:m]
    sign = torch.randint(0, 2, (m,), generator=g, device=device) * 2 - 1
    k = torch.randint(16, 41, (m,), generator=g, device=device)
    x[idx] = torch.ldexp(x[idx].float(), (sign * k).float()).to(torch.bfloat16)
    return x.view(torch.int16)


def stress_device(device, n=1 << 28, seed=5, special_fraction=0.01):
    """Same recipe as `stress`, drawn on `device` with torch's Philox."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    c = torch.empty(n, device=device, dtype=torch.float32).cauchy_(generator=g)
    u = torch.rand(n, generator=g, device=device, dtype=torch.float32) * 120.0 - 60.0
    bits = (c * torch.exp2(u)).to(torch.bfloat16).view(torch.int16)
    m = int(round(special_fraction * n))
    idx = torch.randperm(n, generator=g, device=device)[:m]
    kind = torch.randint(0, 4, (m,), generator=g, device=device)
    sign = torch.randint(0, 2, (m,), generator=g, device=device).to(torch.int32) << 15
    payload = torch.randint(1, 128, (m,), generator=g, device=device).to(torch.int32)
    zero = torch.zeros_like(payload)
    pattern = torch.where(kind == 0, zero,
              torch.where(kind == 1, payload,
              torch.where(kind == 2, zero + 0x7F80, payload | 0x7F80)))
    bits[idx] = (sign | pattern).to(torch.int16)
    return bits


def uniform_bits_device(device, n, seed=9):
    """n uniformly random 16-bit patterns (BF16 bit patterns of every kind,
    all 256 exponents about equally often) drawn on `device` with torch's
    Philox; an int16 tensor."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(-32768, 32768, (n,), generator=g, device=device, dtype=torch.int16)
