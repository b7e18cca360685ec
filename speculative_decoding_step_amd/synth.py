"""Seeded synthetic inputs shared by the GPU path's harness and the CPU oracle's tests.

This module holds none of the speculative-decoding arithmetic.  It only turns
(seed, tag, index) into numbers, with the same integer function on the host
(numpy) and on a device (torch), so both sides see bit-identical inputs:

* ``bits32(key, idx)``   a 32-bit hash of the element index (two rounds of the
  "lowbias32" integer finaliser, keyed by the seed and the tensor tag);
* normal-ish values      ``table[bits >> 16]``, where ``table`` holds the
  65,536 mid-point quantiles of N(0, sigma) rounded to the storage dtype (the
  configs draw every weight from N(0, 0.02));
* token ids              ``(bits * V) >> 32``, uniform over [0, V);
* uniforms               ``(bits >> 8) * 2**-24``, exact fp32 on a 24-bit grid.

The device path never takes a float decision: lookup, shifts, xors and
16-bit-split multiplies only, so the host and device results agree bit for bit.
"""
from __future__ import annotations

import zlib

import numpy as np

M32 = 0xFFFFFFFF
_C1 = 0x7FEB352D
_C2 = 0x846CA68B


def tag_of(name: str) -> int:
    """Stable 32-bit tag for a tensor name."""
    return zlib.crc32(name.encode()) & M32


# ---------------------------------------------------------------- host (numpy)

def _lowbias32_np(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.uint32, copy=True)
    x ^= x >> np.uint32(16)
    x *= np.uint32(_C1)
    x ^= x >> np.uint32(15)
    x *= np.uint32(_C2)
    x ^= x >> np.uint32(16)
    return x


def key_of(seed: int, tag: int) -> tuple[int, int]:
    """Two 32-bit keys for one (seed, tag) stream."""
    a = int(_lowbias32_np(np.array([(seed * 0x9E3779B1 + 0x632BE5AB) & M32]))[0])
    b = int(_lowbias32_np(np.array([(a ^ tag) & M32]))[0])
    c = int(_lowbias32_np(np.array([(b + 0x85EBCA77) & M32]))[0])
    return b, c


def bits32_np(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    """uint32 hash of indices [start, start+n) in stream (seed, tag)."""
    k1, k2 = key_of(seed, tag)
    idx = np.arange(start, start + n, dtype=np.uint64)
    assert start + n <= 1 << 32, "per-tensor index space is 32-bit"
    x = idx.astype(np.uint32) ^ np.uint32(k1)
    x = _lowbias32_np(x)
    x = x + np.uint32(k2)
    return _lowbias32_np(x)


_TABLE_CACHE: dict = {}


def _bf16_round_np(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even), returned as float32 values."""
    m, e = np.frexp(x)                      # keep 8 significant bits
    q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return q.astype(np.float32)


def normal_table(sigma: float, dtype: str) -> np.ndarray:
    """65,536 mid-point quantiles of N(0, sigma) rounded to ``dtype`` (as float32 values)."""
    key = (float(sigma), dtype)
    if key not in _TABLE_CACHE:
        from scipy.special import ndtri

        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        t = sigma * ndtri(p)
        if dtype == "bf16":
            t = _bf16_round_np(t)
        elif dtype == "f32":
            t = t.astype(np.float32)
        else:
            raise ValueError(dtype)
        _TABLE_CACHE[key] = t.astype(np.float32)
    return _TABLE_CACHE[key]


def normal_np(seed: int, name: str, shape, sigma: float = 0.02, dtype: str = "bf16") -> np.ndarray:
    """Seeded N(0, sigma)-shaped float32 array whose values are exact in ``dtype``."""
    n = int(np.prod(shape))
    b = bits32_np(seed, tag_of(name), n)
    return normal_table(sigma, dtype)[b >> np.uint32(16)].reshape(shape)


def randint_np(seed: int, name: str, n: int, lo: int, hi: int) -> np.ndarray:
    """n seeded integers uniform in [lo, hi]."""
    b = bits32_np(seed, tag_of(name), n).astype(np.uint64)
    span = np.uint64(hi - lo + 1)
    return (lo + ((b * span) >> np.uint64(32))).astype(np.int64)


def tokens_np(seed: int, name: str, n: int, vocab: int) -> np.ndarray:
    return randint_np(seed, name, n, 0, vocab - 1).astype(np.int32)


def subset_np(seed: int, name: str, n: int, vocab: int) -> np.ndarray:
    """n distinct seeded ids in [0, vocab), ascending: the ids whose hashes are the n
    smallest (ties by id)."""
    b = bits32_np(seed, tag_of(name), vocab)
    order = np.lexsort((np.arange(vocab), b))
    return np.sort(order[:n]).astype(np.int32)


def uniform24_np(seed: int, name: str, n: int) -> np.ndarray:
    """n seeded uniforms in [0, 1), multiples of 2**-24 (exact in float32)."""
    b = bits32_np(seed, tag_of(name), n)
    return ((b >> np.uint32(8)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


# --------------------------------------------------------------- device (torch)

def _mul32_t(x, c: int):
    """(x * c) mod 2**32 for int64 tensors holding values < 2**32, without overflow."""
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & M32


def _lowbias32_t(x):
    x = x ^ (x >> 16)
    x = _mul32_t(x, _C1)
    x = x ^ (x >> 15)
    x = _mul32_t(x, _C2)
    x = x ^ (x >> 16)
    return x


def bits32_t(seed: int, tag: int, n: int, device, start: int = 0):
    import torch

    k1, k2 = key_of(seed, tag)
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    x = _lowbias32_t((idx & M32) ^ k1)
    x = (x + k2) & M32
    return _lowbias32_t(x)


def normal_t(seed: int, name: str, shape, device, sigma: float = 0.02, dtype: str = "bf16",
             chunk: int = 1 << 27):
    """Device twin of :func:`normal_np`; returns a tensor of torch dtype bf16 or f32."""
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    table = torch.from_numpy(normal_table(sigma, dtype)).to(device=device, dtype=tdt)
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=tdt, device=device)
    tag = tag_of(name)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        b = bits32_t(seed, tag, m, device, start=s)
        out[s:s + m] = table[b >> 16]
    return out.view(*shape)


def tokens_t(seed: int, name: str, n: int, vocab: int, device):
    import torch

    b = bits32_t(seed, tag_of(name), n, device)
    return ((b * vocab) >> 32).to(torch.int32)


def uniform24_t(seed: int, name: str, n: int, device):
    import torch

    b = bits32_t(seed, tag_of(name), n, device)
    return (b >> 8).to(torch.float32) * (2.0 ** -24)
