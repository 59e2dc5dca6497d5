"""Oracle of the prefix-cache storage conversions (test infrastructure only).

The cached context is held fixed, in F16 or q8_0 storage ("train: walk the window",
Contents; approval comment: the storage type is the serving side's, and V is kept
token-major rather than transposed, which is what allows block quantisation of it).
A bf16 cache (a plain copy of the bf16 rows) is also supported.

q8_0 is named on that page but not spelled out. It is read here as the ggml Q8_0
block format: along head_dim, each run of 32 consecutive values of one token row of
one KV head forms a block that stores 32 int8 codes and one fp16 scale
d = amax / 127. Exact arithmetic used:

  amax = max |x| over the block (x: fp32 values of bf16 inputs, exact)
  d    = fl32(amax / 127)          IEEE fp32 division, round to nearest even
  d16  = fp16_rne(d)               the stored scale
  q    = clamp(round_half_away_from_zero(fl32(x / d)), -127, 127)   (d = 0 -> q = 0)
  x^   = fl32(f32(d16) * q)        dequantised value, exact in fp32

F16 storage is fp16_rne(fp32(bf16 x)). Every function works on numpy arrays and
returns numpy arrays; fp32 work is done in numpy float32 (IEEE, correctly rounded).
"""
from __future__ import annotations

import numpy as np

QK8_0 = 32  # values per q8_0 block


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits).astype(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def from_torch_bf16(t) -> np.ndarray:
    """A torch bf16 CPU tensor -> float32 numpy array of the same values."""
    import torch
    bits = t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return bf16_bits_to_f32(bits)


def to_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp16, round to nearest even (numpy's IEEE conversion)."""
    with np.errstate(over="ignore"):   # overflow -> inf, as IEEE RNE says
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def _round_half_away(r: np.ndarray) -> np.ndarray:
    # r is fp32; in fp64 both |r| + 0.5 and the floor are exact for |r| < 2^52.
    r64 = r.astype(np.float64)
    return np.sign(r64) * np.floor(np.abs(r64) + 0.5)


def quantise_q8_0(x: np.ndarray):
    """x float32 [..., D] (D % 32 == 0) -> (qs int8 [..., D], d float16 [..., D/32])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    if D % QK8_0:
        raise ValueError("q8_0 needs head_dim % 32 == 0")
    blk = x.reshape(x.shape[:-1] + (D // QK8_0, QK8_0))
    amax = np.abs(blk).max(axis=-1)
    d = amax / np.float32(127.0)                    # fp32 / fp32 -> fp32, RNE
    assert d.dtype == np.float32
    safe = np.where(d == 0, np.float32(1.0), d)
    r = blk / safe[..., None]                       # fp32, RNE
    q = np.clip(_round_half_away(r), -127, 127)
    q = np.where((d == 0)[..., None], 0.0, q).astype(np.int8)
    return q.reshape(x.shape), d.astype(np.float16)


def dequantise_q8_0(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    """(qs int8 [..., D], d float16 [..., D/32]) -> float32 [..., D], exact."""
    qs = np.asarray(qs)
    D = qs.shape[-1]
    blk = qs.reshape(qs.shape[:-1] + (D // QK8_0, QK8_0)).astype(np.float32)
    x = blk * np.asarray(d).astype(np.float32)[..., None]
    return x.reshape(qs.shape)


def build_prefix(x: np.ndarray, cache_type: str) -> dict:
    """Convert raw rows x (float32 values of bf16 inputs, [..., D]) to cache storage.

    Returns {"values": fp64 values the attention reads, plus the stored arrays}:
      "f16":  {"f16": float16}
      "bf16": {"bits": uint16}
      "q8_0": {"qs": int8, "d": float16}
    """
    x = np.asarray(x, dtype=np.float32)
    if cache_type == "f16":
        h = to_f16(x)
        return {"values": h.astype(np.float64), "f16": h}
    if cache_type == "bf16":
        bits = f32_to_bf16_rne(x)
        return {"values": bf16_bits_to_f32(bits).astype(np.float64), "bits": bits}
    if cache_type == "q8_0":
        qs, d = quantise_q8_0(x)
        return {"values": dequantise_q8_0(qs, d).astype(np.float64), "qs": qs, "d": d}
    raise ValueError(f"unknown cache type {cache_type!r}")


def append_rows(x: np.ndarray, cache_type: str) -> dict:
    """The cache rows [P, P+C) an append of the chunk's K or V writes.

    After its step a chunk's K/V are written into the cache, where the following
    chunks read them ("train: walk the window", What it is); the stored form is the
    cache's own type.
    """
    return build_prefix(x, cache_type)
