"""Seeded synthetic inputs for prefix-KV chunk attention.

This module is shared by the tests, the benchmark and the oracle's checks. It holds
*no* arithmetic of the method itself: it only draws random numbers, scales them and
rounds them to bf16 (the storage type of every live tensor). Building a prefix cache
in F16 / BF16 / q8_0 form from the raw bf16 prefix rows is method arithmetic and is
done separately by each side (the oracle's converters on the CPU, the library's
append kernels on the GPU).

Workloads follow the shapes the pages train at:
  * chunks of 256 and 512 tokens ("train: walk the window", Contents and the
    "Measured on the 5090" table: chunk parameter a multiple of 256, default 512);
  * a 63k-token window ("train: walk the window", What it is) -> P = 63,488, C = 512;
  * 16,384-token contexts ("Training Large Context Models On Low VRAM", Key Takeaways).
The pages train on conversation windows and evaluation sets that are not available
here; these seeded tensors of the same shapes stand in for them.

Recipe (all values drawn as float32 from ``numpy.random.default_rng(seed)``,
multiplied, then rounded to bf16 with round-to-nearest-even via torch):
  draw order: Q, Kc, Vc, prefix K, prefix V, dO, outlier masks (K then V),
  per-head scales (Q, K, V).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

CACHE_F16 = "f16"
CACHE_BF16 = "bf16"
CACHE_Q8_0 = "q8_0"
CACHE_TYPES = (CACHE_F16, CACHE_BF16, CACHE_Q8_0)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one chunk step."""

    name: str
    batch: int          # B: independent windows in one call
    n_heads_q: int      # Hq
    n_heads_kv: int     # Hkv (Hq % Hkv == 0); query head h reads KV head h // (Hq/Hkv)
    head_dim: int       # D
    prefix_len: int     # P: frozen cached tokens
    chunk_len: int      # C: trainable chunk tokens
    cache_type: str     # storage type of the prefix cache
    seed: int
    qkv_std: float      # multiplier of N(0,1) for Q, Kc, Vc
    prefix_std: float   # multiplier of N(0,1) for the raw prefix K/V
    do_std: float       # multiplier of N(0,1) for dO
    outlier_frac: float = 0.0   # Bernoulli fraction of prefix elements multiplied by 8
    head_scale: Optional[tuple] = None  # (lo, hi): per-head U[lo,hi] scale of Q/K/V

    @property
    def group(self) -> int:
        return self.n_heads_q // self.n_heads_kv

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads. Index 0 is the small case the oracle finishes in well under a
# second; index 3 (8B-like, P=16384, C=512, bf16 prefix) is the headline one.
WORKLOADS = (
    Workload("tiny", 1, 2, 1, 64, 256, 64, CACHE_F16, seed=0,
             qkv_std=0.125, prefix_std=0.125, do_std=1.0),
    Workload("walk1.5b", 4, 12, 2, 128, 4096, 256, CACHE_F16, seed=1,
             qkv_std=0.1, prefix_std=0.1, do_std=1e-2),
    Workload("q8_0-16k", 2, 12, 2, 128, 16384, 512, CACHE_Q8_0, seed=2,
             qkv_std=0.1, prefix_std=1.0, do_std=1e-2, outlier_frac=0.01),
    Workload("8b-16k", 4, 32, 8, 128, 16384, 512, CACHE_BF16, seed=3,
             qkv_std=0.1, prefix_std=0.1, do_std=1e-2),
    Workload("long-63k", 1, 40, 8, 128, 63488, 512, CACHE_Q8_0, seed=4,
             qkv_std=0.1, prefix_std=0.1, do_std=1e-2, head_scale=(0.5, 2.0)),
)
WORKLOAD_BY_NAME = {w.name: w for w in WORKLOADS}
HEADLINE = WORKLOADS[3]


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 numpy -> torch bf16 (round to nearest even), CPU."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def make_inputs(w: Workload) -> dict:
    """Draw the seeded tensors of one chunk step.

    Returns torch CPU tensors:
      q   bf16 [B][Hq][C][D]      kc, vc bf16 [B][Hkv][C][D]  (the chunk's own keys)
      kp, vp bf16 [B][Hkv][P][D]  (raw prefix rows, before any cache conversion)
      do  bf16 [B][Hq][C][D]
    """
    B, Hq, Hkv, D, P, C = (w.batch, w.n_heads_q, w.n_heads_kv, w.head_dim,
                           w.prefix_len, w.chunk_len)
    rng = np.random.default_rng(w.seed)

    def normal(shape, std):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return x

    q = normal((B, Hq, C, D), w.qkv_std)
    kc = normal((B, Hkv, C, D), w.qkv_std)
    vc = normal((B, Hkv, C, D), w.qkv_std)
    kp = normal((B, Hkv, P, D), w.prefix_std)
    vp = normal((B, Hkv, P, D), w.prefix_std)
    do = normal((B, Hq, C, D), w.do_std)
    if w.outlier_frac > 0.0:
        mk = rng.random(size=kp.shape, dtype=np.float32) < w.outlier_frac
        mv = rng.random(size=vp.shape, dtype=np.float32) < w.outlier_frac
        kp[mk] *= np.float32(8.0)
        vp[mv] *= np.float32(8.0)
    if w.head_scale is not None:
        lo, hi = w.head_scale
        sq = rng.uniform(lo, hi, size=Hq).astype(np.float32)
        sk = rng.uniform(lo, hi, size=Hkv).astype(np.float32)
        sv = rng.uniform(lo, hi, size=Hkv).astype(np.float32)
        q *= sq[None, :, None, None]
        kc *= sk[None, :, None, None]
        kp *= sk[None, :, None, None]
        vc *= sv[None, :, None, None]
        vp *= sv[None, :, None, None]
    return {"q": to_bf16(q), "kc": to_bf16(kc), "vc": to_bf16(vc),
            "kp": to_bf16(kp), "vp": to_bf16(vp), "do": to_bf16(do)}


def small(name="small", *, batch=1, n_heads_q=2, n_heads_kv=1, head_dim=64,
          prefix_len=100, chunk_len=37, cache_type=CACHE_F16, seed=123,
          qkv_std=0.5, prefix_std=0.5, do_std=1.0, outlier_frac=0.0,
          head_scale=None) -> Workload:
    """An ad-hoc workload for edge cases (ragged P and C, G = 1, D = 64, ...)."""
    return Workload(name, batch, n_heads_q, n_heads_kv, head_dim, prefix_len,
                    chunk_len, cache_type, seed, qkv_std, prefix_std, do_std,
                    outlier_frac, head_scale)


# ---------------------------------------------------------------------------------
# Row-sparse linear backward ("stop-gradient through context tokens", Mechanism and
# its single-GPU microbenchmark: a 1.7B dense model at sequence length 2048, kept
# fractions 0.62, 0.5, 0.2, 0.1). No weights or data of that model are available;
# these seeded tensors have the shapes of one decoder layer's projections.

@dataclasses.dataclass(frozen=True)
class RowSparseShape:
    name: str
    in_features: int
    out_features: int


# One decoder layer of a 1.7B-class dense model (hidden 2048, 16 query heads x 128,
# MLP 6144): the projections whose backward the page makes row-sparse.
LAYER_1_7B = (
    RowSparseShape("q_proj", 2048, 2048),
    RowSparseShape("o_proj", 2048, 2048),
    RowSparseShape("gate_proj", 2048, 6144),
    RowSparseShape("up_proj", 2048, 6144),
    RowSparseShape("down_proj", 6144, 2048),
)


def kept_rows(n_rows: int, keep_frac: float, seed: int, mean_span: int = 96) -> np.ndarray:
    """Sorted int32 indices of round(keep_frac * n_rows) kept rows, laid out as reply
    spans between context gaps (the rows a loss reads come in runs): about
    K / mean_span spans whose lengths, and the gaps around them, are random
    compositions of K and N - K."""
    rng = np.random.default_rng(seed)
    k = int(round(keep_frac * n_rows))
    if k == 0:
        return np.zeros(0, dtype=np.int32)
    s = max(1, min(k, n_rows - k + 1, k // mean_span))

    def composition(total, parts, min_part):
        cuts = np.sort(rng.choice(np.arange(1, total - parts * (min_part - 1)), parts - 1,
                                  replace=False)) if parts > 1 else np.zeros(0, dtype=np.int64)
        edges = np.concatenate([[0], cuts, [total - parts * (min_part - 1)]])
        return np.diff(edges) + (min_part - 1)

    spans = composition(k, s, 1)
    gaps = composition(n_rows - k + 2, s + 1, 1) - np.array([1] + [0] * (s - 1) + [1])
    rows, pos = [], 0
    for i in range(s):
        pos += int(gaps[i])
        rows.append(np.arange(pos, pos + int(spans[i])))
        pos += int(spans[i])
    out = np.concatenate(rows).astype(np.int32)
    assert len(out) == k and out[-1] < n_rows
    return out


def row_sparse_inputs(n_rows: int, in_features: int, out_features: int, keep_frac: float,
                      seed: int) -> dict:
    """x bf16 [N][in] ~ N(0, 1), w bf16 [out][in] ~ N(0, 0.02^2), dy bf16 [N][out]
    ~ N(0, 0.01^2) (drawn in that order, torch CPU tensors) and keep int32 [K]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_rows, in_features), dtype=np.float32)
    w = rng.standard_normal((out_features, in_features), dtype=np.float32) * np.float32(0.02)
    dy = rng.standard_normal((n_rows, out_features), dtype=np.float32) * np.float32(0.01)
    keep = kept_rows(n_rows, keep_frac, seed + 1)
    return {"x": to_bf16(x), "w": to_bf16(w), "dy": to_bf16(dy),
            "keep": torch.from_numpy(keep)}
