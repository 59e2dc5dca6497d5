"""GPU parity at the largest chunk the boundary accepts, on sampled outputs.

A full oracle of C = 65536 chunk rows is out of reach, but every sampled output has an
exact small formulation (the oracle's own definition, re-sliced):
  * rows [a, a + n) of the chunk are the whole chunk of a call whose cache is
    [cache ; chunk keys 0..a-1] (tests/_slices.py, pinned against the full oracle in
    test_oracle_slices.py): O, LSE and dQ of those rows come from a small oracle call;
  * dK/dV of chunk keys [a, C) get contributions from rows >= a only: the same call
    with n = C - a returns them as its chunk dK/dV.
Cases: C = 65536 (the maximum, 512 key blocks of 128, q8_0 cache) and C = 9000 with
one (window, KV head), whose 71 key blocks are too many for per-block row splits, so
the dK/dV rows are split uniformly.
"""
import numpy as np
import pytest
import torch

import synthetic
from _gpu import TOL, Case, f64, rel_l2
from _slices import chunk_slice

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import prefix_kv_attention_amd  # noqa: F401  (fails loudly without libpka.so)


def _oracle_slice(case, kpv, vpv, a, n):
    """Oracle outputs of chunk rows / keys [a, a+n) of every (window 0, KV head)."""
    w, x = case.w, case.cpu
    G = w.group
    out = []
    for kv in range(w.n_heads_kv):
        hs = slice(kv * G, (kv + 1) * G)
        e = a + n   # rows / keys past the slice play no part
        out.append(chunk_slice(f64(x["q"][0, hs, :e]), f64(x["kc"][0, kv, :e]),
                               f64(x["vc"][0, kv, :e]), kpv[0, kv], vpv[0, kv],
                               f64(x["do"][0, hs, :e]), w.softmax_scale, a, n))
    return out


def _check(case, got, a, n, keys=False):
    w = case.w
    G = w.group
    o, lse, dq, dk, dv = got
    kpv, vpv = case.oracle_prefix()
    ref = _oracle_slice(case, kpv, vpv, a, n)
    errs = {}
    for kv, (ro, rl, rdq, rdk, rdv) in enumerate(ref):
        hs = slice(kv * G, (kv + 1) * G)
        errs.setdefault("o", []).append(rel_l2(f64(o[0, hs, a:a + n]), ro))
        errs.setdefault("dq", []).append(rel_l2(f64(dq[0, hs, a:a + n]), rdq))
        errs.setdefault("lse_abs", []).append(float(np.abs(f64(lse[0, hs, a:a + n]) - rl).max()))
        if keys:
            errs.setdefault("dk", []).append(rel_l2(f64(dk[0, kv, a:a + n]), rdk))
            errs.setdefault("dv", []).append(rel_l2(f64(dv[0, kv, a:a + n]), rdv))
    errs = {k: max(v) for k, v in errs.items()}
    bad = {k: v for k, v in errs.items() if not v <= TOL[k]}
    assert not bad, f"{w.name} rows [{a}, {a + n}): {bad} (all: {errs})"


LIMITS = [
    (synthetic.small("max-chunk-q8", batch=1, prefix_len=300, chunk_len=65536, n_heads_q=4,
                     n_heads_kv=1, head_dim=128, cache_type="q8_0", qkv_std=0.3,
                     prefix_std=1.0, seed=71),
     [(0, 64), (32768 - 17, 40), (65536 - 96, 96)]),
    (synthetic.small("c9000-uniform-split", batch=1, prefix_len=500, chunk_len=9000,
                     n_heads_q=2, n_heads_kv=1, head_dim=64, cache_type="bf16", qkv_std=0.3,
                     prefix_std=0.3, seed=72),
     [(0, 64), (4000, 64), (9000 - 1100, 1100)]),
]


@pytest.mark.parametrize("w,slices", LIMITS, ids=[c[0].name for c in LIMITS])
def test_largest_chunks_sampled(w, slices):
    print(f"{w.name} P{w.prefix_len} C{w.chunk_len} G{w.group} {w.cache_type}", flush=True)
    case = Case(w)
    o, lse = case.fwd()
    dq, dk, dv = case.bwd(o, lse)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    for a, n in slices:
        _check(case, (o, lse, dq, dk, dv), a, n, keys=(a + n == w.chunk_len))
