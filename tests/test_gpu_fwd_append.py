"""GPU tests of the forward fused with the re-decode into the cache
(pka_chunk_attn_fwd_append).

The fused launch must change no value: O and LSE bitwise equal to pka_chunk_attn_fwd
and the cache bitwise equal to what pka_kv_append_* writes (both of which are checked
against the oracle elsewhere). Cases cover every cache type, D = 64 and 128, ragged
windows and prefix splits (several workgroups share the append of one unit). A
prefill walk builds a whole context chunk by chunk with WindowWalk.decode and must
leave the same cache as one append of all the rows, and its last chunk's outputs
must match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import DEV, TOL, f64, rel_l2
from oracle.cache import from_torch_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import prefix_kv_attention_amd  # noqa: F401  (fails loudly without libpka.so)


def _cache_like(pka, c):
    n = pka.PrefixCache.empty(c.cache_type, c.batch, c.n_heads_kv, c.capacity, c.head_dim, DEV)
    for a, b in ((n.k, c.k), (n.v, c.v), (n.k_scale, c.k_scale), (n.v_scale, c.v_scale)):
        if a is not None:
            a.copy_(b)
    return n


def _same_cache(a, b):
    for x, y in ((a.k, b.k), (a.v, b.v), (a.k_scale, b.k_scale), (a.v_scale, b.v_scale)):
        if x is not None:
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


CASES = [
    (synthetic.small("fa-q8", batch=2, prefix_len=700, chunk_len=100, n_heads_q=6,
                     n_heads_kv=2, head_dim=128, cache_type="q8_0", prefix_std=1.0, seed=61),
     None),
    (synthetic.small("fa-f16-d64", batch=1, prefix_len=513, chunk_len=70, n_heads_q=4,
                     n_heads_kv=1, head_dim=64, cache_type="f16", seed=62), None),
    (synthetic.small("fa-bf16-split", batch=1, prefix_len=3000, chunk_len=256, n_heads_q=2,
                     n_heads_kv=1, head_dim=128, cache_type="bf16", seed=63), None),
    (synthetic.small("fa-ragged-q8", batch=3, prefix_len=800, chunk_len=64, n_heads_q=4,
                     n_heads_kv=2, head_dim=128, cache_type="q8_0", prefix_std=1.0, seed=64),
     [800, 0, 333]),
]


@pytest.mark.parametrize("w,lens", CASES, ids=[c[0].name for c in CASES])
def test_fused_equals_forward_then_append(w, lens):
    import prefix_kv_attention_amd as pka
    print(f"{w.name} P{w.prefix_len} C{w.chunk_len} {w.cache_type} lens={lens}", flush=True)
    inp = synthetic.make_inputs(w)
    d = {k: inp[k].to(DEV) for k in ("q", "kc", "vc")}
    cap = w.prefix_len + w.chunk_len + 17
    base = pka.PrefixCache.empty(w.cache_type, w.batch, w.n_heads_kv, cap, w.head_dim, DEV)
    for t in (base.k, base.v, base.k_scale, base.v_scale):
        if t is not None:
            t.view(torch.uint8).fill_(0x5A)     # rows nobody writes keep this pattern
    pka.kv_append(inp["kp"].to(DEV), inp["vp"].to(DEV), base, 0)
    plens = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    ref_cache, fused_cache = _cache_like(pka, base), _cache_like(pka, base)
    o1, l1 = pka.chunk_attn_fwd(d["q"], d["kc"], d["vc"], ref_cache, w.prefix_len,
                                w.softmax_scale, prefix_lens=plens)
    pka.kv_append(d["kc"], d["vc"], ref_cache, w.prefix_len, prefix_lens=plens)
    o2, l2 = pka.chunk_attn_fwd_append(d["q"], d["kc"], d["vc"], fused_cache, w.prefix_len,
                                       w.softmax_scale, prefix_lens=plens)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    _same_cache(ref_cache, fused_cache)


@pytest.mark.parametrize("ct", ["q8_0", "bf16"])
def test_prefill_walk_builds_the_cache(ct):
    """Phase 1: fill a context into the cache chunk by chunk with the fused launch."""
    import prefix_kv_attention_amd as pka
    C, n = 96, 4
    w = synthetic.small("prefill", batch=2, prefix_len=C * n, chunk_len=C, n_heads_q=4,
                        n_heads_kv=2, head_dim=128, cache_type=ct, prefix_std=0.5, seed=65)
    full = synthetic.make_inputs(w)          # kp / vp: the whole context's K/V rows
    walk_cache = pka.PrefixCache.empty(ct, w.batch, w.n_heads_kv, C * n, w.head_dim, DEV)
    walk = pka.WindowWalk(walk_cache, [0] * w.batch, w.softmax_scale)
    rng = np.random.default_rng(7)
    for s in range(n):
        k = full["kp"][:, :, s * C:(s + 1) * C].contiguous()
        v = full["vp"][:, :, s * C:(s + 1) * C].contiguous()
        qn = rng.standard_normal((w.batch, w.n_heads_q, C, w.head_dim), dtype=np.float32) * 0.5
        q = torch.from_numpy(qn).to(torch.bfloat16)
        o, lse = walk.decode(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert walk.lens == [C * n] * w.batch
    ref_cache = pka.PrefixCache.empty(ct, w.batch, w.n_heads_kv, C * n, w.head_dim, DEV)
    pka.kv_append(full["kp"].to(DEV), full["vp"].to(DEV), ref_cache, 0)
    torch.cuda.synchronize()
    _same_cache(ref_cache, walk_cache)
    # the last chunk against the oracle (its prefix: the first n - 1 chunks)
    P = C * (n - 1)
    kp = oracle.build_prefix(from_torch_bf16(full["kp"][:, :, :P]), ct)["values"]
    vp = oracle.build_prefix(from_torch_bf16(full["vp"][:, :, :P]), ct)["values"]
    kc = f64(full["kp"][:, :, P:])
    vc = f64(full["vp"][:, :, P:])
    ro, rl = oracle.chunk_fwd(f64(q), kc, vc, kp, vp, w.softmax_scale)
    assert rel_l2(f64(o), ro) <= TOL["o"]
    assert float(np.abs(f64(lse) - rl).max()) <= TOL["lse_abs"]
