"""GPU parity of the prefix gradient (pka_prefix_kv_grad) against the fp64 oracle.

dK/dV of the last H cached prefix rows from the chunk queries -- the gradient a
stop-gradient prefix drops ("train: walk the window", Why it's a draft: the exact
reverse pass with horizon H). The oracle is group_bwd_prefix (pinned in
test_oracle_prefix_grad.py) on the cache values as the attention reads them.
Bar: relative L2 2e-2, as for the chunk's own dK/dV; rows of windows shorter than
the horizon are exactly zero.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import DEV, Case, f64, rel_l2
from test_gpu_ragged import Ragged

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import prefix_kv_attention_amd  # noqa: F401  (fails loudly without libpka.so)


def _device_grads(pka, w, dev, cache, lens, horizon, plens=None):
    o, lse = pka.chunk_attn_fwd(dev["q"], dev["kc"], dev["vc"], cache, w.prefix_len,
                                w.softmax_scale, prefix_lens=plens)
    delta = torch.empty(lse.shape, dtype=torch.float32, device=DEV)
    pka.chunk_attn_bwd(dev["q"], dev["kc"], dev["vc"], cache, w.prefix_len, w.softmax_scale,
                       o, lse, dev["do"], delta=delta, prefix_lens=plens)
    dk, dv = pka.prefix_kv_grad(dev["q"], cache, w.prefix_len, w.softmax_scale, lse, dev["do"],
                                delta, horizon, prefix_lens=plens)
    torch.cuda.synchronize()
    return f64(dk), f64(dv)


def _oracle_grads(w, inp, kpv, vpv, lens, horizon, groups):
    """Oracle dK/dV [H][D] of the sampled (b, kv) groups, aligned like the device rows."""
    G = w.group
    out = {}
    for b, kv in groups:
        P_b = lens[b]
        hs = slice(kv * G, (kv + 1) * G)
        dkp, dvp = oracle.group_bwd_prefix(
            f64(inp["q"][b, hs]), f64(inp["kc"][b, kv]), f64(inp["vc"][b, kv]),
            kpv[b, kv, :P_b], vpv[b, kv, :P_b], w.softmax_scale, f64(inp["do"][b, hs]))
        dk = np.zeros((horizon, w.head_dim))
        dv = np.zeros((horizon, w.head_dim))
        n = min(horizon, P_b)            # row h <-> cache row P_b - H + h
        if n:
            dk[horizon - n:] = dkp[P_b - n:]
            dv[horizon - n:] = dvp[P_b - n:]
        out[(b, kv)] = (dk, dv)
    return out


def _compare(got_k, got_v, ref, lens, horizon, label):
    ak, rk, av, rv = [], [], [], []
    for (b, kv), (dk, dv) in ref.items():
        ak.append(got_k[b, kv].ravel())
        rk.append(dk.ravel())
        av.append(got_v[b, kv].ravel())
        rv.append(dv.ravel())
        missing = max(0, horizon - lens[b])
        assert np.all(got_k[b, kv, :missing] == 0.0) and np.all(got_v[b, kv, :missing] == 0.0)
    ek = rel_l2(np.concatenate(ak), np.concatenate(rk))
    ev = rel_l2(np.concatenate(av), np.concatenate(rv))
    assert ek <= TOL and ev <= TOL, f"{label}: dK {ek:.3g} dV {ev:.3g}"
    return ek, ev


UNIFORM = [
    (synthetic.small("pg-all-f16", batch=2, prefix_len=300, chunk_len=70, n_heads_q=4,
                     n_heads_kv=2, head_dim=128, cache_type="f16", seed=51), 300),
    (synthetic.small("pg-part-bf16-d64", batch=1, prefix_len=513, chunk_len=64, n_heads_q=6,
                     n_heads_kv=2, head_dim=64, cache_type="bf16", seed=52), 200),
    (synthetic.small("pg-q8", batch=1, prefix_len=900, chunk_len=100, n_heads_q=5,
                     n_heads_kv=1, head_dim=128, cache_type="q8_0", prefix_std=1.0,
                     outlier_frac=0.01, seed=53), 384),
    # one (window, KV head) and many query rows: the rows are split over workgroups
    (synthetic.small("pg-split", batch=1, prefix_len=500, chunk_len=1024, n_heads_q=4,
                     n_heads_kv=1, head_dim=128, cache_type="bf16", qkv_std=0.3,
                     prefix_std=0.3, seed=54), 128),
]


@pytest.mark.parametrize("w,horizon", UNIFORM, ids=[u[0].name for u in UNIFORM])
def test_prefix_grad_parity(w, horizon):
    import prefix_kv_attention_amd as pka
    print(f"{w.name} P{w.prefix_len} H{horizon} C{w.chunk_len} {w.cache_type}", flush=True)
    case = Case(w)
    lens = [w.prefix_len] * w.batch
    dk, dv = _device_grads(pka, w, case.dev, case.cache, lens, horizon)
    kpv, vpv = case.oracle_prefix()
    ref = _oracle_grads(w, case.cpu, kpv, vpv, lens, horizon, case.all_groups())
    _compare(dk, dv, ref, lens, horizon, w.name)


def test_prefix_grad_ragged_windows_shorter_than_horizon():
    import prefix_kv_attention_amd as pka
    lens = [300, 50, 0]
    w = synthetic.small("pg-ragged", batch=3, prefix_len=300, chunk_len=48, n_heads_q=4,
                        n_heads_kv=2, head_dim=128, cache_type="q8_0", prefix_std=1.0, seed=55)
    r = Ragged(w, lens)
    H = 128
    dk, dv = _device_grads(pka, w, r.dev, r.cache, lens, H, plens=r.plens)
    groups = [(b, kv) for b in range(w.batch) for kv in range(w.n_heads_kv)]
    ref = _oracle_grads(w, r.inp, r.prefix_vals[0], r.prefix_vals[1], lens, H, groups)
    _compare(dk, dv, ref, lens, H, "ragged")


def test_prefix_grad_full_size_sampled():
    """q8_0 16k workload at full size, horizon 2048, one sampled (window, KV head)."""
    import prefix_kv_attention_amd as pka
    w = synthetic.WORKLOADS[2]
    H = 2048
    print(f"{w.name} full size, H{H}", flush=True)
    case = Case(w)
    lens = [w.prefix_len] * w.batch
    dk, dv = _device_grads(pka, w, case.dev, case.cache, lens, H)
    assert np.isfinite(dk).all() and np.isfinite(dv).all()
    kpv, vpv = case.oracle_prefix()
    ref = _oracle_grads(w, case.cpu, kpv, vpv, lens, H, [(1, 1)])
    _compare(dk, dv, ref, lens, H, w.name)
