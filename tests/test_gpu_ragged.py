"""GPU parity of ragged windows and of the chunk walk, through the C-ABI.

Ragged windows: one call serves B windows whose cached prefixes have different
lengths P_b (pka_dims.prefix_lens); window b's chunk row i attends to its own cache
rows 0..P_b-1 and chunk rows 0..i, and its append writes rows [P_b, P_b + C). The
oracle computes every window on its own, from its own P_b prefix rows.

The walk ("train: walk the window", What it is: train a chunk against the cached
prefix, re-decode it into the cache, move on) runs several chunks of a ragged batch
through WindowWalk and checks every step against the oracle on the concatenation
of the initial prefix and the chunks appended so far.

Bars as in test_gpu_parity: O 1e-2, dQ/dK/dV 2e-2 relative L2, LSE 5e-3 absolute,
appended rows bit-exact.
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


def _oracle_cache_rows(raw_bf16, cache_type):
    """Oracle cache values (fp64) of raw bf16 rows [..][rows][D] in a storage type."""
    return oracle.build_prefix(from_torch_bf16(raw_bf16), cache_type)["values"]


def _oracle_window(w, inp, b, kp_vals, vp_vals, P_b):
    """Oracle outputs of window b with prefix rows [0, P_b) of kp_vals / vp_vals."""
    G = w.group
    out = {k: [] for k in ("o", "lse", "dq", "dk", "dv")}
    for kv in range(w.n_heads_kv):
        hs = slice(kv * G, (kv + 1) * G)
        q = f64(inp["q"][b, hs])
        kc, vc = f64(inp["kc"][b, kv]), f64(inp["vc"][b, kv])
        do = f64(inp["do"][b, hs])
        kp, vp = kp_vals[b, kv, :P_b], vp_vals[b, kv, :P_b]
        o, lse = oracle.group_fwd(q, kc, vc, kp, vp, w.softmax_scale)
        dq, dk, dv, _ = oracle.group_bwd(q, kc, vc, kp, vp, w.softmax_scale, do)
        for k, val in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            out[k].append(val)
    return {k: np.stack(v) for k, v in out.items()}


def _check_windows(w, inp, prefix_vals, lens, o, lse, dq, dk, dv, label):
    """Compare every window of the device outputs with the per-window oracle."""
    kpv, vpv = prefix_vals
    G = w.group
    acc = {k: ([], []) for k in ("o", "dq", "dk", "dv")}
    lse_err = 0.0
    for b, P_b in enumerate(lens):
        ref = _oracle_window(w, inp, b, kpv, vpv, P_b)
        gpu = {"o": f64(o[b]).reshape(w.n_heads_kv, G, w.chunk_len, w.head_dim),
               "dq": f64(dq[b]).reshape(w.n_heads_kv, G, w.chunk_len, w.head_dim),
               "dk": f64(dk[b]), "dv": f64(dv[b])}
        for k in acc:
            acc[k][0].append(gpu[k].ravel())
            acc[k][1].append(ref[k].ravel())
        lse_gpu = f64(lse[b]).reshape(w.n_heads_kv, G, w.chunk_len)
        lse_err = max(lse_err, float(np.abs(lse_gpu - ref["lse"]).max()))
    errs = {k: rel_l2(np.concatenate(a), np.concatenate(r)) for k, (a, r) in acc.items()}
    errs["lse_abs"] = lse_err
    bad = {k: v for k, v in errs.items() if not v <= TOL[k]}
    assert not bad, f"{label}: {bad} (all: {errs})"
    return errs


class Ragged:
    """Device inputs of one ragged chunk step; the cache holds the longest prefix."""

    def __init__(self, w, lens, extra_capacity=0):
        import prefix_kv_attention_amd as pka
        self.pka, self.w, self.lens = pka, w, list(lens)
        assert max(lens) == w.prefix_len
        self.inp = synthetic.make_inputs(w)
        self.dev = {k: v.to(DEV) for k, v in self.inp.items() if k not in ("kp", "vp")}
        self.cache = pka.PrefixCache.empty(w.cache_type, w.batch, w.n_heads_kv,
                                           w.prefix_len + w.chunk_len + extra_capacity,
                                           w.head_dim, DEV)
        if w.prefix_len > 0:   # rows past a window's own P_b are written but never read
            pka.kv_append(self.inp["kp"].to(DEV), self.inp["vp"].to(DEV), self.cache, 0)
        self.plens = torch.tensor(self.lens, dtype=torch.int32, device=DEV)
        self.prefix_vals = (_oracle_cache_rows(self.inp["kp"], w.cache_type),
                            _oracle_cache_rows(self.inp["vp"], w.cache_type))

    def run(self, plens=None):
        d, w = self.dev, self.w
        plens = self.plens if plens is None else plens
        o, lse = self.pka.chunk_attn_fwd(d["q"], d["kc"], d["vc"], self.cache, w.prefix_len,
                                         w.softmax_scale, prefix_lens=plens)
        dq, dk, dv = self.pka.chunk_attn_bwd(d["q"], d["kc"], d["vc"], self.cache,
                                             w.prefix_len, w.softmax_scale, o, lse, d["do"],
                                             prefix_lens=plens)
        torch.cuda.synchronize()
        return o, lse, dq, dk, dv


RAGGED = [
    (synthetic.small("rag-f16", batch=4, prefix_len=700, chunk_len=70, n_heads_q=4,
                     n_heads_kv=2, head_dim=128, cache_type="f16", seed=41),
     [0, 100, 333, 700]),
    (synthetic.small("rag-bf16-d64", batch=3, prefix_len=513, chunk_len=64, n_heads_q=6,
                     n_heads_kv=2, head_dim=64, cache_type="bf16", seed=42),
     [513, 1, 64]),
    (synthetic.small("rag-q8", batch=3, prefix_len=900, chunk_len=100, n_heads_q=5,
                     n_heads_kv=1, head_dim=128, cache_type="q8_0", prefix_std=1.0,
                     outlier_frac=0.01, seed=43),
     [900, 257, 0]),
    # few (window, KV head) units: the prefix is split over workgroups per window
    (synthetic.small("rag-split", batch=2, prefix_len=3000, chunk_len=128, n_heads_q=2,
                     n_heads_kv=1, head_dim=128, cache_type="bf16", qkv_std=0.3,
                     prefix_std=0.3, seed=44),
     [3000, 700]),
]


@pytest.mark.parametrize("w,lens", RAGGED, ids=[r[0].name for r in RAGGED])
def test_ragged_parity(w, lens):
    print(f"{w.name} P_b={lens} C{w.chunk_len} {w.cache_type}", flush=True)
    r = Ragged(w, lens)
    _check_windows(w, r.inp, r.prefix_vals, lens, *r.run(), label=w.name)


def test_ragged_prefix_lens_are_clamped():
    """Entries above prefix_len act as prefix_len, negative ones as 0."""
    w = synthetic.small("rag-clamp", batch=3, prefix_len=300, chunk_len=40, n_heads_q=2,
                        n_heads_kv=1, head_dim=64, cache_type="bf16", seed=45)
    r = Ragged(w, [300, 0, 120])
    ref = r.run()
    wild = torch.tensor([1 << 30, -5, 120], dtype=torch.int32, device=DEV)
    got = r.run(plens=wild)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


@pytest.mark.parametrize("ct", ["q8_0", "f16", "bf16"])
def test_ragged_append_bitexact(ct):
    """Appends land at each window's own prefix end; other rows keep their bits."""
    import prefix_kv_attention_amd as pka
    lens = [17, 0, 200]
    w = synthetic.small("rag-app", batch=3, prefix_len=200, chunk_len=33, n_heads_q=2,
                        n_heads_kv=2, head_dim=128, cache_type=ct, prefix_std=1.0, seed=46)
    r = Ragged(w, lens)
    before_k = r.cache.k.clone()
    before_ks = None if r.cache.k_scale is None else r.cache.k_scale.clone()
    pka.kv_append(r.dev["kc"], r.dev["vc"], r.cache, w.prefix_len, prefix_lens=r.plens)
    torch.cuda.synchronize()
    want_k = oracle.build_prefix(from_torch_bf16(r.inp["kc"]), ct)
    want_v = oracle.build_prefix(from_torch_bf16(r.inp["vc"]), ct)
    for b, P_b in enumerate(lens):
        rows = slice(P_b, P_b + w.chunk_len)
        for got, want in ((r.cache.k, want_k), (r.cache.v, want_v)):
            g = got[b, :, rows].cpu()
            if ct == "q8_0":
                assert np.array_equal(g.numpy(), want["qs"][b])
            elif ct == "f16":
                assert np.array_equal(g.view(torch.int16).numpy(), want["f16"][b].view(np.int16))
            else:
                assert np.array_equal(g.view(torch.int16).numpy(), want["bits"][b].view(np.int16))
        if ct == "q8_0":
            for got, want in ((r.cache.k_scale, want_k), (r.cache.v_scale, want_v)):
                g = got[b, :, rows].cpu().view(torch.int16).numpy()
                assert np.array_equal(g, want["d"][b].view(np.int16))
        # rows before the window's prefix end are untouched
        assert torch.equal(r.cache.k[b, :, :P_b], before_k[b, :, :P_b])
        if before_ks is not None:
            assert torch.equal(r.cache.k_scale[b, :, :P_b], before_ks[b, :, :P_b])


@pytest.mark.parametrize("ct", ["q8_0", "bf16"])
def test_walk_ragged_three_chunks(ct):
    """Three chunk steps of a ragged batch: each step's outputs equal the oracle over
    the initial prefix plus the chunks appended before it."""
    import prefix_kv_attention_amd as pka
    lens0 = [50, 300, 128]
    C, steps = 64, 3
    base = synthetic.small("walk-rag", batch=3, prefix_len=max(lens0), chunk_len=C,
                           n_heads_q=4, n_heads_kv=2, head_dim=128, cache_type=ct,
                           prefix_std=0.5, seed=47)
    r = Ragged(base, lens0, extra_capacity=C * steps)
    walk = pka.WindowWalk(r.cache, lens0, base.softmax_scale)
    # oracle prefix per window: list of raw bf16 row blocks, grown by every chunk
    raw_k = [[r.inp["kp"][b, :, :P]] for b, P in enumerate(lens0)]
    raw_v = [[r.inp["vp"][b, :, :P]] for b, P in enumerate(lens0)]
    for s in range(steps):
        w = base if s == 0 else base.with_(seed=base.seed + 100 * s)
        inp = r.inp if s == 0 else synthetic.make_inputs(w)
        dev = {k: inp[k].to(DEV) for k in ("q", "kc", "vc", "do")}
        lens = list(walk.lens)
        print(f"walk step {s}: P_b={lens} {ct}", flush=True)
        o, lse, dq, dk, dv = walk.step(dev["q"], dev["kc"], dev["vc"], dev["do"])
        torch.cuda.synchronize()
        Pm = max(lens)
        kpv = np.zeros((w.batch, w.n_heads_kv, Pm, w.head_dim))
        vpv = np.zeros_like(kpv)
        for b in range(w.batch):
            kb = torch.cat(raw_k[b], dim=1)
            vb = torch.cat(raw_v[b], dim=1)
            assert kb.shape[1] == lens[b]
            if lens[b]:
                kpv[b, :, :lens[b]] = _oracle_cache_rows(kb, ct)
                vpv[b, :, :lens[b]] = _oracle_cache_rows(vb, ct)
        _check_windows(w, inp, (kpv, vpv), lens, o, lse, dq, dk, dv, f"walk step {s}")
        for b in range(w.batch):
            raw_k[b].append(inp["kc"][b])
            raw_v[b].append(inp["vc"][b])
        assert walk.lens == [p + C for p in lens]
