"""A chunk step captured in a HIP graph and replayed.

The library makes no allocation, memset or synchronisation inside its calls, so one
step (forward, backward, append into the cache; the forward and the append as separate
calls or as one fused launch) can be captured with torch.cuda.graph
and replayed, which removes the launch overhead of small workloads. The kernels are
deterministic: every replay must reproduce the eager step bitwise (O, LSE, dQ, dK, dV
and the appended cache rows). Replays are separated by eager work and synchronisation,
and each is checked.
"""
import pytest
import torch

import synthetic
from _gpu import DEV

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import prefix_kv_attention_amd  # noqa: F401  (fails loudly without libpka.so)


GRAPH_CASES = [
    synthetic.small("graph-q8-split", batch=2, prefix_len=3000, chunk_len=200, n_heads_q=6,
                    n_heads_kv=2, head_dim=128, cache_type="q8_0", prefix_std=1.0, seed=81),
    synthetic.small("graph-f16-d64", batch=3, prefix_len=400, chunk_len=96, n_heads_q=4,
                    n_heads_kv=1, head_dim=64, cache_type="f16", seed=82),
]


@pytest.mark.parametrize("fused", [False, True], ids=["fwd-then-append", "fwd_append"])
@pytest.mark.parametrize("w", GRAPH_CASES, ids=lambda w: w.name)
def test_step_graph_replays_match_eager(w, fused):
    import prefix_kv_attention_amd as pka
    print(f"{w.name} P{w.prefix_len} C{w.chunk_len} {w.cache_type} fused={fused}", flush=True)
    x = synthetic.make_inputs(w)
    d = {k: v.to(DEV) for k, v in x.items()}
    B, Hq, Hkv, D, P, C = w.batch, w.n_heads_q, w.n_heads_kv, w.head_dim, w.prefix_len, w.chunk_len
    sc = w.softmax_scale
    cache = pka.PrefixCache.empty(w.cache_type, B, Hkv, P + C, D, DEV)
    pka.kv_append(d["kp"], d["vp"], cache, 0)
    q, kc, vc, do = d["q"], d["kc"], d["vc"], d["do"]
    dims = pka.make_dims(B, Hq, Hkv, D, P, C, sc)
    nf, nb = pka.fwd_workspace_bytes(dims), pka.bwd_workspace_bytes(dims)
    assert nf > 0 or nb > 0 or w.name == "graph-f16-d64"
    ws_f = torch.empty(max(nf, 1), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)
    outs = {"o": torch.empty_like(q), "lse": torch.empty((B, Hq, C), dtype=torch.float32,
                                                         device=DEV),
            "dq": torch.empty_like(q), "dk": torch.empty_like(kc), "dv": torch.empty_like(vc)}

    def step():
        if fused:   # the bench's step: forward and append in one launch, then backward
            pka.chunk_attn_fwd_append(q, kc, vc, cache, P, sc, o=outs["o"], lse=outs["lse"],
                                      ws=ws_f)
        else:
            pka.chunk_attn_fwd(q, kc, vc, cache, P, sc, o=outs["o"], lse=outs["lse"], ws=ws_f)
        pka.chunk_attn_bwd(q, kc, vc, cache, P, sc, outs["o"], outs["lse"], do, dq=outs["dq"],
                           dk=outs["dk"], dv=outs["dv"], ws=ws_b)
        if not fused:
            pka.kv_append(kc, vc, cache, P)

    def snapshot():
        snap = {k: v.clone() for k, v in outs.items()}
        snap["ck"] = cache.k[:, :, P:].clone()
        snap["cv"] = cache.v[:, :, P:].clone()
        if cache.k_scale is not None:
            snap["cks"] = cache.k_scale[:, :, P:].clone()
        return snap

    step()
    torch.cuda.synchronize()
    ref = snapshot()

    # capture on a side stream (torch's recipe), after a warm-up there
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs.values():      # eager work between replays: clobber the outputs
            t.zero_()
        cache.k[:, :, P:].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"replay {rep}: {k} differs from the eager step"
