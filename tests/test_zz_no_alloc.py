"""pka_chunk_attn_bwd_noalloc (the backward with the library's own fixed workspace, for
callers that cannot allocate) against pka_chunk_attn_bwd with a caller workspace: the
same kernels and plan, so every output must match bit for bit. Two calls in a row on
one GPU, the second with a smaller input (the array keeps the first call's contents),
then a shape whose workspace exceeds the fixed size, which must be refused before any
launch.
"""
import pytest
import torch

import synthetic
from _gpu import DEV, Case

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _check_case(w):
    import prefix_kv_attention_amd as pka
    print(f"{w.name}: B{w.batch} Hq{w.n_heads_q} Hkv{w.n_heads_kv} D{w.head_dim} "
          f"P{w.prefix_len} C{w.chunk_len} {w.cache_type}", flush=True)
    case = Case(w)
    d = case.dev
    o, lse = case.fwd()
    ref_delta = torch.empty(lse.shape, dtype=torch.float32, device=DEV)
    ref = case.bwd(o, lse, delta=ref_delta)
    dq, dk, dv = (torch.full_like(t, 7.0) for t in ref)
    delta = torch.full_like(ref_delta, 3.0)
    out = pka.chunk_attn_bwd_noalloc(d["q"], d["kc"], d["vc"], case.cache, w.prefix_len,
                                     w.softmax_scale, o, lse, d["do"], dq, dk, dv,
                                     delta=delta)
    torch.cuda.synchronize()
    for a, b in zip(out + (delta,), ref + (ref_delta,)):
        assert torch.equal(_bits(a), _bits(b))


def test_noalloc_matches_the_workspace_call_twice_then_smaller():
    import prefix_kv_attention_amd as pka
    big = synthetic.WORKLOAD_BY_NAME["q8_0-16k"]        # prefix and row splits: 62 MiB
    small = synthetic.small("noalloc-small", batch=2, prefix_len=900, chunk_len=130,
                            n_heads_q=6, n_heads_kv=2, head_dim=64, cache_type="f16",
                            qkv_std=0.5, prefix_std=0.5)
    dims = [pka.make_dims(w.batch, w.n_heads_q, w.n_heads_kv, w.head_dim, w.prefix_len,
                          w.chunk_len, w.softmax_scale) for w in (big, small)]
    need = [pka.bwd_workspace_bytes(x) for x in dims]
    assert need[0] > need[1] > 0
    assert need[0] <= pka.BWD_NOALLOC_MAX_WORKSPACE
    _check_case(big)
    _check_case(small)


def test_noalloc_headline_shape():
    _check_case(synthetic.HEADLINE)


def test_noalloc_refuses_shapes_beyond_its_workspace():
    import prefix_kv_attention_amd as pka
    # 8 windows x 64 heads x 65,536 chunk rows: delta alone is 128 MiB of fp32
    B, Hq, Hkv, D, P, C = 8, 64, 64, 64, 0, 65536
    dims = pka.make_dims(B, Hq, Hkv, D, P, C, 0.125)
    assert pka.bwd_workspace_bytes(dims) > pka.BWD_NOALLOC_MAX_WORKSPACE
    q = torch.zeros((1, 1, 1, 8), dtype=torch.bfloat16, device=DEV)   # never read
    cache = pka.PrefixCache.empty("bf16", B, Hkv, 1, D, DEV)
    from prefix_kv_attention_amd import _lib, _ptr, _stream
    import ctypes
    cd = cache.desc()
    st = _lib.pka_chunk_attn_bwd_noalloc(ctypes.byref(dims), _ptr(q), _ptr(q), _ptr(q),
                                         ctypes.byref(cd), _ptr(q), _ptr(q), _ptr(q),
                                         _ptr(q), _ptr(q), _ptr(q), None, _stream(q.device))
    assert pka.STATUS[st] == "PKA_ERR_WORKSPACE"
    assert b"fixed" in _lib.pka_last_error()
