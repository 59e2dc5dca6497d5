"""Whole caches built on the GPU at the workloads' full sizes, byte for byte against the
oracle's converters: every prefix row [0, P) written by one append of the raw bf16
rows, then the chunk's rows [P, P + C) written by the step's append
("train: walk the window", What it is: each trained chunk is re-decoded into the
cache; Contents: the cache constants are F16 or q8_0). q8_0 codes and fp16 scales,
F16 and bf16 values must all be bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import DEV, Case
from oracle.cache import from_torch_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import prefix_kv_attention_amd  # noqa: F401  (fails loudly without libpka.so)


def _u16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("w", synthetic.WORKLOADS[1:], ids=lambda w: w.name)
def test_full_cache_bitexact(w):
    import prefix_kv_attention_amd as pka
    print(f"{w.name}: {w.cache_type} cache of {w.batch} x {w.n_heads_kv} x "
          f"{w.prefix_len + w.chunk_len} rows", flush=True)
    case = Case(w)
    pka.kv_append(case.dev["kc"], case.dev["vc"], case.cache, w.prefix_len)
    torch.cuda.synchronize()
    P, C = w.prefix_len, w.chunk_len
    for name, pre, chunk in (("k", "kp", "kc"), ("v", "vp", "vc")):
        raw = np.concatenate([from_torch_bf16(case.cpu[pre]), from_torch_bf16(case.cpu[chunk])],
                             axis=2)                                  # [B][Hkv][P+C][D]
        ref = oracle.build_prefix(raw, w.cache_type)
        store = getattr(case.cache, name)[:, :, :P + C]
        if w.cache_type == "q8_0":
            scale = getattr(case.cache, name + "_scale")[:, :, :P + C]
            got_q = store.cpu().numpy()
            got_d = _u16(scale)
            bad_q = np.argwhere(got_q != ref["qs"])
            bad_d = np.argwhere(got_d != ref["d"].view(np.uint16))
            assert bad_q.size == 0, f"{name}: {len(bad_q)} codes differ, first {bad_q[:3]}"
            assert bad_d.size == 0, f"{name}: {len(bad_d)} scales differ, first {bad_d[:3]}"
        elif w.cache_type == "f16":
            np.testing.assert_array_equal(_u16(store), ref["f16"].view(np.uint16))
        else:
            np.testing.assert_array_equal(_u16(store), ref["bits"])
        del raw, ref
