"""GPU parity of the row-sparse linear backward (pka_row_sparse_linear_bwd) against
the fp64 oracle ("stop-gradient through context tokens", Mechanism).

Tolerances. The inputs are bf16 (exact in fp64) and the kernels accumulate in fp32:
  * dW is written in fp32. A sum of K bf16 products accumulated in fp32 has a
    relative error of order sqrt(K) * 2^-24 (K = 2048: 3e-6); the bar is 1e-4 relative
    L2, far below what a wrong row, feature or sign produces.
  * dX is written in bf16: rounding alone gives about 2^-9 / sqrt(3) = 1.1e-3 relative
    L2; the bar is 1e-2 (the forward output's bar).
  * dX rows that are not kept must be exactly zero.
Cases span several 128 x 128 tiles with ragged kept-row counts (K not a multiple of
the 64-row k-stage or of the 128-row tile), a single kept row, no kept row, every row
kept, few kept rows (the dX product split over output features into a workspace, 2
and 8 splits), grids of over 500 tiles (both products, ragged K), an unsorted kept
list, entries outside [0, N), one product at a time,
and the projection shapes of a 1.7B-class layer at sequence length 2048 (kept
fraction 0.5, checked in full against the oracle).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import DEV, f64, rel_l2

pytestmark = pytest.mark.gpu

TOL_DW, TOL_DX = 1e-4, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import prefix_kv_attention_amd  # noqa: F401  (fails loudly without libpka.so)


def run(inp, keep=None, want_dw=True, want_dx=True):
    import prefix_kv_attention_amd as pka
    keep = inp["keep"] if keep is None else keep
    dw, dx = pka.row_sparse_linear_bwd(inp["x"].to(DEV), inp["w"].to(DEV), inp["dy"].to(DEV),
                                       keep.to(DEV), want_dw=want_dw, want_dx=want_dx)
    torch.cuda.synchronize()
    return dw, dx


def check(inp, dw, dx, keep=None):
    keep = (inp["keep"] if keep is None else keep).numpy().astype(np.int64)
    n = inp["x"].shape[0]
    valid = keep[(keep >= 0) & (keep < n)]
    rdw, rdx = oracle.row_sparse_linear_bwd(f64(inp["x"]), f64(inp["w"]), f64(inp["dy"]),
                                            valid)
    if dw is not None:
        e = rel_l2(f64(dw), rdw)
        assert e <= TOL_DW, f"dW rel L2 {e:.3e}"
    if dx is not None:
        gx = f64(dx)
        e = rel_l2(gx, rdx)
        assert e <= TOL_DX, f"dX rel L2 {e:.3e}"
        other = np.setdiff1d(np.arange(n), valid)
        assert np.all(gx[other] == 0.0), "a row that is not kept got a nonzero gradient"


CASES = [  # (name, N, in, out, kept fraction, seed)
    ("ragged-k150", 300, 256, 384, 0.5, 1),
    ("tiles-3x5", 640, 384, 640, 0.62, 2),
    ("k1", 512, 128, 128, 1 / 512, 3),
    ("all-kept", 256, 256, 128, 1.0, 4),
    ("frac0.1-dx-split2", 2048, 256, 512, 0.1, 5),
    ("dx-split8-ragged", 700, 256, 2048, 0.19, 12),
    ("big-dw-grid-k350", 700, 2048, 4096, 0.5, 13),        # 512 dW tiles, ragged K
    ("big-dx-grid-k2058", 2100, 4096, 256, 0.98, 14),      # 544 dX tiles, ragged K
]


@pytest.mark.parametrize("name,n,fin,fout,frac,seed", CASES, ids=[c[0] for c in CASES])
def test_row_sparse_matches_oracle(name, n, fin, fout, frac, seed):
    import prefix_kv_attention_amd as pka
    inp = synthetic.row_sparse_inputs(n, fin, fout, frac, seed)
    k = inp["keep"].numel()
    print(f"{name} N{n} in{fin} out{fout} K{k} ws {pka.row_sparse_workspace_bytes(n, k, fin, fout)}",
          flush=True)
    if "split" in name:
        assert pka.row_sparse_workspace_bytes(n, k, fin, fout) > 0
    dw, dx = run(inp)
    check(inp, dw, dx)


def test_no_row_kept():
    inp = synthetic.row_sparse_inputs(200, 128, 256, 0.0, 6)
    assert inp["keep"].numel() == 0
    dw, dx = run(inp)
    assert not dw.any() and not dx.float().any()


def test_unsorted_keep_and_out_of_range_entries():
    inp = synthetic.row_sparse_inputs(400, 256, 256, 0.5, 7)
    k = inp["keep"].numpy()
    rng = np.random.default_rng(8)
    shuffled = torch.from_numpy(rng.permutation(k).astype(np.int32))
    dw, dx = run(inp, keep=shuffled)
    check(inp, dw, dx, keep=shuffled)
    # entries outside [0, N) add nothing and write nothing
    bad = torch.from_numpy(np.concatenate([[-5], k[:50], [400, 10**6], k[50:]]).astype(np.int32))
    dw2, dx2 = run(inp, keep=bad)
    check(inp, dw2, dx2, keep=bad)


def test_one_product_at_a_time():
    inp = synthetic.row_sparse_inputs(300, 256, 128, 0.4, 9)
    dw, dx = run(inp, want_dx=False)
    assert dx is None
    check(inp, dw, None)
    dw, dx = run(inp, want_dw=False)
    assert dw is None
    check(inp, None, dx)


def test_deterministic():
    inp = synthetic.row_sparse_inputs(640, 384, 640, 0.5, 10)
    a = run(inp)
    b = run(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("proj", synthetic.LAYER_1_7B, ids=lambda s: s.name)
def test_layer_1_7b_seq2048_full(proj):
    """Full-size projections at N = 2048 tokens, kept fraction 0.5 (all outputs)."""
    print(f"{proj.name} in{proj.in_features} out{proj.out_features}", flush=True)
    inp = synthetic.row_sparse_inputs(2048, proj.in_features, proj.out_features, 0.5, 11)
    dw, dx = run(inp)
    check(inp, dw, dx)
