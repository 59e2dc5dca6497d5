"""Pins of the oracle's row-sparse linear backward -- CPU only.

oracle.row_sparse_linear_bwd gives dW = dY[keep]^T X[keep] and dX (kept rows
dY[keep] W, other rows zero) of y = x W^T ("stop-gradient through context tokens",
Mechanism). It is tied to:
  * torch autograd (fp64) of the dense layer y = x @ W^T with the upstream gradient
    zeroed on the rows not kept -- the reference the page checks its own kernel
    against ("row-sparse linear backward == dense torch.where(detach) reference");
  * a brute-force sum over rows, output features and input features on tiny shapes;
  * special cases: every row kept (plain dense backward), no row kept (all zero);
  * additivity of dW over disjoint sets of kept rows;
and planted mistakes (W transposed, the first K rows instead of the kept ones, dW
transposed) must each break the autograd pin.
"""
import numpy as np
import pytest
import torch

from oracle.row_sparse import row_sparse_flops, row_sparse_linear_bwd


def rel(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))


def case(n, fin, fout, frac, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, fin))
    w = rng.standard_normal((fout, fin)) * 0.1
    dy = rng.standard_normal((n, fout))
    keep = np.sort(rng.choice(n, size=int(round(frac * n)), replace=False))
    return x, w, dy, keep


def autograd_ref(x, w, dy, keep):
    """Dense backward of y = x @ w^T with dY zeroed outside `keep` (torch, fp64)."""
    mask = np.zeros(x.shape[0], dtype=bool)
    mask[keep] = True
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    y = xt @ wt.T
    g = torch.where(torch.tensor(mask)[:, None], torch.tensor(dy), torch.zeros(()))
    y.backward(g)
    return wt.grad.numpy(), xt.grad.numpy()


def pin_autograd(fn, x, w, dy, keep, tol=1e-12):
    dw, dx = fn(x, w, dy, keep)
    rdw, rdx = autograd_ref(x, w, dy, keep)
    return dw.shape == rdw.shape and dx.shape == rdx.shape and \
        rel(dw, rdw) <= tol and rel(dx, rdx) <= tol


SHAPES = [(37, 24, 40, 0.62, 1), (64, 48, 48, 0.5, 2), (50, 32, 16, 0.1, 3),
          (20, 8, 12, 1.0, 4)]


@pytest.mark.parametrize("n,fin,fout,frac,seed", SHAPES)
def test_matches_autograd_of_masked_dense_layer(n, fin, fout, frac, seed):
    x, w, dy, keep = case(n, fin, fout, frac, seed)
    assert pin_autograd(row_sparse_linear_bwd, x, w, dy, keep)


def test_rows_not_kept_get_exactly_zero():
    x, w, dy, keep = case(40, 16, 24, 0.3, 5)
    _, dx = row_sparse_linear_bwd(x, w, dy, keep)
    other = np.setdiff1d(np.arange(40), keep)
    assert np.all(dx[other] == 0.0)
    assert np.all(np.abs(dx[keep]).sum(axis=1) > 0)


def test_brute_force_tiny():
    x, w, dy, keep = case(7, 3, 5, 0.5, 6)
    dw, dx = row_sparse_linear_bwd(x, w, dy, keep)
    for o in range(5):
        for i in range(3):
            s = 0.0
            for r in keep:
                s += dy[r, o] * x[r, i]
            assert abs(dw[o, i] - s) <= 1e-12 * max(1.0, abs(s))
    for r in range(7):
        for i in range(3):
            s = sum(dy[r, o] * w[o, i] for o in range(5)) if r in set(keep) else 0.0
            assert abs(dx[r, i] - s) <= 1e-12 * max(1.0, abs(s))


def test_every_row_kept_is_the_dense_backward():
    x, w, dy, _ = case(30, 12, 20, 0.5, 7)
    dw, dx = row_sparse_linear_bwd(x, w, dy, np.arange(30))
    assert rel(dw, dy.T @ x) <= 1e-14 and rel(dx, dy @ w) <= 1e-14


def test_no_row_kept_is_zero():
    x, w, dy, _ = case(9, 4, 6, 0.5, 8)
    dw, dx = row_sparse_linear_bwd(x, w, dy, np.zeros(0, dtype=np.int64))
    assert dw.shape == (6, 4) and dx.shape == (9, 4)
    assert not dw.any() and not dx.any()


def test_dw_adds_over_disjoint_kept_sets():
    x, w, dy, keep = case(48, 16, 20, 0.75, 9)
    a, b = keep[::2], keep[1::2]
    dw, dx = row_sparse_linear_bwd(x, w, dy, keep)
    dwa, dxa = row_sparse_linear_bwd(x, w, dy, a)
    dwb, dxb = row_sparse_linear_bwd(x, w, dy, b)
    assert rel(dw, dwa + dwb) <= 1e-14 and rel(dx, dxa + dxb) <= 1e-14


def test_flop_count():
    assert row_sparse_flops(1024, 2048, 6144) == 4 * 1024 * 2048 * 6144


# Planted mistakes (square W, so every variant has valid shapes): each must fail the
# autograd pin.
def _w_transposed(x, w, dy, keep):
    dw, dx = row_sparse_linear_bwd(x, w, dy, keep)
    dx = np.zeros_like(x)
    dx[keep] = dy[keep] @ w.T
    return dw, dx


def _first_rows(x, w, dy, keep):
    k = len(keep)
    dw = dy[keep].T @ x[:k]
    return dw, row_sparse_linear_bwd(x, w, dy, keep)[1]


def _dw_transposed(x, w, dy, keep):
    dw, dx = row_sparse_linear_bwd(x, w, dy, keep)
    return dw.T, dx


@pytest.mark.parametrize("bad", [_w_transposed, _first_rows, _dw_transposed])
def test_planted_mistakes_fail_the_pin(bad):
    x, w, dy, keep = case(40, 24, 24, 0.5, 10)
    assert pin_autograd(row_sparse_linear_bwd, x, w, dy, keep)
    assert not pin_autograd(bad, x, w, dy, keep)
