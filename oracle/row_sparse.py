"""fp64 oracle of the row-sparse linear backward (test infrastructure only).

What is computed ("stop-gradient through context tokens", Mechanism): a linear layer
y = x W^T keeps its full-row forward, and its backward is compacted to the kept rows,
the token rows that some loss component reads:

  dW        = dY[keep]^T X[keep]          ([out][in])
  dX[keep]  = dY[keep] W                  ([K][in] rows, scattered back to `keep`)
  dX[other] = 0

It equals the dense backward of y = x W^T when the upstream gradient is zero on the
rows not kept: the page applies it only where a gradient mask has already zeroed
those rows, and its own correctness check compares it with that dense reference.

`keep` lists distinct row indices of x (the page builds it with nonzero() of the
keep mask, so it is increasing); W is [out][in], x is [N][in], dY is [N][out].
"""
from __future__ import annotations

import numpy as np


def row_sparse_linear_bwd(x: np.ndarray, w: np.ndarray, dy: np.ndarray,
                          keep: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(dW [out][in], dX [N][in]) in fp64 from x [N][in], w [out][in], dy [N][out] and
    the kept row indices `keep` (int, distinct)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    keep = np.asarray(keep, dtype=np.int64)
    xk = x[keep]                     # [K][in]
    dyk = dy[keep]                   # [K][out]
    dw = dyk.T @ xk                  # [out][in]
    dx = np.zeros_like(x)
    dx[keep] = dyk @ w               # [K][in]
    return dw, dx


def row_sparse_flops(n_keep: int, in_features: int, out_features: int) -> int:
    """Multiply-adds x 2 of both products: dW and dX[keep] are each K*in*out MACs."""
    return 2 * 2 * n_keep * in_features * out_features
