"""Per-element error bounds of the GPU's bf16 / fp32 arithmetic, for sampled parity.

One relative-L2 norm over a whole tensor can hide a few wrong rows, so the sampled
full-size parity tests also check every output element against a first-order bound
on what the GPU's roundings can do to it. The bound follows the GPU's arithmetic step
by step, using the oracle's fp64 intermediates (probabilities P, dP = dO Vf^T, Delta,
dS) and absolute values of the operands. Notation, per (query row i, key j, dim d):

  u     = 2^-8: twice the unit roundoff of bf16 round-to-nearest (the factor 2 covers
          the second-order terms that the first-order sums below drop);
  g(n)  = n 2^-24: worst-case relative error of an fp32 sum of n products;
  rk_j, rv_j = u for a prefix row of an F16 / q8_0 cache (the MFMA reads it rounded
          to bf16), 0 for a bf16 cache row and for the chunk's own rows (exact);
  Aqk   = |Q| |Kf|^T,  Adv = |dO| |Vf|^T  (fp64 matrices over the allowed pairs).

  scores:   |ds_ij| <= scale (rk_j + g(D)) Aqk_ij
  forward probabilities: relative error e_ij = u + |ds_ij| (bf16 of exp2 of the
            perturbed score); the normaliser sums the same rounded values, so the
            weights move by at most e_ij + ebar_i, ebar = sum_j P_ij e_ij;
  O:        |dO_id| <= ((P o e) |V| + ebar (P |V|) + (P o rv) |V|)_id
                       + g(P + C) (P |V|)_id + u |O_id|
  LSE:      |dLSE_i| <= ebar_i + g(P + C)
  Delta:    |dDelta_i| <= sum_d |dO_id| (bO_id + u |O_id|) + g(D) sum_d |dO_id O_id|
            =: eD_i  (Delta reads the stored bf16 O)
  backward probabilities: P~ = P exp(ds_ij - dLSE_i) to first order: a relative error
            eb_ij = |ds_ij| + 1e-6 (exp2) per element, and the factor exp(-dLSE_i),
            common to the whole row;
  dP:       |d dP_ij| <= (rv_j + g(D)) Adv_ij =: eP_ij
  dS:       dS~ = bf16(P~ (dP~ - Delta~)): per element (eb_ij + u) |dS_ij| + P_ij eP_ij,
            the row factor -dLSE_i dS_ij and the row term -P_ij dDelta_i;
  dQ:       the row terms sum to -dLSE_i dQ_id and -scale dDelta_i (P Kf)_id, so
            |d dQ_id| <= scale [((eb + u + rk + g(n)) |dS| + P eP) |Kf|]_id
                         + scale eD_i |(P Kf)_id| + (bLSE_i + u) |dQ_id|
            (rk: K read rounded; g(n): the sum over n = P + C keys);
  dK (chunk key t, summed over the G heads, m = G C rows; the row terms now differ
      from row to row and are bounded one by one):
            <= scale sum_g [((eb + bLSE + u + g(m)) |dS| + P (eP + eD))^T |Q|]_t + u |dK_t|
  dV:       <= sum_g [((eb + bLSE + u + g(m)) P)^T |dO|]_t + u |dV_t|  (u: bf16 of P)

These are worst-case bounds: rounding errors that cancel (the usual case) leave the
GPU far inside them. `ratio` = max |gpu - oracle| / bound over the elements; parity
needs ratio <= 1. The tests in tests/test_bounds_gate.py check that bf16-rounded
oracle outputs and a GPU-like fp32 forward stay inside, and that wrong or unwritten
rows of sharp inputs fall outside.
"""
from __future__ import annotations

import numpy as np

import oracle

U = 2.0 ** -8
G32 = 2.0 ** -24


def group_reference_and_bounds(q, kc, vc, kp, vp, scale, do, prefix_rounded=False):
    """Oracle outputs of one (window, KV head) and the element bounds above.

    q, do [G][C][D]; kc, vc [C][D]; kp, vp [P][D] (fp64 values as stored in the
    cache). prefix_rounded: the cache is F16 / q8_0, whose values the MFMA reads
    rounded to bf16. Returns (ref, bound) with o, lse, dq, delta [G][C][...] and
    dk, dv [C][D].
    """
    ref = {}
    ref["o"], ref["lse"] = oracle.group_fwd(q, kc, vc, kp, vp, scale)
    ref["dq"], ref["dk"], ref["dv"], ref["delta"] = oracle.group_bwd(
        q, kc, vc, kp, vp, scale, do)
    G, C, D = q.shape
    P = kp.shape[0]
    n = P + C
    kf = np.concatenate([kp, kc], axis=0)
    vf = np.concatenate([vp, vc], axis=0)
    akf, avf = np.abs(kf), np.abs(vf)
    allowed = oracle.allowed_mask(P, C)
    rkv = np.zeros(n)
    if prefix_rounded:
        rkv[:P] = U
    bound = {k: np.zeros_like(ref[k]) for k in ("o", "lse", "dq", "dk", "dv", "delta")}
    for g in range(G):
        s = scale * (q[g] @ kf.T)
        pr, _ = oracle.softmax_probs(s, allowed)
        aq = np.abs(q[g])
        a_do = np.abs(do[g])
        ds_err = scale * (rkv + D * G32)[None, :] * (aq @ akf.T)       # score error
        ds_err = np.where(allowed, ds_err, 0.0)
        e = U + ds_err
        ebar = (pr * e).sum(axis=1)
        pv = pr @ avf
        o = ref["o"][g]
        b_o = (pr * e) @ avf + ebar[:, None] * pv + (pr * rkv[None, :]) @ avf \
            + n * G32 * pv + U * np.abs(o)
        bound["o"][g] = b_o
        b_lse = ebar + n * G32
        bound["lse"][g] = b_lse
        e_d = (a_do * (b_o + U * np.abs(o))).sum(axis=1) + D * G32 * (a_do * np.abs(o)).sum(axis=1)
        bound["delta"][g] = e_d
        eb = ds_err + 1e-6
        e_p = (rkv + D * G32)[None, :] * (a_do @ avf.T)
        ads = np.abs(pr * (do[g] @ vf.T - ref["delta"][g][:, None]))   # |dS|
        w_ds = (eb + U + rkv[None, :] + n * G32) * ads
        bound["dq"][g] = scale * ((w_ds + pr * e_p) @ akf) \
            + scale * e_d[:, None] * np.abs(pr @ kf) + (b_lse + U)[:, None] * np.abs(ref["dq"][g])
        m = G * C
        ebk = eb + b_lse[:, None] + U + m * G32
        w_p = pr * (e_p + e_d[:, None])
        bound["dk"] += scale * ((ebk * ads + w_p)[:, P:].T @ aq)
        bound["dv"] += (ebk * pr)[:, P:].T @ a_do
    bound["dk"] += U * np.abs(ref["dk"])
    bound["dv"] += U * np.abs(ref["dv"])
    return ref, bound


def ratio(got, ref, bound):
    """max over elements of |got - ref| / bound (inf where a NaN appears)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    if not np.all(np.isfinite(err)):
        return float("inf")
    return float((err / np.maximum(bound, 1e-300)).max())


def row_rel_l2(got, ref):
    """Largest relative L2 error of one row (last axis) among rows with a nonzero
    reference."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, ref.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    den = np.linalg.norm(ref, axis=1)
    num = np.linalg.norm(got - ref, axis=1)
    ok = den > 0
    return float((num[ok] / den[ok]).max()) if ok.any() else 0.0
