"""fp64 oracle of chunk attention against a frozen prefix (test infrastructure only).

What is computed (the plain definition; no blocking, no online softmax):

* The chunk's queries attend to the cached context plus the chunk's own keys. The
  context was built by a no-grad forward and is read as a constant
  ("Context-Frozen Training", The Solution: Phase 1 builds the KV cache without
  gradients, Phase 2 runs only the decision tokens against it with gradients).
* The key sequence of one window and one KV head is Kf = [prefix rows 0..P-1 ;
  chunk rows 0..C-1]; chunk query i (token P+i of the window) sees key j iff
  j <= P + i: causal attention offset by the prefix length ("train: walk the
  window", What it is: each reply chunk trains against the cached prefix).
* GQA: query head h reads KV head floor(h / G), G = Hq / Hkv (contiguous groups;
  the pages do not say, this is the usual convention).
* Forward: S = scale * Q Kf^T, masked softmax over allowed keys, O = Pr Vf and the
  per-row log-sum-exp LSE = m + ln(sum exp(S - m)) (natural log).
* Backward from an upstream dO on the chunk rows only: Delta_i = dO_i . O_i,
  dPr = dO Vf^T, dS = Pr * (dPr - Delta), dQ = scale dS Kf,
  dKc = scale dS[:, P:]^T Q and dVc = Pr[:, P:]^T dO summed over the G query heads of
  the KV head. The prefix rows get no gradient at all: the cache is a fixed input
  of the step ("train: walk the window", Why it's a draft; "stop-gradient through
  context tokens", Known gaps: an attention backward split by query that gives
  gradient to the kept queries alone).

The full-window functions (plain causal attention over L tokens, every row a query)
exist only to check the invariants that tie the chunk form to ordinary attention.
"""
from __future__ import annotations

import numpy as np


def kv_head_of(h: int, group: int) -> int:
    """KV head read by query head h when G = group query heads share one KV head."""
    return h // group


def allowed_mask(prefix_len: int, chunk_len: int) -> np.ndarray:
    """bool [C][P+C]: chunk row i may attend key j iff j <= P + i."""
    i = np.arange(chunk_len)[:, None]
    j = np.arange(prefix_len + chunk_len)[None, :]
    return j <= prefix_len + i


def softmax_probs(s: np.ndarray, allowed: np.ndarray):
    """Row softmax of scores s over the allowed entries; returns (Pr, lse).

    Masked entries are exactly 0; lse is the natural log of sum(exp(s)) over the
    allowed entries of each row (computed stably as m + ln(sum exp(s - m))).
    """
    m = np.where(allowed, s, -np.inf).max(axis=1)
    e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    return e / l[:, None], m + np.log(l)


def _head_fwd(q, kf, vf, allowed, scale):
    s = scale * (q @ kf.T)
    pr, lse = softmax_probs(s, allowed)
    return pr @ vf, lse, pr


def group_fwd(q, kc, vc, kp, vp, scale):
    """One (window, KV head): q [G][C][D]; kc, vc [C][D]; kp, vp [P][D] (fp64).

    Returns O [G][C][D] and LSE [G][C].
    """
    q, kc, vc, kp, vp = (np.asarray(a, dtype=np.float64) for a in (q, kc, vc, kp, vp))
    G, C, D = q.shape
    P = kp.shape[0]
    kf = np.concatenate([kp, kc], axis=0)
    vf = np.concatenate([vp, vc], axis=0)
    allowed = allowed_mask(P, C)
    o = np.empty((G, C, D))
    lse = np.empty((G, C))
    for g in range(G):
        o[g], lse[g], _ = _head_fwd(q[g], kf, vf, allowed, scale)
    return o, lse


def group_bwd(q, kc, vc, kp, vp, scale, do):
    """Backward of one (window, KV head) from dO [G][C][D] on the chunk rows.

    Returns dQ [G][C][D], dKc [C][D], dVc [C][D] and Delta [G][C]. The prefix
    rows kp, vp receive nothing.
    """
    q, kc, vc, kp, vp, do = (np.asarray(a, dtype=np.float64)
                             for a in (q, kc, vc, kp, vp, do))
    G, C, D = q.shape
    P = kp.shape[0]
    kf = np.concatenate([kp, kc], axis=0)
    vf = np.concatenate([vp, vc], axis=0)
    allowed = allowed_mask(P, C)
    dq = np.empty((G, C, D))
    dkc = np.zeros((C, D))
    dvc = np.zeros((C, D))
    delta = np.empty((G, C))
    for g in range(G):
        o, _, pr = _head_fwd(q[g], kf, vf, allowed, scale)
        delta[g] = (do[g] * o).sum(axis=1)
        dpr = do[g] @ vf.T
        ds = pr * (dpr - delta[g][:, None])
        dq[g] = scale * (ds @ kf)
        dkc += scale * (ds[:, P:].T @ q[g])
        dvc += pr[:, P:].T @ do[g]
    return dq, dkc, dvc, delta


def group_bwd_prefix(q, kc, vc, kp, vp, scale, do):
    """Gradient of the chunk's loss w.r.t. the cached prefix rows of one (window, KV
    head), from the chunk queries only: dKp [P][D] and dVp [P][D].

    The same masked softmax as group_bwd; every chunk row sees every prefix row, so
    dKp = scale * sum_g dS_g[:, :P]^T Q_g and dVp = sum_g Pr_g[:, :P]^T dO_g. This is
    the gradient a stop-gradient prefix discards ("train: walk the window", Why it's
    a draft: the exact reverse pass with a horizon H; "stop-gradient through context
    tokens", Mechanism: kept queries attend to context k/v, so context dK/dV are
    nonzero and feed the k/v weight gradients).
    """
    q, kc, vc, kp, vp, do = (np.asarray(a, dtype=np.float64)
                             for a in (q, kc, vc, kp, vp, do))
    G, C, D = q.shape
    P = kp.shape[0]
    kf = np.concatenate([kp, kc], axis=0)
    vf = np.concatenate([vp, vc], axis=0)
    allowed = allowed_mask(P, C)
    dkp = np.zeros((P, D))
    dvp = np.zeros((P, D))
    for g in range(G):
        o, _, pr = _head_fwd(q[g], kf, vf, allowed, scale)
        delta = (do[g] * o).sum(axis=1)
        ds = pr * (do[g] @ vf.T - delta[:, None])
        dkp += scale * (ds[:, :P].T @ q[g])
        dvp += pr[:, :P].T @ do[g]
    return dkp, dvp


def _split(q, kc, n_heads_kv):
    B, Hq = q.shape[:2]
    return B, Hq, Hq // n_heads_kv


def chunk_fwd(q, kc, vc, kp, vp, scale):
    """Whole batch: q [B][Hq][C][D], kc/vc [B][Hkv][C][D], kp/vp [B][Hkv][P][D]."""
    Hkv = kc.shape[1]
    B, Hq, G = _split(q, kc, Hkv)
    C, D = q.shape[2:]
    o = np.empty((B, Hq, C, D))
    lse = np.empty((B, Hq, C))
    for b in range(B):
        for kv in range(Hkv):
            hs = [h for h in range(Hq) if kv_head_of(h, G) == kv]
            o[b, hs], lse[b, hs] = group_fwd(q[b, hs], kc[b, kv], vc[b, kv],
                                             kp[b, kv], vp[b, kv], scale)
    return o, lse


def chunk_bwd(q, kc, vc, kp, vp, scale, do):
    """Whole batch backward; returns dQ, dKc, dVc, Delta."""
    Hkv = kc.shape[1]
    B, Hq, G = _split(q, kc, Hkv)
    C, D = q.shape[2:]
    dq = np.empty((B, Hq, C, D))
    dkc = np.empty((B, Hkv, C, D))
    dvc = np.empty((B, Hkv, C, D))
    delta = np.empty((B, Hq, C))
    for b in range(B):
        for kv in range(Hkv):
            hs = [h for h in range(Hq) if kv_head_of(h, G) == kv]
            dq[b, hs], dkc[b, kv], dvc[b, kv], delta[b, hs] = group_bwd(
                q[b, hs], kc[b, kv], vc[b, kv], kp[b, kv], vp[b, kv], scale, do[b, hs])
    return dq, dkc, dvc, delta


def full_causal_fwd(q, k, v, scale):
    """Plain causal attention over a whole window of L tokens.

    q [Hq][L][D], k/v [Hkv][L][D]; row i sees keys j <= i. Returns O, LSE.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    Hq, L, D = q.shape
    G = Hq // k.shape[0]
    allowed = np.tril(np.ones((L, L), dtype=bool))
    o = np.empty((Hq, L, D))
    lse = np.empty((Hq, L))
    for h in range(Hq):
        kv = kv_head_of(h, G)
        o[h], lse[h], _ = _head_fwd(q[h], k[kv], v[kv], allowed, scale)
    return o, lse


def full_causal_bwd(q, k, v, scale, do):
    """Gradients of sum(dO * O) of plain causal attention w.r.t. every row.

    Returns dQ [Hq][L][D], dK [Hkv][L][D], dV [Hkv][L][D].
    """
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    Hq, L, D = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    allowed = np.tril(np.ones((L, L), dtype=bool))
    dq = np.empty((Hq, L, D))
    dk = np.zeros((Hkv, L, D))
    dv = np.zeros((Hkv, L, D))
    for h in range(Hq):
        kv = kv_head_of(h, G)
        o, _, pr = _head_fwd(q[h], k[kv], v[kv], allowed, scale)
        delta = (do[h] * o).sum(axis=1)
        ds = pr * (do[h] @ v[kv].T - delta[:, None])
        dq[h] = scale * (ds @ k[kv])
        dk[kv] += scale * (ds.T @ q[h])
        dv[kv] += pr.T @ do[h]
    return dq, dk, dv
