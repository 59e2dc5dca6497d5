"""Pins of the oracle's prefix gradient (group_bwd_prefix) -- CPU only.

group_bwd_prefix gives dL/dK and dL/dV of the cached prefix rows from the chunk's
queries: what a stop-gradient prefix discards, and what the exact reverse pass with
a horizon ("train: walk the window", Why it's a draft) keeps. It is tied to:
  * central finite differences of L = sum(dO * O) in the prefix rows;
  * torch's scaled_dot_product_attention (fp64) with the prefix NOT detached;
  * full-window causal attention with upstream gradient only on the chunk rows: its
    dK/dV on the prefix rows equal the chunk queries' contribution (the context's
    own queries get zero dS);
and planted mistakes (a dropped scale, the chunk slice instead of the prefix one, a
missing delta) must each break a pin.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.attention as oa
from test_oracle_attention import full_window, rand_case, rel


def prefix_grads(c, fn=None):
    """dKp, dVp [B][Hkv][P][D] of a whole batch through group_bwd_prefix (or fn)."""
    fn = fn or oa.group_bwd_prefix
    B, Hq = c["q"].shape[:2]
    Hkv = c["kc"].shape[1]
    G = Hq // Hkv
    dk = np.zeros_like(c["kp"])
    dv = np.zeros_like(c["vp"])
    for b in range(B):
        for kv in range(Hkv):
            hs = slice(kv * G, (kv + 1) * G)
            dk[b, kv], dv[b, kv] = fn(c["q"][b, hs], c["kc"][b, kv], c["vc"][b, kv],
                                      c["kp"][b, kv], c["vp"][b, kv], c["scale"],
                                      c["do"][b, hs])
    return dk, dv


def pin_fd(c, fn=None, h=1e-6, tol=1e-6):
    dk, dv = prefix_grads(c, fn)
    args = lambda: (c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    ok = True
    for name, grad in (("kp", dk), ("vp", dv)):
        x = c[name]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = (oa.chunk_fwd(*args())[0] * c["do"]).sum()
            x[idx] = old - h
            lm = (oa.chunk_fwd(*args())[0] * c["do"]).sum()
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        ok &= rel(grad, num) <= tol
    return bool(ok)


def pin_torch_undetached(c, fn=None, tol=1e-12):
    dk, dv = prefix_grads(c, fn)
    t = {k: torch.tensor(v) for k, v in c.items() if k != "scale"}
    B, Hq, C, D = t["q"].shape
    Hkv, P = t["kc"].shape[1], t["kp"].shape[2]
    G = Hq // Hkv
    kp = t["kp"].clone().requires_grad_(True)
    vp = t["vp"].clone().requires_grad_(True)
    k = torch.cat([kp, t["kc"]], dim=2).repeat_interleave(G, dim=1)
    v = torch.cat([vp, t["vc"]], dim=2).repeat_interleave(G, dim=1)
    mask = torch.ones(C, P + C, dtype=torch.bool).tril(diagonal=P)
    o = F.scaled_dot_product_attention(t["q"], k, v, attn_mask=mask, scale=c["scale"])
    o.backward(t["do"])
    return rel(dk, kp.grad.numpy()) <= tol and rel(dv, vp.grad.numpy()) <= tol


def pin_full_window(c, fn=None, tol=1e-12):
    dk, dv = prefix_grads(c, fn)
    qf, kf, vf, dof = full_window(c)
    P = c["kp"].shape[2]
    ok = True
    for b in range(qf.shape[0]):
        _, fdk, fdv = oa.full_causal_bwd(qf[b], kf[b], vf[b], c["scale"], dof[b])
        ok &= rel(fdk[:, :P], dk[b]) <= tol and rel(fdv[:, :P], dv[b]) <= tol
    return bool(ok)


PINS = (pin_fd, pin_torch_undetached, pin_full_window)
SHAPES = [dict(P=5), dict(Hq=2, Hkv=2, P=4), dict(Hq=4, Hkv=2, P=6, C=4), dict(P=1, C=1)]


@pytest.mark.parametrize("shape", SHAPES, ids=str)
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_prefix_grad_pins(pin, shape):
    assert pin(rand_case(**shape))


def test_prefix_grad_nonzero_and_p0_empty():
    dk, dv = prefix_grads(rand_case(P=5))
    assert np.abs(dk).max() > 1e-3 and np.abs(dv).max() > 1e-3
    dk0, dv0 = prefix_grads(rand_case(P=0))
    assert dk0.shape[2] == 0 and dv0.shape[2] == 0


def _variant(mistake):
    def fn(q, kc, vc, kp, vp, scale, do):
        G, C, D = q.shape
        P = kp.shape[0]
        kf = np.concatenate([kp, kc])
        vf = np.concatenate([vp, vc])
        allowed = oa.allowed_mask(P, C)
        dkp = np.zeros((P, D))
        dvp = np.zeros((P, D))
        for g in range(G):
            o, _, pr = oa._head_fwd(q[g], kf, vf, allowed, scale)
            delta = 0.0 if mistake == "no_delta" else (do[g] * o).sum(axis=1)[:, None]
            ds = pr * (do[g] @ vf.T - delta)
            # chunk_slice: the last P key columns instead of the first P
            sl = slice(C, P + C) if mistake == "chunk_slice" else slice(0, P)
            sc = 1.0 if mistake == "no_scale" else scale
            dkp += sc * (ds[:, sl].T @ q[g])
            dvp += pr[:, sl].T @ do[g]
        return dkp, dvp
    return fn


@pytest.mark.parametrize("mistake", ["no_scale", "chunk_slice", "no_delta"])
def test_planted_mistake_is_caught(mistake):
    c = rand_case(Hq=4, Hkv=2, P=6, C=4)
    assert not all(pin(c, _variant(mistake)) for pin in PINS)
