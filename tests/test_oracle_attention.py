"""Pins of the fp64 attention oracle -- CPU only.

The oracle is tied to things other than itself:
  * brute-force central finite differences of L = sum(dO * O);
  * torch's scaled_dot_product_attention (fp64, CPU) with an explicit bottom-right
    mask, the prefix detached and autograd (the detach reference of "stop-gradient
    through context tokens", Correctness tests); P = 0 against torch's own causal
    mode and GQA expansion;
  * the four invariants: softmax rows sum to 1; chunk rows equal the rows of plain
    full-window causal attention; with upstream gradient only on the chunk, dQ and
    the chunk's dK/dV equal the full-window gradients on those rows while the prefix
    rows get exactly zero dQ; P = 0 is plain causal attention;
  * closed forms and shift invariances.
A last group plants plausible mistakes into the oracle and checks that some pin
fails for each, so that the pins are known to bite.
"""
import contextlib

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.attention as oa


def rand_case(B=1, Hq=2, Hkv=1, D=8, P=5, C=3, seed=0, std=1.0):
    rng = np.random.default_rng(seed)
    n = lambda *s: rng.standard_normal(s) * std
    return dict(q=n(B, Hq, C, D), kc=n(B, Hkv, C, D), vc=n(B, Hkv, C, D),
                kp=n(B, Hkv, P, D), vp=n(B, Hkv, P, D), do=n(B, Hq, C, D),
                scale=1.0 / np.sqrt(D))


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


SHAPES = [dict(P=0), dict(P=5), dict(Hq=2, Hkv=2, P=5), dict(Hq=4, Hkv=2, P=4, C=4)]


# ----------------------------------------------------------------- pins as checks
def pin_finite_differences(c, h=1e-6, tol=1e-6):
    """Central differences of L = sum(dO * O) match dQ, dKc, dVc."""
    args = (c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    dq, dkc, dvc, _ = oa.chunk_bwd(*args, c["do"])
    ok = True
    for name, grad in (("q", dq), ("kc", dkc), ("vc", dvc)):
        x = c[name]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = (oa.chunk_fwd(*args)[0] * c["do"]).sum()
            x[idx] = old - h
            lm = (oa.chunk_fwd(*args)[0] * c["do"]).sum()
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        ok &= rel(grad, num) <= tol
    return bool(ok)


def torch_reference(c):
    """fp64 SDPA with explicit mask, KV heads repeated, prefix detached, autograd."""
    t = {k: torch.tensor(v) for k, v in c.items() if k != "scale"}
    B, Hq, C, D = t["q"].shape
    Hkv, P = t["kc"].shape[1], t["kp"].shape[2]
    G = Hq // Hkv
    q = t["q"].clone().requires_grad_(True)
    kc = t["kc"].clone().requires_grad_(True)
    vc = t["vc"].clone().requires_grad_(True)
    k = torch.cat([t["kp"].detach(), kc], dim=2).repeat_interleave(G, dim=1)
    v = torch.cat([t["vp"].detach(), vc], dim=2).repeat_interleave(G, dim=1)
    mask = torch.ones(C, P + C, dtype=torch.bool).tril(diagonal=P)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=c["scale"])
    o.backward(t["do"])
    # LSE through the same library routine: with V = one-hot rows the output is the
    # probability matrix itself, and lse_i = s_ij - ln(p_ij) for an allowed j.
    eye = torch.eye(P + C, dtype=torch.float64).expand(B, Hq, P + C, P + C)
    pr = F.scaled_dot_product_attention(q.detach(), k.detach(), eye, attn_mask=mask,
                                        scale=c["scale"])
    s = c["scale"] * (q.detach() @ k.detach().transpose(-1, -2))
    j = P + torch.arange(C)          # the diagonal key, always allowed
    i = torch.arange(C)
    lse = s[..., i, j] - torch.log(pr[..., i, j])
    return (o.detach().numpy(), lse.numpy(), q.grad.numpy(), kc.grad.numpy(),
            vc.grad.numpy(), pr.numpy(), mask.numpy())


def pin_torch(c, tol=1e-12):
    args = (c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    o, lse = oa.chunk_fwd(*args)
    dq, dkc, dvc, _ = oa.chunk_bwd(*args, c["do"])
    to, tlse, tdq, tdk, tdv, _, _ = torch_reference(c)
    return (rel(o, to) <= tol and np.abs(lse - tlse).max() <= 1e-10
            and rel(dq, tdq) <= tol and rel(dkc, tdk) <= tol and rel(dvc, tdv) <= tol)


def pin_p0_causal(c, tol=1e-12):
    """P = 0: torch's own causal mode (top-left == bottom-right) and GQA expansion."""
    c = dict(c)
    c["kp"] = c["kp"][:, :, :0]
    c["vp"] = c["vp"][:, :, :0]
    args = (c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    o, _ = oa.chunk_fwd(*args)
    dq, dkc, dvc, _ = oa.chunk_bwd(*args, c["do"])
    q = torch.tensor(c["q"], requires_grad=True)
    k = torch.tensor(c["kc"], requires_grad=True)
    v = torch.tensor(c["vc"], requires_grad=True)
    to = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=c["scale"],
                                        enable_gqa=True)
    to.backward(torch.tensor(c["do"]))
    return (rel(o, to.detach().numpy()) <= tol and rel(dq, q.grad.numpy()) <= tol
            and rel(dkc, k.grad.numpy()) <= tol and rel(dvc, v.grad.numpy()) <= tol)


def full_window(c):
    """The same window as plain causal attention over L = P + C rows."""
    B, Hq, C, D = c["q"].shape
    P = c["kp"].shape[2]
    rng = np.random.default_rng(99)
    qp = rng.standard_normal((B, Hq, P, D))     # the context's own queries
    qf = np.concatenate([qp, c["q"]], axis=2)
    kf = np.concatenate([c["kp"], c["kc"]], axis=2)
    vf = np.concatenate([c["vp"], c["vc"]], axis=2)
    dof = np.concatenate([np.zeros((B, Hq, P, D)), c["do"]], axis=2)
    return qf, kf, vf, dof


def pin_full_window(c, tol=1e-12):
    """Chunk rows == full-window rows; chunk-only dO -> prefix-row dQ exactly 0."""
    args = (c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    o, lse = oa.chunk_fwd(*args)
    dq, dkc, dvc, _ = oa.chunk_bwd(*args, c["do"])
    qf, kf, vf, dof = full_window(c)
    P = c["kp"].shape[2]
    ok = True
    for b in range(qf.shape[0]):
        fo, flse = oa.full_causal_fwd(qf[b], kf[b], vf[b], c["scale"])
        fdq, fdk, fdv = oa.full_causal_bwd(qf[b], kf[b], vf[b], c["scale"], dof[b])
        ok &= rel(fo[:, P:], o[b]) <= tol and np.abs(flse[:, P:] - lse[b]).max() <= 1e-12
        ok &= bool(np.all(fdq[:, :P] == 0.0))
        ok &= rel(fdq[:, P:], dq[b]) <= tol
        ok &= rel(fdk[:, P:], dkc[b]) <= tol and rel(fdv[:, P:], dvc[b]) <= tol
    return bool(ok)


ALL_PINS = (pin_finite_differences, pin_torch, pin_p0_causal, pin_full_window)


# ----------------------------------------------------------------- the pins hold
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_finite_differences(shape):
    assert pin_finite_differences(rand_case(**shape))


@pytest.mark.parametrize("shape", SHAPES + [dict(B=2, Hq=6, Hkv=2, D=16, P=37, C=11)], ids=str)
def test_torch_sdpa_detached_prefix(shape):
    assert pin_torch(rand_case(**shape))


@pytest.mark.parametrize("shape", [dict(Hq=4, Hkv=2, C=7), dict(Hq=6, Hkv=3, C=5, D=16)], ids=str)
def test_p0_is_plain_causal(shape):
    assert pin_p0_causal(rand_case(**shape))


@pytest.mark.parametrize("shape", SHAPES + [dict(Hq=6, Hkv=2, D=16, P=20, C=9)], ids=str)
def test_full_window_invariants(shape):
    c = rand_case(**shape)
    assert pin_full_window(c)
    # The stop-gradient is a truncation: full-window attention would give the
    # prefix keys a non-zero gradient ("train: walk the window", Why it's a draft).
    if c["kp"].shape[2] > 0:
        qf, kf, vf, dof = full_window(c)
        _, fdk, fdv = oa.full_causal_bwd(qf[0], kf[0], vf[0], c["scale"], dof[0])
        assert np.abs(fdk[:, :c["kp"].shape[2]]).max() > 0


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(3)
    P, C = 50, 17
    s = rng.standard_normal((C, P + C)) * 5
    allowed = oa.allowed_mask(P, C)
    pr, lse = oa.softmax_probs(s, allowed)
    assert np.abs(pr.sum(axis=1) - 1).max() <= 1e-14
    assert np.all(pr[~allowed] == 0.0)
    assert np.all(pr[allowed] > 0.0)
    # the mask: row i sees exactly P + i + 1 keys
    np.testing.assert_array_equal(allowed.sum(axis=1), P + 1 + np.arange(C))


def test_lse_matches_torch_probabilities():
    c = rand_case(B=1, Hq=4, Hkv=2, D=16, P=30, C=9, seed=5, std=2.0)
    _, lse = oa.chunk_fwd(c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    _, tlse, *_ = torch_reference(c)
    assert np.abs(lse - tlse).max() <= 1e-10


# ----------------------------------------------------------------- closed forms
def test_zero_queries_closed_form():
    c = rand_case(Hq=4, Hkv=2, D=16, P=11, C=6, seed=4)
    c["q"][:] = 0.0
    args = (c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    o, lse = oa.chunk_fwd(*args)
    dq, dkc, dvc, _ = oa.chunk_bwd(*args, c["do"])
    P, C = 11, 6
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(P + 1 + np.arange(C)), lse.shape),
                               rtol=0, atol=1e-14)
    for b in range(1):
        for h in range(4):
            vf = np.concatenate([c["vp"][b, h // 2], c["vc"][b, h // 2]])
            for i in range(C):
                np.testing.assert_allclose(o[b, h, i], vf[:P + i + 1].mean(axis=0),
                                           rtol=1e-13, atol=1e-15)
    assert np.all(dkc == 0.0)       # dK = scale dS^T Q with Q = 0: exactly zero
    assert np.abs(dvc).max() > 0


def test_constant_values_closed_form():
    c = rand_case(Hq=2, Hkv=1, D=8, P=9, C=5, seed=6)
    const = np.linspace(-1, 1, 8)
    c["vp"][:] = const
    c["vc"][:] = const
    args = (c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    o, _ = oa.chunk_fwd(*args)
    dq, dkc, _, _ = oa.chunk_bwd(*args, c["do"])
    assert np.abs(o - const).max() <= 1e-14
    assert np.abs(dq).max() <= 1e-13 and np.abs(dkc).max() <= 1e-13


def test_single_token_closed_form():
    c = rand_case(Hq=3, Hkv=1, D=8, P=0, C=1, seed=8)
    args = (c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    o, lse = oa.chunk_fwd(*args)
    dq, dkc, dvc, _ = oa.chunk_bwd(*args, c["do"])
    np.testing.assert_array_equal(o[0, :, 0], np.broadcast_to(c["vc"][0, 0, 0], (3, 8)))
    np.testing.assert_allclose(lse[0, :, 0], c["scale"] * (c["q"][0, :, 0] @ c["kc"][0, 0, 0]),
                               rtol=1e-13)
    np.testing.assert_allclose(dvc[0, 0, 0], c["do"][0, :, 0].sum(axis=0), rtol=1e-14)
    assert np.abs(dq).max() <= 1e-15 and np.abs(dkc).max() <= 1e-15


def test_shift_invariance():
    c = rand_case(Hq=4, Hkv=2, D=8, P=7, C=5, seed=9)
    args = lambda c: (c["q"], c["kc"], c["vc"], c["kp"], c["vp"], c["scale"])
    o, lse = oa.chunk_fwd(*args(c))
    dq, dkc, dvc, _ = oa.chunk_bwd(*args(c), c["do"])
    shift = np.random.default_rng(1).standard_normal(8)
    ck = dict(c, kp=c["kp"] + shift, kc=c["kc"] + shift)
    o2, lse2 = oa.chunk_fwd(*args(ck))
    dq2, dkc2, dvc2, _ = oa.chunk_bwd(*args(ck), c["do"])
    assert rel(o2, o) <= 1e-12 and rel(dq2, dq) <= 1e-12
    assert rel(dkc2, dkc) <= 1e-12 and rel(dvc2, dvc) <= 1e-12
    np.testing.assert_allclose(lse2, lse + c["scale"] * (c["q"] @ shift), rtol=0, atol=1e-12)
    cv = dict(c, vp=c["vp"] + shift, vc=c["vc"] + shift)
    o3, lse3 = oa.chunk_fwd(*args(cv))
    dq3, dkc3, dvc3, _ = oa.chunk_bwd(*args(cv), c["do"])
    assert rel(o3, o + shift) <= 1e-12 and np.abs(lse3 - lse).max() == 0
    assert rel(dq3, dq) <= 1e-12 and rel(dkc3, dkc) <= 1e-12 and rel(dvc3, dvc) <= 1e-12


# ----------------------------------------------------------------- planted mistakes
@contextlib.contextmanager
def planted(name, fn):
    old = getattr(oa, name)
    setattr(oa, name, fn)
    try:
        yield
    finally:
        setattr(oa, name, old)


def _bwd_variant(mistake):
    """group_bwd with one plausible mistake planted (for pin sensitivity only)."""
    def group_bwd(q, kc, vc, kp, vp, scale, do):
        G, C, D = q.shape
        P = kp.shape[0]
        kf = np.concatenate([kp, kc])
        vf = np.concatenate([vp, vc])
        allowed = oa.allowed_mask(P, C)
        dq = np.empty((G, C, D)); dkc = np.zeros((C, D)); dvc = np.zeros((C, D))
        delta = np.empty((G, C))
        for g in range(G):
            o, _, pr = oa._head_fwd(q[g], kf, vf, allowed, scale)
            delta[g] = (do[g] * o).sum(axis=1)
            dpr = do[g] @ vf.T
            ds = pr * dpr if mistake == "no_delta" else pr * (dpr - delta[g][:, None])
            dq[g] = (1.0 if mistake == "dq_no_scale" else scale) * (ds @ kf)
            dkc += (1.0 if mistake == "dk_no_scale" else scale) * (ds[:, P:].T @ q[g])
            src = ds if mistake == "dv_uses_ds" else pr
            dvc += src[:, P:].T @ do[g]
            if mistake == "dk_off_by_one":
                dkc[:] = np.roll(dkc, 1, axis=0)
        return dq, dkc, dvc, delta
    return group_bwd


def _fwd_variant(mistake):
    def head_fwd(q, kf, vf, allowed, scale):
        s = (1.0 if mistake == "no_scale" else scale) * (q @ kf.T)
        if mistake == "mask_after_normalising":
            e = np.exp(s - s.max(axis=1)[:, None])
            pr = np.where(allowed, e / e.sum(axis=1)[:, None], 0.0)
            return pr @ vf, s.max(axis=1) + np.log(e.sum(axis=1)), pr
        pr, lse = oa.softmax_probs(s, allowed)
        if mistake == "lse_log2":
            lse = lse / np.log(2.0)
        return pr @ vf, lse, pr
    return head_fwd


MISTAKES = [
    ("allowed_mask", lambda P, C: np.arange(P + C)[None, :] <= np.arange(C)[:, None] + max(P - 1, 0)),
    ("allowed_mask", lambda P, C: np.arange(P + C)[None, :] <= np.arange(C)[:, None] + P + 1),
    ("kv_head_of", lambda h, g: h % 2),
    ("group_bwd", _bwd_variant("no_delta")),
    ("group_bwd", _bwd_variant("dq_no_scale")),
    ("group_bwd", _bwd_variant("dk_no_scale")),
    ("group_bwd", _bwd_variant("dv_uses_ds")),
    ("group_bwd", _bwd_variant("dk_off_by_one")),
    ("_head_fwd", _fwd_variant("no_scale")),
    ("_head_fwd", _fwd_variant("lse_log2")),
    ("_head_fwd", _fwd_variant("mask_after_normalising")),
]


@pytest.mark.parametrize("mistake", range(len(MISTAKES)))
def test_planted_mistake_is_caught(mistake):
    name, fn = MISTAKES[mistake]
    case = lambda: rand_case(B=1, Hq=4, Hkv=2, D=8, P=5, C=4, seed=21)
    with planted(name, fn):
        results = []
        for pin in ALL_PINS:
            try:
                with np.errstate(all="ignore"):
                    results.append(pin(case()))
            except Exception:
                results.append(False)
    assert not all(results), f"no pin caught planted mistake {mistake}"
