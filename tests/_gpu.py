"""Shared setup of GPU parity tests: one chunk step on the device and its oracle.

The device side builds its prefix cache with the library's own append kernel from
the raw bf16 prefix rows; the oracle builds its cache from the same rows with its
own converters. The two never exchange values.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synthetic
from oracle.cache import from_torch_bf16

DEV = "cuda:0"


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def f64(t):
    """A torch tensor (bf16 / f32, any device) -> fp64 numpy of the same values."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return from_torch_bf16(t).astype(np.float64)
    return t.to(torch.float64).numpy()


class Case:
    """Inputs of one workload on the device plus lazily computed oracle values."""

    def __init__(self, w: synthetic.Workload, extra_capacity: int = 0, inputs=None):
        import prefix_kv_attention_amd as pka
        self.pka = pka
        self.w = w
        self.cpu = inputs if inputs is not None else synthetic.make_inputs(w)
        self.dev = {k: v.to(DEV) for k, v in self.cpu.items() if k not in ("kp", "vp")}
        B, Hkv, D, P, C = w.batch, w.n_heads_kv, w.head_dim, w.prefix_len, w.chunk_len
        self.capacity = P + C + extra_capacity
        self.cache = pka.PrefixCache.empty(w.cache_type, B, Hkv, self.capacity, D, DEV)
        if P > 0:
            pka.kv_append(self.cpu["kp"].to(DEV), self.cpu["vp"].to(DEV), self.cache, 0)
        self._oracle_prefix = None

    # ---------------------------------------------------------------- device
    def fwd(self):
        d = self.dev
        return self.pka.chunk_attn_fwd(d["q"], d["kc"], d["vc"], self.cache,
                                       self.w.prefix_len, self.w.softmax_scale)

    def bwd(self, o, lse, delta=None):
        d = self.dev
        return self.pka.chunk_attn_bwd(d["q"], d["kc"], d["vc"], self.cache,
                                       self.w.prefix_len, self.w.softmax_scale, o, lse,
                                       d["do"], delta=delta)

    # ---------------------------------------------------------------- oracle
    def oracle_prefix(self):
        """Oracle cache values of the prefix rows: (K, V) fp64 [B][Hkv][P][D]."""
        if self._oracle_prefix is None:
            kp = from_torch_bf16(self.cpu["kp"])
            vp = from_torch_bf16(self.cpu["vp"])
            self._oracle_prefix = (oracle.build_prefix(kp, self.w.cache_type)["values"],
                                   oracle.build_prefix(vp, self.w.cache_type)["values"])
        return self._oracle_prefix

    def oracle_group(self, b, kv):
        """Oracle forward and backward of one (window, KV head)."""
        G = self.w.group
        hs = slice(kv * G, (kv + 1) * G)
        kpv, vpv = self.oracle_prefix()
        q = f64(self.cpu["q"][b, hs])
        kc = f64(self.cpu["kc"][b, kv])
        vc = f64(self.cpu["vc"][b, kv])
        do = f64(self.cpu["do"][b, hs])
        sc = self.w.softmax_scale
        o, lse = oracle.group_fwd(q, kc, vc, kpv[b, kv], vpv[b, kv], sc)
        dq, dk, dv, delta = oracle.group_bwd(q, kc, vc, kpv[b, kv], vpv[b, kv], sc, do)
        return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)

    def all_groups(self):
        return [(b, kv) for b in range(self.w.batch) for kv in range(self.w.n_heads_kv)]


def compare_groups(case: Case, groups, o, lse, dq, dk, dv, delta=None):
    """Relative L2 over the sampled groups (concatenated) and max |LSE| error."""
    G = case.w.group
    acc = {k: ([], []) for k in ("o", "dq", "dk", "dv", "delta")}
    lse_err = 0.0
    for b, kv in groups:
        ref = case.oracle_group(b, kv)
        hs = slice(kv * G, (kv + 1) * G)
        for name, gpu in (("o", o[b, hs]), ("dq", dq[b, hs]), ("dk", dk[b, kv]),
                          ("dv", dv[b, kv])):
            acc[name][0].append(f64(gpu).ravel())
            acc[name][1].append(ref[name].ravel())
        if delta is not None:
            acc["delta"][0].append(f64(delta[b, hs]).ravel())
            acc["delta"][1].append(ref["delta"].ravel())
        lse_err = max(lse_err, float(np.abs(f64(lse[b, hs]) - ref["lse"]).max()))
    out = {k: rel_l2(np.concatenate(a), np.concatenate(r)) for k, (a, r) in acc.items() if a}
    out["lse_abs"] = lse_err
    return out


def sample_groups(case: Case, n: int = 4):
    """n (window, KV head) groups spread over the batch: the first, the last and
    interior ones (all of them when there are at most n)."""
    groups = case.all_groups()
    if len(groups) <= n:
        return groups
    idx = sorted({round(k * (len(groups) - 1) / (n - 1)) for k in range(n)})
    return [groups[i] for i in idx]


def compare_groups_bounded(case: Case, groups, o, lse, dq, dk, dv):
    """As compare_groups, plus the worst per-(window, head) relative L2, the worst
    per-row relative L2, and the largest ratio of an element's error to its
    first-order rounding bound (tests/_bounds.py; parity needs ratio <= 1)."""
    from _bounds import group_reference_and_bounds, ratio, row_rel_l2
    G = case.w.group
    sc = case.w.softmax_scale
    kpv, vpv = case.oracle_prefix()
    acc = {k: ([], []) for k in ("o", "dq", "dk", "dv")}
    worst_head = {k: 0.0 for k in acc}
    worst_row = {k: 0.0 for k in acc}
    worst_ratio = {k: 0.0 for k in ("o", "lse", "dq", "dk", "dv")}
    lse_err = 0.0
    for b, kv in groups:
        hs = slice(kv * G, (kv + 1) * G)
        ref, bnd = group_reference_and_bounds(
            f64(case.cpu["q"][b, hs]), f64(case.cpu["kc"][b, kv]), f64(case.cpu["vc"][b, kv]),
            kpv[b, kv], vpv[b, kv], sc, f64(case.cpu["do"][b, hs]),
            prefix_rounded=case.w.cache_type != "bf16")
        got = {"o": f64(o[b, hs]), "dq": f64(dq[b, hs]), "dk": f64(dk[b, kv]),
               "dv": f64(dv[b, kv]), "lse": f64(lse[b, hs])}
        for name in acc:
            acc[name][0].append(got[name].ravel())
            acc[name][1].append(ref[name].ravel())
            heads = [(got[name], ref[name])] if name in ("dk", "dv") else \
                [(got[name][g], ref[name][g]) for g in range(G)]
            for gg, rr in heads:
                worst_head[name] = max(worst_head[name], rel_l2(gg, rr))
            worst_row[name] = max(worst_row[name], row_rel_l2(got[name], ref[name]))
        for name in worst_ratio:
            worst_ratio[name] = max(worst_ratio[name], ratio(got[name], ref[name], bnd[name]))
        lse_err = max(lse_err, float(np.abs(got["lse"] - ref["lse"]).max()))
    out = {k: rel_l2(np.concatenate(a), np.concatenate(r)) for k, (a, r) in acc.items()}
    out["lse_abs"] = lse_err
    out["worst_head_rel_l2"] = worst_head
    out["worst_row_rel_l2"] = worst_row
    out["bound_ratio"] = worst_ratio
    out["groups"] = [list(g) for g in groups]
    return out


def assert_bounded(errs: dict, label: str):
    """Stated bars on the sampled groups, and every element within its bound."""
    assert_within(errs, label)
    bad = {k: v for k, v in errs["bound_ratio"].items() if not v <= 1.0}
    assert not bad, f"{label}: elements outside their rounding bound {bad} (all: {errs})"


# Tolerances: relative L2 1e-2 for O and 2e-2 for dQ/dK/dV (bf16 operands, fp32
# accumulation); LSE feeds the backward, so it is gated at 5e-3 absolute.
TOL = dict(o=1e-2, dq=2e-2, dk=2e-2, dv=2e-2, delta=2e-2, lse_abs=5e-3)


def assert_within(errs: dict, label: str):
    bad = {k: v for k, v in errs.items() if k in TOL and not v <= TOL[k]}
    assert not bad, f"{label}: {bad} (all: {errs})"
