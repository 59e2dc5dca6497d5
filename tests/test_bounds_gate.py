"""The per-element rounding bound of the sampled full-size parity tests (tests/_bounds.py),
checked on the CPU: bf16-rounded oracle outputs and an fp32 forward with bf16
probabilities stay inside it; with unit-scale inputs (distinct rows), outputs holding a
neighbour's row, half a row of another head or an unwritten row fall outside it.
"""
import numpy as np
import pytest

import oracle
import synthetic
from _bounds import group_reference_and_bounds, ratio, row_rel_l2
from oracle.cache import from_torch_bf16, bf16_bits_to_f32, f32_to_bf16_rne


def _bf16(x):
    return bf16_bits_to_f32(f32_to_bf16_rne(np.asarray(x, np.float32))).astype(np.float64)


def _group(ct, std):
    w = synthetic.small("gate", prefix_len=4096, chunk_len=64, n_heads_q=2, n_heads_kv=1,
                        head_dim=128, cache_type=ct, qkv_std=std, prefix_std=std,
                        do_std=1e-2, seed=21)
    t = synthetic.make_inputs(w)
    f = lambda x: from_torch_bf16(x).astype(np.float64)
    q, kc, vc, do = f(t["q"][0]), f(t["kc"][0, 0]), f(t["vc"][0, 0]), f(t["do"][0])
    kp = oracle.build_prefix(from_torch_bf16(t["kp"][0, 0]), ct)["values"]
    vp = oracle.build_prefix(from_torch_bf16(t["vp"][0, 0]), ct)["values"]
    ref, bnd = group_reference_and_bounds(q, kc, vc, kp, vp, w.softmax_scale, do,
                                          prefix_rounded=ct != "bf16")
    return dict(w=w, q=q, kc=kc, vc=vc, kp=kp, vp=vp, do=do, ref=ref, bnd=bnd)


@pytest.fixture(scope="module", params=[("bf16", 0.1), ("q8_0", 0.1), ("bf16", 1.0),
                                        ("q8_0", 1.0)], ids=lambda p: f"{p[0]}-std{p[1]}")
def group(request):
    return _group(*request.param)


def test_bf16_rounded_oracle_is_inside(group):
    ref, bnd = group["ref"], group["bnd"]
    for k in ("o", "dq", "dk", "dv"):
        assert ratio(_bf16(ref[k]), ref[k], bnd[k]) <= 0.5, k


def test_fp32_forward_with_bf16_probabilities_is_inside(group):
    """A forward computed the GPU's way in fp32 (operands rounded to bf16, bf16
    probabilities, fp32 sums, bf16 output) stays inside the O and LSE bounds."""
    g = group
    P = g["kp"].shape[0]
    C = g["q"].shape[1]
    kf = _bf16(np.concatenate([g["kp"], g["kc"]])).astype(np.float32)
    vf = _bf16(np.concatenate([g["vp"], g["vc"]])).astype(np.float32)
    allowed = oracle.allowed_mask(P, C)
    worst = 0.0
    for h in range(g["q"].shape[0]):
        s = np.float32(g["w"].softmax_scale) * (g["q"][h].astype(np.float32) @ kf.T)
        m = np.where(allowed, s, -np.inf).max(axis=1, keepdims=True)
        p = np.where(allowed, _bf16(np.exp(s - m)), 0.0).astype(np.float32)
        lsum = p.sum(axis=1, keepdims=True)
        o = _bf16((p @ vf) / lsum)
        lse = (m + np.log(lsum))[:, 0]
        worst = max(worst, ratio(o, g["ref"]["o"][h], g["bnd"]["o"][h]),
                    ratio(lse, g["ref"]["lse"][h], g["bnd"]["lse"][h]))
    assert worst <= 1.0
    print(f"fp32 forward: largest error / bound {worst:.3f}")


def _unit(group):
    if group["w"].qkv_std < 1.0:
        pytest.skip("near-uniform softmax: neighbouring rows are almost equal")
    return group["ref"], group["bnd"]


@pytest.mark.parametrize("name", ["o", "dq"])
def test_wrong_rows_are_outside(group, name):
    ref, bnd = (x[name] for x in _unit(group))
    got = ref.copy()
    got[0, 40] = ref[0, 41]                          # a row holding its neighbour
    assert ratio(got, ref, bnd) > 1.0
    got = ref.copy()
    got[1, 10, :64] = ref[0, 10, :64]                # half a row from the other head
    assert ratio(got, ref, bnd) > 1.0
    got = ref.copy()
    got[0, 63] = 0.0                                 # a row never written
    assert ratio(got, ref, bnd) > 1.0
    assert row_rel_l2(got, ref) == pytest.approx(1.0)


@pytest.mark.parametrize("name", ["dk", "dv"])
def test_wrong_key_rows_are_outside(group, name):
    ref, bnd = (x[name] for x in _unit(group))
    got = ref.copy()
    got[5] = ref[6]
    assert ratio(got, ref, bnd) > 1.0
    got = ref.copy()
    got[30, 64:] = ref[31, 64:]
    assert ratio(got, ref, bnd) > 1.0


def test_unwritten_rows_are_outside_for_workload_scale_inputs(group):
    """At the workloads' own scale (std 0.1) a row left at zero is still caught in O
    and in dK / dV."""
    if group["w"].qkv_std >= 1.0:
        pytest.skip("covered above")
    for name, idx in (("o", (0, 63)), ("dk", (30,)), ("dv", (30,))):
        ref, bnd = group["ref"][name], group["bnd"][name]
        got = ref.copy()
        got[idx] = 0.0
        assert ratio(got, ref, bnd) > 1.0, name
