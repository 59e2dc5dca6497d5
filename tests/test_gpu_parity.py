"""GPU parity of the HIP path against the fp64 oracle, through the C-ABI.

Bars: q8_0 / F16 / bf16 appends and the q8_0 dequant hook bit-exact; O within 1e-2
relative L2, dQ / dK / dV within 2e-2, LSE within 5e-3 absolute; bitwise run-to-run
determinism. Small shapes (several tiles, ragged tails, splits) are compared in
full; the three large workloads run at their full sizes with the launch
configuration the benchmark times and are compared on sampled (window, KV head)
groups that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import (DEV, Case, assert_bounded, assert_within, compare_groups,
                  compare_groups_bounded, f64, rel_l2, sample_groups)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import prefix_kv_attention_amd  # noqa: F401  (fails loudly without libpka.so)


def _label(w):
    return (f"{w.name} B{w.batch} Hq{w.n_heads_q} Hkv{w.n_heads_kv} D{w.head_dim} "
            f"P{w.prefix_len} C{w.chunk_len} {w.cache_type}")


EDGE = [
    synthetic.small("p0", prefix_len=0, chunk_len=64, head_dim=64),
    synthetic.small("ragged", prefix_len=100, chunk_len=37, head_dim=64),
    synthetic.small("c1", prefix_len=300, chunk_len=1, n_heads_q=6, n_heads_kv=1,
                    head_dim=128, cache_type="bf16"),
    synthetic.small("g5-q8", prefix_len=1000, chunk_len=100, n_heads_q=5, n_heads_kv=1,
                    head_dim=128, cache_type="q8_0", prefix_std=1.0),
    synthetic.small("g1-b2", batch=2, prefix_len=64, chunk_len=64, n_heads_q=2,
                    n_heads_kv=2, head_dim=128),
    synthetic.small("g3-d64-q8", batch=2, prefix_len=513, chunk_len=130, n_heads_q=6,
                    n_heads_kv=2, head_dim=64, cache_type="q8_0"),
    synthetic.small("split-bf16", prefix_len=2000, chunk_len=256, n_heads_q=4,
                    n_heads_kv=1, head_dim=128, cache_type="bf16"),
    synthetic.small("sharp-f16", prefix_len=700, chunk_len=90, n_heads_q=4, n_heads_kv=2,
                    head_dim=128, qkv_std=1.0, prefix_std=1.0),
    synthetic.small("g6-c512", batch=1, prefix_len=1500, chunk_len=512, n_heads_q=6,
                    n_heads_kv=1, head_dim=128, cache_type="q8_0", qkv_std=0.1,
                    prefix_std=1.0, do_std=1e-2, outlier_frac=0.01),
    # prefix split of dQ without a row split of dK/dV (128 dQ units, 256 dK/dV units)
    synthetic.small("dq-split-only", batch=2, prefix_len=2048, chunk_len=2048, n_heads_q=8,
                    n_heads_kv=8, head_dim=64, cache_type="bf16", qkv_std=0.3, prefix_std=0.3),
    # row split of dK/dV without a prefix split of dQ (256 dQ units, 64 dK/dV units)
    synthetic.small("dkv-split-only", batch=8, prefix_len=128, chunk_len=64, n_heads_q=128,
                    n_heads_kv=8, head_dim=64, cache_type="f16", qkv_std=0.3, prefix_std=0.3),
    # very sharp softmax (logit std ~9 and ~4): the forward raises its reference max
    # often and most probabilities underflow
    synthetic.small("very-sharp-bf16", prefix_len=1000, chunk_len=130, n_heads_q=4,
                    n_heads_kv=1, head_dim=128, cache_type="bf16", qkv_std=3.0,
                    prefix_std=3.0),
    # plain causal attention over a long chunk: every tile crosses the chunk
    synthetic.small("p0-c2048", batch=1, prefix_len=0, chunk_len=2048, n_heads_q=4,
                    n_heads_kv=2, head_dim=128, cache_type="bf16", qkv_std=0.3),
]


def _full_parity(case: Case):
    o, lse = case.fwd()
    delta = torch.empty(lse.shape, dtype=torch.float32, device=DEV)
    dq, dk, dv = case.bwd(o, lse, delta=delta)
    torch.cuda.synchronize()
    errs = compare_groups(case, case.all_groups(), o, lse, dq, dk, dv, delta)
    assert_within(errs, _label(case.w))
    return errs


@pytest.mark.parametrize("w", EDGE, ids=lambda w: w.name)
def test_parity_edge_shapes(w):
    print(_label(w), flush=True)
    _full_parity(Case(w))


@pytest.mark.parametrize("w", synthetic.WORKLOADS[:2], ids=lambda w: w.name)
def test_parity_small_workloads(w):
    print(_label(w), flush=True)
    errs = _full_parity(Case(w))
    print(errs, flush=True)


def _sampled_full_size(w, lse_fixed_bar=True):
    print(_label(w), flush=True)
    case = Case(w)
    o, lse = case.fwd()
    dq, dk, dv = case.bwd(o, lse)
    torch.cuda.synchronize()
    # properties that hold at any size: finite outputs
    for t in (o, dq, dk, dv, lse):
        assert torch.isfinite(t.float()).all()
    errs = compare_groups_bounded(case, sample_groups(case, 4), o, lse, dq, dk, dv)
    print(errs, flush=True)
    if not lse_fixed_bar:
        # Keys far from unit scale read through bf16 move the LSE by up to
        # scale * 2^-8 * sum_d |q_d k_d| (tests/_bounds.py), above the fixed 5e-3 bar
        # that assumes unit-scale logits: LSE is gated by its element bound alone.
        errs = dict(errs)
        errs.pop("lse_abs")
    assert_bounded(errs, _label(w))
    return errs


@pytest.mark.parametrize("w", synthetic.WORKLOADS[2:], ids=lambda w: w.name)
def test_parity_full_size_sampled(w):
    """Full-size launch with the benchmark's configuration; the oracle recomputes four
    (window, KV head) groups (first, last and interior ones). Gates: the stated
    relative-L2 bars over the sampled groups, and every element of O, LSE, dQ, dK, dV
    within its first-order rounding bound (tests/_bounds.py); the worst per-head and
    per-row relative L2 are printed."""
    _sampled_full_size(w)


@pytest.mark.parametrize("w", synthetic.WORKLOADS[2:], ids=lambda w: w.name)
def test_parity_full_size_sampled_unit_scale(w):
    """The same launches with unit-scale Q, K, V and prefix (logits ~ N(0, 1) and
    wider): the workloads' own 0.1 scale makes the softmax nearly uniform, so rows
    differ little; at unit scale a row computed from wrong keys, a wrong head or a
    wrong mask falls outside the element bound (checked on the CPU in
    tests/test_bounds_gate.py)."""
    _sampled_full_size(w.with_(name=w.name + "-unit", qkv_std=1.0, prefix_std=1.0,
                               seed=w.seed + 100), lse_fixed_bar=w.cache_type == "bf16")


def _cache_bits(cache, rows=None):
    sl = slice(None) if rows is None else rows
    out = {}
    if cache.cache_type == "q8_0":
        out["qs_k"] = cache.k[:, :, sl].cpu().numpy()
        out["qs_v"] = cache.v[:, :, sl].cpu().numpy()
        out["d_k"] = cache.k_scale[:, :, sl].cpu().view(torch.int16).numpy().view(np.uint16)
        out["d_v"] = cache.v_scale[:, :, sl].cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        out["k"] = cache.k[:, :, sl].cpu().view(torch.int16).numpy().view(np.uint16)
        out["v"] = cache.v[:, :, sl].cpu().view(torch.int16).numpy().view(np.uint16)
    return out


def _oracle_bits(x_f32, cache_type):
    c = oracle.build_prefix(x_f32, cache_type)
    if cache_type == "q8_0":
        return c["qs"], c["d"].view(np.uint16)
    if cache_type == "f16":
        return c["f16"].view(np.uint16), None
    return c["bits"], None


def _assert_rows_bitexact(cache, rows, k_f32, v_f32):
    got = _cache_bits(cache, rows)
    kq, kd = _oracle_bits(k_f32, cache.cache_type)
    vq, vd = _oracle_bits(v_f32, cache.cache_type)
    if cache.cache_type == "q8_0":
        np.testing.assert_array_equal(got["qs_k"], kq)
        np.testing.assert_array_equal(got["qs_v"], vq)
        np.testing.assert_array_equal(got["d_k"], kd)
        np.testing.assert_array_equal(got["d_v"], vd)
    else:
        np.testing.assert_array_equal(got["k"], kq)
        np.testing.assert_array_equal(got["v"], vq)


@pytest.mark.parametrize("ct", ["q8_0", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_append_bitexact(ct, D):
    w = synthetic.small(f"app-{ct}", batch=2, n_heads_q=4, n_heads_kv=2, head_dim=D,
                        prefix_len=333, chunk_len=77, cache_type=ct, prefix_std=1.0,
                        outlier_frac=0.01, seed=5)
    print(_label(w), flush=True)
    case = Case(w)
    import prefix_kv_attention_amd as pka
    pka.kv_append(case.dev["kc"], case.dev["vc"], case.cache, w.prefix_len)
    torch.cuda.synchronize()
    from oracle.cache import from_torch_bf16
    _assert_rows_bitexact(case.cache, slice(0, w.prefix_len),
                          from_torch_bf16(case.cpu["kp"]), from_torch_bf16(case.cpu["vp"]))
    _assert_rows_bitexact(case.cache, slice(w.prefix_len, w.prefix_len + w.chunk_len),
                          from_torch_bf16(case.cpu["kc"]), from_torch_bf16(case.cpu["vc"]))


def test_append_q8_0_special_blocks():
    """Zero blocks, exact ties and negative amax written by the GPU quantiser."""
    import prefix_kv_attention_amd as pka
    from oracle.cache import from_torch_bf16
    x = np.zeros((1, 1, 8, 64), np.float32)
    x[0, 0, 1, 0] = 127.0
    x[0, 0, 1, 1:31] = np.arange(30) + 0.5          # exact ties with d = 1
    x[0, 0, 2, 32] = -127.0
    x[0, 0, 2, 33:40] = -(np.arange(7) + 0.5)
    x[0, 0, 3, :] = 1e-3                            # tiny block
    x[0, 0, 4, 5] = 8.0
    x[0, 0, 4, 6] = 0.03125
    kb = torch.from_numpy(x).to(torch.bfloat16)
    cache = pka.PrefixCache.empty("q8_0", 1, 1, 8, 64, DEV)
    pka.kv_append_q8_0(kb.to(DEV), kb.to(DEV), cache, 0)
    torch.cuda.synchronize()
    _assert_rows_bitexact(cache, slice(0, 8), from_torch_bf16(kb), from_torch_bf16(kb))


def test_dequant_hook_bitexact():
    import prefix_kv_attention_amd as pka
    w = synthetic.small("deq", batch=2, n_heads_kv=2, n_heads_q=2, head_dim=128,
                        prefix_len=200, chunk_len=8, cache_type="q8_0", prefix_std=1.0,
                        outlier_frac=0.01)
    case = Case(w)
    f32, bf = pka.kv_dequant_q8_0(case.cache, 17, 150)
    torch.cuda.synchronize()
    from oracle.cache import from_torch_bf16
    for i, name in enumerate(("kp", "vp")):
        x = from_torch_bf16(case.cpu[name])
        qs, d = oracle.quantise_q8_0(x)
        ref = oracle.dequantise_q8_0(qs, d)[:, :, 17:167]
        np.testing.assert_array_equal(f32[i].cpu().numpy(), ref)
        np.testing.assert_array_equal(
            bf[i].cpu().view(torch.int16).numpy().view(np.uint16), oracle.f32_to_bf16_rne(ref))


def test_dequant_hook_overflowing_scale():
    """A block with amax above 127 * 65504 gets an infinite fp16 scale. The hook runs
    the attention staging's own conversion, so it must give what the plain product
    f32(d16) * q gives: +-inf for nonzero codes and NaN for zero codes (and the bf16
    operand bits of the same values), exactly as the oracle's dequantiser."""
    import prefix_kv_attention_amd as pka
    from oracle.cache import from_torch_bf16
    x = np.zeros((1, 1, 4, 64), np.float32)
    x[0, 0, 0, :32] = np.linspace(-3e7, 3e7, 32)     # scale overflows
    x[0, 0, 0, 10] = 0.0                              # ... with a zero code
    x[0, 0, 1, 32:] = 1.0e9                           # scale overflows, every code 127
    x[0, 0, 2, 5] = 8.0e6                             # largest finite scale region
    x[0, 0, 3, :] = np.arange(64) - 31.5              # ordinary block
    kb = torch.from_numpy(x).to(torch.bfloat16)
    cache = pka.PrefixCache.empty("q8_0", 1, 1, 4, 64, DEV)
    pka.kv_append_q8_0(kb.to(DEV), kb.to(DEV), cache, 0)
    f32, bf = pka.kv_dequant_q8_0(cache, 0, 4)
    torch.cuda.synchronize()
    qs, d = oracle.quantise_q8_0(from_torch_bf16(kb))
    assert np.isinf(d.astype(np.float32)).sum() >= 2, "the planted blocks must overflow"
    with np.errstate(invalid="ignore"):
        ref = oracle.dequantise_q8_0(qs, d)
    for i in range(2):
        got = f32[i].cpu().numpy()
        np.testing.assert_array_equal(got, ref)          # NaN positions must match too
        fin = np.isfinite(ref)
        gbits = bf[i].cpu().view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(gbits[fin], oracle.f32_to_bf16_rne(ref[fin]))
        assert np.array_equal(np.isnan(bf[i].cpu().float().numpy()), np.isnan(ref))
        inf = np.isinf(ref)
        np.testing.assert_array_equal(gbits[inf], oracle.f32_to_bf16_rne(ref[inf]))


def test_very_sharp_q8_lse_within_operand_rounding_bound():
    """Large keys from a q8_0 cache (2 % outliers x8 at std 2: |k| up to ~50) and a
    sharp softmax. The MFMA reads each dequantised key rounded to bf16 (relative error
    <= 2^-8), so a score moves by at most scale * 2^-8 * sum_d |q_d k_d|; LSE is
    1-Lipschitz in the scores (sup norm), and the row sum of bf16 probabilities adds
    <= 2^-8 relative. Each row's LSE error must stay within that bound (the fixed 5e-3
    bar assumes unit-scale logits); O, dQ, dK, dV keep the standard bars."""
    w = synthetic.small("very-sharp-q8", batch=2, prefix_len=700, chunk_len=70, n_heads_q=6,
                        n_heads_kv=2, head_dim=64, cache_type="q8_0", qkv_std=2.0,
                        prefix_std=2.0, outlier_frac=0.02)
    print(_label(w), flush=True)
    case = Case(w)
    o, lse = case.fwd()
    dq, dk, dv = case.bwd(o, lse)
    torch.cuda.synchronize()
    groups = case.all_groups()
    errs = compare_groups(case, groups, o, lse, dq, dk, dv)
    print(errs, flush=True)
    assert_within({k: v for k, v in errs.items() if k != "lse_abs"}, _label(w))
    kpv, _ = case.oracle_prefix()
    G, P = w.group, w.prefix_len
    worst = 0.0
    for b, kv in groups:
        hs = slice(kv * G, (kv + 1) * G)
        q = np.abs(f64(case.cpu["q"][b, hs]))                           # [G][C][D]
        kf = np.abs(np.concatenate([kpv[b, kv], f64(case.cpu["kc"][b, kv])]))
        allowed = oracle.allowed_mask(P, w.chunk_len)                   # [C][P+C]
        mag = np.where(allowed[None], q @ kf.T, 0.0).max(axis=2)         # [G][C]
        bound = w.softmax_scale * 2.0 ** -8 * mag + 2.0 ** -8 + 1e-4
        err = np.abs(f64(lse[b, hs]) - case.oracle_group(b, kv)["lse"])
        assert np.all(err <= bound), f"(b={b}, kv={kv}): LSE error above its bound"
        worst = max(worst, float((err / bound).max()))
    print(f"largest LSE error / bound: {worst:.3f}", flush=True)


def test_closed_form_zero_queries():
    """Q = 0: LSE = ln(P + i + 1); O = mean of allowed values; dK exactly zero."""
    w = synthetic.small("q0", prefix_len=777, chunk_len=70, n_heads_q=4, n_heads_kv=2,
                        head_dim=128, cache_type="bf16")
    inputs = synthetic.make_inputs(w)
    inputs["q"].zero_()
    case = Case(w, inputs=inputs)
    o, lse = case.fwd()
    dq, dk, dv = case.bwd(o, lse)
    torch.cuda.synchronize()
    want = np.log(w.prefix_len + 1 + np.arange(w.chunk_len))
    assert np.abs(f64(lse) - want).max() <= 1e-5
    assert bool((dk == 0).all())
    errs = compare_groups(case, case.all_groups(), o, lse, dq, dk, dv)
    assert_within({k: v for k, v in errs.items() if k != "dk"}, "q0")


@pytest.mark.parametrize("ct", ["q8_0", "f16", "bf16"])
def test_closed_form_constant_values(ct):
    """V = c for every key (prefix and chunk): O = c, and since dP_ij = dO_i . c = Delta_i
    for every key, dS = 0, so dQ and dK vanish (up to fp32 rounding of the two equal
    dot products). c = 127/128 is exact in bf16, in F16 and in q8_0 (scale 2^-7, codes
    127), so the cache holds c exactly for every cache type."""
    c = 127.0 / 128.0
    w = synthetic.small(f"vconst-{ct}", batch=2, prefix_len=700, chunk_len=90, n_heads_q=6,
                        n_heads_kv=2, head_dim=128, cache_type=ct, qkv_std=0.5, prefix_std=0.5)
    inputs = synthetic.make_inputs(w)
    inputs["vc"].fill_(c)
    inputs["vp"].fill_(c)
    case = Case(w, inputs=inputs)
    o, lse = case.fwd()
    dq, dk, dv = case.bwd(o, lse)
    torch.cuda.synchronize()
    assert np.abs(f64(o) - c).max() <= 2.0 ** -9 * c
    # dP~ - Delta~ subtracts two fp32 sums of the same D products dO_id c, each within
    # D 2^-24 c |dO_i|_1 of the exact value, so |dS_ij| <= P_ij e_i with
    # e_i = 2 D 2^-24 c |dO_i|_1 (1 + 2^-8 for a rounded key read); then
    # |dQ_id| <= scale e_i max_j |K_jd| and |dK_td| <= scale sum_{g,i} e_gi |Q_gid|.
    D, G = w.head_dim, w.group
    e = 2 * D * 2.0 ** -24 * c * np.abs(f64(case.cpu["do"])).sum(-1) * (1 + 2.0 ** -8)
    kpv, _ = case.oracle_prefix()
    kmax = np.maximum(np.abs(kpv).max(axis=2), np.abs(f64(case.cpu["kc"])).max(axis=2))
    bq = w.softmax_scale * e[..., None] * np.repeat(kmax, G, axis=1)[:, :, None, :]
    assert np.all(np.abs(f64(dq)) <= bq)
    aq = np.abs(f64(case.cpu["q"])) * e[..., None]                       # [B][Hq][C][D]
    bk = w.softmax_scale * aq.reshape(w.batch, w.n_heads_kv, G * w.chunk_len, D).sum(2)
    assert np.all(np.abs(f64(dk)) <= bk[:, :, None, :])
    errs = compare_groups(case, case.all_groups(), o, lse, dq, dk, dv)
    assert_within({k: v for k, v in errs.items() if k in ("o", "dv", "lse_abs")}, w.name)


@pytest.mark.parametrize("ct", ["q8_0", "bf16"])
def test_closed_form_single_token(ct):
    """C = 1 and P = 0: the one query sees only its own key, so its probability is 1:
    O = V_0 and dV = dO exactly, LSE = scale q . k, and dS = dP - Delta = dO . V_0 -
    dO . O = 0, so dQ and dK vanish (up to fp32 rounding of two equal dot products)."""
    w = synthetic.small(f"c1p0-{ct}", batch=3, prefix_len=0, chunk_len=1, n_heads_q=4,
                        n_heads_kv=4, head_dim=128, cache_type=ct, qkv_std=1.0)
    case = Case(w)
    o, lse = case.fwd()
    dq, dk, dv = case.bwd(o, lse)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), case.cpu["vc"])           # G = 1: one query head per KV head
    assert torch.equal(dv.cpu(), case.cpu["do"])
    q = f64(case.cpu["q"])
    k = f64(case.cpu["kc"])
    assert np.abs(f64(lse) - w.softmax_scale * (q * k).sum(-1)).max() <= 1e-5
    # dS = P (dP~ - Delta~): two fp32 sums of the same D products, each within
    # D 2^-24 |dO|.|V| of the exact value, and P = 1 + O(1e-6)
    e = 2.05 * w.head_dim * 2.0 ** -24 * (np.abs(f64(case.cpu["do"])) *
                                          np.abs(f64(case.cpu["vc"]))).sum(-1)
    assert np.all(np.abs(f64(dq)) <= w.softmax_scale * e[..., None] * np.abs(k))
    assert np.all(np.abs(f64(dk)) <= w.softmax_scale * e[..., None] * np.abs(q))


@pytest.mark.parametrize("w", [synthetic.WORKLOADS[1], EDGE[3], EDGE[6]], ids=lambda w: w.name)
def test_bitwise_determinism(w):
    """Same inputs twice -> identical bits (no atomics; fixed-order split merges)."""
    case = Case(w)
    runs = []
    for _ in range(2):
        o, lse = case.fwd()
        dq, dk, dv = case.bwd(o, lse)
        runs.append([t.clone() for t in (o, lse, dq, dk, dv)])
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)
    for a, b in zip(*runs):
        assert torch.equal(bits(a), bits(b))


@pytest.mark.parametrize("ct", ["q8_0", "f16"])
def test_walk_two_chunks(ct):
    """Chunk 1 at P, append it, then chunk 2 at P + C reads chunk 1 from the cache."""
    import prefix_kv_attention_amd as pka
    from oracle.cache import from_torch_bf16
    w1 = synthetic.small("walk1", prefix_len=400, chunk_len=96, n_heads_q=6, n_heads_kv=2,
                         head_dim=128, cache_type=ct, seed=31)
    case = Case(w1, extra_capacity=96)
    o, lse = case.fwd()
    case.bwd(o, lse)
    pka.kv_append(case.dev["kc"], case.dev["vc"], case.cache, w1.prefix_len)
    w2 = w1.with_(prefix_len=w1.prefix_len + w1.chunk_len, seed=32)
    inp2 = synthetic.make_inputs(w2)
    # The next chunk's cache is the first cache plus the appended chunk.
    inp2["kp"] = torch.cat([case.cpu["kp"], case.cpu["kc"]], dim=2)
    inp2["vp"] = torch.cat([case.cpu["vp"], case.cpu["vc"]], dim=2)
    case2 = Case.__new__(Case)
    case2.pka, case2.w, case2.cpu = pka, w2, inp2
    case2.dev = {k: v.to(DEV) for k, v in inp2.items() if k not in ("kp", "vp")}
    case2.capacity, case2.cache, case2._oracle_prefix = case.capacity, case.cache, None
    o2, lse2 = case2.fwd()
    dq2, dk2, dv2 = case2.bwd(o2, lse2)
    torch.cuda.synchronize()
    errs = compare_groups(case2, case2.all_groups(), o2, lse2, dq2, dk2, dv2)
    assert_within(errs, "walk step 2")
    _assert_rows_bitexact(case.cache, slice(w1.prefix_len, w2.prefix_len),
                          from_torch_bf16(case.cpu["kc"]), from_torch_bf16(case.cpu["vc"]))


def test_autograd_function_and_stop_gradient():
    import prefix_kv_attention_amd as pka
    w = synthetic.small("ag", prefix_len=150, chunk_len=40, n_heads_q=4, n_heads_kv=2,
                        head_dim=64, cache_type="bf16")
    case = Case(w)
    q = case.dev["q"].clone().requires_grad_(True)
    k = case.dev["kc"].clone().requires_grad_(True)
    v = case.dev["vc"].clone().requires_grad_(True)
    cache_k = case.cache.k
    cache_k.requires_grad_(False)
    o = pka.chunk_attention(q, k, v, case.cache, w.prefix_len, w.softmax_scale)
    o.backward(case.dev["do"])
    o2, lse2 = case.fwd()
    dq, dk, dv = case.bwd(o2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)
    assert case.cache.k.grad is None and case.cache.v.grad is None


def test_error_paths_raise_before_launch():
    import prefix_kv_attention_amd as pka
    w = synthetic.small("err", prefix_len=64, chunk_len=16)
    case = Case(w)
    small = pka.PrefixCache.empty("f16", 1, 1, 10, 64, DEV)
    with pytest.raises(pka.PkaError, match="CAPACITY"):
        pka.chunk_attn_fwd(case.dev["q"], case.dev["kc"], case.dev["vc"], small, 64, 0.125)
    with pytest.raises(pka.PkaError, match="UNSUPPORTED"):
        pka.kv_append_q8_0(case.dev["kc"], case.dev["vc"], case.cache, 64)
    q96 = torch.zeros((1, 2, 16, 96), dtype=torch.bfloat16, device=DEV)
    c96 = pka.PrefixCache.empty("f16", 1, 1, 80, 96, DEV)
    with pytest.raises(pka.PkaError, match="UNSUPPORTED"):
        pka.chunk_attn_fwd(q96, q96[:, :1].contiguous(), q96[:, :1].contiguous(), c96, 64, 0.1)


def test_binding_rejects_mismatched_tensors():
    """The C entry points see bare pointers: the binding checks every tensor's shape,
    dtype, device and layout first and raises ValueError without launching."""
    import prefix_kv_attention_amd as pka
    w = synthetic.small("shapes", prefix_len=64, chunk_len=16, n_heads_q=4, n_heads_kv=2)
    case = Case(w)
    d, P, sc = case.dev, w.prefix_len, w.softmax_scale
    q, k, v = d["q"], d["kc"], d["vc"]
    o, lse = pka.chunk_attn_fwd(q, k, v, case.cache, P, sc)
    torch.cuda.synchronize()
    bad_calls = {
        "v shorter": lambda: pka.chunk_attn_fwd(q, k, v[:, :, :8].contiguous(), case.cache, P, sc),
        "o shape": lambda: pka.chunk_attn_fwd(q, k, v, case.cache, P, sc, o=o[:, :2].contiguous()),
        "lse dtype": lambda: pka.chunk_attn_fwd(q, k, v, case.cache, P, sc, lse=lse.double()),
        "q on cpu": lambda: pka.chunk_attn_fwd(q.cpu(), k, v, case.cache, P, sc),
        "q transposed": lambda: pka.chunk_attn_fwd(q.transpose(2, 3), k, v, case.cache, P, sc),
        "ws on cpu": lambda: pka.chunk_attn_fwd(q, k, v, case.cache, P, sc,
                                                ws=torch.empty(1 << 20, dtype=torch.uint8)),
        "cache batch": lambda: pka.chunk_attn_fwd(
            q, k, v, pka.PrefixCache.empty("f16", 2, 2, P + 16, 64, DEV), P, sc),
        "dk shape": lambda: pka.chunk_attn_bwd(q, k, v, case.cache, P, sc, o, lse, d["do"],
                                               dk=torch.empty_like(q)),
        "delta shape": lambda: pka.chunk_attn_bwd(
            q, k, v, case.cache, P, sc, o, lse, d["do"],
            delta=torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)),
        "d_o dtype": lambda: pka.chunk_attn_bwd(q, k, v, case.cache, P, sc, o, lse,
                                                d["do"].float()),
        "prefix dk shape": lambda: pka.prefix_kv_grad(
            q, case.cache, P, sc, lse, d["do"], torch.zeros_like(lse), 32,
            dk=torch.empty((1, 2, 16, 64), dtype=torch.float32, device=DEV)),
        "append v shape": lambda: pka.kv_append(k, v[:, :1].contiguous(), case.cache, P),
        "cache dtype": lambda: pka.PrefixCache(
            "bf16", case.cache.k, case.cache.v),   # an f16 cache's tensors as bf16
        "q8 scales": lambda: pka.PrefixCache(
            "q8_0", torch.empty((1, 2, 80, 64), dtype=torch.int8, device=DEV),
            torch.empty((1, 2, 80, 64), dtype=torch.int8, device=DEV)),
    }
    for name, call in bad_calls.items():
        with pytest.raises(ValueError):
            call()
            pytest.fail(f"{name}: no error")
    torch.cuda.synchronize()
    o2, lse2 = pka.chunk_attn_fwd(q, k, v, case.cache, P, sc)   # the good call still works
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("ct", ["q8_0", "f16", "bf16"])
def test_forward_backward_leave_cache_untouched(ct):
    """The prefix is read-only and stop-gradient: fwd and bwd change no cache byte."""
    w = synthetic.small(f"ro-{ct}", batch=2, prefix_len=640, chunk_len=96, n_heads_q=4,
                        n_heads_kv=2, head_dim=128, cache_type=ct, prefix_std=1.0)
    case = Case(w, extra_capacity=32)
    before = [t.clone() for t in (case.cache.k, case.cache.v, case.cache.k_scale,
                                  case.cache.v_scale) if t is not None]
    o, lse = case.fwd()
    case.bwd(o, lse)
    torch.cuda.synchronize()
    after = [t for t in (case.cache.k, case.cache.v, case.cache.k_scale, case.cache.v_scale)
             if t is not None]
    for a, b in zip(before, after):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_parity_group1_full_width():
    """G = 1 (no GQA) at the headline's P and C, sampled groups."""
    _sampled_full_size(synthetic.HEADLINE.with_(name="g1-16k", batch=2, n_heads_q=8,
                                                n_heads_kv=8, seed=9))
