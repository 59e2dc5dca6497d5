"""Pins of the oracle's cache conversions (q8_0, F16, bf16) -- CPU only.

Each check ties oracle/cache.py to something other than itself: hand-derived blocks
(tests/golden/q8_0_blocks.txt), algebraic properties of the q8_0 definition, an
independent re-derivation with Python's float division and struct rounding, and
torch's own fp16 / bf16 conversions.
"""
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q8_0_blocks.txt")


def load_golden():
    cases, cur = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0]}
                cases.append(cur)
            elif key == "x":
                cur["x"] = [float(v) for v in vals]
            elif key == "d16":
                cur["d16"] = int(vals[0], 16)
            elif key == "q":
                cur["q"] = [int(v) for v in vals]
    return cases


def pad32(v, dtype):
    a = np.zeros(32, dtype=dtype)
    a[:len(v)] = v
    return a


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c["name"])
def test_q8_0_hand_blocks(case):
    x = pad32(case["x"], np.float32)
    qs, d = oracle.quantise_q8_0(x[None, :])
    assert int(d.view(np.uint16)[0, 0]) == case["d16"]
    np.testing.assert_array_equal(qs[0], pad32(case["q"], np.int8))
    # dequantise is exactly d16 * q
    back = oracle.dequantise_q8_0(qs, d)
    exp = np.float32(np.float16(np.uint16(case["d16"]).view(np.float16))) * pad32(case["q"], np.float32)
    np.testing.assert_array_equal(back[0], exp)


def _prefix_sample(n_rows=4096, seed=2):
    """Rows drawn by the q8_0 workload's recipe (N(0,1), 1% outliers x8, bf16)."""
    w = synthetic.WORKLOAD_BY_NAME["q8_0-16k"].with_(
        batch=1, n_heads_kv=1, n_heads_q=1, prefix_len=n_rows, chunk_len=1, seed=seed)
    t = synthetic.make_inputs(w)
    return oracle.cache.from_torch_bf16(t["kp"]).reshape(-1, w.head_dim)


def test_q8_0_properties():
    x = _prefix_sample()
    qs, d = oracle.quantise_q8_0(x)
    blk = x.reshape(-1, 32)
    q = qs.reshape(-1, 32).astype(np.int32)
    d32 = (np.abs(blk).max(axis=1) / np.float32(127))
    # max |q| == 127 in every non-zero block; codes stay in [-127, 127]
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert q.min() >= -127 and q.max() <= 127
    # odd symmetry: quant(-x) == -quant(x) with the same scale
    qn, dn = oracle.quantise_q8_0(-x)
    np.testing.assert_array_equal(qn, -qs)
    np.testing.assert_array_equal(dn, d)
    # error bound: |x - d16 q| <= d/2 + 127 |d - d16| (plus fp32 rounding of x/d)
    d16 = d.reshape(-1).astype(np.float64)
    err = np.abs(blk.astype(np.float64) - d16[:, None] * q)
    bound = d32.astype(np.float64) * (0.5 + 1e-6) + 127 * np.abs(d32 - d16)
    assert np.all(err <= bound[:, None])


def _py_quant_block(vals):
    """Independent q8_0 of one block: Python doubles + struct rounding to fp32/fp16."""
    f32 = lambda v: struct.unpack("<f", struct.pack("<f", v))[0]
    amax = max(abs(v) for v in vals)
    # a/b of two fp32 values computed in double then rounded to fp32 equals the
    # correctly rounded fp32 quotient (53 >= 2*24 + 2).
    d = f32(amax / 127.0)
    d16 = struct.unpack("<H", struct.pack("<e", d))[0]
    out = []
    for v in vals:
        if d == 0.0:
            out.append(0)
            continue
        r = f32(v / d)
        n = math.floor(abs(r) + 0.5)
        out.append(int(max(-127, min(127, n if r >= 0 else -n))))
    return d16, out


def test_q8_0_independent_rederivation():
    x = _prefix_sample(n_rows=1024, seed=7)
    blocks = x.reshape(-1, 32)
    qs, d = oracle.quantise_q8_0(x)
    qs = qs.reshape(-1, 32)
    dbits = d.reshape(-1).view(np.uint16)
    for i in range(blocks.shape[0]):
        d16, q = _py_quant_block([float(v) for v in blocks[i]])
        assert d16 == int(dbits[i]), i
        assert q == [int(c) for c in qs[i]], i


def test_q8_0_exact_ties_away_from_zero():
    # With amax = 127 the scale is exactly 1, so x/d = x and k + 0.5 are exact ties.
    ks = np.arange(0, 126, dtype=np.float32)
    x = np.zeros((len(ks), 32), np.float32)
    x[:, 0] = 127.0
    x[:, 1] = ks + 0.5
    x[:, 2] = -(ks + 0.5)
    qs, _ = oracle.quantise_q8_0(x)
    np.testing.assert_array_equal(qs[:, 1], (ks + 1).astype(np.int8))
    np.testing.assert_array_equal(qs[:, 2], -(ks + 1).astype(np.int8))


def test_f16_matches_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 0.1,
        rng.standard_normal(10000).astype(np.float32) * 1e-5,     # fp16 subnormals
        rng.standard_normal(10000).astype(np.float32) * 3e4,      # near overflow
    ])
    x = oracle.cache.from_torch_bf16(torch.from_numpy(x).to(torch.bfloat16))
    ours = oracle.to_f16(x).view(np.uint16)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(200000).astype(np.float32)
    # exact ties: low 16 bits = 0x8000, both parities of the kept lsb
    u = rng.integers(0, 2**31, 5000, dtype=np.uint32) & np.uint32(0xFFFF0000)
    ties = ((u | np.uint32(0x8000)) & np.uint32(0x7F7FFFFF)).view(np.float32)
    x = np.concatenate([x, ties])
    ours = oracle.f32_to_bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_build_prefix_values_are_stored_values():
    x = _prefix_sample(n_rows=64)
    for t in ("f16", "bf16", "q8_0"):
        c = oracle.build_prefix(x, t)
        assert c["values"].dtype == np.float64 and c["values"].shape == x.shape
    c = oracle.build_prefix(x, "bf16")
    np.testing.assert_array_equal(c["values"], x.astype(np.float64))  # bf16 in, bf16 out
