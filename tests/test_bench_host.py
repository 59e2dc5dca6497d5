"""Host logic of bench.py, on the CPU: the FLOP and byte counts behind `value` and
`roofline`, the rule that ties a committed traffic figure to the kernel sources it was
taken on, and the refusal of more than one GPU.

The counts are pinned to brute force over the allowed (query, key) pairs of a small
window and to the pair count of the method's causal mask: every chunk row sees the
whole frozen prefix plus its own chunk prefix ("Context-Frozen Training", Phase 2;
"train: walk the window", What it is).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synthetic  # noqa: E402


def brute_pairs(P, C):
    prefix = sum(1 for t in range(C) for j in range(P + t + 1) if j < P)
    chunk = sum(1 for t in range(C) for j in range(P + t + 1) if j >= P)
    return prefix, chunk


@pytest.mark.parametrize("P,C", [(0, 1), (5, 3), (17, 9), (64, 33)])
def test_pairs_match_brute_force(P, C):
    w = synthetic.small(prefix_len=P, chunk_len=C)
    assert bench.pairs(w) == brute_pairs(P, C)


def test_flops_of_the_8b_workload():
    w = synthetic.WORKLOAD_BY_NAME["8b-16k"]
    B, Hq, D, P, C = 4, 32, 128, 16384, 512
    allowed = C * P + C * (C + 1) // 2          # every row: P prefix keys + t + 1 chunk keys
    per_contraction = 2 * B * Hq * D * allowed  # one multiply-add per (pair, head, dim)
    fwd, bwd, dq = bench.flops(w)
    assert fwd == 2 * per_contraction           # S = Q K^T and O = P V
    assert dq == 3 * per_contraction            # S recompute, dP = dO V^T, dQ = dS K
    # dK and dV exist for chunk keys only (the prefix is stop-gradient)
    assert bwd == dq + 2 * (2 * B * Hq * D * (C * (C + 1) // 2))
    assert fwd + bwd == 1_404_513_026_048    # per step: 1.40 TFLOP


def test_prefix_bytes_per_cache_format():
    w = synthetic.WORKLOAD_BY_NAME["8b-16k"]
    rows = 4 * 8 * 16384
    assert bench.prefix_bytes(w) == 2 * rows * 128 * 2          # bf16 K and V
    q8 = w.with_(cache_type=synthetic.CACHE_Q8_0)
    # q8_0: per 32 values, 32 int8 codes + one fp16 scale = 34 bytes
    assert bench.prefix_bytes(q8) == 2 * rows * (128 // 32) * 34


def test_traffic_figure_is_dropped_when_the_kernel_sources_change(monkeypatch):
    fig = bench.read_traffic("bwd_dq")
    if fig is None:
        pytest.skip("the committed counters predate the current kernel sources")
    assert fig > 0
    monkeypatch.setattr(bench, "source_digest", lambda files: "0000000000000000")
    assert bench.read_traffic("bwd_dq") is None
    assert bench.read_traffic("no_such_kernel") is None


def test_source_digest_covers_every_named_file():
    one = bench.source_digest(["attn_bwd.hip"])
    both = bench.source_digest(["attn_bwd.hip", "pka_device.hpp"])
    assert len(one) == 16 and one != both
    assert bench.source_digest(["attn_bwd.hip"]) == one


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_code_text_ignores_comments_and_layout_but_not_code():
    a = 'int x = 1; // one\n/* two\n   lines */ float y = f("a//b", \'/\');\n'
    b = 'int x = 1;   // uno\n\nfloat y = f("a//b", \'/\');'
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(a.replace("x = 1", "x = 2"))
    assert '"a//b"' in bench.code_text(a)          # a literal is not a comment
