"""Oracle for prefix-KV chunk attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation of what the hot path computes:
masked-softmax attention of a trainable chunk against a frozen prefix plus the
chunk's own keys (forward and analytic backward, fp64), the cache conversions
(q8_0 quantise / dequantise and F16 storage, in exact fp32 / fp16 arithmetic), and
the row-sparse linear backward of the projections next to attention (fp64).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from here. The product (the HIP library and its
Python binding) shares no code with this package and never calls it.

Pins (what ties each function to something other than itself) live in
``tests/test_oracle_*.py``: finite differences, torch's scaled_dot_product_attention
with the prefix detached, full-window invariants, closed forms, shift invariances,
hand-derived q8_0 blocks and an independent re-derivation of q8_0 with Python's own
float and struct rounding, and torch autograd of a dense linear layer with the
upstream gradient masked. No function here is "parity unpinned".
"""
from .attention import (  # noqa: F401
    allowed_mask, kv_head_of, group_fwd, group_bwd, group_bwd_prefix, chunk_fwd, chunk_bwd,
    full_causal_fwd, full_causal_bwd, softmax_probs,
)
from .cache import (  # noqa: F401
    QK8_0, bf16_bits_to_f32, f32_to_bf16_rne, quantise_q8_0, dequantise_q8_0,
    to_f16, build_prefix, append_rows,
)
from .row_sparse import row_sparse_linear_bwd, row_sparse_flops  # noqa: F401
