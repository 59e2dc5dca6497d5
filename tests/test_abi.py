"""C-ABI tests that need no GPU: the library loads, exports every entry point that
include/pka.h declares, and refuses bad arguments on the host before any HIP call
(so nothing here launches a kernel)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pka.h")
LIB = os.path.join(ROOT, "prefix_kv_attention_amd", "libpka.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pka_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def pka():
    if not os.path.exists(LIB):
        pytest.fail("libpka.so is not built (python prefix_kv_attention_amd/build.py)")
    import prefix_kv_attention_amd as m
    return m


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("pka_chunk_attn_fwd", "pka_chunk_attn_fwd_append", "pka_chunk_attn_bwd",
              "pka_kv_append_q8_0",
              "pka_kv_append_f16", "pka_kv_append_bf16", "pka_kv_dequant_q8_0",
              "pka_fwd_workspace_bytes", "pka_bwd_workspace_bytes", "pka_prefix_kv_grad",
              "pka_prefix_kv_grad_workspace_bytes", "pka_status_string",
              "pka_last_error", "pka_profile_enable", "pka_profile_reset", "pka_profile_read"):
        assert n in names


def test_every_declared_symbol_is_exported(pka):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pka_[a-z0-9_]+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        getattr(pka.lib, n)      # resolvable through ctypes as well


# Fake, 16-byte aligned device addresses: every call below must fail validation,
# so none of them is ever dereferenced.
A = 0x7F0000000000
MIS = A + 8


def dims(pka, **kw):
    d = dict(batch=1, n_heads_q=4, n_heads_kv=2, head_dim=128, prefix_len=256,
             chunk_len=64, softmax_scale=0.125)
    d.update(kw)
    return pka.make_dims(**d)


def cache(pka, **kw):
    c = dict(type=pka.CACHE_F16, head_dim=128, capacity=512, k=A, v=A, k_scale=None,
             v_scale=None)
    c.update(kw)
    return pka.CacheDesc(c["type"], c["head_dim"], c["capacity"], c["k"], c["v"],
                         c["k_scale"], c["v_scale"])


def fwd(pka, d, c, ptrs=None, ws=None, ws_bytes=0):
    p = dict(q=A, k=A, v=A, o=A, lse=A)
    p.update(ptrs or {})
    st = pka.lib.pka_chunk_attn_fwd(ctypes.byref(d) if d is not None else None, p["q"], p["k"],
                                    p["v"], ctypes.byref(c) if c is not None else None,
                                    p["o"], p["lse"], ws, ws_bytes, None)
    return st, pka.lib.pka_last_error().decode()


def bwd(pka, d, c, ptrs=None, ws=A, ws_bytes=1 << 40, delta=None):
    p = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A)
    p.update(ptrs or {})
    st = pka.lib.pka_chunk_attn_bwd(ctypes.byref(d), p["q"], p["k"], p["v"], ctypes.byref(c),
                                    p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                                    delta, ws, ws_bytes, None)
    return st, pka.lib.pka_last_error().decode()


CASES_FWD = [
    ("null dims", lambda pka: (None, cache(pka), None), 1),
    ("hq % hkv", lambda pka: (dims(pka, n_heads_q=5), cache(pka), None), 2),
    ("batch 0", lambda pka: (dims(pka, batch=0), cache(pka), None), 2),
    ("head_dim 96", lambda pka: (dims(pka, head_dim=96), cache(pka, head_dim=96), None), 3),
    ("chunk 0", lambda pka: (dims(pka, chunk_len=0), cache(pka), None), 2),
    ("chunk too long", lambda pka: (dims(pka, chunk_len=65537), cache(pka), None), 2),
    ("negative prefix", lambda pka: (dims(pka, prefix_len=-1), cache(pka), None), 2),
    ("seq overflow", lambda pka: (dims(pka, prefix_len=2**31 - 10), cache(pka), None), 2),
    ("scale 0", lambda pka: (dims(pka, softmax_scale=0.0), cache(pka), None), 2),
    ("scale nan", lambda pka: (dims(pka, softmax_scale=float("nan")), cache(pka), None), 2),
    ("null q", lambda pka: (dims(pka), cache(pka), {"q": None}), 1),
    ("null lse", lambda pka: (dims(pka), cache(pka), {"lse": None}), 1),
    ("misaligned o", lambda pka: (dims(pka), cache(pka), {"o": MIS}), 5),
    ("null cache", lambda pka: (dims(pka), None, None), 1),
    ("cache type 9", lambda pka: (dims(pka), cache(pka, type=9), None), 3),
    ("cache head_dim", lambda pka: (dims(pka), cache(pka, head_dim=64), None), 2),
    ("capacity < P", lambda pka: (dims(pka), cache(pka, capacity=255), None), 4),
    ("null cache k", lambda pka: (dims(pka), cache(pka, k=None), None), 1),
    ("misaligned cache v", lambda pka: (dims(pka), cache(pka, v=MIS), None), 5),
    ("q8_0 no scales", lambda pka: (dims(pka), cache(pka, type=2), None), 1),
    ("q8_0 misaligned scale", lambda pka: (dims(pka), cache(pka, type=2, k_scale=A,
                                                             v_scale=MIS), None), 5),
]


@pytest.mark.parametrize("name,make,want", CASES_FWD, ids=[c[0] for c in CASES_FWD])
def test_fwd_validation(pka, name, make, want):
    d, c, ptrs = make(pka)
    st, msg = fwd(pka, d, c, ptrs)
    assert st == want, (name, st, msg)
    assert msg


def test_fwd_workspace_required_when_split(pka):
    d = dims(pka, batch=1, n_heads_q=2, n_heads_kv=1, prefix_len=16384, chunk_len=64)
    need = pka.fwd_workspace_bytes(d)
    assert need > 0
    st, msg = fwd(pka, d, cache(pka, capacity=20000))
    assert st == 6 and "workspace" in msg
    st, _ = fwd(pka, d, cache(pka, capacity=20000), ws=A, ws_bytes=need - 1)
    assert st == 6
    st, _ = fwd(pka, d, cache(pka, capacity=20000), ws=MIS, ws_bytes=need)
    assert st == 5


def test_bwd_validation(pka):
    d = dims(pka)
    need = pka.bwd_workspace_bytes(d)
    assert need >= 1 * 4 * 64 * 4
    assert bwd(pka, d, cache(pka), ws=None)[0] == 6
    assert bwd(pka, d, cache(pka), ws=A, ws_bytes=need - 1)[0] == 6
    assert bwd(pka, d, cache(pka), ptrs={"do": None})[0] == 1
    assert bwd(pka, d, cache(pka), ptrs={"dk": MIS})[0] == 5
    assert bwd(pka, d, cache(pka), delta=MIS)[0] == 5
    assert bwd(pka, d, cache(pka, capacity=100))[0] == 4
    assert bwd(pka, dims(pka, n_heads_kv=3), cache(pka))[0] == 2


def test_backward_rejects_query_rows_of_one_kv_head_over_4gib(pka):
    # 256 query heads per KV head x 65536 rows x 128 values x 2 bytes = 4 GiB: the
    # backward kernels address one KV head's Q / dO rows with 32-bit byte offsets.
    d = dims(pka, n_heads_q=256, n_heads_kv=1, chunk_len=65536)
    st, msg = bwd(pka, d, cache(pka))
    assert st == 2 and "4 GiB" in msg, (st, msg)
    st = pka.lib.pka_prefix_kv_grad(ctypes.byref(d), 64, A, ctypes.byref(cache(pka)), A, A, A,
                                    A, A, A, 1 << 40, None)
    assert st == 2 and "4 GiB" in pka.lib.pka_last_error().decode()


def test_append_validation(pka):
    lib = pka.lib
    d = dims(pka, prefix_len=500, chunk_len=64)
    c = cache(pka, capacity=563)                       # P + C = 564 > capacity
    assert lib.pka_kv_append_f16(ctypes.byref(d), A, A, ctypes.byref(c), None) == 4
    c = cache(pka, capacity=600, type=pka.CACHE_F16)
    assert lib.pka_kv_append_q8_0(ctypes.byref(d), A, A, ctypes.byref(c), None) == 3
    assert lib.pka_kv_append_bf16(ctypes.byref(d), A, A, ctypes.byref(c), None) == 3
    assert lib.pka_kv_append_f16(ctypes.byref(d), None, A, ctypes.byref(c), None) == 1
    assert lib.pka_kv_append_f16(ctypes.byref(d), A, MIS, ctypes.byref(c), None) == 5
    cq = cache(pka, capacity=600, type=pka.CACHE_Q8_0)
    assert lib.pka_kv_append_q8_0(ctypes.byref(d), A, A, ctypes.byref(cq), None) == 1
    assert lib.pka_kv_append_f16(None, A, A, ctypes.byref(c), None) == 1


def test_dequant_validation(pka):
    lib = pka.lib
    cq = cache(pka, capacity=100, type=pka.CACHE_Q8_0, k_scale=A, v_scale=A)
    assert lib.pka_kv_dequant_q8_0(ctypes.byref(cq), 1, 1, 50, 51, A, None, None) == 4
    assert lib.pka_kv_dequant_q8_0(ctypes.byref(cq), 1, 1, 0, 0, A, None, None) == 2
    assert lib.pka_kv_dequant_q8_0(ctypes.byref(cq), 1, 1, 0, 10, None, None, None) == 1
    assert lib.pka_kv_dequant_q8_0(ctypes.byref(cq), 1, 1, 0, 10, A, MIS, None) == 5
    cf = cache(pka, capacity=100, type=pka.CACHE_F16)
    assert lib.pka_kv_dequant_q8_0(ctypes.byref(cf), 1, 1, 0, 10, A, None, None) == 3


def test_status_strings_and_profile_ids(pka):
    for st in range(8):
        assert pka.lib.pka_status_string(st)
    ms, n, dr = ctypes.c_double(), ctypes.c_int64(), ctypes.c_int64()
    assert pka.lib.pka_profile_read(99, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(dr)) == 2
    assert pka.lib.pka_profile_read(0, None, None, None) == 1


def test_workspace_plan(pka):
    # The headline shape fills the chip without splitting the prefix.
    assert pka.fwd_workspace_bytes(dims(pka, batch=4, n_heads_q=32, n_heads_kv=8,
                                        prefix_len=16384, chunk_len=512)) == 0
    # Few (window, KV head) units: split, with partials sized by the split count.
    d3 = dims(pka, batch=2, n_heads_q=12, n_heads_kv=2, prefix_len=16384, chunk_len=512)
    nrow = 2 * 12 * 512
    ws = pka.fwd_workspace_bytes(d3)
    assert ws >= 2 * nrow * 129 * 4 and ws % 256 == 0
    assert pka.bwd_workspace_bytes(d3) >= nrow * 4 + 2 * nrow * 128 * 4
    # invalid dims -> 0
    assert pka.fwd_workspace_bytes(dims(pka, head_dim=80)) == 0


def test_struct_layout_matches_the_header(pka, tmp_path):
    """The ctypes mirrors of pka_dims and pka_cache have the C compiler's layout."""
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "pka.h"\n'
        "int main(void) {\n"
        '  printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(pka_dims),'
        " offsetof(pka_dims, prefix_len), offsetof(pka_dims, chunk_len),"
        " offsetof(pka_dims, softmax_scale), offsetof(pka_dims, prefix_lens),"
        " sizeof(pka_cache));\n  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", f"-I{os.path.dirname(HEADER)}", str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    D = pka.Dims
    want = [ctypes.sizeof(D), D.prefix_len.offset, D.chunk_len.offset, D.softmax_scale.offset,
            D.prefix_lens.offset, ctypes.sizeof(pka.CacheDesc)]
    assert got == want


def test_prefix_lens_alignment_is_checked(pka):
    """A misaligned per-window prefix array is refused before any launch."""
    d = dims(pka)
    d.prefix_lens = A + 2
    st, msg = fwd(pka, d, cache(pka))
    assert st == 5 and "prefix_lens" in msg
    c = cache(pka, capacity=600, type=pka.CACHE_F16)
    assert pka.lib.pka_kv_append_f16(ctypes.byref(d), A, A, ctypes.byref(c), None) == 5


def test_prefix_kv_grad_validation(pka):
    lib = pka.lib
    d = dims(pka)                                    # P = 256
    c = cache(pka)

    def call(horizon, ptrs=None, ws=None, ws_bytes=0, dd=d, cc=c):
        p = dict(q=A, lse=A, do=A, delta=A, dk=A, dv=A)
        p.update(ptrs or {})
        st = lib.pka_prefix_kv_grad(ctypes.byref(dd), horizon, p["q"], ctypes.byref(cc),
                                    p["lse"], p["do"], p["delta"], p["dk"], p["dv"], ws,
                                    ws_bytes, None)
        return st, lib.pka_last_error().decode()

    assert call(257)[0] == 2 and call(-1)[0] == 2          # horizon outside [0, P]
    assert call(64, {"delta": None})[0] == 1
    assert call(64, {"dk": MIS})[0] == 5
    assert call(64, cc=cache(pka, capacity=100))[0] == 4
    assert call(64, dd=dims(pka, n_heads_kv=3))[0] == 2
    # few units and many query rows -> row splits with an fp32 partial workspace
    dl = dims(pka, chunk_len=1024)
    need = pka.prefix_kv_grad_workspace_bytes(dl, 64)
    assert need >= 2 * 1 * 2 * 64 * 128 * 4 and need % 256 == 0
    st, msg = call(64, dd=dl)
    assert st == 6 and "workspace" in msg
    assert call(64, ws=MIS, ws_bytes=need, dd=dl)[0] == 5
    # horizon 0 is valid and writes nothing (no launch, so fake pointers are fine)
    assert call(0)[0] == 0
    assert pka.prefix_kv_grad_workspace_bytes(d, 300) == 0     # invalid -> 0


def test_fwd_append_validation(pka):
    """The fused forward + append needs the capacity of the append (P + C rows)."""
    lib = pka.lib
    d = dims(pka, prefix_len=500, chunk_len=64)

    def call(c):
        st = lib.pka_chunk_attn_fwd_append(ctypes.byref(d), A, A, A, ctypes.byref(c), A, A,
                                           A, 1 << 40, None)
        return st, lib.pka_last_error().decode()

    st, msg = call(cache(pka, capacity=563))       # enough for P, not for P + C
    assert st == 4 and "capacity" in msg
    assert call(cache(pka, capacity=600, type=pka.CACHE_Q8_0))[0] == 1   # no scales
    assert call(cache(pka, capacity=600, k=MIS))[0] == 5


def test_row_sparse_validation(pka):
    """Row-sparse backward: refused on the host before any launch."""
    lib = pka.lib

    def call(n=256, k=128, fin=256, fout=384, x=A, w=A, dy=A, keep=A, dw=A, dx=A, d=True,
             ws=A, ws_bytes=1 << 40):
        dd = pka.RsDims(n, k, fin, fout)
        st = lib.pka_row_sparse_linear_bwd(ctypes.byref(dd) if d else None, x, w, dy, keep,
                                           dw, dx, ws, ws_bytes, None)
        return st, lib.pka_last_error().decode()

    assert call(d=False)[0] == 1
    assert call(n=0, k=0)[0] == 2
    assert call(k=-1)[0] == 2
    assert call(k=257)[0] == 2                        # more kept rows than rows
    st, msg = call(fin=200)
    assert st == 3 and "multiples of 128" in msg
    assert call(fout=64)[0] == 3
    assert call(dy=None)[0] == 1
    assert call(x=None)[0] == 1                       # dw needs x
    assert call(w=None, dx=A, dw=None)[0] == 1        # dx needs w
    assert call(keep=None)[0] == 1
    assert call(keep=A + 2)[0] == 5
    assert call(dx=MIS)[0] == 5
    assert call(dw=MIS)[0] == 5
    assert call(dw=None, dx=None)[0] == 0             # nothing asked: nothing launched
    # few kept rows: the dX product is split over the output features into a workspace
    need = pka.row_sparse_workspace_bytes(512, 128, 256, 2048)
    assert need >= 2 * 128 * 256 * 4 and need % 256 == 0
    st, msg = call(n=512, k=128, fin=256, fout=2048, ws=None)
    assert st == 6 and "workspace" in msg
    assert call(n=512, k=128, fin=256, fout=2048, ws=A, ws_bytes=need - 1)[0] == 6
    assert call(n=512, k=128, fin=256, fout=2048, ws=MIS, ws_bytes=need)[0] == 5
    # many tiles: no split, no workspace; invalid dims: 0
    assert pka.row_sparse_workspace_bytes(4096, 4096, 4096, 4096) == 0
    assert pka.row_sparse_workspace_bytes(512, 128, 200, 2048) == 0


def test_rs_dims_layout_matches_the_header(pka, tmp_path):
    src = tmp_path / "rs_layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "pka.h"\n'
        "int main(void) {\n"
        '  printf("%zu %zu %zu %zu\\n", sizeof(pka_rs_dims), offsetof(pka_rs_dims, n_keep),'
        " offsetof(pka_rs_dims, in_features), offsetof(pka_rs_dims, out_features));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "rs_layout"
    subprocess.run(["gcc", "-std=c99", f"-I{os.path.dirname(HEADER)}", str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    R = pka.RsDims
    assert got == [ctypes.sizeof(R), R.n_keep.offset, R.in_features.offset,
                   R.out_features.offset]


def _dkv_splits(batch, hq, hkv, C, cus=256, kb=128):
    """The chunk dK/dV split rule, restated: one workgroup per (window, KV head, block
    of 128 keys); while the CU budget allows, another split goes to the block whose
    workgroups have the most 64-row steps (first on ties), each block keeping >= 2
    steps per split and at most 16 splits. Returns the largest split count."""
    G, groups, nkb = hq // hkv, batch * hkv, -(-C // kb)
    if groups * nkb >= cus:
        return 1
    steps = [-(-(G * (C - k * kb)) // 64) for k in range(nkb)]
    cnt = [1] * nkb
    for _ in range(cus // groups - nkb):
        best, load = -1, 0
        for k in range(nkb):
            if cnt[k] >= min(steps[k] // 2, 16):
                continue
            lk = -(-steps[k] // cnt[k])
            if lk > load:
                best, load = k, lk
        if best < 0:
            break
        cnt[best] += 1
    return max(cnt)


def _dkv_beside(batch, hq, hkv, P, C, cus=256):
    """The rule for running the chunk dK/dV units beside the dQ row blocks, restated.
    dQ grid: one workgroup per 256 packed rows of a (window, KV head); when those are
    fewer than the CUs, the key tiles are split (each split keeps >= 8 tiles, at most 16
    splits). Beside: every unit (one per 128-key block) has an idle CU, and a unit's
    64-row steps (all rows of the group) are no more than one dQ workgroup's key tiles."""
    G = hq // hkv
    units = batch * hkv * -(-(G * C) // 256)
    split = 1
    if units < cus:
        split = min(cus // units, max(1, -(-(P + 1) // 64) // 8), 16)
    nblk = units * split
    dq_tiles = -(-(-(-(P + C) // 64)) // split)
    kv_units = batch * hkv * -(-C // 128)
    return nblk < cus and kv_units <= cus - nblk and -(-(G * C) // 64) <= dq_tiles


@pytest.mark.parametrize("shape", [(4, 32, 8, 16384, 512), (2, 12, 2, 16384, 512),
                                   (1, 40, 8, 63488, 512), (1, 4, 1, 1000, 130),
                                   (8, 32, 8, 4096, 512)])
def test_bwd_workspace_follows_the_dkv_split_rule(pka, shape):
    B, hq, hkv, P, C = shape
    d = dims(pka, batch=B, n_heads_q=hq, n_heads_kv=hkv, prefix_len=P, chunk_len=C)
    a256 = lambda n: (n + 255) // 256 * 256
    nrow = B * hq * C
    # dK/dV units beside the dQ blocks are not split
    beside = _dkv_beside(B, hq, hkv, P, C)
    split = 1 if beside else _dkv_splits(B, hq, hkv, C)
    if shape == (2, 12, 2, 16384, 512):
        assert beside                            # 16 units, 16 idle CUs, 48 <= 53 tiles
    if shape == (1, 40, 8, 63488, 512):
        assert not beside                        # 32 units for 16 idle CUs
    want = a256(nrow * 4)
    if split > 1:
        want += a256(split * 2 * B * hkv * C * 128 * 4)
    ws = pka.bwd_workspace_bytes(d)
    if pka.fwd_workspace_bytes(d) == 0:          # no prefix split: delta + dK/dV partials
        assert ws == want, (ws, want, split)
    else:                                        # plus the dQ partials of the split
        assert ws > want and (ws - want) % (nrow * 128 * 4) == 0
    if shape == (4, 32, 8, 16384, 512):
        assert split == 3                        # blocks of 32, 24, 16, 8 steps: 3, 2, 2, 1
