"""Python binding of libpka (prefix-KV chunk attention on MI355X).

Argument marshalling only: every computation runs in the HIP kernels of
``libpka.so`` (built by ``python prefix_kv_attention_amd/build.py``). PyTorch
provides device memory and the current HIP stream. Importing this package raises
if the library is missing; there is no fallback implementation.

Names follow the C entry points of include/pka.h without the ``pka_`` prefix:
``chunk_attn_fwd``, ``chunk_attn_fwd_append``, ``chunk_attn_bwd``,
``chunk_attn_bwd_noalloc``, ``kv_append_q8_0``,
``kv_append_f16``, ``kv_append_bf16``, ``kv_dequant_q8_0``, ``prefix_kv_grad``,
``fwd_workspace_bytes``, ``bwd_workspace_bytes``, ``prefix_kv_grad_workspace_bytes``,
``row_sparse_linear_bwd``, ``row_sparse_workspace_bytes``, ``profile_*``. ``chunk_attention`` wraps forward and backward in an
autograd function whose cache inputs get no gradient (the cache is a fixed input:
"train: walk the window", Why it's a draft). ``WindowWalk`` drives the
chunk loop of a batch of windows: step, append, advance every window's prefix.

Every call takes ``prefix_len`` (an int: the prefix of every window, or the
largest one) and optionally ``prefix_lens``, a CUDA int32 tensor [B] of the
windows' own prefix lengths (ragged windows; entries clamped to [0, prefix_len]).

The C entry points take bare device pointers and cannot see tensor sizes, so every
tensor is checked here (shape, dtype, device, contiguity) before the call: a wrong
one raises ValueError and nothing is launched.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpka.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python prefix_kv_attention_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

CACHE_F16, CACHE_BF16, CACHE_Q8_0 = 0, 1, 2
CACHE_TYPE_BY_NAME = {"f16": CACHE_F16, "bf16": CACHE_BF16, "q8_0": CACHE_Q8_0}
STATUS = {0: "PKA_OK", 1: "PKA_ERR_NULL", 2: "PKA_ERR_DIMS", 3: "PKA_ERR_UNSUPPORTED",
          4: "PKA_ERR_CAPACITY", 5: "PKA_ERR_ALIGN", 6: "PKA_ERR_WORKSPACE", 7: "PKA_ERR_HIP"}
KERNELS = {"fwd": 0, "fwd_combine": 1, "bwd_prep": 2, "bwd_dq": 3, "bwd_dkdv": 4,
           "bwd_dq_reduce": 5, "append": 6, "dequant": 7, "bwd_dkdv_reduce": 8,
           "prefix_kv": 9, "prefix_kv_reduce": 10, "rs_zero": 11, "rs_dx": 12, "rs_dw": 13,
           "rs_dx_reduce": 14}


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_heads_q", ctypes.c_int32),
                ("n_heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("prefix_len", ctypes.c_int64), ("chunk_len", ctypes.c_int64),
                ("softmax_scale", ctypes.c_float), ("prefix_lens", ctypes.c_void_p)]


class RsDims(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int64), ("n_keep", ctypes.c_int64),
                ("in_features", ctypes.c_int32), ("out_features", ctypes.c_int32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


_P = ctypes.POINTER
_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
_SIGS = {
    "pka_fwd_workspace_bytes": (_sz, [_P(Dims)]),
    "pka_bwd_workspace_bytes": (_sz, [_P(Dims)]),
    "pka_chunk_attn_fwd": (ctypes.c_int, [_P(Dims), _vp, _vp, _vp, _P(CacheDesc), _vp, _vp,
                                          _vp, _sz, _vp]),
    "pka_chunk_attn_fwd_append": (ctypes.c_int, [_P(Dims), _vp, _vp, _vp, _P(CacheDesc), _vp,
                                                 _vp, _vp, _sz, _vp]),
    "pka_chunk_attn_bwd": (ctypes.c_int, [_P(Dims), _vp, _vp, _vp, _P(CacheDesc), _vp, _vp,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "pka_chunk_attn_bwd_noalloc": (ctypes.c_int, [_P(Dims), _vp, _vp, _vp, _P(CacheDesc), _vp,
                                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pka_prefix_kv_grad_workspace_bytes": (_sz, [_P(Dims), _i64]),
    "pka_prefix_kv_grad": (ctypes.c_int, [_P(Dims), _i64, _vp, _P(CacheDesc), _vp, _vp, _vp,
                                          _vp, _vp, _vp, _sz, _vp]),
    "pka_kv_append_q8_0": (ctypes.c_int, [_P(Dims), _vp, _vp, _P(CacheDesc), _vp]),
    "pka_kv_append_f16": (ctypes.c_int, [_P(Dims), _vp, _vp, _P(CacheDesc), _vp]),
    "pka_kv_append_bf16": (ctypes.c_int, [_P(Dims), _vp, _vp, _P(CacheDesc), _vp]),
    "pka_kv_dequant_q8_0": (ctypes.c_int, [_P(CacheDesc), _i32, _i32, _i64, _i64, _vp, _vp,
                                           _vp]),
    "pka_row_sparse_linear_bwd_workspace_bytes": (_sz, [_P(RsDims)]),
    "pka_row_sparse_linear_bwd": (ctypes.c_int, [_P(RsDims), _vp, _vp, _vp, _vp, _vp, _vp,
                                                 _vp, _sz, _vp]),
    "pka_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pka_last_error": (ctypes.c_char_p, []),
    "pka_profile_enable": (ctypes.c_int, [_i32]),
    "pka_profile_select": (ctypes.c_int, [ctypes.c_uint32]),
    "pka_profile_reset": (ctypes.c_int, []),
    "pka_profile_read": (ctypes.c_int, [_i32, _P(ctypes.c_double), _P(_i64), _P(_i64)]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args
lib = _lib


class PkaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.pka_last_error().decode() or _lib.pka_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def _check(status: int, where: str):
    if status != 0:
        raise PkaError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_dims(batch, n_heads_q, n_heads_kv, head_dim, prefix_len, chunk_len,
              softmax_scale, prefix_lens=None) -> Dims:
    if prefix_lens is not None:
        if (prefix_lens.dtype != torch.int32 or not prefix_lens.is_cuda
                or not prefix_lens.is_contiguous() or prefix_lens.numel() != int(batch)):
            raise ValueError("prefix_lens must be a contiguous CUDA int32 tensor of "
                             f"{int(batch)} entries")
    return Dims(int(batch), int(n_heads_q), int(n_heads_kv), int(head_dim),
                int(prefix_len), int(chunk_len), float(softmax_scale),
                None if prefix_lens is None else prefix_lens.data_ptr())


class PrefixCache:
    """Device tensors of a prefix cache [B][Hkv][capacity][D] in one storage type."""

    def __init__(self, cache_type: str, k, v, k_scale=None, v_scale=None):
        if cache_type not in CACHE_TYPE_BY_NAME:
            raise ValueError(f"unknown cache type {cache_type!r}")
        if not isinstance(k, torch.Tensor) or k.dim() != 4:
            raise ValueError("cache k must be a 4-D tensor [B][Hkv][capacity][D]")
        dt = {"q8_0": torch.int8, "f16": torch.float16, "bf16": torch.bfloat16}[cache_type]
        _tensor(k, "cache k", k.shape, dt, k.device)
        _tensor(v, "cache v", k.shape, dt, k.device)
        if cache_type == "q8_0":
            sshape = tuple(k.shape[:3]) + (k.shape[3] // 32,)
            _tensor(k_scale, "cache k_scale", sshape, torch.float16, k.device)
            _tensor(v_scale, "cache v_scale", sshape, torch.float16, k.device)
        elif k_scale is not None or v_scale is not None:
            raise ValueError(f"a {cache_type} cache has no scales")
        self.cache_type = cache_type
        self.k, self.v, self.k_scale, self.v_scale = k, v, k_scale, v_scale
        self.batch, self.n_heads_kv, self.capacity, self.head_dim = k.shape

    def check_for(self, batch, n_heads_kv, head_dim, device):
        """Raise unless this cache serves windows of these dimensions on `device`."""
        if (self.batch, self.n_heads_kv, self.head_dim) != (batch, n_heads_kv, head_dim):
            raise ValueError(f"cache is [B={self.batch}][Hkv={self.n_heads_kv}][.]"
                             f"[D={self.head_dim}], the call needs [B={batch}]"
                             f"[Hkv={n_heads_kv}][.][D={head_dim}]")
        if self.k.device != device:
            raise ValueError(f"cache is on {self.k.device}, the call on {device}")

    @classmethod
    def empty(cls, cache_type, batch, n_heads_kv, capacity, head_dim, device="cuda"):
        shape = (batch, n_heads_kv, capacity, head_dim)
        if cache_type == "q8_0":
            sshape = (batch, n_heads_kv, capacity, head_dim // 32)
            return cls(cache_type,
                       torch.empty(shape, dtype=torch.int8, device=device),
                       torch.empty(shape, dtype=torch.int8, device=device),
                       torch.empty(sshape, dtype=torch.float16, device=device),
                       torch.empty(sshape, dtype=torch.float16, device=device))
        dt = torch.float16 if cache_type == "f16" else torch.bfloat16
        return cls(cache_type, torch.empty(shape, dtype=dt, device=device),
                   torch.empty(shape, dtype=dt, device=device))

    def desc(self) -> CacheDesc:
        return CacheDesc(CACHE_TYPE_BY_NAME[self.cache_type], int(self.head_dim),
                         int(self.capacity), self.k.data_ptr(), self.v.data_ptr(),
                         self.k_scale.data_ptr() if self.k_scale is not None else None,
                         self.v_scale.data_ptr() if self.v_scale is not None else None)


def _tensor(t, name, shape, dtype, device):
    """Raise unless t is a contiguous `dtype` CUDA tensor of `shape` on `device`."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ws_bytes(ws, device):
    """Size in bytes of a caller's workspace tensor (None: 0)."""
    if ws is None:
        return 0
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != device \
            or not ws.is_contiguous():
        raise ValueError(f"ws must be a contiguous tensor on {device}")
    return ws.numel() * ws.element_size()


def _chunk_inputs(q, k, v, cache, prefix_len, scale, prefix_lens):
    """Check q [B][Hq][C][D], k and v [B][Hkv][C][D] (bf16) against each other and the
    cache; return the dims of the call."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4 or not isinstance(k, torch.Tensor) \
            or k.dim() != 4:
        raise ValueError("q and k must be 4-D tensors")
    B, Hq, C, D = q.shape
    Hkv = k.shape[1]
    _tensor(q, "q", (B, Hq, C, D), torch.bfloat16, q.device)
    _tensor(k, "k", (B, Hkv, C, D), torch.bfloat16, q.device)
    _tensor(v, "v", (B, Hkv, C, D), torch.bfloat16, q.device)
    cache.check_for(B, Hkv, D, q.device)
    return make_dims(B, Hq, Hkv, D, prefix_len, C, scale, prefix_lens)


def fwd_workspace_bytes(dims: Dims) -> int:
    return int(_lib.pka_fwd_workspace_bytes(ctypes.byref(dims)))


def bwd_workspace_bytes(dims: Dims) -> int:
    return int(_lib.pka_bwd_workspace_bytes(ctypes.byref(dims)))


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def chunk_attn_fwd(q, k, v, cache: PrefixCache, prefix_len: int, scale: float,
                   o=None, lse=None, ws=None, prefix_lens=None):
    """O [B][Hq][C][D] bf16 and LSE [B][Hq][C] f32 of the chunk against the prefix."""
    dims = _chunk_inputs(q, k, v, cache, prefix_len, scale, prefix_lens)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _tensor(o, "o", q.shape, torch.bfloat16, q.device)
    _tensor(lse, "lse", q.shape[:3], torch.float32, q.device)
    if ws is None:
        ws = _workspace(fwd_workspace_bytes(dims), q.device)
    nws = _ws_bytes(ws, q.device)
    cd = cache.desc()
    _check(_lib.pka_chunk_attn_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                   ctypes.byref(cd), _ptr(o), _ptr(lse), _ptr(ws), nws,
                                   _stream(q.device)),
           "pka_chunk_attn_fwd")
    return o, lse


def chunk_attn_fwd_append(q, k, v, cache: PrefixCache, prefix_len: int, scale: float,
                          o=None, lse=None, ws=None, prefix_lens=None):
    """chunk_attn_fwd and the append of k, v to cache rows [P_b, P_b + C) in one launch."""
    dims = _chunk_inputs(q, k, v, cache, prefix_len, scale, prefix_lens)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _tensor(o, "o", q.shape, torch.bfloat16, q.device)
    _tensor(lse, "lse", q.shape[:3], torch.float32, q.device)
    if ws is None:
        ws = _workspace(fwd_workspace_bytes(dims), q.device)
    nws = _ws_bytes(ws, q.device)
    cd = cache.desc()
    _check(_lib.pka_chunk_attn_fwd_append(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                          ctypes.byref(cd), _ptr(o), _ptr(lse), _ptr(ws),
                                          nws, _stream(q.device)),
           "pka_chunk_attn_fwd_append")
    return o, lse


def chunk_attn_bwd(q, k, v, cache: PrefixCache, prefix_len: int, scale: float, o, lse,
                   d_o, dq=None, dk=None, dv=None, delta=None, ws=None, prefix_lens=None):
    """dQ (chunk rows), dK and dV (the chunk's own keys); the prefix gets nothing."""
    dims = _chunk_inputs(q, k, v, cache, prefix_len, scale, prefix_lens)
    _tensor(o, "o", q.shape, torch.bfloat16, q.device)
    _tensor(d_o, "d_o", q.shape, torch.bfloat16, q.device)
    _tensor(lse, "lse", q.shape[:3], torch.float32, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _tensor(dq, "dq", q.shape, torch.bfloat16, q.device)
    _tensor(dk, "dk", k.shape, torch.bfloat16, q.device)
    _tensor(dv, "dv", k.shape, torch.bfloat16, q.device)
    if delta is not None:
        _tensor(delta, "delta", q.shape[:3], torch.float32, q.device)
    if ws is None:
        ws = _workspace(bwd_workspace_bytes(dims), q.device)
    nws = _ws_bytes(ws, q.device)
    cd = cache.desc()
    _check(_lib.pka_chunk_attn_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                   ctypes.byref(cd), _ptr(o), _ptr(lse), _ptr(d_o),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta), _ptr(ws),
                                   nws, _stream(q.device)),
           "pka_chunk_attn_bwd")
    return dq, dk, dv


# Size of the library's own backward workspace (pka.h: PKA_BWD_NOALLOC_MAX_WORKSPACE).
BWD_NOALLOC_MAX_WORKSPACE = 96 << 20


def chunk_attn_bwd_noalloc(q, k, v, cache: PrefixCache, prefix_len: int, scale: float, o,
                           lse, d_o, dq, dk, dv, delta=None, prefix_lens=None):
    """chunk_attn_bwd through pka_chunk_attn_bwd_noalloc: the caller passes every output
    and the library uses its own fixed per-GPU workspace, so the call allocates nothing
    (usable under graph capture). Calls on one GPU must not overlap in time."""
    dims = _chunk_inputs(q, k, v, cache, prefix_len, scale, prefix_lens)
    _tensor(o, "o", q.shape, torch.bfloat16, q.device)
    _tensor(d_o, "d_o", q.shape, torch.bfloat16, q.device)
    _tensor(lse, "lse", q.shape[:3], torch.float32, q.device)
    _tensor(dq, "dq", q.shape, torch.bfloat16, q.device)
    _tensor(dk, "dk", k.shape, torch.bfloat16, q.device)
    _tensor(dv, "dv", k.shape, torch.bfloat16, q.device)
    if delta is not None:
        _tensor(delta, "delta", q.shape[:3], torch.float32, q.device)
    cd = cache.desc()
    _check(_lib.pka_chunk_attn_bwd_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                           ctypes.byref(cd), _ptr(o), _ptr(lse), _ptr(d_o),
                                           _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta),
                                           _stream(q.device)),
           "pka_chunk_attn_bwd_noalloc")
    return dq, dk, dv


def prefix_kv_grad_workspace_bytes(dims: Dims, horizon: int) -> int:
    return int(_lib.pka_prefix_kv_grad_workspace_bytes(ctypes.byref(dims), int(horizon)))


def prefix_kv_grad(q, cache: PrefixCache, prefix_len: int, scale: float, lse, d_o, delta,
                   horizon: int, dk=None, dv=None, ws=None, prefix_lens=None):
    """dK, dV (f32 [B][Hkv][H][D]) of the last `horizon` cache rows of every window from
    the chunk queries; row h is cache row P_b - H + h (zero where P_b < H). lse is the
    forward's, delta the backward's (chunk_attn_bwd(..., delta=...))."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor")
    B, Hq, C, D = q.shape
    Hkv = cache.n_heads_kv
    _tensor(q, "q", q.shape, torch.bfloat16, q.device)
    _tensor(d_o, "d_o", q.shape, torch.bfloat16, q.device)
    _tensor(lse, "lse", q.shape[:3], torch.float32, q.device)
    _tensor(delta, "delta", q.shape[:3], torch.float32, q.device)
    cache.check_for(B, Hkv, D, q.device)
    if int(horizon) < 0:
        raise ValueError("horizon must be >= 0")
    dims = make_dims(B, Hq, Hkv, D, prefix_len, C, scale, prefix_lens)
    shape = (B, Hkv, int(horizon), D)
    dk = torch.empty(shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(shape, dtype=torch.float32, device=q.device) if dv is None else dv
    _tensor(dk, "dk", shape, torch.float32, q.device)
    _tensor(dv, "dv", shape, torch.float32, q.device)
    if ws is None:
        ws = _workspace(prefix_kv_grad_workspace_bytes(dims, horizon), q.device)
    nws = _ws_bytes(ws, q.device)
    cd = cache.desc()
    _check(_lib.pka_prefix_kv_grad(ctypes.byref(dims), int(horizon), _ptr(q), ctypes.byref(cd),
                                   _ptr(lse), _ptr(d_o), _ptr(delta), _ptr(dk), _ptr(dv),
                                   _ptr(ws), nws, _stream(q.device)),
           "pka_prefix_kv_grad")
    return dk, dv


def _append(fn, name, k, v, cache: PrefixCache, prefix_len: int, prefix_lens=None):
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise ValueError("k must be a 4-D tensor")
    B, Hkv, C, D = k.shape
    _tensor(k, "k", k.shape, torch.bfloat16, k.device)
    _tensor(v, "v", k.shape, torch.bfloat16, k.device)
    cache.check_for(B, Hkv, D, k.device)
    dims = make_dims(B, Hkv, Hkv, D, prefix_len, C, 1.0, prefix_lens)
    cd = cache.desc()
    _check(fn(ctypes.byref(dims), _ptr(k), _ptr(v), ctypes.byref(cd), _stream(k.device)), name)


def kv_append_q8_0(k, v, cache: PrefixCache, prefix_len: int, prefix_lens=None):
    """Quantise the chunk's K/V (bf16 [B][Hkv][C][D]) into cache rows [P, P+C)."""
    _append(_lib.pka_kv_append_q8_0, "pka_kv_append_q8_0", k, v, cache, prefix_len,
            prefix_lens)


def kv_append_f16(k, v, cache: PrefixCache, prefix_len: int, prefix_lens=None):
    _append(_lib.pka_kv_append_f16, "pka_kv_append_f16", k, v, cache, prefix_len, prefix_lens)


def kv_append_bf16(k, v, cache: PrefixCache, prefix_len: int, prefix_lens=None):
    _append(_lib.pka_kv_append_bf16, "pka_kv_append_bf16", k, v, cache, prefix_len,
            prefix_lens)


def kv_append(k, v, cache: PrefixCache, prefix_len: int, prefix_lens=None):
    """Append in the cache's own storage type."""
    {"q8_0": kv_append_q8_0, "f16": kv_append_f16, "bf16": kv_append_bf16}[
        cache.cache_type](k, v, cache, prefix_len, prefix_lens)


def kv_dequant_q8_0(cache: PrefixCache, row0: int, rows: int, want_bf16: bool = True):
    """(f32, bf16 or None) [2][B][Hkv][rows][D]: cache rows as the attention reads them."""
    if int(row0) < 0 or int(rows) < 0:
        raise ValueError("row0 and rows must be >= 0")
    shape = (2, cache.batch, cache.n_heads_kv, int(rows), cache.head_dim)
    out = torch.empty(shape, dtype=torch.float32, device=cache.k.device)
    outb = torch.empty(shape, dtype=torch.bfloat16, device=cache.k.device) if want_bf16 else None
    cd = cache.desc()
    _check(_lib.pka_kv_dequant_q8_0(ctypes.byref(cd), cache.batch, cache.n_heads_kv, row0, rows,
                                    _ptr(out), _ptr(outb), _stream(cache.k.device)),
           "pka_kv_dequant_q8_0")
    return out, outb


def row_sparse_workspace_bytes(n_rows: int, n_keep: int, in_features: int,
                               out_features: int) -> int:
    return int(_lib.pka_row_sparse_linear_bwd_workspace_bytes(
        ctypes.byref(RsDims(n_rows, n_keep, in_features, out_features))))


def row_sparse_linear_bwd(x, w, dy, keep, dw=None, dx=None, ws=None, want_dw=True,
                          want_dx=True):
    """Backward of y = x @ w.T on the kept rows only ("stop-gradient through context
    tokens", Mechanism): dw = dy[keep]^T x[keep] (f32 [out][in]) and dx (bf16 [N][in],
    dy[keep] @ w on the kept rows, zero elsewhere). x [N][in], w [out][in], dy [N][out]
    bf16 on one GPU; keep: int32 tensor [K] of distinct row indices on that GPU; ws: a
    uint8 workspace of row_sparse_workspace_bytes(...) bytes (allocated if None).
    Returns (dw, dx); a product not wanted is skipped and returned as None."""
    if x.dim() != 2 or w.dim() != 2 or dy.dim() != 2:
        raise ValueError("x, w, dy must be 2-D")
    n, fin = x.shape
    fout = w.shape[0]
    _tensor(x, "x", (n, fin), torch.bfloat16, x.device)
    _tensor(w, "w", (fout, fin), torch.bfloat16, x.device)
    _tensor(dy, "dy", (n, fout), torch.bfloat16, x.device)
    if keep.dim() != 1:
        raise ValueError("keep must be 1-D")
    _tensor(keep, "keep", (keep.shape[0],), torch.int32, x.device)
    if want_dw:
        dw = torch.empty((fout, fin), dtype=torch.float32, device=x.device) if dw is None else dw
        _tensor(dw, "dw", (fout, fin), torch.float32, x.device)
    else:
        dw = None
    if want_dx:
        dx = torch.empty_like(x) if dx is None else dx
        _tensor(dx, "dx", (n, fin), torch.bfloat16, x.device)
    else:
        dx = None
    dims = RsDims(n, keep.shape[0], fin, fout)
    if ws is None and dx is not None:
        ws = _workspace(int(_lib.pka_row_sparse_linear_bwd_workspace_bytes(ctypes.byref(dims))),
                        x.device)
    nws = _ws_bytes(ws, x.device)
    _check(_lib.pka_row_sparse_linear_bwd(ctypes.byref(dims), _ptr(x), _ptr(w), _ptr(dy),
                                          _ptr(keep), _ptr(dw), _ptr(dx), _ptr(ws), nws,
                                          _stream(x.device)),
           "pka_row_sparse_linear_bwd")
    return dw, dx


class _ChunkAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cache, prefix_len, scale, prefix_lens):
        o, lse = chunk_attn_fwd(q, k, v, cache, prefix_len, scale, prefix_lens=prefix_lens)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cache, ctx.prefix_len, ctx.scale = cache, prefix_len, scale
        ctx.prefix_lens = prefix_lens
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = chunk_attn_bwd(q, k, v, ctx.cache, ctx.prefix_len, ctx.scale, o, lse,
                                    d_o.contiguous(), prefix_lens=ctx.prefix_lens)
        return dq, dk, dv, None, None, None, None


def chunk_attention(q, k, v, cache: PrefixCache, prefix_len: int, scale: float,
                    prefix_lens=None):
    """Autograd op: O of the chunk; gradients reach q, k, v only (never the cache)."""
    return _ChunkAttention.apply(q, k, v, cache, prefix_len, scale, prefix_lens)


class WindowWalk:
    """The chunk loop over a batch of windows ("train: walk the window", What it is and
    Contents): each step trains one chunk of every window against that window's cached
    prefix, then re-decodes the chunk into the cache and advances the prefix by C.

    Windows may start at different prefix lengths (ragged). The device tensor of the
    per-window lengths and the host-side maximum are kept in step; the caller owns the
    cache, whose capacity bounds the walk.
    """

    def __init__(self, cache: PrefixCache, prefix_lens, scale: float):
        self.cache = cache
        self.scale = float(scale)
        self.lens = [int(p) for p in prefix_lens]
        if len(self.lens) != cache.batch or min(self.lens) < 0:
            raise ValueError("one non-negative prefix length per window of the cache")
        self._dev = torch.tensor(self.lens, dtype=torch.int32, device=cache.k.device)

    @property
    def prefix_len(self) -> int:
        return max(self.lens)

    def _plens(self):
        return None if len(set(self.lens)) == 1 else self._dev

    def forward(self, q, k, v):
        return chunk_attn_fwd(q, k, v, self.cache, self.prefix_len, self.scale,
                              prefix_lens=self._plens())

    def backward(self, q, k, v, o, lse, d_o, delta=None):
        return chunk_attn_bwd(q, k, v, self.cache, self.prefix_len, self.scale, o, lse, d_o,
                              delta=delta, prefix_lens=self._plens())

    def advance(self, k, v):
        """Append the chunk's K/V at every window's prefix end, then P_b += C."""
        C = k.shape[2]
        if self.prefix_len + C > self.cache.capacity:
            raise ValueError(f"cache capacity {self.cache.capacity} < "
                             f"{self.prefix_len + C} rows")
        kv_append(k, v, self.cache, self.prefix_len, prefix_lens=self._plens())
        self.lens = [p + C for p in self.lens]
        self._dev += C

    def decode(self, q, k, v):
        """No-grad forward of one chunk fused with its append (the pass that builds the
        cache): (o, lse); then P_b += C."""
        C = k.shape[2]
        if self.prefix_len + C > self.cache.capacity:
            raise ValueError(f"cache capacity {self.cache.capacity} < "
                             f"{self.prefix_len + C} rows")
        o, lse = chunk_attn_fwd_append(q, k, v, self.cache, self.prefix_len, self.scale,
                                       prefix_lens=self._plens())
        self.lens = [p + C for p in self.lens]
        self._dev += C
        return o, lse

    def step(self, q, k, v, d_o):
        """Forward, backward and append of one chunk: (o, lse, dq, dk, dv)."""
        o, lse = self.forward(q, k, v)
        dq, dk, dv = self.backward(q, k, v, o, lse, d_o)
        self.advance(k, v)
        return o, lse, dq, dk, dv


def profile_enable(on: bool = True):
    _check(_lib.pka_profile_enable(1 if on else 0), "pka_profile_enable")


def profile_select(kernels=None):
    """Bracket only the named kernels (None: all) while profiling is enabled."""
    mask = 0xFFFFFFFF if kernels is None else sum(1 << KERNELS[k] for k in kernels)
    _check(_lib.pka_profile_select(mask), "pka_profile_select")


def profile_reset():
    _check(_lib.pka_profile_reset(), "pka_profile_reset")


def profile_read(kernel: str):
    """(total_ms, launches, dropped) of one kernel since the last reset."""
    ms, n, dr = ctypes.c_double(), ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.pka_profile_read(KERNELS[kernel], ctypes.byref(ms), ctypes.byref(n),
                                 ctypes.byref(dr)), "pka_profile_read")
    return ms.value, n.value, dr.value
