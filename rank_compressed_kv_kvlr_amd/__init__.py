"""Python binding of libkvlr: decode attention over a rank-compressed KV cache
on AMD MI355X (gfx950).

Argument marshalling only. Every step of the computation runs in the HIP
kernels of ``libkvlr.so`` (see ``include/kvlr.h`` for the ABI); torch is
used for device memory and the current stream. Importing this module fails
if the library has not been built (``python -m rank_compressed_kv_kvlr_amd.build``);
there is no fallback.

Entry points mirror the C ABI:

* ``prefill_compress(desc, K, V, start, P_K, P_V, lat_k, lat_v)`` stores
  K P_K, V P_V for tokens start .. start + n - 1 (StiefAttention technical
  summary, "Mecanismo Central" item 5);
* ``append(desc, k_new, v_new, pos, P_K, P_V, lat_k, lat_v)`` stores one
  token per batch row at row pos[b];
* ``decode_attn(desc, q, P_K, P_V, lat_k, lat_v, seq_lens, scale, out, workspace)``
  computes softmax((K_lat P_K^T) q * scale) (V_lat P_V^T) in latent order;
* ``decode_attn_latent(desc, q_lat, lat_k, lat_v, seq_lens, scale, o_lat)``
  is the folded form: q_lat = q P_K in, o_lat out (P_V^T left to the caller).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "KvlrError", "Desc", "F32", "BF16", "Q43", "VALUES_PER_HEAD", "VALUES_JOINT", "lib", "version", "status_string",
    "cache_elems", "decode_workspace_bytes", "decode_plan", "decode_counter_bytes",
    "prefill_compress", "append", "decode_attn", "decode_attn_noalloc", "append_decode_attn", "decode_partials", "decode_combine", "decode_attn_latent",
    "hadamard_bases", "q43_outlier", "q43_row_bytes",
    "alloc_cache", "alloc_workspace", "pack_bases", "block_view", "latent_rows", "cap_rows", "k_tiled_index",
    "v_joint_index",
]

F32, BF16, Q43 = 0, 1, 2
# status codes (kvlr_status)
OK, ERR_NULL, ERR_SHAPE, ERR_RANK, ERR_DTYPE, ERR_WORKSPACE, ERR_HIP, ERR_ARG, ERR_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8
VALUES_PER_HEAD, VALUES_JOINT = 0, 1
SPLIT_BALANCED = -1   # split_tokens asking kvlr_decode_attn for the balanced plan
STATIC_SCRATCH_BYTES = 16 << 20   # the library's static decode scratch (kvlr_decode_attn_noalloc)
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvlr.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m rank_compressed_kv_kvlr_amd.build`")

# torch ships its own HIP runtime (soname libamdhip64.so.7). Loading it before
# libkvlr.so lets the library bind to that same runtime; loading libkvlr.so
# first would map the system runtime as well, and two HIP runtimes in one
# process do not share devices, streams or allocations.
import torch  # noqa: E402,F401


class _CDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("r_k", ctypes.POINTER(ctypes.c_int32)), ("r_v", ctypes.POINTER(ctypes.c_int32)),
                ("in_dtype", ctypes.c_int32), ("latent_dtype", ctypes.c_int32), ("value_mode", ctypes.c_int32)]


lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_D = ctypes.POINTER(_CDesc)
_SZ = ctypes.POINTER(ctypes.c_size_t)
_I32P = ctypes.POINTER(ctypes.c_int32)
lib.kvlr_version.restype = ctypes.c_int
lib.kvlr_status_string.restype = ctypes.c_char_p
lib.kvlr_status_string.argtypes = [ctypes.c_int]
lib.kvlr_cache_elems.argtypes = [_D, _SZ, _SZ]
lib.kvlr_decode_workspace_bytes.argtypes = [_D, ctypes.c_int32, _SZ]
lib.kvlr_decode_plan.argtypes = [_D, ctypes.c_int32, _I32P, _I32P]
lib.kvlr_decode_counter_bytes.argtypes = [_D, _SZ]
lib.kvlr_prefill_compress.argtypes = [_D, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P]
lib.kvlr_append.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P]
lib.kvlr_decode_attn.argtypes = [_D, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, ctypes.c_size_t,
                                 ctypes.c_int32, _P]
lib.kvlr_decode_attn_noalloc.argtypes = [_D, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, ctypes.c_int32, _P]
lib.kvlr_decode_partials.argtypes = [_D, _P, _P, _P, _P, _P, ctypes.c_float, _P, ctypes.c_size_t, ctypes.c_int32, _P]
lib.kvlr_decode_combine.argtypes = [_D, _P, _P, ctypes.c_size_t, ctypes.c_int32, _P, _P]
lib.kvlr_decode_attn_latent.argtypes = [_D, _P, _P, _P, _P, ctypes.c_float, _P, _P, ctypes.c_size_t,
                                        ctypes.c_int32, _P]
lib.kvlr_append_decode_attn.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                        ctypes.c_size_t, ctypes.c_int32, _P]
lib.kvlr_hadamard_bases.argtypes = [_D, _P, _P, _P, _P, _P]


class _CLayer(ctypes.Structure):
    """kvlr_layer (kvlr.h): the arguments of kvlr_decode_attn for one layer."""
    _fields_ = [("desc", _D), ("q", _P), ("P_K", _P), ("P_V", _P), ("lat_k", _P), ("lat_v", _P),
                ("seq_lens", _P), ("scale", ctypes.c_float), ("out", _P), ("workspace", _P),
                ("workspace_bytes", ctypes.c_size_t), ("split_tokens", ctypes.c_int32)]


lib.kvlr_decode_attn_layers.argtypes = [ctypes.POINTER(_CLayer), ctypes.c_int32, ctypes.c_int32, _P]
MAX_LANES = 4   # KVLR_MAX_LANES
for _f in ("kvlr_cache_elems", "kvlr_decode_workspace_bytes", "kvlr_decode_plan", "kvlr_decode_counter_bytes", "kvlr_prefill_compress",
           "kvlr_append", "kvlr_decode_attn", "kvlr_decode_partials", "kvlr_decode_combine",
           "kvlr_decode_attn_latent", "kvlr_hadamard_bases", "kvlr_append_decode_attn", "kvlr_decode_attn_noalloc"):
    getattr(lib, _f).restype = ctypes.c_int


class KvlrError(RuntimeError):
    def __init__(self, code: int, where: str = ""):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


def version() -> int:
    return lib.kvlr_version()


def status_string(code: int) -> str:
    return lib.kvlr_status_string(code).decode()


def _check(code: int, where: str):
    if code != 0:
        raise KvlrError(code, where)


class Desc:
    """One layer's cache shape (mirrors ``kvlr_desc``); keeps the rank arrays alive."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, capacity: int,
                 r_k, r_v, in_dtype: int = BF16, latent_dtype: int = BF16, value_mode: int = VALUES_PER_HEAD):
        rk = np.broadcast_to(np.asarray(r_k, dtype=np.int32), (n_kv_heads,)).copy()
        rv = np.broadcast_to(np.asarray(r_v, dtype=np.int32), (n_kv_heads,)).copy()
        self.r_k, self.r_v = rk, rv
        self.batch, self.n_q_heads, self.n_kv_heads = batch, n_q_heads, n_kv_heads
        self.head_dim, self.capacity = head_dim, capacity
        self.in_dtype, self.latent_dtype, self.value_mode = in_dtype, latent_dtype, value_mode
        self._c = _CDesc(batch, n_q_heads, n_kv_heads, head_dim, capacity,
                         rk.ctypes.data_as(_I32P), rv.ctypes.data_as(_I32P), in_dtype, latent_dtype, value_mode)

    @property
    def ptr(self):
        return ctypes.byref(self._c)

    @property
    def pointer(self):
        """A kvlr_desc* value (for structures that hold one)."""
        return ctypes.pointer(self._c)

    @property
    def G(self):
        return self.n_q_heads // self.n_kv_heads

    def rank_offsets(self, which: str):
        r = self.r_k if which == "k" else self.r_v
        return np.concatenate([[0], np.cumsum(r)]).astype(np.int64)


def cache_elems(desc: Desc):
    k, v = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.kvlr_cache_elems(desc.ptr, ctypes.byref(k), ctypes.byref(v)), "kvlr_cache_elems")
    return k.value, v.value


def decode_workspace_bytes(desc: Desc, split_tokens: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib.kvlr_decode_workspace_bytes(desc.ptr, split_tokens, ctypes.byref(n)), "kvlr_decode_workspace_bytes")
    return n.value


def decode_plan(desc: Desc, split_tokens: int = 0):
    ns, length = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.kvlr_decode_plan(desc.ptr, split_tokens, ctypes.byref(ns), ctypes.byref(length)), "kvlr_decode_plan")
    return ns.value, length.value


# ---------------------------------------------------------------------------
# torch-facing helpers (device memory and streams only)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_of(code: int):
    torch = _torch()
    return {BF16: torch.bfloat16, F32: torch.float32, Q43: torch.uint8}[code]


def q43_outlier(r: int) -> int:
    """Channels of the 4-bit outlier block of a 4/3-bit row of rank r (layout in kvlr.h)."""
    return 16 * max(1, (r + 40) // 80)


def q43_row_bytes(r: int) -> int:
    """Bytes one token takes in a 4/3-bit cache of rank r (tiles of 32 tokens, layout in kvlr.h)."""
    no = q43_outlier(r)
    return 8 + no // 2 + 3 * (r - no) // 8


def _row_storage(desc, r: int) -> int:
    return q43_row_bytes(r) if desc.latent_dtype == Q43 else r


def _stream():
    torch = _torch()
    return _P(torch.cuda.current_stream().cuda_stream)


def _need(t, name: str, dtype, numel: Optional[int] = None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return _P(t.data_ptr())


def alloc_cache(desc: Desc, device="cuda"):
    """Flat latent caches (lat_k, lat_v) in the ABI layout."""
    torch = _torch()
    nk, nv = cache_elems(desc)
    dt = _dtype_of(desc.latent_dtype)
    return torch.empty(nk, dtype=dt, device=device), torch.empty(nv, dtype=dt, device=device)


def decode_counter_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.kvlr_decode_counter_bytes(desc.ptr, ctypes.byref(n)), "kvlr_decode_counter_bytes")
    return n.value


def alloc_workspace(desc: Desc, split_tokens: int = 0, device="cuda"):
    """Decode workspace with its counter region zeroed (as kvlr_decode_attn requires)."""
    torch = _torch()
    n = decode_workspace_bytes(desc, split_tokens)
    return torch.zeros((n + 3) // 4, dtype=torch.float32, device=device)


def pack_bases(bases: Sequence, device="cuda"):
    """Per-head [d][r_h] arrays -> one packed fp32 device tensor."""
    torch = _torch()
    flat = np.concatenate([np.ascontiguousarray(b, dtype=np.float32).ravel() for b in bases])
    return torch.from_numpy(flat).to(device)


def cap_rows(desc: Desc) -> int:
    """Rows allocated per (batch row, KV head) block: capacity rounded up to 16 (to 32 for
    4/3-bit caches, which store tiles of 32 tokens)."""
    g = 32 if desc.latent_dtype == Q43 else 16
    return (desc.capacity + g - 1) // g * g


def block_view(lat, desc: Desc, which: str, b: int, h: int):
    """The raw storage block of (batch row b, KV head h), 1-D: cap_rows * r elements
    (cap_rows * q43_row_bytes(r) bytes for 4/3-bit rows)."""
    ranks = desc.r_k if which == "k" else desc.r_v
    sizes = [_row_storage(desc, int(x)) for x in ranks]
    rows = cap_rows(desc)
    if which == "v" and desc.value_mode == VALUES_JOINT:   # one block per batch row, shared by the heads
        return lat[rows * b * sizes[0]:rows * (b + 1) * sizes[0]]
    start = rows * (b * sum(sizes) + sum(sizes[:h]))
    return lat[start:start + rows * sizes[h]]


def k_tiled_index(T: int, r: int):
    """Element offsets [T][r] of bf16 key latents inside a block (MFMA operand order, see kvlr.h)."""
    t = np.arange(T)[:, None]
    j = np.arange(r)[None, :]
    np_ = r // 32
    base = (t >> 4) * 16 * r
    n = t & 15
    pair = base + (j >> 5) * 512 + ((j >> 3) & 3) * 128 + n * 8 + (j & 7)
    jj = j - 32 * np_
    tail = base + np_ * 512 + (jj >> 2) * 64 + n * 4 + (jj & 3)
    return np.where(j < 32 * np_, pair, tail)


def v_joint_index(T: int, r: int):
    """Element offsets [T][r] of bf16 value latents inside a block (per head, or a batch row's
    joint block; value-product operand order, see kvlr.h)."""
    t = np.arange(T)[:, None]
    j = np.arange(r)[None, :]
    np_ = r // 32
    base = (t >> 4) * 16 * r
    q, e = (t & 15) >> 2, t & 3
    pair = base + (j >> 5) * 512 + q * 128 + (j & 15) * 8 + ((j >> 4) & 1) * 4 + e
    tail = base + np_ * 512 + q * 64 + (j - 32 * np_) * 4 + e
    return np.where(j < 32 * np_, pair, tail)


def latent_rows(lat, desc: Desc, which: str, b: int, h: int):
    """Logical latent rows [capacity][r] of (b, h) (a gather for bf16 latents, which are stored
    in operand order; a view otherwise). 4/3-bit caches store tiles of 32 tokens, not rows: this
    returns the block's bytes (cap_rows * q43_row_bytes(r)) as they are."""
    torch = _torch()
    r = int((desc.r_k if which == "k" else desc.r_v)[h])
    blk = block_view(lat, desc, which, b, h)
    if desc.latent_dtype == BF16:
        index = k_tiled_index if which == "k" else v_joint_index
        idx = torch.from_numpy(index(desc.capacity, r).ravel()).to(blk.device)
        return blk[idx].view(desc.capacity, r)
    if desc.latent_dtype == Q43:
        return blk
    return blk[:desc.capacity * r].view(desc.capacity, r)


def _basis_numel(desc: Desc, which: str) -> int:
    return int(desc.head_dim * (desc.r_k if which == "k" else desc.r_v).sum())


def prefill_compress(desc: Desc, K, V, start: int, P_K, P_V, lat_k, lat_v):
    """Store latents of K, V [B][n][Hkv][d] (in_dtype) at cache rows start .. start+n-1."""
    torch = _torch()
    n_tok = K.shape[1] if K is not None and K.dim() == 4 else 0
    shape = (desc.batch, n_tok, desc.n_kv_heads, desc.head_dim)
    for t, name in ((K, "K"), (V, "V")):
        if t is None or tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}")
    nk, nv = cache_elems(desc)
    ind = _dtype_of(desc.in_dtype)
    lad = _dtype_of(desc.latent_dtype)
    args = (_need(K, "K", ind), _need(V, "V", ind), start, n_tok,
            _need(P_K, "P_K", torch.float32, _basis_numel(desc, "k")),
            _need(P_V, "P_V", torch.float32, _basis_numel(desc, "v")),
            _need(lat_k, "lat_k", lad, nk), _need(lat_v, "lat_v", lad, nv))
    _check(lib.kvlr_prefill_compress(desc.ptr, *args, _stream()), "kvlr_prefill_compress")


def append(desc: Desc, k_new, v_new, pos, P_K, P_V, lat_k, lat_v):
    """Store one token per batch row: k_new, v_new [B][Hkv][d] at row pos[b] (device int32 [B])."""
    torch = _torch()
    n = desc.batch * desc.n_kv_heads * desc.head_dim
    nk, nv = cache_elems(desc)
    ind = _dtype_of(desc.in_dtype)
    lad = _dtype_of(desc.latent_dtype)
    args = (_need(k_new, "k_new", ind, n), _need(v_new, "v_new", ind, n),
            _need(pos, "pos", torch.int32, desc.batch),
            _need(P_K, "P_K", torch.float32, _basis_numel(desc, "k")),
            _need(P_V, "P_V", torch.float32, _basis_numel(desc, "v")),
            _need(lat_k, "lat_k", lad, nk), _need(lat_v, "lat_v", lad, nv))
    _check(lib.kvlr_append(desc.ptr, *args, _stream()), "kvlr_append")


def decode_attn(desc: Desc, q, P_K, P_V, lat_k, lat_v, seq_lens, scale: Optional[float] = None,
                out=None, workspace=None, split_tokens: int = 0):
    """o [B][Hq][d] fp32 for queries q [B][Hq][d] fp32 over rows t < seq_lens[b]."""
    torch = _torch()
    if scale is None:
        scale = 1.0 / math.sqrt(desc.head_dim)
    nq = desc.batch * desc.n_q_heads * desc.head_dim
    if out is None:
        out = torch.empty((desc.batch, desc.n_q_heads, desc.head_dim), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(desc, split_tokens, q.device)
    nk, nv = cache_elems(desc)
    lad = _dtype_of(desc.latent_dtype)
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (_need(q, "q", torch.float32, nq),
            _need(P_K, "P_K", torch.float32, _basis_numel(desc, "k")),
            _need(P_V, "P_V", torch.float32, _basis_numel(desc, "v")),
            _need(lat_k, "lat_k", lad, nk), _need(lat_v, "lat_v", lad, nv),
            _need(seq_lens, "seq_lens", torch.int32, desc.batch), ctypes.c_float(scale),
            _need(out, "out", torch.float32, nq), _need(workspace, "workspace", workspace.dtype),
            ctypes.c_size_t(ws_bytes), split_tokens)
    _check(lib.kvlr_decode_attn(desc.ptr, *args, _stream()), "kvlr_decode_attn")
    return out


def decode_attn_layers(layers: Sequence[dict], lanes: int = 2):
    """kvlr_decode_attn_layers: one decode_attn per entry of `layers` (dicts with the keys
    desc, q, P_K, P_V, lat_k, lat_v, seq_lens, out, workspace, and optionally scale and
    split_tokens), whose kernels may overlap across `lanes` streams; returns the outputs."""
    torch = _torch()
    arr = (_CLayer * max(len(layers), 1))()
    keep = []
    for i, L in enumerate(layers):
        desc = L["desc"]
        nq = desc.batch * desc.n_q_heads * desc.head_dim
        nk, nv = cache_elems(desc)
        lad = _dtype_of(desc.latent_dtype)
        ws = L["workspace"]
        scale = L.get("scale")
        if scale is None:
            scale = 1.0 / math.sqrt(desc.head_dim)
        arr[i] = _CLayer(desc.pointer, _need(L["q"], "q", torch.float32, nq),
                         _need(L["P_K"], "P_K", torch.float32, _basis_numel(desc, "k")),
                         _need(L["P_V"], "P_V", torch.float32, _basis_numel(desc, "v")),
                         _need(L["lat_k"], "lat_k", lad, nk), _need(L["lat_v"], "lat_v", lad, nv),
                         _need(L["seq_lens"], "seq_lens", torch.int32, desc.batch), scale,
                         _need(L["out"], "out", torch.float32, nq), _need(ws, "workspace", ws.dtype),
                         ws.numel() * ws.element_size(), int(L.get("split_tokens", 0)))
        keep.append(desc)
    _check(lib.kvlr_decode_attn_layers(arr, len(layers), lanes, _stream()), "kvlr_decode_attn_layers")
    return [L["out"] for L in layers]


def decode_attn_noalloc(desc: Desc, q, P_K, P_V, lat_k, lat_v, seq_lens, scale: Optional[float] = None,
                        out=None, split_tokens: int = 0):
    """decode_attn without a workspace argument: the library's static device scratch
    (STATIC_SCRATCH_BYTES per device) serves as the workspace; nothing is allocated
    by the call when `out` is given."""
    torch = _torch()
    if scale is None:
        scale = 1.0 / math.sqrt(desc.head_dim)
    nq = desc.batch * desc.n_q_heads * desc.head_dim
    if out is None:
        out = torch.empty((desc.batch, desc.n_q_heads, desc.head_dim), dtype=torch.float32, device=q.device)
    nk, nv = cache_elems(desc)
    lad = _dtype_of(desc.latent_dtype)
    args = (_need(q, "q", torch.float32, nq),
            _need(P_K, "P_K", torch.float32, _basis_numel(desc, "k")),
            _need(P_V, "P_V", torch.float32, _basis_numel(desc, "v")),
            _need(lat_k, "lat_k", lad, nk), _need(lat_v, "lat_v", lad, nv),
            _need(seq_lens, "seq_lens", torch.int32, desc.batch), ctypes.c_float(scale),
            _need(out, "out", torch.float32, nq), split_tokens)
    _check(lib.kvlr_decode_attn_noalloc(desc.ptr, *args, _stream()), "kvlr_decode_attn_noalloc")
    return out


def append_decode_attn(desc: Desc, k_new, v_new, pos, q, P_K, P_V, lat_k, lat_v, seq_lens,
                       scale: Optional[float] = None, out=None, workspace=None, split_tokens: int = 0):
    """append(...) then decode_attn(...) as one call (one launch for bf16 per-head caches)."""
    torch = _torch()
    if scale is None:
        scale = 1.0 / math.sqrt(desc.head_dim)
    n = desc.batch * desc.n_kv_heads * desc.head_dim
    nq = desc.batch * desc.n_q_heads * desc.head_dim
    if out is None:
        out = torch.empty((desc.batch, desc.n_q_heads, desc.head_dim), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(desc, split_tokens, q.device)
    nk, nv = cache_elems(desc)
    ind = _dtype_of(desc.in_dtype)
    lad = _dtype_of(desc.latent_dtype)
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (_need(k_new, "k_new", ind, n), _need(v_new, "v_new", ind, n),
            _need(pos, "pos", torch.int32, desc.batch), _need(q, "q", torch.float32, nq),
            _need(P_K, "P_K", torch.float32, _basis_numel(desc, "k")),
            _need(P_V, "P_V", torch.float32, _basis_numel(desc, "v")),
            _need(lat_k, "lat_k", lad, nk), _need(lat_v, "lat_v", lad, nv),
            _need(seq_lens, "seq_lens", torch.int32, desc.batch), ctypes.c_float(scale),
            _need(out, "out", torch.float32, nq), _need(workspace, "workspace", workspace.dtype),
            ctypes.c_size_t(ws_bytes), split_tokens)
    _check(lib.kvlr_append_decode_attn(desc.ptr, *args, _stream()), "kvlr_append_decode_attn")
    return out


def decode_partials(desc: Desc, q, P_K, lat_k, lat_v, seq_lens, workspace, scale: Optional[float] = None,
                    split_tokens: int = 0):
    """First stage of decode_attn: per-split softmax records into `workspace`."""
    torch = _torch()
    if scale is None:
        scale = 1.0 / math.sqrt(desc.head_dim)
    nk, nv = cache_elems(desc)
    lad = _dtype_of(desc.latent_dtype)
    args = (_need(q, "q", torch.float32, desc.batch * desc.n_q_heads * desc.head_dim),
            _need(P_K, "P_K", torch.float32, _basis_numel(desc, "k")),
            _need(lat_k, "lat_k", lad, nk), _need(lat_v, "lat_v", lad, nv),
            _need(seq_lens, "seq_lens", torch.int32, desc.batch), ctypes.c_float(scale),
            _need(workspace, "workspace", workspace.dtype),
            ctypes.c_size_t(workspace.numel() * workspace.element_size()), split_tokens)
    _check(lib.kvlr_decode_partials(desc.ptr, *args, _stream()), "kvlr_decode_partials")


def decode_combine(desc: Desc, P_V, workspace, out, split_tokens: int = 0):
    """Second stage of decode_attn: merge split records and back-project by P_V^T into out [B][Hq][d]."""
    torch = _torch()
    args = (_need(P_V, "P_V", torch.float32, _basis_numel(desc, "v")),
            _need(workspace, "workspace", workspace.dtype),
            ctypes.c_size_t(workspace.numel() * workspace.element_size()), split_tokens,
            _need(out, "out", torch.float32, desc.batch * desc.n_q_heads * desc.head_dim))
    _check(lib.kvlr_decode_combine(desc.ptr, *args, _stream()), "kvlr_decode_combine")
    return out


def decode_attn_latent(desc: Desc, q_lat, lat_k, lat_v, seq_lens, scale: Optional[float] = None, o_lat=None,
                       workspace=None, split_tokens: int = 0):
    """Folded decode: q_lat [B][Hq][max r_k] (query in key latent space) -> o_lat [B][Hq][max r_v]."""
    torch = _torch()
    if scale is None:
        scale = 1.0 / math.sqrt(desc.head_dim)
    rk_max, rv_max = int(desc.r_k.max()), int(desc.r_v.max())
    if o_lat is None:
        o_lat = torch.empty((desc.batch, desc.n_q_heads, rv_max), dtype=torch.float32, device=q_lat.device)
    if workspace is None:
        workspace = alloc_workspace(desc, split_tokens, q_lat.device)
    nk, nv = cache_elems(desc)
    lad = _dtype_of(desc.latent_dtype)
    args = (_need(q_lat, "q_lat", torch.float32, desc.batch * desc.n_q_heads * rk_max),
            _need(lat_k, "lat_k", lad, nk), _need(lat_v, "lat_v", lad, nv),
            _need(seq_lens, "seq_lens", torch.int32, desc.batch), ctypes.c_float(scale),
            _need(o_lat, "o_lat", torch.float32, desc.batch * desc.n_q_heads * rv_max),
            _need(workspace, "workspace", workspace.dtype),
            ctypes.c_size_t(workspace.numel() * workspace.element_size()), split_tokens)
    _check(lib.kvlr_decode_attn_latent(desc.ptr, *args, _stream()), "kvlr_decode_attn_latent")
    return o_lat


def hadamard_bases(desc: Desc, P_K, P_V, out_K=None, out_V=None):
    """Fold the block-wise Hadamard rotation into packed bases (in place when no outputs are given)."""
    torch = _torch()
    nk, nv = _basis_numel(desc, "k"), _basis_numel(desc, "v")
    out_K = P_K if out_K is None else out_K
    out_V = P_V if out_V is None else out_V
    args = (_need(P_K, "P_K", torch.float32, nk), _need(P_V, "P_V", torch.float32, nv),
            _need(out_K, "out_K", torch.float32, nk), _need(out_V, "out_V", torch.float32, nv))
    _check(lib.kvlr_hadamard_bases(desc.ptr, *args, _stream()), "kvlr_hadamard_bases")
    return out_K, out_V
