"""GPU side of the seeded generator: fills device tensors with the same bits as
``synth.host.kv_rows``. Uses ``libkvlr_synth.so`` built from ``csrc/synth_gen.hip``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import host
from .configs import Config

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvlr_synth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (bind to torch's HIP runtime, see rank_compressed_kv_kvlr_amd)
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing; run __graft_entry__.build() first")
        _lib = ctypes.CDLL(_LIB_PATH)
        _lib.synth_fill_kv.restype = ctypes.c_int
        _lib.synth_fill_kv.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
        _lib.synth_touch.restype = ctypes.c_int
        _lib.synth_touch.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p]
        _lib.synth_copy.restype = ctypes.c_int
        _lib.synth_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
        _lib.synth_stream_read.restype = ctypes.c_int
        _lib.synth_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_void_p]
    return _lib


def _stream_ptr(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class KVGenerator:
    """Holds one layer's per-channel statistics on the device and fills K or V rows."""

    def __init__(self, cfg: Config, layer: int, device="cuda"):
        import torch
        self.cfg, self.layer = cfg, layer
        self.stats = host.kv_stats(cfg, layer)
        self.dev = {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in self.stats.items()}

    def fill(self, kind: str, out, t0: int = 0):
        """out: contiguous device tensor [B][n_tok][Hkv][d] of float32 or bfloat16."""
        import torch
        cfg = self.cfg
        assert out.is_cuda and out.is_contiguous() and out.dim() == 4
        B, n_tok, H, d = out.shape
        assert H == cfg.Hkv and d == cfg.d
        is_bf16 = {torch.bfloat16: 1, torch.float32: 0}[out.dtype]
        key = host.stream_key(cfg, self.layer, host.KIND_K if kind == "k" else host.KIND_V)
        rc = lib().synth_fill_kv(ctypes.c_void_p(out.data_ptr()), is_bf16, B, n_tok, t0, H, d,
                                 ctypes.c_uint64(key), ctypes.c_void_p(self.dev["mu_" + kind].data_ptr()),
                                 ctypes.c_void_p(self.dev["sigma_" + kind].data_ptr()),
                                 ctypes.c_void_p(self.dev["mult_" + kind].data_ptr()), _stream_ptr(torch))
        if rc != 0:
            raise RuntimeError(f"synth_fill_kv failed with {rc}")
        return out

    def make(self, kind: str, B: int, n_tok: int, t0: int = 0):
        import torch
        dt = torch.bfloat16 if self.cfg.in_dtype == "bf16" else torch.float32
        out = torch.empty((B, n_tok, self.cfg.Hkv, self.cfg.d), dtype=dt, device="cuda")
        return self.fill(kind, out, t0)


def touch(buf, salt: int = 0):
    """Overwrite a device scratch tensor (evicts caches between timed calls)."""
    import torch
    nbytes = buf.numel() * buf.element_size()
    rc = lib().synth_touch(ctypes.c_void_p(buf.data_ptr()), ctypes.c_uint64(nbytes - nbytes % 16),
                           ctypes.c_uint32(salt & 0xFFFFFFFF), _stream_ptr(torch))
    if rc != 0:
        raise RuntimeError(f"synth_touch failed with {rc}")


def copy(src, dst):
    """Plain device copy of src into dst (same byte size): a known-size traffic reference."""
    import torch
    nbytes = src.numel() * src.element_size()
    assert nbytes == dst.numel() * dst.element_size() and nbytes % 16 == 0
    rc = lib().synth_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                          ctypes.c_uint64(nbytes), _stream_ptr(torch))
    if rc != 0:
        raise RuntimeError(f"synth_copy failed with {rc}")


def stream_read(src, sink, workgroups: int = 512):
    """Non-temporal streaming read of all of src (a byte size that is a multiple of 16), in
    `workgroups` contiguous chunks: the achievable read bandwidth. sink: an int32 device
    tensor of at least 2048 elements."""
    import torch
    nbytes = src.numel() * src.element_size()
    assert nbytes % 16 == 0 and sink.dtype == torch.int32 and sink.numel() >= 2048
    assert 1 <= workgroups <= 2048
    rc = lib().synth_stream_read(ctypes.c_void_p(src.data_ptr()), ctypes.c_uint64(nbytes),
                                 ctypes.c_void_p(sink.data_ptr()), ctypes.c_int(workgroups), _stream_ptr(torch))
    if rc != 0:
        raise RuntimeError(f"synth_stream_read failed with {rc}")
