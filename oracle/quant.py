"""Mixed-precision latent storage: plain reference of what the quantised cache holds.

Test infrastructure only (see the package docstring).

Source: STAR-KV technical summary, "Metodologia" section 3 (mixed-precision
quantisation aware of the low rank). The latent channels come ordered by
singular value, so the leading channels carry the large magnitudes. The
latent dimension is split into an "outlier" block (the first 20% of the
channels) and an "inlier" block (the other 80%). Each block is rotated by
its own Hadamard transform, and then quantised: the outlier block with more
bits (4 in the page's example), the inlier block with fewer (3). The
Hadamard factors are folded into the projection matrices, so the rotation
costs nothing at run time ("Zero Overhead" bullet). "Risultati Chiave" quotes
3.2 bits on average, which is 0.2 * 4 + 0.8 * 3.

Readings where the page leaves a step open:

* block sizes: the outlier block is the first n_o = 16 * max(1, round(r / 80))
  channels (exactly 20% at r = 80, the nearest multiple of 16 otherwise) and
  the inlier block is the rest;
* "independent Hadamard per block": every run of 16 channels is rotated by
  the normalised 16 x 16 Sylvester Hadamard matrix H16 / 4 (entries +-1/4).
  The rotation is block-diagonal, so no rotation crosses the outlier/inlier
  boundary, and it is folded into the bases as P' = P R;
* quantiser: per token and per block, asymmetric round-to-nearest over
  [min, max] with 2^bits - 1 steps. The step and the minimum are stored as
  IEEE half floats. The code is decided in fp32, in the order written in
  `quantize_block`, so any fp32 implementation takes the same decision;
* dequantised value: step * code + minimum.

Storage of one token row of rank r (little-endian bytes):

  [0:2] step of the outlier block, [2:4] its minimum, [4:6] step of the
  inlier block, [6:8] its minimum (fp16; both zero when there is no inlier
  block), then the outlier codes, two per byte (channel 2k in the low
  nibble of byte k), then the inlier codes as one bit stream (channel c in
  bits 3c .. 3c+2), zero padding to a multiple of 4 bytes.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16
BITS_OUTLIER = 4
BITS_INLIER = 3


def hadamard(n: int) -> np.ndarray:
    """Normalised Sylvester Hadamard matrix of order n (a power of two): H_1 = [1],
    H_2m = [[H_m, H_m], [H_m, -H_m]], divided by sqrt(n)."""
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == n, "order must be a power of two"
    return H / np.sqrt(n)


def n_outlier(r: int) -> int:
    """Channels in the outlier block: 20% of r, as a multiple of 16 (at least 16)."""
    return BLOCK * max(1, int(np.floor(r / 80 + 0.5)))


def rotation(r: int) -> np.ndarray:
    """Block-diagonal R = diag(H16, ..., H16) of order r (r a multiple of 16)."""
    R = np.zeros((r, r))
    H = hadamard(BLOCK)
    for k in range(0, r, BLOCK):
        R[k:k + BLOCK, k:k + BLOCK] = H
    return R


def fuse_bases(P) -> np.ndarray:
    """Bases with the Hadamard factors folded in: P' = P R."""
    P = np.asarray(P, np.float64)
    return P @ rotation(P.shape[1])


def quantize_block(x, bits: int):
    """Asymmetric round-to-nearest of one block of fp32 values.

    Every step is an fp32 (or fp16 storage) operation, in this order:
      lo = min(x), hi = max(x)
      step = fp16(fp32(hi - lo) / (2^bits - 1))      division in fp32
      base = fp16(lo)
      code = clamp(rint(fp32(x - base) * fp32(1 / step)), 0, 2^bits - 1)
    with code = 0 everywhere when step == 0. Returns (codes uint8, step, base)
    with step and base as numpy float16.
    """
    x = np.asarray(x, np.float32)
    L = np.float32(2 ** bits - 1)
    lo, hi = np.float32(x.min()), np.float32(x.max())
    step = np.float16(np.float32(hi - lo) / L)
    base = np.float16(lo)
    if np.float32(step) == 0:
        return np.zeros(x.shape, np.uint8), step, base
    inv = np.float32(1.0) / np.float32(step)
    t = np.float32(x - np.float32(base)) * inv
    codes = np.clip(np.rint(t.astype(np.float32)), 0, L).astype(np.uint8)
    return codes, step, base


def quantize_row(x, r: int = None):
    """One token row of r fp32 latents -> (codes [r] uint8, (step_o, base_o, step_i, base_i))."""
    x = np.asarray(x, np.float32)
    r = x.shape[0] if r is None else r
    no = n_outlier(r)
    co, so, bo = quantize_block(x[:no], BITS_OUTLIER)
    if r > no:
        ci, si, bi = quantize_block(x[no:], BITS_INLIER)
    else:
        ci, si, bi = np.zeros(0, np.uint8), np.float16(0), np.float16(0)
    return np.concatenate([co, ci]), (so, bo, si, bi)


def dequantize_row(codes, meta, r: int = None) -> np.ndarray:
    """float64 values step * code + base of one row."""
    codes = np.asarray(codes, np.float64)
    r = codes.shape[0] if r is None else r
    no = n_outlier(r)
    so, bo, si, bi = (float(m) for m in meta)
    out = np.empty(r)
    out[:no] = so * codes[:no] + bo
    out[no:] = si * codes[no:] + bi
    return out


def row_bytes(r: int) -> int:
    """Bytes of one stored row of rank r."""
    no = n_outlier(r)
    n = 8 + no // 2 + (3 * (r - no) + 7) // 8
    return (n + 3) // 4 * 4


def pack_row(codes, meta, r: int = None) -> np.ndarray:
    """Codes and block parameters -> the stored bytes of one row (uint8 [row_bytes(r)])."""
    codes = np.asarray(codes, np.int64)
    r = codes.shape[0] if r is None else r
    no = n_outlier(r)
    out = np.zeros(row_bytes(r), np.uint8)
    out[0:8] = np.array(meta, dtype=np.float16).view(np.uint8)
    for c in range(no):
        out[8 + c // 2] |= np.uint8((codes[c] & 0xF) << (4 * (c % 2)))
    base = 8 + no // 2
    for c in range(r - no):
        v = int(codes[no + c]) & 0x7
        for bit in range(3):
            pos = 3 * c + bit
            if (v >> bit) & 1:
                out[base + pos // 8] |= np.uint8(1 << (pos % 8))
    return out


def unpack_row(raw, r: int):
    """Stored bytes of one row -> (codes [r] uint8, (step_o, base_o, step_i, base_i) as float16)."""
    raw = np.asarray(raw, np.uint8)
    no = n_outlier(r)
    meta = tuple(raw[0:8].view(np.float16))
    codes = np.zeros(r, np.uint8)
    for c in range(no):
        codes[c] = (raw[8 + c // 2] >> (4 * (c % 2))) & 0xF
    base = 8 + no // 2
    for c in range(r - no):
        v = 0
        for bit in range(3):
            pos = 3 * c + bit
            v |= ((int(raw[base + pos // 8]) >> (pos % 8)) & 1) << bit
        codes[no + c] = v
    return codes, meta


def quantize_rows(X32):
    """Rows [T][r] of fp32 latents -> (codes [T][r], meta [T][4] float16)."""
    X32 = np.asarray(X32, np.float32)
    T, r = X32.shape
    codes = np.zeros((T, r), np.uint8)
    meta = np.zeros((T, 4), np.float16)
    for t in range(T):
        codes[t], m = quantize_row(X32[t], r)
        meta[t] = m
    return codes, meta


def dequantize_rows(codes, meta) -> np.ndarray:
    """float64 [T][r] from codes [T][r] and meta [T][4]."""
    codes = np.asarray(codes)
    return np.stack([dequantize_row(codes[t], meta[t]) for t in range(codes.shape[0])]) if len(codes) else \
        np.zeros((0, codes.shape[1] if codes.ndim == 2 else 0))


def stored_latents(X, P_fused) -> np.ndarray:
    """What the quantised cache reconstructs for rows X [T][d]: the fp32 latents
    X P' (computed in float64, rounded once to fp32) quantised and dequantised."""
    lat = (np.asarray(X, np.float64) @ np.asarray(P_fused, np.float64)).astype(np.float32)
    codes, meta = quantize_rows(lat)
    return dequantize_rows(codes, meta)


def decode_head_quantized(q_heads, K, V, P_K, P_V, scale) -> np.ndarray:
    """Decode over a quantised cache for the G query heads of one KV head.

    The bases get the Hadamard factors folded in (P' = P R), the cache holds
    the quantised latents of K P'_K and V P'_V, and attention runs in latent
    order on the dequantised values: q~ = q P'_K, s = K^_lat q~ * scale,
    o = softmax(s) V^_lat P'_V^T. R is orthogonal, so with exact latents this
    equals the unquantised result; the difference is the storage error.
    """
    from .kvlr_oracle import decode_head_latent
    PKf, PVf = fuse_bases(P_K), fuse_bases(P_V)
    Kl = stored_latents(K, PKf)
    Vl = stored_latents(V, PVf)
    return decode_head_latent(q_heads, Kl, Vl, PKf, PVf, scale)
