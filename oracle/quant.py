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

Storage (the cache layout of kvlr.h, written out here as plain loops). A
block of rows (one KV head of one batch row) is cut into tiles of 32
consecutive tokens; a tile of rank r takes 32 * row_bytes(r) bytes, with
row_bytes(r) = 8 + n_o / 2 + 3 n_i / 8 (n_o outlier, n_i = r - n_o inlier
channels, both multiples of 16). Token u of a tile (0 <= u < 32) sits in
"slot" 8 ((u mod 16) div 4) + 4 (u div 16) + (u mod 4). Inside a tile:

* bytes [0, 256): the block parameters as half floats, parameter P of the
  token in slot s at byte 64 (s div 8) + 16 P + 2 (s mod 8); P = 0 outlier
  step, 1 outlier minimum, 2 inlier step, 3 inlier minimum (the inlier pair
  is zero when there is no inlier block);
* then n_o / 16 outlier groups of 16 channels, 256 bytes each: 64 words, word
  w = n + 16 kq (0 <= n < 16, 0 <= kq < 4); byte i (0..3) of word w holds two
  4-bit codes, block 0 in the low nibble and block 1 in the high nibble;
* then n_i / 16 inlier groups of 16 channels, 192 bytes each: position w
  owns bytes 3w .. 3w + 2 as a little-endian 24-bit field that holds 8 codes
  of 3 bits, code e at bits 3e .. 3e + 2, where e names (block, i) as
  e = 0..7 -> (0,0) (0,2) (1,0) (1,2) (0,1) (0,3) (1,1) (1,3).

What (block, n, kq, i) means depends on the kind of latent, so that every
position holds what one lane of the decode kernel feeds to its matrix
products:

* keys:   token 16 block + n, channel (of the group) 4 kq + i;
* values: token 16 block + 4 kq + i, channel (of the group) n.
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


TILE = 32
KINDS = ("k", "v")
# (block, i) of the code at position e of a 24-bit inlier field
INLIER_FIELD = ((0, 0), (0, 2), (1, 0), (1, 2), (0, 1), (0, 3), (1, 1), (1, 3))


def row_bytes(r: int) -> int:
    """Bytes one token takes in the cache at rank r (meta, outlier nibbles, inlier 3-bit codes)."""
    no = n_outlier(r)
    return 8 + no // 2 + 3 * (r - no) // 8


def tile_bytes(r: int) -> int:
    """Bytes of one tile of 32 tokens."""
    return TILE * row_bytes(r)


def slot(u: int) -> int:
    """Position of tile token u (0..31) in the parameter arrays."""
    return 8 * ((u % 16) // 4) + 4 * (u // 16) + (u % 4)


def lane_code(kind: str, n: int, kq: int, block: int, i: int):
    """(token in the tile, channel in the 16-channel group) held at (block, n, kq, i)."""
    if kind == "k":
        return 16 * block + n, 4 * kq + i
    return 16 * block + 4 * kq + i, n


def pack_tile(codes, meta, r: int, kind: str) -> np.ndarray:
    """Codes [32][r] and block parameters [32][4] (float16) of one tile -> its bytes."""
    codes = np.asarray(codes, np.int64)
    meta = np.asarray(meta, np.float16)
    no = n_outlier(r)
    out = np.zeros(tile_bytes(r), np.uint8)
    for u in range(TILE):
        s = slot(u)
        for P in range(4):
            off = 64 * (s // 8) + 16 * P + 2 * (s % 8)
            out[off:off + 2] = np.array([meta[u, P]], np.float16).view(np.uint8)
    for g in range(no // BLOCK):
        base = 256 + 256 * g
        for n in range(16):
            for kq in range(4):
                w = n + 16 * kq
                for i in range(4):
                    for block in range(2):
                        tok, ch = lane_code(kind, n, kq, block, i)
                        out[base + 4 * w + i] |= np.uint8((int(codes[tok, BLOCK * g + ch]) & 0xF) << (4 * block))
    for g in range((r - no) // BLOCK):
        base = 256 + 256 * (no // BLOCK) + 192 * g
        for n in range(16):
            for kq in range(4):
                w = n + 16 * kq
                field = 0
                for e, (block, i) in enumerate(INLIER_FIELD):
                    tok, ch = lane_code(kind, n, kq, block, i)
                    field |= (int(codes[tok, no + BLOCK * g + ch]) & 0x7) << (3 * e)
                out[base + 3 * w:base + 3 * w + 3] = np.frombuffer(field.to_bytes(3, "little"), np.uint8)
    return out


def unpack_tile(raw, r: int, kind: str):
    """Bytes of one tile -> (codes [32][r] uint8, meta [32][4] float16)."""
    raw = np.asarray(raw, np.uint8)
    no = n_outlier(r)
    codes = np.zeros((TILE, r), np.uint8)
    meta = np.zeros((TILE, 4), np.float16)
    for u in range(TILE):
        s = slot(u)
        for P in range(4):
            off = 64 * (s // 8) + 16 * P + 2 * (s % 8)
            meta[u, P] = raw[off:off + 2].copy().view(np.float16)[0]
    for g in range(no // BLOCK):
        base = 256 + 256 * g
        for n in range(16):
            for kq in range(4):
                w = n + 16 * kq
                for i in range(4):
                    for block in range(2):
                        tok, ch = lane_code(kind, n, kq, block, i)
                        codes[tok, BLOCK * g + ch] = (int(raw[base + 4 * w + i]) >> (4 * block)) & 0xF
    for g in range((r - no) // BLOCK):
        base = 256 + 256 * (no // BLOCK) + 192 * g
        for n in range(16):
            for kq in range(4):
                w = n + 16 * kq
                field = int.from_bytes(bytes(raw[base + 3 * w:base + 3 * w + 3]), "little")
                for e, (block, i) in enumerate(INLIER_FIELD):
                    tok, ch = lane_code(kind, n, kq, block, i)
                    codes[tok, no + BLOCK * g + ch] = (field >> (3 * e)) & 0x7
    return codes, meta


def unpack_block(raw, T: int, r: int, kind: str):
    """The first T tokens of a block (its bytes, whole tiles) -> (codes [T][r], meta [T][4])."""
    raw = np.asarray(raw, np.uint8)
    n_tiles = (T + TILE - 1) // TILE
    codes = np.zeros((n_tiles * TILE, r), np.uint8)
    meta = np.zeros((n_tiles * TILE, 4), np.float16)
    tb = tile_bytes(r)
    for k in range(n_tiles):
        codes[k * TILE:(k + 1) * TILE], meta[k * TILE:(k + 1) * TILE] = unpack_tile(raw[k * tb:(k + 1) * tb], r, kind)
    return codes[:T], meta[:T]


def pack_block(codes, meta, r: int, kind: str) -> np.ndarray:
    """Codes [T][r] and meta [T][4] of the first T tokens -> the bytes of whole tiles (tokens
    past T zero)."""
    codes = np.asarray(codes)
    T = codes.shape[0]
    n_tiles = (T + TILE - 1) // TILE
    c = np.zeros((n_tiles * TILE, r), np.int64)
    m = np.zeros((n_tiles * TILE, 4), np.float16)
    c[:T], m[:T] = codes, meta
    return np.concatenate([pack_tile(c[k * TILE:(k + 1) * TILE], m[k * TILE:(k + 1) * TILE], r, kind)
                           for k in range(n_tiles)]) if n_tiles else np.zeros(0, np.uint8)


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
