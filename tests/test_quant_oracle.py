"""Pins of the quantised-latent oracle (oracle/quant.py) to facts outside it,
and a planted-mistake battery: each wrong variant fails at least one pin."""
from __future__ import annotations

import json
import os
import types

import numpy as np
import pytest

import oracle
from oracle import quant as qo

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_examples.json")


def _orth(rng, d, r):
    Q, _ = np.linalg.qr(rng.standard_normal((d, r)))
    return Q


# ---------------------------------------------------------------------------
# pins: each returns True when the implementation `m` passes
# ---------------------------------------------------------------------------
def pin_hadamard(m) -> bool:
    """Textbook H2 = [[1, 1], [1, -1]] / sqrt 2; H16 has entries +-1/4 and H H^T = I;
    R is block-diagonal and orthogonal; folding R into orthonormal bases keeps them
    orthonormal and keeps their span (P' P'^T = P P^T)."""
    ok = np.allclose(m.hadamard(2), np.array([[1, 1], [1, -1]]) / np.sqrt(2), atol=0, rtol=1e-15)
    H = m.hadamard(16)
    ok &= bool(np.all(np.abs(np.abs(H) - 0.25) == 0))
    ok &= np.allclose(H @ H.T, np.eye(16), atol=1e-15)
    R = m.rotation(48)
    ok &= np.allclose(R @ R.T, np.eye(48), atol=1e-14)
    ok &= bool(np.all(R[:16, 16:] == 0) and np.all(R[16:32, 32:] == 0) and np.all(R[32:, :32] == 0))
    rng = np.random.default_rng(31)
    P = _orth(rng, 128, 64)
    Pf = m.fuse_bases(P)
    ok &= np.allclose(Pf.T @ Pf, np.eye(64), atol=1e-13)
    ok &= np.allclose(Pf @ Pf.T, P @ P.T, atol=1e-13)
    return bool(ok)


def pin_block_sizes(m) -> bool:
    """r = 80 splits into 16 outlier (20%) and 64 inlier channels, i.e. 3.2 bits per
    channel, the page's figure; every rank takes the whole number of 16-channel
    Hadamard blocks nearest to 20% of its channels."""
    ok = m.n_outlier(80) == 16
    bits = (m.n_outlier(80) * m.BITS_OUTLIER + (80 - m.n_outlier(80)) * m.BITS_INLIER) / 80
    ok &= abs(bits - 3.2) < 1e-12
    for r in range(16, 129, 16):
        # the whole 16-channel block count closest to 20% of r, at least one block
        want = min((16, 32), key=lambda c: abs(c - 0.2 * r))
        ok &= m.n_outlier(r) == want
    return bool(ok)


def pin_golden(m) -> bool:
    """Hand-derived quantiser and byte-layout examples in tests/golden/quant_examples.json."""
    g = json.load(open(GOLDEN))
    ok = True
    for c in g["quantize_block"]:
        codes, step, base = m.quantize_block(np.array(c["x"], np.float32), c["bits"])
        ok &= list(map(int, codes)) == c["codes"] and float(step) == c["step"] and float(base) == c["base"]
        if "dequantized" in c:   # a block on its own: dequantised with its own step and base
            deq = float(step) * np.asarray(codes, np.float64) + float(base)
            ok &= np.array_equal(deq, np.array(c["dequantized"]))
    for t in g["pack_tile"]:
        r, kind = t["r"], t["kind"]
        codes = np.zeros((m.TILE, r), np.int64)
        meta = np.zeros((m.TILE, 4), np.float16)
        for tok, ch, c in t["codes"]:
            codes[tok, ch] = c
        for tok, P, v in t["meta"]:
            meta[tok, P] = v
        want = np.zeros(t["tile_bytes"], np.uint8)
        for off, v in t["bytes"].items():
            want[int(off)] = v
        raw = m.pack_tile(codes, meta, r, kind)
        ok &= len(raw) == m.tile_bytes(r) and np.array_equal(raw, want)
        c2, m2 = m.unpack_tile(want, r, kind)
        ok &= np.array_equal(c2, codes) and np.array_equal(m2.view(np.uint16), meta.view(np.uint16))
    rb = g["row_bytes"]
    ok &= all(m.row_bytes(int(r)) == v for r, v in rb.items() if r != "note")
    return bool(ok)


def pin_quantizer_properties(m) -> bool:
    """Codes stay in [0, 2^b - 1]; every value inside the stored range is reproduced
    within half a step (plus the half-float rounding of the base); values on an exact
    grid are reproduced exactly; a constant block stores step 0 and its value."""
    rng = np.random.default_rng(32)
    ok = True
    for bits in (3, 4):
        L = 2 ** bits - 1
        for _ in range(200):
            x = (rng.standard_normal(16) * rng.uniform(0.01, 30)).astype(np.float32)
            codes, step, base = m.quantize_block(x, bits)
            ok &= bool(codes.max() <= L)
            s, b = float(step), float(base)
            deq = s * codes.astype(np.float64) + b
            inside = (x >= b) & (x <= b + L * s)
            ok &= bool(np.all(np.abs(deq - x)[inside] <= s / 2 * (1 + 1e-6) + 1e-30))
        grid = (np.float32(-3.0) + np.float32(0.25) * np.arange(L + 1)).astype(np.float32)
        codes, step, base = m.quantize_block(grid, bits)
        ok &= list(map(int, codes)) == list(range(L + 1)) and float(step) == 0.25 and float(base) == -3.0
        codes, step, base = m.quantize_block(np.full(9, 1.5, np.float32), bits)
        ok &= bool(np.all(codes == 0)) and float(step) == 0.0 and float(base) == 1.5
    return bool(ok)


def pin_tile_round_trip(m) -> bool:
    """pack/unpack are inverse on random codes and parameters for every rank and both kinds,
    every byte of a tile is used (a tile holds exactly 32 rows of 3.2-bit-class codes), the
    outlier block is quantised with 4 bits and the inlier block with 3 (a row whose inlier
    block spans many steps never stores a code above 7 there)."""
    rng = np.random.default_rng(33)
    ok = True
    for r in range(16, 129, 16):
        no = m.n_outlier(r)
        ok &= m.tile_bytes(r) * 8 == m.TILE * (64 + 4 * no + 3 * (r - no))
        for kind in ("k", "v"):
            T = 45
            codes = np.concatenate([rng.integers(0, 16, (T, no)), rng.integers(0, 8, (T, r - no))], 1).astype(np.uint8)
            meta = rng.standard_normal((T, 4)).astype(np.float16)
            raw = m.pack_block(codes, meta, r, kind)
            ok &= len(raw) == 2 * m.tile_bytes(r)
            c2, m2 = m.unpack_block(raw, T, r, kind)
            ok &= np.array_equal(c2, codes) and np.array_equal(m2.view(np.uint16), meta.view(np.uint16))
            # all-ones codes and parameters fill every bit of a tile
            full = m.pack_tile(np.concatenate([np.full((32, no), 15), np.full((32, r - no), 7)], 1),
                               np.full((32, 4), np.float16(np.frombuffer(b"\xff\x7b", np.float16)[0])), r, kind)
            ok &= bool(np.all(full[256:] == 255)) and bool(np.all(full[:256].view(np.uint16) == 0x7BFF))
        x = np.linspace(-4, 4, r).astype(np.float32)
        cq, _ = m.quantize_row(x, r)
        ok &= int(cq[:no].max()) == 15 and (r == no or int(cq[no:].max()) == 7)
    return bool(ok)


def pin_decode_quantized(m) -> bool:
    """Decode over the quantised cache equals reconstruct-then-attend on the dequantised
    rows (associativity), equals the exact result when every latent lies on the grid,
    and stays within the storage error of the unquantised decode."""
    rng = np.random.default_rng(34)
    d, T, G, r = 32, 40, 2, 32
    P_K, P_V = _orth(rng, d, r), _orth(rng, d, r)
    K, V = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    q = rng.standard_normal((G, d))
    got = m.decode_head_quantized(q, K, V, P_K, P_V, 0.2)
    PKf, PVf = m.fuse_bases(P_K), m.fuse_bases(P_V)
    Kh = m.stored_latents(K, PKf) @ PKf.T
    Vh = m.stored_latents(V, PVf) @ PVf.T
    ref = np.stack([oracle.attend_reconstructed(qi, Kh, Vh, np.eye(d), np.eye(d), 0.2) for qi in q])
    ok = np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    exact = oracle.decode_head_latent(q, K @ PKf, V @ PVf, PKf, PVf, 0.2)
    ok &= float(np.linalg.norm(got - exact) / np.linalg.norm(exact)) < 0.3
    # latents on an exact grid: rows that are multiples of 1/8 in [-1, 0.875] (4-bit span)
    Xl = rng.integers(-8, 8, (T, r)) / 8.0
    Xl[:, 0], Xl[:, 1] = -1.0, 0.875                               # full 4-bit outlier range
    Xl[:, m.n_outlier(r)], Xl[:, m.n_outlier(r) + 1] = -0.5, 0.375   # 8 steps of 1/8 inlier
    Xl[:, m.n_outlier(r):] = np.clip(Xl[:, m.n_outlier(r):], -0.5, 0.375)
    codes, meta = m.quantize_rows(Xl.astype(np.float32))
    ok &= np.array_equal(m.dequantize_rows(codes, meta), Xl)
    return bool(ok)


PINS = {
    "hadamard": pin_hadamard,
    "block_sizes": pin_block_sizes,
    "golden": pin_golden,
    "quantizer_properties": pin_quantizer_properties,
    "tile_round_trip": pin_tile_round_trip,
    "decode_quantized": pin_decode_quantized,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    assert PINS[name](qo), name


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------
def _variant(**override):
    ns = types.SimpleNamespace(**{k: getattr(qo, k) for k in dir(qo) if not k.startswith("_")})
    for k, v in override.items():
        setattr(ns, k, v)
    return ns


def _floor_block(x, bits):
    x = np.asarray(x, np.float32)
    L = np.float32(2 ** bits - 1)
    step = np.float16(np.float32(x.max() - x.min()) / L)
    base = np.float16(x.min())
    if float(step) == 0:
        return np.zeros(x.shape, np.uint8), step, base
    t = (x - np.float32(base)) * (np.float32(1) / np.float32(step))
    return np.clip(np.floor(t), 0, L).astype(np.uint8), step, base


def _no_clamp_block(x, bits):
    x = np.asarray(x, np.float32)
    L = np.float32(2 ** bits - 1)
    step = np.float16(np.float32(x.max() - x.min()) / L)
    base = np.float16(x.min())
    if float(step) == 0:
        return np.zeros(x.shape, np.uint8), step, base
    t = (x - np.float32(base)) * (np.float32(1) / np.float32(step))
    return np.rint(t).astype(np.int64).astype(np.uint8), step, base


def _swapped_nibbles(codes, meta, r, kind):
    raw = qo.pack_tile(codes, meta, r, kind)
    seg = raw[256:256 + 256 * (qo.n_outlier(r) // 16)]
    raw[256:256 + len(seg)] = ((seg & 0xF) << 4) | (seg >> 4)
    return raw


def _meta_in_token_order(codes, meta, r, kind):
    raw = qo.pack_tile(codes, np.zeros((32, 4), np.float16), r, kind)
    meta = np.asarray(meta, np.float16)
    for u in range(32):
        for P in range(4):
            off = 64 * (u // 8) + 16 * P + 2 * (u % 8)
            raw[off:off + 2] = np.array([meta[u, P]], np.float16).view(np.uint8)
    return raw


def _kinds_swapped(codes, meta, r, kind):
    return qo.pack_tile(codes, meta, r, "v" if kind == "k" else "k")


def _unnormalised_hadamard(n):
    return qo.hadamard(n) * np.sqrt(n)


def _three_bit_outliers(x, r=None):
    x = np.asarray(x, np.float32)
    r = x.shape[0] if r is None else r
    no = qo.n_outlier(r)
    co, so, bo = qo.quantize_block(x[:no], 3)
    ci, si, bi = qo.quantize_block(x[no:], 3) if r > no else (np.zeros(0, np.uint8), np.float16(0), np.float16(0))
    return np.concatenate([co, ci]), (so, bo, si, bi)


MUTANTS = {
    "floor_instead_of_round": _variant(quantize_block=_floor_block),
    "no_clamp": _variant(quantize_block=_no_clamp_block),
    "swapped_nibbles": _variant(pack_tile=_swapped_nibbles),
    "key_value_layouts_swapped": _variant(pack_tile=_kinds_swapped),
    "parameters_in_token_order": _variant(pack_tile=_meta_in_token_order),
    "unnormalised_hadamard": _variant(hadamard=_unnormalised_hadamard),
    "quarter_outliers": _variant(n_outlier=lambda r: 16 * max(1, int(np.floor(r / 64 + 0.5)))),
    "three_bit_outliers": _variant(quantize_row=_three_bit_outliers),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant):
    m = MUTANTS[mutant]
    failed = []
    for name, pin in PINS.items():
        try:
            ok = pin(m)
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"planted mistake {mutant} passed every pin"
