"""The oracle against facts that the pages and the mathematics fix (CPU only)."""
from __future__ import annotations

import types

import numpy as np
import scipy.special
import pytest
import torch

import oracle
from oracle import kvlr_oracle as ko
from tests import oracle_pins as pins


@pytest.mark.parametrize("name", sorted(pins.PINS))
def test_pin(name):
    fn, bound = pins.PINS[name]
    err = fn(oracle)
    assert np.isfinite(err) and err <= bound, f"{name}: {err} > {bound}"


def test_bf16_round_matches_torch_on_float32_values():
    """bf16 rounding of float32-representable values equals torch's float32 -> bfloat16 (nearest even)."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-20, 20, 200000),
                        [0.0, -0.0, 1.0, -1.0, 2.0 ** -126, 3.0e38 / 2]]).astype(np.float32)
    # exact halfway cases: 8 significant bits plus a trailing half ulp, both parities
    mant = rng.integers(128, 256, 5000).astype(np.float64)
    ties = ((mant + 0.5) * 2.0 ** rng.integers(-60, 60, 5000)).astype(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_ties_to_even():
    assert oracle.bf16_round(1.0 + 2.0 ** -8) == 1.0            # tie, even neighbour is 1.0
    assert oracle.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6   # tie, rounds up to even
    assert oracle.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7


def test_decode_empty_row_is_zero():
    rng = np.random.default_rng(0)
    d = 8
    P = [np.linalg.qr(rng.standard_normal((d, 3)))[0]]
    q = rng.standard_normal((2, 2, d))
    K = rng.standard_normal((2, 4, 1, d))
    out = oracle.decode(q, K, K, P, P, [0, 4], 0.3)
    assert np.all(out[0] == 0) and np.all(np.abs(out[1]) > 0)


def test_decode_latents_matches_decode():
    rng = np.random.default_rng(1)
    B, T, Hkv, G, d = 2, 30, 2, 3, 16
    rk, rv = [4, 8], [6, 2]
    P_K = [np.linalg.qr(rng.standard_normal((d, r)))[0] for r in rk]
    P_V = [np.linalg.qr(rng.standard_normal((d, r)))[0] for r in rv]
    K, V = rng.standard_normal((B, T, Hkv, d)), rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, Hkv * G, d))
    lens = [30, 17]
    lat_k = [[oracle.compress(K[b, :, h], P_K[h]) for h in range(Hkv)] for b in range(B)]
    lat_v = [[oracle.compress(V[b, :, h], P_V[h]) for h in range(Hkv)] for b in range(B)]
    a = oracle.decode(q, K, V, P_K, P_V, lens, 0.25)
    b = oracle.decode_latents(q, lat_k, lat_v, P_K, P_V, lens, 0.25)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


def test_grouped_head_decode_equals_per_head_definition():
    """decode_head_reconstructed (rows reconstructed once for the G query heads of a KV
    head) gives attend_reconstructed's result for every head, bit for bit, and the
    textbook attention over the reconstructed rows."""
    rng = np.random.default_rng(5)
    d, T, G = 16, 40, 3
    P_K = np.linalg.qr(rng.standard_normal((d, 5)))[0]
    P_V = np.linalg.qr(rng.standard_normal((d, 7)))[0]
    K, V = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    q = rng.standard_normal((G, d))
    got = oracle.decode_head_reconstructed(q, K, V, P_K, P_V, 0.4)
    ref = np.stack([oracle.attend_reconstructed(qi, K, V, P_K, P_V, 0.4) for qi in q])
    assert np.array_equal(got, ref)
    Kt, Vt = K @ P_K @ P_K.T, V @ P_V @ P_V.T
    text = np.stack([scipy.special.softmax(Kt @ qi * 0.4) @ Vt for qi in q])
    assert np.abs(got - text).max() <= 1e-12 * np.abs(text).max()
    assert np.all(oracle.decode_head_reconstructed(q, K[:0], V[:0], P_K, P_V, 0.4) == 0)
    assert oracle.decode_head_reconstructed(q, K[:0], V[:0], P_K, P_V, 0.4).shape == (G, d)


# --------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# --------------------------------------------------------------------------
def _impl(**override):
    ns = types.SimpleNamespace(attend_reconstructed=ko.attend_reconstructed, attend_latent=ko.attend_latent,
                               decode=ko.decode, compress=ko.compress, attend_folded=ko.attend_folded,
                               decode_folded=ko.decode_folded)
    for k, v in override.items():
        setattr(ns, k, v)
    return ns


def _decode_with(attend, head_of=ko.kv_head_of, len_shift=0):
    def decode(q, K, V, P_K, P_V, lens, scale):
        q = np.asarray(q, np.float64)
        B, Hq, d = q.shape
        Hkv = len(P_K)
        out = np.zeros((B, Hq, d))
        for b in range(B):
            T = int(lens[b]) + len_shift
            for i in range(Hq):
                h = head_of(i, Hq, Hkv)
                out[b, i] = attend(q[b, i], K[b, :T, h, :], V[b, :T, h, :], P_K[h], P_V[h], scale)
        return out
    return decode


def _m_no_reconstruction(q, K, V, P_K, P_V, scale):
    if len(K) == 0:
        return np.zeros(np.asarray(P_K).shape[0])
    return ko.softmax(np.asarray(K) @ q * scale) @ np.asarray(V)


def _m_rank_scale(q, K, V, P_K, P_V, scale):
    return ko.attend_reconstructed(q, K, V, P_K, P_V, 1.0 / np.sqrt(np.asarray(P_K).shape[1]))


def _m_swapped_value_basis(q, K, V, P_K, P_V, scale):
    return ko.attend_reconstructed(q, K, V, P_K, P_K if np.shape(P_K) == np.shape(P_V) else P_V, scale) \
        if np.shape(P_K) == np.shape(P_V) else _swap_generic(q, K, V, P_K, P_V, scale)


def _swap_generic(q, K, V, P_K, P_V, scale):
    # use the key basis for the values, truncated/padded to the value rank
    P_K, P_V = np.asarray(P_K), np.asarray(P_V)
    r = min(P_K.shape[1], P_V.shape[1])
    return ko.attend_reconstructed(q, K, V, P_K, P_K[:, :r], scale)


def _m_no_max_shift(q, K, V, P_K, P_V, scale):
    K = np.asarray(K, np.float64)
    if K.shape[0] == 0:
        return np.zeros(np.asarray(P_K).shape[0])
    Kt = ko.reconstruct(ko.compress(K, P_K), P_K)
    Vt = ko.reconstruct(ko.compress(V, P_V), P_V)
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.exp(Kt @ q * scale)
        return (w / w.sum()) @ Vt


def _m_sign(q, K, V, P_K, P_V, scale):
    return ko.attend_reconstructed(q, K, V, P_K, P_V, -scale)


def _m_latent_backproj_with_key_basis(q, K_lat, V_lat, P_K, P_V, scale):
    P_K, P_V = np.asarray(P_K), np.asarray(P_V)
    if np.shape(K_lat)[0] == 0:
        return np.zeros(P_V.shape[0])
    p = ko.softmax(np.asarray(K_lat) @ (np.asarray(q) @ P_K) * scale)
    B = P_K if P_K.shape == P_V.shape else P_K[:, :P_V.shape[1]] if P_K.shape[1] >= P_V.shape[1] else P_V
    return (p @ np.asarray(V_lat)) @ B.T


def _m_max_weight_normaliser(q, K, V, P_K, P_V, scale):
    K = np.asarray(K, np.float64)
    if K.shape[0] == 0:
        return np.zeros(np.asarray(P_K).shape[0])
    Kt = ko.reconstruct(ko.compress(K, P_K), P_K)
    Vt = ko.reconstruct(ko.compress(V, P_V), P_V)
    s = Kt @ q * scale
    w = np.exp(s - s.max())
    return (w / w.max()) @ Vt


def _m_folded_unscaled(q_lat, K_lat, V_lat, scale):
    return ko.attend_folded(q_lat, K_lat, V_lat, 1.0)


def _folded_with(attend, head_of=ko.kv_head_of):
    def decode_folded(q_lat, lat_k, lat_v, lens, scale, Hkv):
        q_lat = np.asarray(q_lat, np.float64)
        B, Hq = q_lat.shape[:2]
        rv_max = max(np.asarray(lat_v[0][h]).shape[1] for h in range(Hkv))
        out = np.zeros((B, Hq, rv_max))
        for b in range(B):
            T = int(lens[b])
            for i in range(Hq):
                h = head_of(i, Hq, Hkv)
                Kl, Vl = np.asarray(lat_k[b][h]), np.asarray(lat_v[b][h])
                out[b, i, :Vl.shape[1]] = attend(q_lat[b, i, :Kl.shape[1]], Kl[:T], Vl[:T], scale)
        return out
    return decode_folded


def _m_folded_key_latents_as_values(q_lat, K_lat, V_lat, scale):
    K_lat, V_lat = np.asarray(K_lat), np.asarray(V_lat)
    if K_lat.shape[0] == 0:
        return np.zeros(V_lat.shape[1])
    r = min(K_lat.shape[1], V_lat.shape[1])
    out = np.zeros(V_lat.shape[1])
    out[:r] = ko.softmax(K_lat @ q_lat * scale) @ K_lat[:, :r]
    return out


MUTANTS = {
    "dropped_reconstruction": _impl(attend_reconstructed=_m_no_reconstruction,
                                    decode=_decode_with(_m_no_reconstruction)),
    "rank_instead_of_head_dim_scale": _impl(attend_reconstructed=_m_rank_scale, decode=_decode_with(_m_rank_scale)),
    "key_basis_for_values": _impl(attend_reconstructed=_m_swapped_value_basis,
                                  decode=_decode_with(_m_swapped_value_basis)),
    "no_max_shift": _impl(attend_reconstructed=_m_no_max_shift, decode=_decode_with(_m_no_max_shift)),
    "score_sign": _impl(attend_reconstructed=_m_sign, decode=_decode_with(_m_sign)),
    "latent_backprojection_basis": _impl(attend_latent=_m_latent_backproj_with_key_basis),
    "wrong_normaliser": _impl(attend_reconstructed=_m_max_weight_normaliser,
                              decode=_decode_with(_m_max_weight_normaliser)),
    "head_mapping_modulo": _impl(decode=_decode_with(ko.attend_reconstructed,
                                                     head_of=lambda i, Hq, Hkv: i % Hkv)),
    "length_off_by_one": _impl(decode=_decode_with(ko.attend_reconstructed, len_shift=1)),
    "folded_unscaled": _impl(attend_folded=_m_folded_unscaled, decode_folded=_folded_with(_m_folded_unscaled)),
    "folded_head_mapping_modulo": _impl(decode_folded=_folded_with(ko.attend_folded,
                                                                   head_of=lambda i, Hq, Hkv: i % Hkv)),
    "folded_key_latents_as_values": _impl(attend_folded=_m_folded_key_latents_as_values,
                                          decode_folded=_folded_with(_m_folded_key_latents_as_values)),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant):
    impl = MUTANTS[mutant]
    failed = []
    for name in pins.PINS:
        kw = {"quick": True} if name in ("brute_force", "folded") else {}
        try:
            ok = pins.check(name, impl, **kw)
        except Exception:  # a crash is a caught mistake too
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"planted mistake {mutant} passed every pin"
