"""Pins of the joint-value oracle (oracle/joint.py) and planted mistakes."""
from __future__ import annotations

import types

import numpy as np
import pytest

import oracle
from oracle import brute
from oracle import joint as jo


def _orth(rng, n, r):
    Q, _ = np.linalg.qr(rng.standard_normal((n, r)))
    return Q


def _case(seed, B=2, T=9, Hkv=2, G=2, d=4, rk=2, r=5, lens=None):
    rng = np.random.default_rng(seed)
    Hq = Hkv * G
    P_K = [_orth(rng, d, rk) for _ in range(Hkv)]
    P_J = _orth(rng, Hkv * d, r)
    K = rng.standard_normal((B, T, Hkv, d))
    V = rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, Hq, d))
    lens = [T, max(0, T - 4)] if lens is None else lens
    return q, K, V, P_K, P_J, lens


def pin_block_diagonal_is_per_head(m) -> bool:
    """A block-diagonal joint basis (head h's rows live only in its own column block)
    is per-head value decomposition: equals the per-head decode with those blocks."""
    rng = np.random.default_rng(51)
    B, T, Hkv, G, d, rv = 2, 11, 3, 2, 4, 3
    q, K, V, P_K, _, lens = _case(51, B, T, Hkv, G, d, 2, 1)
    P_V = [_orth(rng, d, rv) for _ in range(Hkv)]
    P_J = np.zeros((Hkv * d, Hkv * rv))
    for h in range(Hkv):
        P_J[h * d:(h + 1) * d, h * rv:(h + 1) * rv] = P_V[h]
    a = m.decode_joint(q, K, V, P_K, P_J, lens, 0.4)
    b = oracle.decode(q, K, V, P_K, P_V, lens, 0.4)
    return bool(np.abs(a - b).max() <= 1e-12 * np.abs(b).max())


def pin_full_rank_is_exact(m) -> bool:
    """r = Hkv d: the joint reconstruction is exact, so values are uncompressed (the
    per-head decode with identity value bases)."""
    q, K, V, P_K, _, lens = _case(52, r=1)
    Hkv, d = len(P_K), len(P_K[0])
    P_J = _orth(np.random.default_rng(53), Hkv * d, Hkv * d)
    a = m.decode_joint(q, K, V, P_K, P_J, lens, 0.3)
    b = oracle.decode(q, K, V, P_K, [np.eye(d)] * Hkv, lens, 0.3)
    return bool(np.abs(a - b).max() <= 1e-12 * np.abs(b).max())


def pin_rotation_invariance(m) -> bool:
    """Only span(P_J) matters: P_J -> P_J O for orthogonal O leaves the output unchanged."""
    q, K, V, P_K, P_J, lens = _case(54)
    O = _orth(np.random.default_rng(55), P_J.shape[1], P_J.shape[1])
    a = m.decode_joint(q, K, V, P_K, P_J, lens, 0.5)
    b = m.decode_joint(q, K, V, P_K, P_J @ O, lens, 0.5)
    return bool(np.abs(a - b).max() <= 1e-12 * np.abs(a).max())


def pin_latent_order(m) -> bool:
    """Latent order (q~, scores on key latents, p V_lat, then the head's rows of P_J)
    equals the definition order (associativity)."""
    q, K, V, P_K, P_J, lens = _case(56, T=13)
    B, Hq, d = q.shape
    Hkv = len(P_K)
    G = Hq // Hkv
    ref = m.decode_joint(q, K, V, P_K, P_J, lens, 0.2)
    worst = 0.0
    for b in range(B):
        T = lens[b]
        V_lat = m.joint_latents(V[b, :T].reshape(T, Hkv * d), P_J)
        for h in range(Hkv):
            got = m.decode_joint_latent_head(q[b, h * G:(h + 1) * G], K[b, :T, h] @ P_K[h], V_lat, P_K[h],
                                             m.joint_slice(P_J, h, d), 0.2)
            worst = max(worst, float(np.abs(got - ref[b, h * G:(h + 1) * G]).max()))
    return worst <= 1e-12 * np.abs(ref).max()


def pin_brute_force(m) -> bool:
    """Tiny shapes against the 50-digit scalar brute force (ragged and empty rows)."""
    worst = 0.0
    for seed, (T, Hkv, G, d, rk, r) in enumerate([(3, 2, 1, 2, 1, 3), (2, 2, 2, 3, 2, 2), (4, 3, 1, 2, 2, 4)]):
        q, K, V, P_K, P_J, _ = _case(60 + seed, 2, T, Hkv, G, d, rk, r)
        lens = [T, 0 if seed == 0 else T - 1]
        got = m.decode_joint(q, K, V, P_K, P_J, lens, 0.7)
        ref = brute.decode_joint_brute(q.tolist(), K.tolist(), V.tolist(), [p.tolist() for p in P_K], P_J.tolist(),
                                       lens, 0.7)
        ref = np.array([[[float(x) for x in row] for row in bb] for bb in ref])
        worst = max(worst, float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300)))
    return worst <= 1e-13


PINS = {
    "block_diagonal_is_per_head": pin_block_diagonal_is_per_head,
    "full_rank_is_exact": pin_full_rank_is_exact,
    "rotation_invariance": pin_rotation_invariance,
    "latent_order": pin_latent_order,
    "brute_force": pin_brute_force,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    assert PINS[name](jo), name


def _variant(**override):
    ns = types.SimpleNamespace(**{k: getattr(jo, k) for k in dir(jo) if not k.startswith("_")})
    for k, v in override.items():
        setattr(ns, k, v)
    return ns


def _wrong_slice(P_J, h, d):
    P_J = np.asarray(P_J, np.float64)
    n = P_J.shape[0] // d
    return P_J[((h + 1) % n) * d:((h + 1) % n + 1) * d]


def _decode_with(slice_fn=jo.joint_slice, latents=jo.joint_latents, own_head_only=False):
    def decode_joint(q, K, V, P_K, P_J, lens, scale):
        q = np.asarray(q, np.float64)
        K = np.asarray(K, np.float64)
        V = np.asarray(V, np.float64)
        B, Hq, d = q.shape
        Hkv = len(P_K)
        out = np.zeros((B, Hq, d))
        for b in range(B):
            T = int(lens[b])
            if T == 0:
                continue
            for i in range(Hq):
                h = i // (Hq // Hkv)
                Vsrc = V[b, :T].copy()
                if own_head_only:       # a head's latent built from its own values only
                    mask = np.zeros_like(Vsrc)
                    mask[:, h] = Vsrc[:, h]
                    Vsrc = mask
                V_lat = latents(Vsrc.reshape(T, Hkv * d), P_J)
                Kt = oracle.reconstruct(oracle.compress(K[b, :T, h], P_K[h]), P_K[h])
                Vt = oracle.reconstruct(V_lat, slice_fn(P_J, h, d))
                out[b, i] = oracle.softmax(Kt @ q[b, i] * scale) @ Vt
        return out
    return decode_joint


MUTANTS = {
    "neighbour_head_slice": _variant(decode_joint=_decode_with(slice_fn=_wrong_slice), joint_slice=_wrong_slice),
    "latent_from_own_head_only": _variant(decode_joint=_decode_with(own_head_only=True)),
    "transposed_latent": _variant(decode_joint=_decode_with(
        latents=lambda Va, P: np.asarray(Va) @ np.asarray(P)[::-1])),
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
