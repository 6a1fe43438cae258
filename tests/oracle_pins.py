"""Pins of the float64 oracle to facts outside itself.

Each pin takes an implementation namespace `impl` with the oracle's
interface (attend_reconstructed, attend_latent, decode, compress) so that
tests can run the same battery against deliberately wrong variants and show
that every planted mistake fails at least one pin. A pin returns the
largest error it saw; `check` compares it with the pin's bound.
"""
from __future__ import annotations

import json
import os

import numpy as np
import scipy.special

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def _orth(rng, d, r):
    Q, _ = np.linalg.qr(rng.standard_normal((d, r)))
    return Q


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


def pin_full_rank_textbook(impl) -> float:
    """r = d: P P^T = I, so the result is textbook softmax(K q * scale) V (scipy softmax)."""
    rng = np.random.default_rng(11)
    worst = 0.0
    for d, T in ((8, 9), (16, 33)):
        P_K, P_V = _orth(rng, d, d), _orth(rng, d, d)
        K, V, q = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal(d)
        scale = 1 / np.sqrt(d)
        ref = scipy.special.softmax(K @ q * scale) @ V
        worst = max(worst, _rel(impl.attend_reconstructed(q, K, V, P_K, P_V, scale), ref))
    return worst


def pin_rotation_invariance(impl) -> float:
    """Output depends only on span(P): P -> P O for orthogonal O (QR's R is a change of coordinates)."""
    rng = np.random.default_rng(12)
    worst = 0.0
    d, T = 16, 40
    for r_k, r_v in ((4, 7), (9, 3)):
        P_K, P_V = _orth(rng, d, r_k), _orth(rng, d, r_v)
        O_K, O_V = _orth(rng, r_k, r_k), _orth(rng, r_v, r_v)
        K, V, q = rng.standard_normal((T, d)) * 2, rng.standard_normal((T, d)), rng.standard_normal(d)
        a = impl.attend_reconstructed(q, K, V, P_K, P_V, 0.25)
        b = impl.attend_reconstructed(q, K, V, P_K @ O_K, P_V @ O_V, 0.25)
        worst = max(worst, _rel(a, b))
        a = impl.attend_latent(q, impl.compress(K, P_K), impl.compress(V, P_V), P_K, P_V, 0.25)
        b = impl.attend_latent(q, impl.compress(K, P_K @ O_K), impl.compress(V, P_V @ O_V),
                               P_K @ O_K, P_V @ O_V, 0.25)
        worst = max(worst, _rel(a, b))
    return worst


def pin_modes_agree(impl) -> float:
    """Reconstruct-then-attend equals the latent order (associativity)."""
    rng = np.random.default_rng(13)
    worst = 0.0
    for d, T, r_k, r_v in ((16, 50, 5, 11), (32, 7, 32, 3)):
        P_K, P_V = _orth(rng, d, r_k), _orth(rng, d, r_v)
        K, V, q = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal(d)
        a = impl.attend_reconstructed(q, K, V, P_K, P_V, 0.3)
        b = impl.attend_latent(q, impl.compress(K, P_K), impl.compress(V, P_V), P_K, P_V, 0.3)
        worst = max(worst, _rel(a, b))
    return worst


def brute_cases(quick=False):
    """(seed, B, T, Hkv, G, d, r_k, r_v, lens) tiny shapes for the mpmath brute force."""
    cases = []
    seed = 100
    dims = (2, 4) if quick else (2, 4, 8)
    Ts = (1, 3) if quick else (1, 2, 3, 5)
    for d in dims:
        ranks = sorted({1, max(1, d // 2), d}) if (quick or d == 8) else range(1, d + 1)
        for r in ranks:
            for T in Ts:
                for G in (1, 2):
                    seed += 1
                    lens = [T, max(0, T - 1)]     # second row ragged (and empty when T = 1)
                    cases.append((seed, 2, T, 2, G, d, r, max(1, d - r + 1), lens))
    return cases


def pin_brute_force(impl, quick=False) -> float:
    """Batch, grouped-query and ragged lengths against the 50-digit scalar brute force."""
    worst = 0.0
    for seed, B, T, Hkv, G, d, r_k, r_v, lens in brute_cases(quick):
        rng = np.random.default_rng(seed)
        Hq = Hkv * G
        P_K = [_orth(rng, d, r_k) for _ in range(Hkv)]
        P_V = [_orth(rng, d, r_v) for _ in range(Hkv)]
        K = rng.standard_normal((B, T, Hkv, d))
        V = rng.standard_normal((B, T, Hkv, d))
        q = rng.standard_normal((B, Hq, d))
        scale = 1 / np.sqrt(d)
        got = impl.decode(q, K, V, P_K, P_V, lens, scale)
        ref = brute.decode_brute(q.tolist(), K.tolist(), V.tolist(),
                                 [p.tolist() for p in P_K], [p.tolist() for p in P_V], lens, scale)
        ref = np.array([[[float(x) for x in row] for row in bb] for bb in ref])
        den = max(np.abs(ref).max(), 1e-300)
        worst = max(worst, float(np.abs(got - ref).max() / den))
    return worst


def pin_large_scores(impl) -> float:
    """Scores near +-1000 (exp would overflow without the max shift) against the brute force."""
    rng = np.random.default_rng(14)
    d, T, r = 4, 3, 2
    P_K, P_V = _orth(rng, d, r), _orth(rng, d, r)
    q = rng.standard_normal(d) * 3.0
    # every score gets a common offset of +1000 along w, where (w P_K P_K^T) . q = 1
    u = P_K @ P_K.T @ q
    w = u / (u @ q)
    K = rng.standard_normal((T, d)) + 1000.0 * w
    V = rng.standard_normal((T, d))
    got = impl.attend_reconstructed(q, K, V, P_K, P_V, 1.0)
    ref = np.array([float(x) for x in brute.attend_brute(q, K, V, P_K, P_V, 1.0)])
    if not np.all(np.isfinite(got)):
        return float("inf")
    return _rel(got, ref)


def pin_closed_forms(impl) -> float:
    """T=1 gives v P_V P_V^T; q=0 gives the mean of V~; T=2 is a sigmoid mix; V in span(P_V) is lossless."""
    rng = np.random.default_rng(15)
    d, r_k, r_v = 12, 5, 4
    P_K, P_V = _orth(rng, d, r_k), _orth(rng, d, r_v)
    worst = 0.0
    # T = 1: any q
    K, V, q = rng.standard_normal((1, d)), rng.standard_normal((1, d)), rng.standard_normal(d) * 5
    worst = max(worst, _rel(impl.attend_reconstructed(q, K, V, P_K, P_V, 0.2), V[0] @ P_V @ P_V.T))
    # q = 0: uniform weights over T tokens
    T = 23
    K, V = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    ref = (V @ P_V @ P_V.T).mean(axis=0)
    worst = max(worst, _rel(impl.attend_reconstructed(np.zeros(d), K, V, P_K, P_V, 0.2), ref))
    # T = 2: o = sigmoid(s1 - s2) V~_1 + sigmoid(s2 - s1) V~_2 with s_t = (K_t P_K)(q P_K) * scale
    K, V, q = rng.standard_normal((2, d)), rng.standard_normal((2, d)), rng.standard_normal(d)
    s = (K @ P_K) @ (q @ P_K) * 0.7
    Vt = V @ P_V @ P_V.T
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))  # noqa: E731
    ref = sig(s[0] - s[1]) * Vt[0] + sig(s[1] - s[0]) * Vt[1]
    worst = max(worst, _rel(impl.attend_reconstructed(q, K, V, P_K, P_V, 0.7), ref))
    # values inside span(P_V): reconstruction of V is exact
    T = 9
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, r_v)) @ P_V.T
    q = rng.standard_normal(d)
    s = (K @ P_K @ P_K.T) @ q * 0.5
    ref = scipy.special.softmax(s) @ V
    worst = max(worst, _rel(impl.attend_reconstructed(q, K, V, P_K, P_V, 0.5), ref))
    return worst


def pin_folded(impl, quick=False) -> float:
    """Folded form: o = o_lat P_V^T and P_V^T P_V = I give o_lat = o P_V, with o from the
    50-digit brute force; plus T = 1 (o_lat = the one value latent) and q_lat = 0 (the mean)."""
    worst = 0.0
    for seed, B, T, Hkv, G, d, r_k, r_v, lens in brute_cases(quick):
        rng = np.random.default_rng(seed)
        Hq = Hkv * G
        P_K = [_orth(rng, d, r_k) for _ in range(Hkv)]
        P_V = [_orth(rng, d, r_v) for _ in range(Hkv)]
        K = rng.standard_normal((B, T, Hkv, d))
        V = rng.standard_normal((B, T, Hkv, d))
        q = rng.standard_normal((B, Hq, d))
        scale = 1 / np.sqrt(d)
        q_lat = np.stack([np.stack([q[b, i] @ P_K[i // G] for i in range(Hq)]) for b in range(B)])
        lat_k = [[K[b, :, h] @ P_K[h] for h in range(Hkv)] for b in range(B)]
        lat_v = [[V[b, :, h] @ P_V[h] for h in range(Hkv)] for b in range(B)]
        got = impl.decode_folded(q_lat, lat_k, lat_v, lens, scale, Hkv)
        ref = brute.decode_brute(q.tolist(), K.tolist(), V.tolist(),
                                 [p.tolist() for p in P_K], [p.tolist() for p in P_V], lens, scale)
        ref = np.array([[[float(x) for x in row] for row in bb] for bb in ref])
        ref_lat = np.stack([np.stack([ref[b, i] @ P_V[i // G] for i in range(Hq)]) for b in range(B)])
        den = max(np.abs(ref_lat).max(), 1e-300)
        worst = max(worst, float(np.abs(got - ref_lat).max() / den))
    rng = np.random.default_rng(16)
    Kl, Vl, ql = rng.standard_normal((1, 5)), rng.standard_normal((1, 3)), rng.standard_normal(5) * 4
    worst = max(worst, _rel(impl.attend_folded(ql, Kl, Vl, 0.3), Vl[0]))
    Kl, Vl = rng.standard_normal((17, 5)), rng.standard_normal((17, 3))
    worst = max(worst, _rel(impl.attend_folded(np.zeros(5), Kl, Vl, 0.3), Vl.mean(axis=0)))
    return worst


def pin_golden(impl) -> float:
    """Hand-derived examples in tests/golden/hand_examples.json."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    worst = 0.0
    for c in cases:
        got = impl.attend_reconstructed(np.array(c["q"]), np.array(c["K"]), np.array(c["V"]),
                                        np.array(c["P_K"]), np.array(c["P_V"]), c["scale"])
        exp = np.array(c["expected"])
        worst = max(worst, float(np.abs(got - exp).max() / max(1.0, np.abs(exp).max())))
    return worst


PINS = {
    "full_rank_textbook": (pin_full_rank_textbook, 1e-12),
    "rotation_invariance": (pin_rotation_invariance, 1e-12),
    "modes_agree": (pin_modes_agree, 1e-12),
    "brute_force": (pin_brute_force, 1e-13),
    "large_scores": (pin_large_scores, 1e-12),
    "closed_forms": (pin_closed_forms, 1e-12),
    "golden": (pin_golden, 1e-14),
    "folded": (pin_folded, 1e-13),
}


def check(name, impl, **kw) -> bool:
    fn, bound = PINS[name]
    err = fn(impl, **kw) if kw else fn(impl)
    return bool(np.isfinite(err) and err <= bound)
