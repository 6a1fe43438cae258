"""Plain float64 implementation of compressed-KV decode attention (test oracle).

Test infrastructure only; see the package docstring for who may use it.

Notation follows the pages: keys K and values V of one KV head are rows
[T][d]; P_K [d][r_k] and P_V [d][r_v] have orthonormal columns (StiefAttention
technical summary, "Mecanismo Central" item 2, a point on the Stiefel
manifold; item 3, Q of a QR factorisation). Readings where the pages are
silent:

* scores are scaled by a caller-given `scale` (1/sqrt(d) in every workload:
  reconstruction happens before standard attention, so the head dimension d
  and not the rank sets the scale);
* query head i reads KV head i // G with G = Hq / Hkv (grouped-query layout);
* an empty cache (T = 0) gives a zero output row;
* the softmax is the usual max-shifted form with the natural exponential.
"""
from __future__ import annotations

import numpy as np


def bf16_round(x) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even) of float64 x, as float64.

    Written from the definition: x = m * 2**e with 0.5 <= |m| < 1, keep 8
    significant bits of m by round-half-even (numpy.rint), scale back.
    Finite values in the bf16 normal range and zero only.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def compress(X, P) -> np.ndarray:
    """Latent storage of rows X [T][d] in basis P [d][r]: X P (Mecanismo Central, item 5)."""
    return np.asarray(X, np.float64) @ np.asarray(P, np.float64)


def reconstruct(X_lat, P) -> np.ndarray:
    """Full-dimension reconstruction X_lat P^T (Mecanismo Central, item 5)."""
    return np.asarray(X_lat, np.float64) @ np.asarray(P, np.float64).T


def softmax(s) -> np.ndarray:
    """Max-shifted softmax over the last axis; an empty axis gives an empty result."""
    s = np.asarray(s, np.float64)
    if s.shape[-1] == 0:
        return s.copy()
    m = s.max(axis=-1, keepdims=True)
    w = np.exp(s - m)
    return w / w.sum(axis=-1, keepdims=True)


def attend(q, Kt, Vt, scale) -> np.ndarray:
    """Standard softmax attention of one query q [d] over full-dimension rows
    Kt, Vt [T][d]: o = softmax(Kt q * scale) Vt, the attention that follows the
    reconstruction (Mecanismo Central, item 5). Zero row when T = 0.
    """
    Kt = np.asarray(Kt, np.float64)
    Vt = np.asarray(Vt, np.float64)
    if Kt.shape[0] == 0:
        return np.zeros(Vt.shape[1])
    s = (Kt @ np.asarray(q, np.float64)) * scale
    p = softmax(s)
    return p @ Vt


def attend_reconstructed(q, K, V, P_K, P_V, scale) -> np.ndarray:
    """Definition mode for one query vector q [d] over one KV head.

    Reconstruct K~ = (K P_K) P_K^T and V~ = (V P_V) P_V^T, then
    o = softmax(K~ q * scale) V~. Zero row when T = 0.
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    d = K.shape[1] if K.ndim == 2 else np.asarray(P_K).shape[0]
    if K.shape[0] == 0:
        return np.zeros(d)
    Kt = reconstruct(compress(K, P_K), P_K)
    Vt = reconstruct(compress(V, P_V), P_V)
    return attend(q, Kt, Vt, scale)


def attend_latent(q, K_lat, V_lat, P_K, P_V, scale) -> np.ndarray:
    """Latent order for one query vector over one KV head's latents.

    q~ = q P_K; s = K_lat q~ * scale; p = softmax(s); o = (p V_lat) P_V^T.
    """
    P_K = np.asarray(P_K, np.float64)
    P_V = np.asarray(P_V, np.float64)
    K_lat = np.asarray(K_lat, np.float64)
    V_lat = np.asarray(V_lat, np.float64)
    if K_lat.shape[0] == 0:
        return np.zeros(P_V.shape[0])
    qt = np.asarray(q, np.float64) @ P_K
    s = (K_lat @ qt) * scale
    p = softmax(s)
    return (p @ V_lat) @ P_V.T


def kv_head_of(i: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head i: i // (Hq / Hkv)."""
    return i // (Hq // Hkv)


def decode_head_reconstructed(q_heads, K, V, P_K, P_V, scale) -> np.ndarray:
    """Definition mode for the G query heads [G][d] that share one KV head's K, V [T][d]:
    the head's rows are reconstructed once and every query head attends over them
    (the same arithmetic as attend_reconstructed per head)."""
    q_heads = np.asarray(q_heads, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if K.shape[0] == 0:
        return np.zeros((q_heads.shape[0], np.asarray(P_V).shape[0]))
    Kt = reconstruct(compress(K, P_K), P_K)
    Vt = reconstruct(compress(V, P_V), P_V)
    return np.stack([attend(qi, Kt, Vt, scale) for qi in q_heads])


def decode_head_latent(q_heads, K_lat, V_lat, P_K, P_V, scale) -> np.ndarray:
    """Latent order for the G query heads that share one KV head's latents."""
    return np.stack([attend_latent(qi, K_lat, V_lat, P_K, P_V, scale) for qi in np.asarray(q_heads)])


def decode(q, K, V, P_K, P_V, lens, scale) -> np.ndarray:
    """Definition mode over a batch.

    q [B][Hq][d]; K, V [B][T][Hkv][d]; P_K, P_V: per-KV-head lists of [d][r];
    lens [B]: row b attends to tokens t < lens[b]. Returns o [B][Hq][d].
    """
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = len(P_K)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        T = int(lens[b])
        for i in range(Hq):
            h = kv_head_of(i, Hq, Hkv)
            out[b, i] = attend_reconstructed(q[b, i], K[b, :T, h, :], V[b, :T, h, :],
                                             P_K[h], P_V[h], scale)
    return out


def decode_latents(q, lat_k, lat_v, P_K, P_V, lens, scale) -> np.ndarray:
    """Latent order over a batch of latent caches.

    lat_k[b][h], lat_v[b][h]: arrays [>= lens[b]][r] (only the first lens[b]
    rows are read). Returns o [B][Hq][d].
    """
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = len(P_K)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        T = int(lens[b])
        for i in range(Hq):
            h = kv_head_of(i, Hq, Hkv)
            out[b, i] = attend_latent(q[b, i], np.asarray(lat_k[b][h])[:T], np.asarray(lat_v[b][h])[:T],
                                      P_K[h], P_V[h], scale)
    return out


def attend_folded(q_lat, K_lat, V_lat, scale) -> np.ndarray:
    """Folded form for one query over one KV head: the bases live in the caller's
    projections (StiefAttention technical summary, "Mecanismo Central" item 5,
    bases incorporated into the attention linear weights; STAR-KV technical
    summary, "Metodologia" section 2, reconstruction absorbed into the output
    projection). In: q_lat = q P_K [r_k]. Out: o_lat = softmax(K_lat q_lat * scale) V_lat
    [r_v], so that o = o_lat P_V^T. Zero row when T = 0.
    """
    K_lat = np.asarray(K_lat, np.float64)
    V_lat = np.asarray(V_lat, np.float64)
    if K_lat.shape[0] == 0:
        return np.zeros(V_lat.shape[1])
    p = softmax((K_lat @ np.asarray(q_lat, np.float64)) * scale)
    return p @ V_lat


def decode_folded(q_lat, lat_k, lat_v, lens, scale, Hkv: int) -> np.ndarray:
    """Folded form over a batch.

    q_lat [B][Hq][>= r_k(h)] (query head i reads its first r_k entries, h = i // G);
    lat_k[b][h], lat_v[b][h]: [>= lens[b]][r]. Returns o_lat [B][Hq][max r_v],
    entries past a head's r_v zero.
    """
    q_lat = np.asarray(q_lat, np.float64)
    B, Hq = q_lat.shape[:2]
    rv_max = max(np.asarray(lat_v[0][h]).shape[1] for h in range(Hkv))
    out = np.zeros((B, Hq, rv_max))
    for b in range(B):
        T = int(lens[b])
        for i in range(Hq):
            h = kv_head_of(i, Hq, Hkv)
            Kl, Vl = np.asarray(lat_k[b][h]), np.asarray(lat_v[b][h])
            rk, rv = Kl.shape[1], Vl.shape[1]
            out[b, i, :rv] = attend_folded(q_lat[b, i, :rk], Kl[:T], Vl[:T], scale)
    return out
