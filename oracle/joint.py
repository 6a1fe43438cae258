"""Joint value decomposition with per-head keys: plain float64 reference.

Test infrastructure only (see the package docstring).

Source: STAR-KV technical summary, "Metodologia" section 2 (hybrid
decomposition strategy). Joint decomposition (JD) factorises the
concatenated heads, per-head decomposition (HD) each head on its own. Values
are the more sensitive to compression error, so STAR-KV decomposes values
jointly and keys per head. The cost of the joint reconstruction is removed
by folding the reconstruction matrices into the output projection.

Here, for one batch row and Hkv KV heads of size d:

* keys as everywhere else: K_lat[h] = K_h P_K[h], K~_h = K_lat[h] P_K[h]^T;
* values of all heads concatenated per token, V_all = [V_0 ... V_{Hkv-1}]
  ([T][Hkv d]), stored as ONE latent V_lat = V_all P_J with P_J
  [Hkv d][r] (orthonormal columns), shared by every head;
* head h reconstructs its values with its own d rows of P_J:
  V~_h = V_lat P_J[h d:(h+1) d]^T.

So query head i (KV head h = i // G) outputs
  o_i = softmax(K~_h q_i * scale) V~_h.
"""
from __future__ import annotations

import numpy as np

from .kvlr_oracle import compress, kv_head_of, reconstruct, softmax


def joint_slice(P_J, h: int, d: int) -> np.ndarray:
    """Rows of the joint value basis that reconstruct head h: P_J[h d:(h+1) d] ([d][r])."""
    return np.asarray(P_J, np.float64)[h * d:(h + 1) * d]


def joint_latents(V_all, P_J) -> np.ndarray:
    """Joint value latents V_all P_J for rows V_all [T][Hkv d]."""
    return np.asarray(V_all, np.float64) @ np.asarray(P_J, np.float64)


def decode_joint(q, K, V, P_K, P_J, lens, scale) -> np.ndarray:
    """Definition order over a batch: reconstruct keys per head and values from the
    joint latent, then softmax attention.

    q [B][Hq][d]; K, V [B][T][Hkv][d]; P_K: per-head [d][r_k]; P_J [Hkv d][r];
    lens [B]. Returns o [B][Hq][d]; empty rows give zero.
    """
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
        V_lat = joint_latents(V[b, :T].reshape(T, Hkv * d), P_J)
        for i in range(Hq):
            h = kv_head_of(i, Hq, Hkv)
            Kt = reconstruct(compress(K[b, :T, h], P_K[h]), P_K[h])
            Vt = reconstruct(V_lat, joint_slice(P_J, h, d))
            out[b, i] = softmax(Kt @ q[b, i] * scale) @ Vt
    return out


def decode_joint_latent_head(q_heads, K_lat, V_lat, P_K, P_J_slice, scale) -> np.ndarray:
    """Latent order for the G query heads of one KV head: q~ = q P_K,
    p = softmax(K_lat q~ * scale), o = (p V_lat) P_J_slice^T. V_lat is the joint latent."""
    K_lat = np.asarray(K_lat, np.float64)
    V_lat = np.asarray(V_lat, np.float64)
    P_K = np.asarray(P_K, np.float64)
    S = np.asarray(P_J_slice, np.float64)
    out = []
    for qi in np.asarray(q_heads, np.float64):
        if K_lat.shape[0] == 0:
            out.append(np.zeros(S.shape[0]))
            continue
        p = softmax(K_lat @ (qi @ P_K) * scale)
        out.append((p @ V_lat) @ S.T)
    return np.stack(out)
