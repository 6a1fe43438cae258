"""50-digit brute force of reconstructed attention on tiny shapes (test oracle).

Test infrastructure only. Scalar loops in mpmath, no numpy arithmetic, so
that it checks the float64 oracle from outside: every sum is written out
element by element from the definition (StiefAttention technical summary,
"Mecanismo Central" item 5: latents K P_K, reconstruction before attention).
"""
from __future__ import annotations

import mpmath

mpmath.mp.dps = 50


def _mp(x):
    return mpmath.mpf(float(x))


def attend_brute(q, K, V, P_K, P_V, scale):
    """One query vector over one KV head; inputs are nested sequences of floats.

    Returns a list of d mpmath numbers.
    """
    T = len(K)
    d = len(P_K)
    r_k = len(P_K[0]) if d else 0
    r_v = len(P_V[0]) if d else 0
    if T == 0:
        return [mpmath.mpf(0)] * d
    # reconstructed rows
    Kt, Vt = [], []
    for t in range(T):
        kl = [mpmath.fsum(_mp(K[t][i]) * _mp(P_K[i][j]) for i in range(d)) for j in range(r_k)]
        vl = [mpmath.fsum(_mp(V[t][i]) * _mp(P_V[i][j]) for i in range(d)) for j in range(r_v)]
        Kt.append([mpmath.fsum(kl[j] * _mp(P_K[i][j]) for j in range(r_k)) for i in range(d)])
        Vt.append([mpmath.fsum(vl[j] * _mp(P_V[i][j]) for j in range(r_v)) for i in range(d)])
    s = [mpmath.fsum(Kt[t][i] * _mp(q[i]) for i in range(d)) * _mp(scale) for t in range(T)]
    w = [mpmath.exp(x) for x in s]          # no shift needed at 50 digits for tiny scores
    Z = mpmath.fsum(w)
    return [mpmath.fsum(w[t] * Vt[t][i] for t in range(T)) / Z for i in range(d)]


def decode_brute(q, K, V, P_K, P_V, lens, scale):
    """Batch version: q [B][Hq][d], K/V [B][T][Hkv][d], per-head P lists, lens [B]."""
    B, Hq = len(q), len(q[0])
    Hkv = len(P_K)
    G = Hq // Hkv
    out = []
    for b in range(B):
        row = []
        for i in range(Hq):
            h = i // G
            T = int(lens[b])
            Kb = [[K[b][t][h][c] for c in range(len(K[b][t][h]))] for t in range(T)]
            Vb = [[V[b][t][h][c] for c in range(len(V[b][t][h]))] for t in range(T)]
            row.append(attend_brute(q[b][i], Kb, Vb, P_K[h], P_V[h], scale))
        out.append(row)
    return out


def decode_joint_brute(q, K, V, P_K, P_J, lens, scale):
    """Joint values (STAR-KV technical summary, "Metodologia" section 2): the values of
    all heads of a token concatenated, V_lat = V_all P_J, head h reconstructed with rows
    h d .. (h+1) d - 1 of P_J. Keys per head as in decode_brute. Nested lists in, mpmath out."""
    B, Hq = len(q), len(q[0])
    Hkv = len(P_K)
    G = Hq // Hkv
    d = len(P_K[0])
    r = len(P_J[0])
    out = []
    for b in range(B):
        T = int(lens[b])
        vlat = [[mpmath.fsum(_mp(V[b][t][hh][c]) * _mp(P_J[hh * d + c][j]) for hh in range(Hkv) for c in range(d))
                 for j in range(r)] for t in range(T)]
        row = []
        for i in range(Hq):
            h = i // G
            if T == 0:
                row.append([mpmath.mpf(0)] * d)
                continue
            rk = len(P_K[h][0])
            Kt = []
            for t in range(T):
                kl = [mpmath.fsum(_mp(K[b][t][h][c]) * _mp(P_K[h][c][j]) for c in range(d)) for j in range(rk)]
                Kt.append([mpmath.fsum(kl[j] * _mp(P_K[h][c][j]) for j in range(rk)) for c in range(d)])
            Vt = [[mpmath.fsum(vlat[t][j] * _mp(P_J[h * d + c][j]) for j in range(r)) for c in range(d)]
                  for t in range(T)]
            s = [mpmath.fsum(Kt[t][c] * _mp(q[b][i][c]) for c in range(d)) * _mp(scale) for t in range(T)]
            w = [mpmath.exp(x) for x in s]
            Z = mpmath.fsum(w)
            row.append([mpmath.fsum(w[t] * Vt[t][c] for t in range(T)) / Z for c in range(d)])
        out.append(row)
    return out
