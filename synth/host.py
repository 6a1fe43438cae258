"""Host-side (numpy) seeded draws for the synthetic workloads.

Small arrays (queries, bases, rank tables, lengths, per-channel statistics,
outlier channels) are drawn with ``numpy.random.default_rng`` on a
``SeedSequence`` keyed by (1000 + workload id, layer, batch row, head, kind,
extra), one independent stream per slice, so any slice can be regenerated
alone.

Bulk key/value rows use a counter-based generator so that a slice can be
regenerated without generating everything before it, and so that the HIP
kernel in ``csrc/synth_gen.hip`` can produce the same bits on the GPU:

* word(key, n) = SplitMix64 output for state ``key + n * 0x9E3779B97F4A7C15``
  (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014: the mixing function with constants 0xBF58476D1CE4E5B9 and
  0x94D049BB133111EB and shifts 30, 27, 31);
* element e takes words 3e+1, 3e+2, 3e+3, i.e. twelve 16-bit uniforms u_k,
  and z = (sum u_k - 6 * 65536) / 65536, the Irwin-Hall sum of twelve
  uniforms, a zero-mean unit-variance stand-in for N(0, 1) that both sides
  compute exactly (every z is a multiple of 2**-16 below 6 in magnitude);
* x = mu_j + sigma_j * z in float64 with two separate roundings (no fused
  multiply-add), then x * outlier_multiplier (1 or 8, exact), then the
  storage encoding: float32 by round-to-nearest-even, or bf16 by
  round-to-nearest-even taken directly from float64.

The element counter of key/value row (b, t, h, j) is
``(((b << 20) | t) * Hkv + h) * d + j``, independent of the cache length, so
appended tokens continue the prefill sequence.
"""
from __future__ import annotations

import numpy as np

from .configs import Config

# kinds of seeded streams
KIND_PK, KIND_PV, KIND_KSTAT, KIND_VSTAT, KIND_K, KIND_V, KIND_Q = 0, 1, 2, 3, 4, 5, 6
KIND_OUTLIER, KIND_RANKS, KIND_LENGTHS = 7, 8, 9
KIND_PJ = 10

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1
T_BITS = 20          # token field width in the element counter
MAX_T = 1 << T_BITS


def seed_sequence(cfg: Config, layer: int, b: int, h: int, kind: int, extra: int = 0):
    return np.random.SeedSequence([1000 + cfg.cid, layer, b, h, kind, extra])


def rng(cfg: Config, layer: int, b: int, h: int, kind: int, extra: int = 0):
    return np.random.default_rng(seed_sequence(cfg, layer, b, h, kind, extra))


# --------------------------------------------------------------------------
# counter-based generator (host twin of csrc/synth_gen.hip)
# --------------------------------------------------------------------------
def mix64_scalar(z: int) -> int:
    """SplitMix64 output mixing on a Python int (reference for the vector form)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def stream_key(cfg: Config, layer: int, kind: int) -> int:
    """64-bit key of the bulk stream for (workload, layer, kind)."""
    return mix64_scalar(((1000 + cfg.cid) << 40) ^ (layer << 16) ^ kind)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
    return z ^ (z >> np.uint64(31))


def word(key: int, n: np.ndarray) -> np.ndarray:
    """SplitMix64 word n (n >= 1) of the stream with the given key."""
    n = np.asarray(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(key) + n * np.uint64(GAMMA)
        return _mix64(state)


def irwin_hall_z(key: int, e: np.ndarray) -> np.ndarray:
    """The generator's unit normal stand-in for element counters e (float64, exact)."""
    e = np.asarray(e, dtype=np.uint64)
    total = np.zeros(e.shape, dtype=np.int64)
    with np.errstate(over="ignore"):
        for k in range(3):
            w = word(key, e * np.uint64(3) + np.uint64(k + 1))
            for s in (0, 16, 32, 48):
                total += ((w >> np.uint64(s)) & np.uint64(0xFFFF)).astype(np.int64)
    return (total - 6 * 65536).astype(np.float64) * (1.0 / 65536.0)


def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 (nearest, ties to even) directly; returns uint16 bits.

    Finite inputs in the bf16 normal range (or zero) only.
    """
    u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    with np.errstate(over="ignore"):
        r = (u + np.uint64((1 << 44) - 1) + lsb) & np.uint64(~((1 << 45) - 1) & MASK64)
    f32 = r.view(np.float64).astype(np.float32)       # exact: r holds 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# small seeded arrays
# --------------------------------------------------------------------------
def ranks(cfg: Config, layer: int = 0):
    """Per-KV-head ranks (r_k[Hkv], r_v[Hkv]) as int32 arrays."""
    H = cfg.Hkv
    if cfg.rank_mode == "uniform":
        return np.full(H, cfg.r_k, np.int32), np.full(H, cfg.r_v, np.int32)
    if cfg.rank_mode == "per_head":
        g = rng(cfg, 0, 0, 0, KIND_RANKS)
        choices = np.asarray(cfg.rank_choices, dtype=np.int32)
        rk = g.choice(choices, size=H)
        rv = g.choice(choices, size=H)
        return rk.astype(np.int32), rv.astype(np.int32)
    if cfg.rank_mode == "per_layer_profile":
        prof = rank_profile(cfg)
        return np.full(H, prof[layer, 0], np.int32), np.full(H, prof[layer, 1], np.int32)
    raise ValueError(cfg.rank_mode)


def rank_profile(cfg: Config) -> np.ndarray:
    """Per-layer (r_k, r_v) profile [n_layers][2] under a fixed total budget.

    Start from profile_start everywhere, then apply profile_moves seeded moves
    of +step to one slot and -step to another, skipping moves that would
    leave [lo, hi]. The sum over all slots never changes.
    """
    g = rng(cfg, 0, 0, 0, KIND_RANKS)
    lo, hi = cfg.profile_bounds
    step = cfg.profile_step
    r = np.full(2 * cfg.n_layers, cfg.profile_start, dtype=np.int64)
    for _ in range(cfg.profile_moves):
        a, b = g.choice(r.size, size=2, replace=False)
        if r[a] + step <= hi and r[b] - step >= lo:
            r[a] += step
            r[b] -= step
    return r.reshape(cfg.n_layers, 2).astype(np.int32)


def lengths(cfg: Config) -> np.ndarray:
    """Cached length T_b of each batch row (before any decode step)."""
    if cfg.T is not None:
        return np.full(cfg.B, cfg.T, np.int32)
    lo, hi = cfg.T_range
    g = rng(cfg, 0, 0, 0, KIND_LENGTHS)
    return g.integers(lo, hi, endpoint=True, size=cfg.B).astype(np.int32)


def joint_value_basis(cfg: Config, r: int, layer: int = 0):
    """Orthonormal joint value basis [Hkv d][r]: Q factor of QR of a seeded Gaussian."""
    A = rng(cfg, layer, 0, 0, KIND_PJ).standard_normal((cfg.Hkv * cfg.d, int(r)))
    Q, _ = np.linalg.qr(A)
    return Q


def bases(cfg: Config, layer: int = 0):
    """Orthonormal bases per KV head: Q factor of QR of a seeded Gaussian d x r.

    Returns (P_K, P_V): lists over heads of float64 [d][r] arrays.
    """
    rk, rv = ranks(cfg, layer)
    PK, PV = [], []
    for h in range(cfg.Hkv):
        for kind, r, out in ((KIND_PK, rk[h], PK), (KIND_PV, rv[h], PV)):
            A = rng(cfg, layer, 0, h, kind).standard_normal((cfg.d, int(r)))
            Q, _ = np.linalg.qr(A)
            out.append(Q)
    return PK, PV


def kv_stats(cfg: Config, layer: int = 0):
    """Per-channel (mu, sigma) of keys and values and the key outlier multiplier.

    mu_j ~ N(0, variance 0.5), sigma_j ~ U(0.5, 2) per (layer, KV head, K or V).
    Returns dict of float64 [Hkv][d] arrays: mu_k, sigma_k, mu_v, sigma_v, mult_k, mult_v.
    """
    H, d = cfg.Hkv, cfg.d
    out = {n: np.zeros((H, d)) for n in ("mu_k", "sigma_k", "mu_v", "sigma_v")}
    out["mult_k"] = np.ones((H, d))
    out["mult_v"] = np.ones((H, d))
    for h in range(H):
        for kind, tag in ((KIND_KSTAT, "k"), (KIND_VSTAT, "v")):
            g = rng(cfg, layer, 0, h, kind)
            out["mu_" + tag][h] = g.normal(0.0, np.sqrt(0.5), d)
            out["sigma_" + tag][h] = g.uniform(0.5, 2.0, d)
        if cfg.n_outliers:
            ch = rng(cfg, layer, 0, h, KIND_OUTLIER).choice(d, size=cfg.n_outliers, replace=False)
            out["mult_k"][h, ch] = cfg.outlier_scale
    return out


def queries(cfg: Config, layer: int = 0, step: int = 0) -> np.ndarray:
    """q ~ N(0, 1), float32 [B][Hq][d]; a fresh draw per (layer, decode step)."""
    g = rng(cfg, layer, 0, 0, KIND_Q, step)
    return g.standard_normal((cfg.B, cfg.Hq, cfg.d)).astype(np.float32)


# --------------------------------------------------------------------------
# bulk key/value rows
# --------------------------------------------------------------------------
def kv_values_f64(cfg: Config, layer: int, kind: str, b: int, t0: int, n: int,
                  heads=None, stats=None) -> np.ndarray:
    """Pre-encoding float64 values x[t][h][j] for tokens t0..t0+n of batch row b."""
    assert kind in ("k", "v")
    assert 0 <= t0 and t0 + n <= MAX_T
    heads = list(range(cfg.Hkv)) if heads is None else list(heads)
    stats = kv_stats(cfg, layer) if stats is None else stats
    key = stream_key(cfg, layer, KIND_K if kind == "k" else KIND_V)
    d, H = cfg.d, cfg.Hkv
    t = np.arange(t0, t0 + n, dtype=np.uint64)[:, None, None]
    hh = np.asarray(heads, dtype=np.uint64)[None, :, None]
    jj = np.arange(d, dtype=np.uint64)[None, None, :]
    e = (((np.uint64(b) << np.uint64(T_BITS)) | t) * np.uint64(H) + hh) * np.uint64(d) + jj
    z = irwin_hall_z(key, e)
    mu = stats["mu_" + kind][heads][None]
    sg = stats["sigma_" + kind][heads][None]
    ml = stats["mult_" + kind][heads][None]
    prod = sg * z
    x = mu + prod
    return x * ml


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage encoding of generated values: float32 array or uint16 bf16 bits."""
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f64(x)
    raise ValueError(dtype)


def decode_to_f64(enc: np.ndarray, dtype: str) -> np.ndarray:
    """float64 value of an encoded array (the exact value the GPU receives)."""
    if dtype == "f32":
        return enc.astype(np.float64)
    return bf16_bits_to_f64(enc)


def kv_rows(cfg: Config, layer: int, kind: str, b: int, t0: int, n: int, heads=None, stats=None):
    """Encoded key or value rows [n][len(heads)][d] exactly as the GPU generator writes them."""
    return encode(kv_values_f64(cfg, layer, kind, b, t0, n, heads, stats), cfg.in_dtype)
