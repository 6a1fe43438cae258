"""Builders shared by the GPU tests: a workload slice on the device (through
the C-ABI) and the oracle's float64 reference for any (batch row, KV head).

Inputs on both sides come from the seeded generator (synth): the device
draws bulk rows with its HIP twin, the host regenerates the same bits with
numpy for the rows the oracle checks. Nothing is copied from the GPU into
the oracle.
"""
from __future__ import annotations

import os
import sys
from dataclasses import dataclass, field

import numpy as np

import oracle
from synth import host
from synth.configs import Config


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bases32(P_list):
    """The fp32 bases the GPU receives, as float64 (oracle input)."""
    return [p.astype(np.float32).astype(np.float64) for p in P_list]


@dataclass
class Case:
    cfg: Config
    layer: int
    desc: object
    PK: list
    PV: list
    pk: object
    pv: object
    lat_k: object
    lat_v: object
    n_rows: int                  # rows written per (b, h): 0 .. n_rows-1
    stats: dict = field(default_factory=dict)

    @property
    def P32K(self):
        return bases32(self.PK)

    @property
    def P32V(self):
        return bases32(self.PV)

    def host_rows(self, kind: str, b: int, h: int, n: int, t0: int = 0) -> np.ndarray:
        """float64 values of K or V rows [n][d] of (b, h), exactly as the device holds its inputs."""
        enc = host.kv_rows(self.cfg, self.layer, kind, b, t0, n, heads=[h], stats=self.stats)
        return host.decode_to_f64(enc, self.cfg.in_dtype)[:, 0, :]

    def reference(self, q: np.ndarray, b: int, h: int, T: int) -> np.ndarray:
        """Oracle output [G][d] of query heads of KV head h for batch row b over rows t < T."""
        G = self.cfg.G
        K = self.host_rows("k", b, h, T)
        V = self.host_rows("v", b, h, T)
        return oracle.decode_head_reconstructed(q[b, h * G:(h + 1) * G].astype(np.float64), K, V,
                                                self.P32K[h], self.P32V[h], 1 / np.sqrt(self.cfg.d))

    def reference_storage_aware(self, q: np.ndarray, b: int, h: int, T: int) -> np.ndarray:
        """Oracle in latent order on latents rounded to the storage dtype (diagnostic)."""
        G = self.cfg.G
        lk = oracle.compress(self.host_rows("k", b, h, T), self.P32K[h])
        lv = oracle.compress(self.host_rows("v", b, h, T), self.P32V[h])
        if self.cfg.latent_dtype == "bf16":
            lk, lv = oracle.bf16_round(lk), oracle.bf16_round(lv)
        else:
            lk, lv = lk.astype(np.float32).astype(np.float64), lv.astype(np.float32).astype(np.float64)
        return oracle.decode_head_latent(q[b, h * G:(h + 1) * G].astype(np.float64), lk, lv,
                                         self.P32K[h], self.P32V[h], 1 / np.sqrt(self.cfg.d))


    def folded_queries(self, q: np.ndarray) -> np.ndarray:
        """q_lat [B][Hq][max r_k] float32 = q P_K per query head (the caller's folded query
        projection, formed on the host from the seeded queries); zero past a head's r_k."""
        cfg = self.cfg
        rk = [p.shape[1] for p in self.PK]
        out = np.zeros((q.shape[0], cfg.Hq, max(rk)), np.float32)
        for i in range(cfg.Hq):
            h = i // cfg.G
            out[:, i, :rk[h]] = (q[:, i].astype(np.float64) @ self.P32K[h]).astype(np.float32)
        return out

    def reference_folded(self, q_lat: np.ndarray, b: int, h: int, T: int) -> np.ndarray:
        """Oracle folded output [G][r_v(h)] for KV head h of batch row b over rows t < T."""
        G = self.cfg.G
        rk = self.PK[h].shape[1]
        lk = oracle.compress(self.host_rows("k", b, h, T), self.P32K[h])
        lv = oracle.compress(self.host_rows("v", b, h, T), self.P32V[h])
        return np.stack([oracle.attend_folded(q_lat[b, i, :rk].astype(np.float64), lk, lv, 1 / np.sqrt(self.cfg.d))
                         for i in range(h * G, (h + 1) * G)])


def dtype_code(kv, name):
    return kv.BF16 if name == "bf16" else kv.F32


def build_case(cfg: Config, layer: int = 0, n_rows: int = None, capacity: int = None, ranks=None,
               chunk: int = None, bases=None) -> Case:
    """Generate K, V on the device and prefill-compress rows 0..n_rows-1 of every (b, h).
    `bases` (per-head lists PK, PV of float64 [d][r] arrays) replaces the seeded bases."""
    import torch

    import rank_compressed_kv_kvlr_amd as kv
    from synth.device import KVGenerator

    rk, rv = host.ranks(cfg, layer) if ranks is None else ranks
    PK, PV = host.bases(cfg, layer) if bases is None else bases
    n_rows = cfg.capacity if n_rows is None else n_rows
    cap = cfg.capacity if capacity is None else capacity
    desc = kv.Desc(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cap, rk, rv, dtype_code(kv, cfg.in_dtype),
                   dtype_code(kv, cfg.latent_dtype))
    say(f"[case] cfg={cfg.name} B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} cap={cap} rows={n_rows} "
        f"rk={list(rk)} rv={list(rv)} in={cfg.in_dtype} lat={cfg.latent_dtype} layer={layer}")
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    lat_k, lat_v = kv.alloc_cache(desc)
    gen = KVGenerator(cfg, layer)
    chunk = chunk or n_rows
    for t0 in range(0, n_rows, chunk):
        n = min(chunk, n_rows - t0)
        K = gen.make("k", cfg.B, n, t0=t0)
        V = gen.make("v", cfg.B, n, t0=t0)
        kv.prefill_compress(desc, K, V, t0, pk, pv, lat_k, lat_v)
        del K, V
    torch.cuda.synchronize()
    return Case(cfg, layer, desc, PK, PV, pk, pv, lat_k, lat_v, n_rows, gen.stats)


def assert_latents_close(got: np.ndarray, X: np.ndarray, P: np.ndarray, dtype: str, exact_frac: float = 0.995):
    """Device latents vs the exact X P (float64).

    bf16: |got - XP| <= ulp_bf16(XP) + 2**-15 * (|X| |P|): one storage rounding
    plus the fp32 accumulation and the high/low basis residual, both bounded
    relative to the sum of absolute products; at least `exact_frac` of the
    entries must equal the correctly rounded value. fp32: the same without
    the storage rounding: n * 2**-24 with n = d <= 256 terms, i.e. 2**-16.
    """
    exact = X @ P
    mag = np.abs(X) @ np.abs(P)
    if dtype == "bf16":
        ulp = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
        bad = np.abs(got - exact) > ulp + mag * 2.0 ** -15
        assert not bad.any(), f"{bad.sum()} latents off by more than one rounding"
        frac = float(np.mean(got == oracle.bf16_round(exact)))
        assert frac >= exact_frac, frac
    else:
        bad = np.abs(got - exact) > mag * 2.0 ** -16
        assert not bad.any(), f"{bad.sum()} latents off"


def rel_l2_rows(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row ||o - o*||_2 / ||o*||_2 over the last axis."""
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return num / np.maximum(den, 1e-300)


def rel_inf_rows(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row max|o - o*| / max|o*| over the last axis."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-300)


def tolerance(cfg: Config):
    """Acceptance metric and bound: fp32 latents 1e-5 (row inf-norm), bf16 latents 2e-2 (row L2)."""
    if cfg.latent_dtype == "f32":
        return rel_inf_rows, 1e-5
    return rel_l2_rows, 2e-2


# ---------------------------------------------------------------------------
# float64 references in worker processes. Regenerating the checked rows on the
# host dominates the full-size checks, so (batch row, KV head) units go to a
# pool of spawned workers (one BLAS thread each); the oracle is called as is.
# ---------------------------------------------------------------------------
def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def oracle_pool(max_workers: int = 16):
    """A process pool for unit references, sized to the host's CPUs (at most max_workers)."""
    import multiprocessing as mp
    n = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    return mp.get_context("spawn").Pool(n, initializer=_one_blas_thread)


def _rows_f64(cfg: Config, layer: int, kind: str, b: int, h: int, n: int) -> np.ndarray:
    return host.decode_to_f64(host.kv_rows(cfg, layer, kind, b, 0, n, heads=[h]), cfg.in_dtype)[:, 0, :]


def unit_reference(job):
    """Oracle output [G][d] of the query heads q_heads [G][d] of KV head h, batch row b,
    over rows t < T (definition order, float64)."""
    cfg, layer, b, h, T, q_heads, PK, PV, scale = job
    K = _rows_f64(cfg, layer, "k", b, h, T)
    V = _rows_f64(cfg, layer, "v", b, h, T)
    return oracle.decode_head_reconstructed(np.asarray(q_heads, np.float64), K, V, PK, PV, scale)


def unit_reference_folded(job):
    """Oracle folded output [G][r_v]: q_lat [G][r_k] in, o_lat out, over rows t < T."""
    cfg, layer, b, h, T, q_lat, PK, PV, scale = job
    lk = oracle.compress(_rows_f64(cfg, layer, "k", b, h, T), PK)
    lv = oracle.compress(_rows_f64(cfg, layer, "v", b, h, T), PV)
    return np.stack([oracle.attend_folded(np.asarray(qi, np.float64), lk, lv, scale) for qi in q_lat])


def unit_reference_steps(job):
    """Oracle outputs [S][G][d] of S decode steps of KV head h, batch row b: step s attends
    over rows t < T0 + s + 1 (the prefill rows and the tokens appended up to step s) with
    its own queries q_steps[s] [G][d]. The rows are reconstructed once (definition order)."""
    cfg, layer, b, h, T0, q_steps, PK, PV, scale = job
    S = len(q_steps)
    Kt = oracle.reconstruct(oracle.compress(_rows_f64(cfg, layer, "k", b, h, T0 + S), PK), PK)
    Vt = oracle.reconstruct(oracle.compress(_rows_f64(cfg, layer, "v", b, h, T0 + S), PV), PV)
    return np.stack([np.stack([oracle.attend(np.asarray(qi, np.float64), Kt[:T0 + s + 1], Vt[:T0 + s + 1], scale)
                               for qi in q_steps[s]]) for s in range(S)])

