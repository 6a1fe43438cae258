"""The seeded input generator (CPU only): determinism, slicing, published definitions."""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

from synth import LLAMA3_32_LAYERS, LLAMA3_LAYER_32K, LONG_CONTEXT_128K, PER_HEAD_RAGGED, WORKLOADS, host


def _exact_bf16(x: float) -> float:
    """Nearest bf16 of x by exact rational comparison (ties to even)."""
    if x == 0:
        return 0.0
    f = Fraction(x)
    e = np.frexp(x)[1]
    ulp = Fraction(2) ** (int(e) - 8)
    lo = (f / ulp).__floor__() * ulp
    hi = lo + ulp
    if f - lo < hi - f:
        return float(lo)
    if hi - f < f - lo:
        return float(hi)
    return float(lo) if (lo / ulp) % 2 == 0 else float(hi)


def test_splitmix_vector_matches_scalar_definition():
    key = host.stream_key(LLAMA3_LAYER_32K, 3, host.KIND_K)
    n = np.array([1, 2, 3, 1000, 2 ** 40 + 7], dtype=np.uint64)
    vec = host.word(key, n)
    ref = [host.mix64_scalar(key + int(i) * host.GAMMA) for i in n]
    assert [int(v) for v in vec] == ref


def test_irwin_hall_values_exact_and_moments():
    z = host.irwin_hall_z(12345, np.arange(400000))
    assert np.all(z * 65536 == np.round(z * 65536)) and np.abs(z).max() < 6
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1.0) < 0.01


def test_bf16_encoder_is_exact_nearest_even():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(3000) * 10.0 ** rng.integers(-10, 10, 3000)
    got = host.bf16_bits_to_f64(host.bf16_bits_from_f64(x))
    ref = np.array([_exact_bf16(float(v)) for v in x])
    assert np.array_equal(got, ref)
    # float32-representable inputs agree with torch's conversion as well
    x32 = x.astype(np.float32)
    t = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(host.bf16_bits_from_f64(x32.astype(np.float64)), t)


def test_slices_regenerate_identically():
    cfg = LONG_CONTEXT_128K.scaled(T=64)
    full = host.kv_values_f64(cfg, 0, "k", 1, 0, 40)
    part = host.kv_values_f64(cfg, 0, "k", 1, 17, 9, heads=[2, 5])
    assert np.array_equal(full[17:26][:, [2, 5]], part)
    assert np.array_equal(host.kv_rows(cfg, 0, "v", 0, 3, 5), host.kv_rows(cfg, 0, "v", 0, 3, 5))
    # different batch rows, layers, kinds and workloads draw different values
    assert not np.array_equal(host.kv_values_f64(cfg, 0, "k", 0, 0, 4), host.kv_values_f64(cfg, 0, "k", 1, 0, 4))
    assert not np.array_equal(host.kv_values_f64(cfg, 0, "k", 0, 0, 4), host.kv_values_f64(cfg, 1, "k", 0, 0, 4))
    assert not np.array_equal(host.kv_values_f64(cfg, 0, "k", 0, 0, 4), host.kv_values_f64(cfg, 0, "v", 0, 0, 4))


def test_channel_statistics_and_outliers():
    cfg = LLAMA3_LAYER_32K
    st = host.kv_stats(cfg, 0)
    x = host.kv_values_f64(cfg, 0, "v", 0, 0, 20000, heads=[3], stats=st)[:, 0, :]
    assert np.allclose(x.mean(0), st["mu_v"][3], atol=0.06)
    assert np.allclose(x.std(0), st["sigma_v"][3], rtol=0.03)
    assert np.all((st["mult_k"] == 8).sum(1) == 4) and np.all(st["mult_v"] == 1)
    assert np.all((st["sigma_k"] >= 0.5) & (st["sigma_k"] <= 2))


@pytest.mark.parametrize("wl", ["single_head_f32", "llama3_8b_layer_32k", "per_head_ranks_ragged", "long_context_128k"])
def test_bases_orthonormal(wl):
    cfg = WORKLOADS[wl]
    PK, PV = host.bases(cfg)
    rk, rv = host.ranks(cfg)
    for h in range(cfg.Hkv):
        for P, r in ((PK[h], rk[h]), (PV[h], rv[h])):
            assert P.shape == (cfg.d, r)
            assert np.abs(P.T @ P - np.eye(r)).max() <= 1e-10
            P32 = P.astype(np.float32).astype(np.float64)
            assert np.abs(P32.T @ P32 - np.eye(r)).max() <= 1e-6


def test_rank_tables():
    rk, rv = host.ranks(PER_HEAD_RAGGED)
    assert set(rk) | set(rv) <= set(PER_HEAD_RAGGED.rank_choices)
    prof = host.rank_profile(LLAMA3_32_LAYERS)
    assert prof.shape == (32, 2) and prof.sum() == 4096
    assert np.all(prof % 16 == 0) and prof.min() >= 16 and prof.max() <= 128
    lens = host.lengths(PER_HEAD_RAGGED)
    assert lens.min() >= 4096 and lens.max() <= 16384 and len(lens) == 16


def test_queries_fresh_per_step():
    cfg = LONG_CONTEXT_128K
    a, b = host.queries(cfg, 0, 0), host.queries(cfg, 0, 1)
    assert a.dtype == np.float32 and a.shape == (2, 32, 128) and not np.array_equal(a, b)
