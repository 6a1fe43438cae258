"""GPU parity of the mixed 4/3-bit latent storage (block-wise Hadamard folded into
the bases, 4-bit outlier and 3-bit inlier blocks per token) against oracle/quant.py."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import quant as qo
from synth import CONFIGS, host
from synth.device import KVGenerator
from tests.gpu_cases import bases32, say

pytestmark = pytest.mark.gpu


def _kv():
    import rank_compressed_kv_kvlr_amd as kv
    return kv


def _rows_bytes(kv, desc, lat, which, b, h, n):
    return kv.latent_rows(lat, desc, which, b, h)[:n].cpu().numpy()


def test_hadamard_fold_matches_oracle(gpu):
    import torch
    kv = _kv()
    rng = np.random.default_rng(41)
    rk, rv = [16, 48, 64, 128], [32, 80, 112, 16]
    d = 128
    PK = [rng.standard_normal((d, r)) for r in rk]
    PV = [rng.standard_normal((d, r)) for r in rv]
    desc = kv.Desc(2, 8, 4, d, 64, rk, rv, kv.BF16, kv.Q43)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    ok, ov = torch.empty_like(pk), torch.empty_like(pv)
    kv.hadamard_bases(desc, pk, pv, ok, ov)
    kv.hadamard_bases(desc, pk, pv)            # in place
    torch.cuda.synchronize()
    assert torch.equal(ok, pk) and torch.equal(ov, pv)
    got_k, got_v = ok.cpu().numpy().astype(np.float64), ov.cpu().numpy().astype(np.float64)
    ref_k = np.concatenate([qo.fuse_bases(P).ravel() for P in bases32(PK)])
    ref_v = np.concatenate([qo.fuse_bases(P).ravel() for P in bases32(PV)])
    # 16-term fp32 sums of values of magnitude ~1: a few ulps
    assert np.abs(got_k - ref_k).max() <= 4e-6 * np.abs(ref_k).max()
    assert np.abs(got_v - ref_v).max() <= 4e-6 * np.abs(ref_v).max()


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_quantised_rows_bit_exact_on_exact_latents(gpu, in_dtype):
    """Integer inputs and bases with entries +-1/16 make every fp32 latent exact, so the
    stored bytes must equal the oracle's byte for byte (compression and append)."""
    import torch
    kv = _kv()
    rng = np.random.default_rng(42)
    B, Hkv, d, T, cap = 2, 3, 128, 150, 160
    rk, rv = [16, 64, 48], [128, 32, 80]
    PK = [rng.choice([-1 / 16, 1 / 16], size=(d, r)) for r in rk]
    PV = [rng.choice([-1 / 16, 1 / 16], size=(d, r)) for r in rv]
    K = rng.integers(-8, 9, size=(B, T, Hkv, d)).astype(np.float32)
    V = rng.integers(-8, 9, size=(B, T, Hkv, d)).astype(np.float32)
    code = kv.BF16 if in_dtype == "bf16" else kv.F32
    tdt = torch.bfloat16 if in_dtype == "bf16" else torch.float32
    desc = kv.Desc(B, Hkv, Hkv, d, cap, rk, rv, code, kv.Q43)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    lk, lv = kv.alloc_cache(desc)
    Kd, Vd = torch.from_numpy(K).to(tdt).cuda(), torch.from_numpy(V).to(tdt).cuda()
    kv.prefill_compress(desc, Kd[:, :T - 1].contiguous(), Vd[:, :T - 1].contiguous(), 0, pk, pv, lk, lv)
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    kv.append(desc, Kd[:, T - 1].contiguous(), Vd[:, T - 1].contiguous(), pos, pk, pv, lk, lv)
    torch.cuda.synchronize()
    for which, X, P, ranks in (("k", K, PK, rk), ("v", V, PV, rv)):
        for b in range(B):
            for h in range(Hkv):
                lat = (X[b, :, h, :].astype(np.float64) @ P[h]).astype(np.float32)
                assert np.array_equal(lat.astype(np.float64), X[b, :, h, :].astype(np.float64) @ P[h])
                want = np.stack([qo.pack_row(*qo.quantize_row(lat[t]), ranks[h]) for t in range(T)])
                got = _rows_bytes(kv, desc, lk if which == "k" else lv, which, b, h, T)
                bad = np.argwhere(got != want)
                assert bad.size == 0, f"{which} b={b} h={h} r={ranks[h]} first mismatches {bad[:5]}"
    say(f"[q43] bit-exact rows ({in_dtype} inputs)")


def test_quantised_compression_matches_oracle(gpu):
    """Realistic rows (llama-shaped workload, folded QR bases): every stored value is within
    one quantisation step of the oracle's, and almost every code is identical."""
    import torch
    kv = _kv()
    cfg = CONFIGS[2].scaled(B=2, T_range=(300, 300))
    rk, rv = host.ranks(cfg)
    PK, PV = host.bases(cfg)
    desc = kv.Desc(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.capacity, rk, rv, kv.BF16, kv.Q43)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    kv.hadamard_bases(desc, pk, pv)
    lk, lv = kv.alloc_cache(desc)
    gen = KVGenerator(cfg, 0)
    T = 300
    kv.prefill_compress(desc, gen.make("k", cfg.B, T), gen.make("v", cfg.B, T), 0, pk, pv, lk, lv)
    torch.cuda.synchronize()
    stats = host.kv_stats(cfg, 0)
    n_codes = n_same = 0
    for which, P, ranks, lat in (("k", PK, rk, lk), ("v", PV, rv, lv)):
        for b in range(cfg.B):
            for h in range(cfg.Hkv):
                X = host.decode_to_f64(host.kv_rows(cfg, 0, which, b, 0, T, heads=[h], stats=stats), "bf16")[:, 0]
                Pf = qo.fuse_bases(bases32([P[h]])[0])
                lat32 = (X @ Pf).astype(np.float32)
                raw = _rows_bytes(kv, desc, lat, which, b, h, T)
                r = int(ranks[h])
                for t in range(T):
                    gc, gm = qo.unpack_row(raw[t], r)
                    wc, wm = qo.quantize_row(lat32[t], r)
                    g = qo.dequantize_row(gc, gm, r)
                    w = qo.dequantize_row(wc, wm, r)
                    step = max(float(wm[0]), float(wm[2]))
                    assert np.abs(g - w).max() <= 1.01 * step + 1e-3 * np.abs(w).max(), (which, b, h, t)
                    n_codes += r
                    n_same += int((gc == wc).sum())
    frac = n_same / n_codes
    say(f"[q43] identical codes {frac:.6f}")
    assert frac >= 0.999, frac
