"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (library-chosen splits). The device generates every row; the
oracle regenerates, bit for bit, only the rows of the sampled (batch row,
KV head) units it checks, and computes their outputs in float64."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import LLAMA3_32_LAYERS, LLAMA3_LAYER_32K, LONG_CONTEXT_128K, PER_HEAD_RAGGED, SINGLE_HEAD_F32, host
from synth.device import KVGenerator
from tests.gpu_cases import build_case, rel_l2_rows, say, tolerance

pytestmark = pytest.mark.gpu


def _kv():
    import rank_compressed_kv_kvlr_amd as kv
    return kv


def _sample(cfg, n, salt):
    """Seeded (b, h) units to check."""
    g = np.random.default_rng(np.random.SeedSequence([7000 + cfg.cid, salt]))
    units = set()
    while len(units) < min(n, cfg.B * cfg.Hkv):
        units.add((int(g.integers(cfg.B)), int(g.integers(cfg.Hkv))))
    return sorted(units)


def _decode(case, q, lens):
    import torch
    kv = _kv()
    out = kv.decode_attn(case.desc, torch.from_numpy(q).cuda(), case.pk, case.pv, case.lat_k, case.lat_v,
                         torch.from_numpy(np.asarray(lens, np.int32)).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _check(case, got, q, lens, units):
    metric, bound = tolerance(case.cfg)
    G = case.cfg.G
    worst = 0.0
    for b, h in units:
        ref = case.reference(q, b, h, int(lens[b]))
        worst = max(worst, float(metric(got[b, h * G:(h + 1) * G], ref).max()))
    say(f"[full] {case.cfg.name} units={units} worst={worst:.3e} bound={bound}")
    assert worst <= bound, worst
    assert np.isfinite(got).all()
    return worst


def test_full_single_head_f32(gpu):
    cfg = SINGLE_HEAD_F32
    case = build_case(cfg)
    q = host.queries(cfg)
    lens = host.lengths(cfg)
    _check(case, _decode(case, q, lens), q, lens, [(0, 0)])


def test_full_llama3_layer_32k(gpu):
    cfg = LLAMA3_LAYER_32K
    case = build_case(cfg, chunk=8192)
    q = host.queries(cfg)
    lens = host.lengths(cfg)
    got = _decode(case, q, lens)
    _check(case, got, q, lens, _sample(cfg, 3, 0))
    # folded form on the same cache: q_lat = q P_K in, o_lat out
    import torch
    kv = _kv()
    q_lat = case.folded_queries(q)
    o_lat = kv.decode_attn_latent(case.desc, torch.from_numpy(q_lat).cuda(), case.lat_k, case.lat_v,
                                  torch.from_numpy(np.asarray(lens, np.int32)).cuda())
    torch.cuda.synchronize()
    o_lat = o_lat.cpu().numpy().astype(np.float64)
    metric, bound = tolerance(cfg)
    worst = 0.0
    for b, h in _sample(cfg, 2, 1):
        ref = case.reference_folded(q_lat, b, h, int(lens[b]))
        worst = max(worst, float(metric(o_lat[b, h * cfg.G:(h + 1) * cfg.G], ref).max()))
    say(f"[full] folded worst={worst:.3e} bound={bound}")
    assert worst <= bound, worst


def test_full_per_head_ranks_ragged(gpu):
    cfg = PER_HEAD_RAGGED
    case = build_case(cfg, chunk=4096)
    q = host.queries(cfg)
    lens = host.lengths(cfg)
    got = _decode(case, q, lens)
    rk, rv = host.ranks(cfg)
    units = _sample(cfg, 4, 0)
    # also the heads with the smallest and largest ranks
    units = sorted(set(units) | {(0, int(np.argmin(rk + rv))), (cfg.B - 1, int(np.argmax(rk + rv)))})
    _check(case, got, q, lens, units)


def test_full_long_context_prefill_and_64_steps(gpu):
    """Prefill-compress 131072 tokens, then 64 x (append one token, attend over all rows)."""
    import torch
    kv = _kv()
    cfg = LONG_CONTEXT_128K
    T = cfg.T
    case = build_case(cfg, n_rows=T, chunk=16384)
    gen = KVGenerator(cfg, 0)
    units = _sample(cfg, 2, 0)
    G = cfg.G
    # oracle state per sampled unit: the reconstructed prefill rows, extended per step
    ref_rows = {}
    for b, h in units:
        K = case.host_rows("k", b, h, T + cfg.decode_steps)
        V = case.host_rows("v", b, h, T + cfg.decode_steps)
        ref_rows[(b, h)] = (K, V)
    check_steps = {0, 31, cfg.decode_steps - 1}
    worst = 0.0
    for s in range(cfg.decode_steps):
        k_new = gen.make("k", cfg.B, 1, t0=T + s)[:, 0].contiguous()
        v_new = gen.make("v", cfg.B, 1, t0=T + s)[:, 0].contiguous()
        pos = torch.full((cfg.B,), T + s, dtype=torch.int32, device="cuda")
        kv.append(case.desc, k_new, v_new, pos, case.pk, case.pv, case.lat_k, case.lat_v)
        q = host.queries(cfg, 0, s)
        lens = np.full(cfg.B, T + s + 1, np.int32)
        got = _decode(case, q, lens)
        assert np.isfinite(got).all(), s
        if s in check_steps:
            for b, h in units:
                K, V = ref_rows[(b, h)]
                ref = oracle.decode_head_reconstructed(q[b, h * G:(h + 1) * G].astype(np.float64), K[:T + s + 1],
                                                       V[:T + s + 1], case.P32K[h], case.P32V[h], 1 / np.sqrt(cfg.d))
                err = float(rel_l2_rows(got[b, h * G:(h + 1) * G], ref).max())
                worst = max(worst, err)
                say(f"[full] step {s} unit {(b, h)} rel_l2={err:.3e}")
    assert worst <= 2e-2, worst


def test_full_32_layers(gpu):
    """All 32 layers, each with its own bases and (r_k, r_v) from the 50%-budget profile."""
    import torch
    cfg = LLAMA3_32_LAYERS
    prof = host.rank_profile(cfg)
    assert int(prof.sum()) == 4096
    worst = 0.0
    for layer in range(cfg.n_layers):
        case = build_case(cfg, layer=layer, chunk=2048)
        q = host.queries(cfg, layer)
        lens = host.lengths(cfg)
        got = _decode(case, q, lens)
        g = np.random.default_rng(np.random.SeedSequence([7004, layer]))
        units = [(int(g.integers(cfg.B)), int(g.integers(cfg.Hkv)))]
        worst = max(worst, _check(case, got, q, lens, units))
        del case
        torch.cuda.empty_cache()
    say(f"[full] 32 layers worst={worst:.3e}")
