"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (library-chosen plans). The device generates every row; the
oracle regenerates, bit for bit, only the rows of the (batch row, KV head)
units it checks, and computes their outputs in float64 (in a pool of worker
processes: the host regeneration dominates).

Coverage per workload:
  single_head_f32        the one unit
  llama3_8b_layer_32k    16 of the 64 units, and 8 units of the folded entry point
  per_head_ranks_ragged  16 units plus the heads with the smallest and largest ranks
  long_context_128k      4 units at every one of the 64 steps, as two calls (append,
                         decode) and as the fused step
  llama3_8b_32_layers    every layer: 4 seeded batch rows x all 8 KV heads
"""
from __future__ import annotations

import numpy as np
import pytest

from synth import LLAMA3_32_LAYERS, LLAMA3_LAYER_32K, LONG_CONTEXT_128K, PER_HEAD_RAGGED, SINGLE_HEAD_F32, host
from synth.device import KVGenerator
from tests.gpu_cases import (build_case, oracle_pool, say, tolerance, unit_reference, unit_reference_folded,
                             unit_reference_steps)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


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


def _jobs(case, q, lens, units):
    G, scale = case.cfg.G, 1 / np.sqrt(case.cfg.d)
    return [(case.cfg, case.layer, b, h, int(lens[b]), q[b, h * G:(h + 1) * G].astype(np.float64),
             case.P32K[h], case.P32V[h], scale) for b, h in units]


def _compare(cfg, got, units, refs, label):
    metric, bound = tolerance(cfg)
    G = cfg.G
    errs = [float(metric(got[b, h * G:(h + 1) * G], ref).max()) for (b, h), ref in zip(units, refs)]
    worst = max(errs)
    say(f"[full] {label} units={len(units)} worst={worst:.3e} median={float(np.median(errs)):.3e} bound={bound}")
    assert worst <= bound, worst
    return worst


def test_full_single_head_f32(gpu):
    cfg = SINGLE_HEAD_F32
    case = build_case(cfg)
    q = host.queries(cfg)
    lens = host.lengths(cfg)
    got = _decode(case, q, lens)
    units = [(0, 0)]
    _compare(cfg, got, units, [unit_reference(j) for j in _jobs(case, q, lens, units)], cfg.name)
    assert np.isfinite(got).all()


def test_full_llama3_layer_32k(gpu):
    import torch
    kv = _kv()
    cfg = LLAMA3_LAYER_32K
    case = build_case(cfg, chunk=8192)
    q = host.queries(cfg)
    lens = host.lengths(cfg)
    units = _sample(cfg, 16, 0)
    funits = _sample(cfg, 8, 1)
    q_lat = case.folded_queries(q)
    G, scale = cfg.G, 1 / np.sqrt(cfg.d)
    fjobs = [(cfg, 0, b, h, int(lens[b]), q_lat[b, h * G:(h + 1) * G, :int(case.PK[h].shape[1])].astype(np.float64),
              case.P32K[h], case.P32V[h], scale) for b, h in funits]
    with oracle_pool() as pool:
        pending = pool.map_async(unit_reference, _jobs(case, q, lens, units))
        fpending = pool.map_async(unit_reference_folded, fjobs)
        got = _decode(case, q, lens)
        assert np.isfinite(got).all()
        # folded form on the same cache: q_lat = q P_K in, o_lat out
        o_lat = kv.decode_attn_latent(case.desc, torch.from_numpy(q_lat).cuda(), case.lat_k, case.lat_v,
                                      torch.from_numpy(np.asarray(lens, np.int32)).cuda())
        torch.cuda.synchronize()
        o_lat = o_lat.cpu().numpy().astype(np.float64)
        refs, frefs = pending.get(), fpending.get()
    _compare(cfg, got, units, refs, cfg.name)
    _compare(cfg, o_lat, funits, frefs, cfg.name + " folded")


def test_full_per_head_ranks_ragged(gpu):
    cfg = PER_HEAD_RAGGED
    case = build_case(cfg, chunk=4096)
    q = host.queries(cfg)
    lens = host.lengths(cfg)
    rk, rv = host.ranks(cfg)
    units = _sample(cfg, 16, 0)
    # also the heads with the smallest and largest ranks
    units = sorted(set(units) | {(0, int(np.argmin(rk + rv))), (cfg.B - 1, int(np.argmax(rk + rv)))})
    with oracle_pool() as pool:
        pending = pool.map_async(unit_reference, _jobs(case, q, lens, units))
        got = _decode(case, q, lens)
        refs = pending.get()
    assert np.isfinite(got).all()
    _compare(cfg, got, units, refs, cfg.name)


def test_full_long_context_prefill_and_64_steps(gpu):
    """Prefill-compress 131072 tokens, then 64 x (append one token, attend over all rows), as two
    calls and as the fused step; 4 units checked at every step of both."""
    import torch
    kv = _kv()
    cfg = LONG_CONTEXT_128K
    T, S, G = cfg.T, cfg.decode_steps, cfg.G
    units = _sample(cfg, 4, 0)
    q_steps = [host.queries(cfg, 0, s) for s in range(S)]
    scale = 1 / np.sqrt(cfg.d)
    case = build_case(cfg, n_rows=T, chunk=16384)
    jobs = [(cfg, 0, b, h, T, np.stack([q_steps[s][b, h * G:(h + 1) * G] for s in range(S)]).astype(np.float64),
             case.P32K[h], case.P32V[h], scale) for b, h in units]
    gen = KVGenerator(cfg, 0)
    ws = kv.alloc_workspace(case.desc)
    outs = {"two_calls": [], "fused": []}
    with oracle_pool() as pool:
        pending = pool.map_async(unit_reference_steps, jobs)
        # both passes write rows T .. T+S-1 with the same bits; step s reads rows < T + s + 1 only
        for path in ("two_calls", "fused"):
            for s in range(S):
                k_new = gen.make("k", cfg.B, 1, t0=T + s)[:, 0].contiguous()
                v_new = gen.make("v", cfg.B, 1, t0=T + s)[:, 0].contiguous()
                pos = torch.full((cfg.B,), T + s, dtype=torch.int32, device="cuda")
                lens = torch.full((cfg.B,), T + s + 1, dtype=torch.int32, device="cuda")
                q = torch.from_numpy(q_steps[s]).cuda()
                if path == "two_calls":
                    kv.append(case.desc, k_new, v_new, pos, case.pk, case.pv, case.lat_k, case.lat_v)
                    o = kv.decode_attn(case.desc, q, case.pk, case.pv, case.lat_k, case.lat_v, lens, workspace=ws)
                else:
                    o = kv.append_decode_attn(case.desc, k_new, v_new, pos, q, case.pk, case.pv, case.lat_k,
                                              case.lat_v, lens, workspace=ws)
                outs[path].append(o.cpu().numpy().astype(np.float64))
            say(f"[full] {cfg.name} {path}: {S} steps done")
        refs = pending.get()   # [unit][S][G][d]
    for path, got in outs.items():
        assert all(np.isfinite(o).all() for o in got), path
        worst = 0.0
        for s in range(S):
            worst = max(worst, _compare(cfg, got[s], units, [r[s] for r in refs], f"{path} step {s}"))
        say(f"[full] {cfg.name} {path} worst over {S} steps x {len(units)} units: {worst:.3e}")


def test_full_32_layers(gpu):
    """All 32 layers, each with its own bases and (r_k, r_v) from the 50%-budget profile; every layer
    checked on 4 seeded batch rows x all 8 KV heads (every (r_k, r_v) pair of the profile)."""
    import torch
    cfg = LLAMA3_32_LAYERS
    prof = host.rank_profile(cfg)
    assert int(prof.sum()) == 4096
    pending = []
    with oracle_pool() as pool:
        for layer in range(cfg.n_layers):
            case = build_case(cfg, layer=layer, chunk=2048)
            q = host.queries(cfg, layer)
            lens = host.lengths(cfg)
            got = _decode(case, q, lens)
            assert np.isfinite(got).all(), layer
            g = np.random.default_rng(np.random.SeedSequence([7004, layer]))
            rows = sorted(int(x) for x in g.choice(cfg.B, size=4, replace=False))
            units = [(b, h) for b in rows for h in range(cfg.Hkv)]
            pending.append((layer, got, units, pool.map_async(unit_reference, _jobs(case, q, lens, units))))
            del case
            torch.cuda.empty_cache()
        say("[full] 32 layers decoded; waiting for the oracle")
        worst = 0.0
        for layer, got, units, res in pending:
            worst = max(worst, _compare(cfg, got, units, res.get(), f"layer {layer}"))
    say(f"[full] 32 layers x 32 units worst={worst:.3e}")
