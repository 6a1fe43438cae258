"""GPU parity of the folded decode (bases folded into the caller's query and
output projections): kvlr_decode_attn_latent against the oracle's folded form
on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import pytest

from synth import LLAMA3_LAYER_32K, WORKLOADS, host
from tests.gpu_cases import build_case, rel_inf_rows, say, tolerance

pytestmark = pytest.mark.gpu


def _kv():
    import rank_compressed_kv_kvlr_amd as kv
    return kv


def _folded(case, q_lat, lens, split=0):
    import torch
    kv = _kv()
    say(f"[folded] lens={list(np.asarray(lens))[:8]} split={split} q_lat={q_lat.shape}")
    o = kv.decode_attn_latent(case.desc, torch.from_numpy(q_lat).cuda(), case.lat_k, case.lat_v,
                              torch.as_tensor(np.asarray(lens, np.int32)).cuda(), split_tokens=split)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64)


def _check(case, got, q_lat, lens, bs=None, heads=None):
    cfg = case.cfg
    metric, bound = tolerance(cfg)
    G = cfg.G
    worst = 0.0
    for b in (range(cfg.B) if bs is None else bs):
        for h in (range(cfg.Hkv) if heads is None else heads):
            rv = case.PV[h].shape[1]
            g = got[b, h * G:(h + 1) * G]
            assert np.all(g[:, rv:] == 0), "entries past r_v must be zero"
            T = int(lens[b])
            if T == 0:
                assert np.all(g == 0), "empty row must be zero"
                continue
            worst = max(worst, float(metric(g[:, :rv], case.reference_folded(q_lat, b, h, T)).max()))
    say(f"[check folded] worst={worst:.3e} (bound {bound})")
    assert worst <= bound, worst
    return worst


@pytest.mark.parametrize("wl,extra", [
    ("single_head_f32", dict(T=2047)),
    ("llama3_8b_layer_32k", dict(B=2, T=1000)),
    ("per_head_ranks_ragged", dict(B=4, T_range=(1, 700))),
    ("llama3_8b_layer_32k", dict(B=2, Hq=10, Hkv=2, T=333, r_k=48, r_v=112)),
    ("single_head_f32", dict(B=2, Hq=3, Hkv=3, T=300, r_k=12, r_v=32)),
])
def test_folded_matches_oracle(gpu, wl, extra):
    cfg = WORKLOADS[wl].scaled(**extra)
    case = build_case(cfg)
    lens = host.lengths(cfg)
    q_lat = case.folded_queries(host.queries(cfg, 0, 0))
    _check(case, _folded(case, q_lat, lens), q_lat, lens)


@pytest.mark.parametrize("lens,split", [([0, 5], 64), ([1, 300], 64), ([257, 0], 0), ([300, 129], 128)])
def test_folded_edge_lengths(gpu, lens, split):
    cfg = LLAMA3_LAYER_32K.scaled(B=2, Hq=8, Hkv=2, T=300)
    case = build_case(cfg)
    q_lat = case.folded_queries(host.queries(cfg, 0, 0))
    lens = np.array(lens, np.int32)
    got = _folded(case, q_lat, lens, split)
    assert np.isfinite(got).all()
    _check(case, got, q_lat, lens)


@pytest.mark.parametrize("wl", ["llama3_8b_layer_32k", "per_head_ranks_ragged"])
def test_folded_back_projects_to_decode_attn(gpu, wl):
    """o_lat P_V^T from the folded call equals kvlr_decode_attn on q with q_lat = q P_K.

    Both sides run the same split records; the back-projection order differs, so fp32
    rounding may differ in the last bits."""
    import torch
    kv = _kv()
    extra = {"llama3_8b_layer_32k": dict(B=2, Hq=16, Hkv=2, T=700), "per_head_ranks_ragged": dict(B=3, T_range=(10, 900))}[wl]
    cfg = WORKLOADS[wl].scaled(**extra)
    case = build_case(cfg)
    lens = host.lengths(cfg)
    q = host.queries(cfg, 0, 0)
    q_lat = case.folded_queries(q)
    o_lat = _folded(case, q_lat, lens)
    full = kv.decode_attn(case.desc, torch.from_numpy(q).cuda(), case.pk, case.pv, case.lat_k, case.lat_v,
                          torch.as_tensor(lens).cuda())
    torch.cuda.synchronize()
    full = full.cpu().numpy().astype(np.float64)
    back = np.zeros_like(full)
    for i in range(cfg.Hq):
        h = i // cfg.G
        rv = case.PV[h].shape[1]
        back[:, i] = o_lat[:, i, :rv] @ case.P32V[h].T
    err = float(rel_inf_rows(back, full).max())
    say(f"[folded vs full] {err:.3e}")
    # q_lat is q P_K rounded to fp32 on the host; the fused path keeps it in fp32 registers
    assert err <= 2e-4, err


def test_folded_counters_left_zero(gpu):
    """A folded call leaves the merge counters at zero, so the workspace is reusable by either call."""
    import torch
    kv = _kv()
    cfg = LLAMA3_LAYER_32K.scaled(B=2, Hq=8, Hkv=2, T=500)
    case = build_case(cfg)
    lens = host.lengths(cfg)
    q_lat = case.folded_queries(host.queries(cfg, 0, 0))
    ws = kv.alloc_workspace(case.desc, 64)
    lens_t = torch.as_tensor(lens).cuda()
    ql = torch.from_numpy(q_lat).cuda()
    a = kv.decode_attn_latent(case.desc, ql, case.lat_k, case.lat_v, lens_t, workspace=ws, split_tokens=64)
    b = kv.decode_attn_latent(case.desc, ql, case.lat_k, case.lat_v, lens_t, workspace=ws, split_tokens=64)
    torch.cuda.synchronize()
    cbytes = kv.decode_counter_bytes(case.desc)
    assert int(ws.view(torch.uint8)[:cbytes].count_nonzero()) == 0
    assert torch.equal(a, b)
