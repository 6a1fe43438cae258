"""kvlr_decode_attn_layers: several independent layers in one call, their kernels spread
over the library's lanes (streams forked from and joined into the caller's stream). The
result must be that of one kvlr_decode_attn per layer, bit for bit, for any lane count,
eagerly and when the call is captured into a HIP graph and replayed."""
from __future__ import annotations

import numpy as np
import pytest

from synth import LLAMA3_32_LAYERS, PER_HEAD_RAGGED, SINGLE_HEAD_F32, host
from tests.gpu_cases import build_case, say, tolerance

pytestmark = pytest.mark.gpu


def _kv():
    import rank_compressed_kv_kvlr_amd as kv
    return kv


def _layers(n_profile=4):
    """Layers of different shapes in one call: per-layer ranks of the 32-layer profile (fixed
    plan), one with per-head ranks and ragged lengths (balanced plan), one fp32 single head."""
    import torch
    kv = _kv()
    out = []
    cfg = LLAMA3_32_LAYERS.scaled(B=4, T=700)
    lens = torch.from_numpy(host.lengths(cfg)).cuda()
    for layer in range(n_profile):
        case = build_case(cfg, layer=layer)
        q = torch.from_numpy(host.queries(cfg, layer)).cuda()
        out.append((cfg, case, q, lens))
    cfg2 = PER_HEAD_RAGGED.scaled(B=3, T_range=(300, 900))
    case2 = build_case(cfg2)
    out.append((cfg2, case2, torch.from_numpy(host.queries(cfg2, 0)).cuda(),
                torch.from_numpy(host.lengths(cfg2)).cuda()))
    cfg3 = SINGLE_HEAD_F32.scaled(T=1000)
    case3 = build_case(cfg3)
    out.append((cfg3, case3, torch.from_numpy(host.queries(cfg3, 0)).cuda(),
                torch.from_numpy(host.lengths(cfg3)).cuda()))
    return out


def _entries(layers):
    import torch
    kv = _kv()
    ents = []
    for cfg, case, q, lens in layers:
        ents.append(dict(desc=case.desc, q=q, P_K=case.pk, P_V=case.pv, lat_k=case.lat_k, lat_v=case.lat_v,
                         seq_lens=lens, out=torch.full((cfg.B, cfg.Hq, cfg.d), float("nan"), device="cuda"),
                         workspace=kv.alloc_workspace(case.desc)))
    return ents


def _sequential(layers):
    import torch
    kv = _kv()
    outs = []
    for cfg, case, q, lens in layers:
        outs.append(kv.decode_attn(case.desc, q, case.pk, case.pv, case.lat_k, case.lat_v, lens))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("lanes", [1, 2, 4])
def test_layers_equal_one_call_per_layer(gpu, lanes):
    import torch
    kv = _kv()
    layers = _layers()
    ref = _sequential(layers)
    ents = _entries(layers)
    say(f"[layers] {len(ents)} layers, lanes={lanes}")
    got = kv.decode_attn_layers(ents, lanes=lanes)
    torch.cuda.synchronize()
    for i, (g, r) in enumerate(zip(got, ref)):
        assert torch.equal(g, r), f"layer {i}"
    for e in ents:   # every call leaves its counter region zero
        nc = kv.decode_counter_bytes(e["desc"]) // 4
        assert (e["workspace"][:nc].view(torch.int32) == 0).all()
    # one unit of the first layer against the oracle as well
    cfg, case, q, lens = layers[0]
    metric, bound = tolerance(cfg)
    T = int(lens[1].item())
    want = case.reference(q.cpu().numpy(), 1, 2, T)
    have = got[0].cpu().numpy()[1, 2 * cfg.G:3 * cfg.G].astype(np.float64)
    assert metric(have, want).max() <= bound


def test_layers_graph_replay_matches_eager(gpu):
    """The forked lanes join the capture: 3 replays with eager work in between, each equal
    to one kvlr_decode_attn per layer."""
    import torch
    kv = _kv()
    layers = _layers(n_profile=3)
    ref = _sequential(layers)
    ents = _entries(layers)
    kv.decode_attn_layers(ents, lanes=2)           # warm-up outside capture (lanes made here)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kv.decode_attn_layers(ents, lanes=2)
    for rep in range(3):
        for e in ents:
            e["out"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (e, r) in enumerate(zip(ents, ref)):
            assert torch.equal(e["out"], r), f"replay {rep} layer {i}"
    say("[layers] graph of a 5-layer call: 3 replays equal the eager calls")


def test_layers_workspace_overlap_rejected(gpu):
    """With more than one lane, layers sharing a workspace could race: rejected before any
    launch; with one lane the same call is ordered on one stream and allowed."""
    import torch
    kv = _kv()
    layers = _layers(n_profile=2)[:2]
    ents = _entries(layers)
    ws = kv.alloc_workspace(ents[0]["desc"])
    for e in ents:
        e["workspace"] = ws
    with pytest.raises(kv.KvlrError) as exc:
        kv.decode_attn_layers(ents, lanes=2)
    assert exc.value.code == kv.ERR_ARG
    assert torch.isnan(ents[0]["out"]).all()       # nothing was launched
    ref = _sequential(layers)
    got = kv.decode_attn_layers(ents, lanes=1)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


def test_layers_with_joint_and_quantised_caches(gpu):
    """Layers whose decode takes other launches: joint bf16 values (projection, split and merge
    kernels, q~ passed through the workspace) and 4/3-bit latents, next to a bf16 layer, over 3
    lanes; equal to one kvlr_decode_attn per layer bit for bit."""
    import torch
    from synth import LLAMA3_LAYER_32K
    from tests.test_gpu_joint import _joint_case
    from tests.test_gpu_quant import _q43_case
    kv = _kv()
    cfg = LLAMA3_LAYER_32K.scaled(B=2, T=900)
    lens = torch.from_numpy(host.lengths(cfg)).cuda()
    q = torch.from_numpy(host.queries(cfg, 0, 0)).cuda()
    jc = _joint_case(cfg, 128)
    qc = _q43_case(cfg)
    bc = build_case(cfg)
    layers = [(jc["desc"], jc["pk"], jc["pj"], jc["lk"], jc["lv"]), (qc["desc"], qc["pk"], qc["pv"], qc["lk"], qc["lv"]),
              (bc.desc, bc.pk, bc.pv, bc.lat_k, bc.lat_v)] * 2
    ref = [kv.decode_attn(d, q, pk, pv, lk, lv, lens) for d, pk, pv, lk, lv in layers]
    torch.cuda.synchronize()
    ents = [dict(desc=d, q=q, P_K=pk, P_V=pv, lat_k=lk, lat_v=lv, seq_lens=lens,
                 out=torch.full((cfg.B, cfg.Hq, cfg.d), float("nan"), device="cuda"), workspace=kv.alloc_workspace(d))
            for d, pk, pv, lk, lv in layers]
    got = kv.decode_attn_layers(ents, lanes=3)
    torch.cuda.synchronize()
    for i, (g, r) in enumerate(zip(got, ref)):
        assert torch.equal(g, r), f"layer {i}"
    say("[layers] joint, 4/3-bit and bf16 layers over 3 lanes equal the one-call results")
