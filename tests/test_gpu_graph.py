"""HIP graph capture of whole decode steps: every entry point enqueues kernels only
(no allocation, no memset, no synchronisation), so a caller can capture a multi-layer
step or a multi-step append + decode loop once and replay it."""
from __future__ import annotations

import numpy as np
import pytest

from synth import LLAMA3_32_LAYERS, LONG_CONTEXT_128K, host
from synth.device import KVGenerator
from tests.gpu_cases import build_case, say

pytestmark = pytest.mark.gpu


def _kv():
    import rank_compressed_kv_kvlr_amd as kv
    return kv


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # warm-up on the side stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_graph_multi_layer_step_matches_eager(gpu):
    """Several layers with their own ranks and bases, captured once, replayed 3 times with
    eager work in between; every replay equals the eager result bit for bit."""
    import torch
    kv = _kv()
    cfg = LLAMA3_32_LAYERS.scaled(B=4, T=700)
    layers = []
    for layer in range(4):
        case = build_case(cfg, layer=layer)
        q = torch.from_numpy(host.queries(cfg, layer)).cuda()
        layers.append((case, q, kv.alloc_workspace(case.desc), torch.empty((cfg.B, cfg.Hq, cfg.d), device="cuda")))
    lens = torch.from_numpy(host.lengths(cfg)).cuda()

    def step():
        for case, q, ws, out in layers:
            kv.decode_attn(case.desc, q, case.pk, case.pv, case.lat_k, case.lat_v, lens, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [out.clone() for *_, out in layers]
    g = _capture(step)
    for rep in range(3):
        for *_, out in layers:
            out.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (case, q, ws, out), e in zip(layers, eager):
            assert torch.equal(out, e), f"replay {rep}"
            nc = kv.decode_counter_bytes(case.desc) // 4
            assert (ws[:nc].view(torch.int32) == 0).all()
    say("[graph] 4-layer step: 3 replays equal the eager step")


@pytest.mark.parametrize("fused", [False, True])
def test_graph_append_decode_loop_matches_eager(gpu, fused):
    """A loop of (append one token, attend over all rows) steps captured as one graph; with
    fused=True each step is one kvlr_append_decode_attn call, compared with the two-call loop."""
    import torch
    kv = _kv()
    cfg = LONG_CONTEXT_128K.scaled(T=2000, decode_steps=8)
    steps = cfg.decode_steps
    T = cfg.T
    gen = KVGenerator(cfg, 0)
    ks = [gen.make("k", cfg.B, 1, t0=T + s)[:, 0].contiguous() for s in range(steps)]
    vs = [gen.make("v", cfg.B, 1, t0=T + s)[:, 0].contiguous() for s in range(steps)]
    qs = [torch.from_numpy(host.queries(cfg, 0, s)).cuda() for s in range(steps)]
    pos = [torch.full((cfg.B,), T + s, dtype=torch.int32, device="cuda") for s in range(steps)]
    lens = [torch.full((cfg.B,), T + s + 1, dtype=torch.int32, device="cuda") for s in range(steps)]

    def run(case, ws, outs, fused_step=False):
        for s in range(steps):
            if fused_step:
                kv.append_decode_attn(case.desc, ks[s], vs[s], pos[s], qs[s], case.pk, case.pv, case.lat_k,
                                      case.lat_v, lens[s], out=outs[s], workspace=ws)
                continue
            kv.append(case.desc, ks[s], vs[s], pos[s], case.pk, case.pv, case.lat_k, case.lat_v)
            kv.decode_attn(case.desc, qs[s], case.pk, case.pv, case.lat_k, case.lat_v, lens[s], out=outs[s],
                           workspace=ws)

    eager_case = build_case(cfg, n_rows=T)
    ws = kv.alloc_workspace(eager_case.desc)
    eager = [torch.empty((cfg.B, cfg.Hq, cfg.d), device="cuda") for _ in range(steps)]
    run(eager_case, ws, eager)
    torch.cuda.synchronize()

    case = build_case(cfg, n_rows=T)
    ws2 = kv.alloc_workspace(case.desc)
    outs = [torch.empty((cfg.B, cfg.Hq, cfg.d), device="cuda") for _ in range(steps)]
    g = _capture(lambda: run(case, ws2, outs, fused))
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()                 # re-appends the same rows at the same positions: same state
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(outs[s], eager[s]), (rep, s)
    say(f"[graph] {steps}-step append + decode loop (fused={fused}): 3 replays equal the eager loop")


def test_graph_other_paths_match_eager(gpu):
    """Joint bf16 values (three launches, q~ through the workspace), 4/3-bit latents, the folded
    entry point and the two-stage form, captured together and replayed 3 times: every replay
    equals the eager calls bit for bit."""
    import torch
    kv = _kv()
    from synth import LLAMA3_LAYER_32K
    from tests.test_gpu_joint import _joint_case
    from tests.test_gpu_quant import _q43_case
    cfg = LLAMA3_LAYER_32K.scaled(B=3, T=900)
    lens = torch.from_numpy(np.array([900, 311, 0], np.int32)).cuda()
    q = torch.from_numpy(host.queries(cfg, 0, 0)).cuda()
    joint = _joint_case(cfg, 128)
    q43 = _q43_case(cfg)
    per_head = build_case(cfg)
    q_lat = torch.randn((cfg.B, cfg.Hq, 64), generator=torch.Generator().manual_seed(5)).cuda()
    ws = [kv.alloc_workspace(joint["desc"]), kv.alloc_workspace(q43["desc"]), kv.alloc_workspace(per_head.desc),
          kv.alloc_workspace(per_head.desc, 128)]
    outs = [torch.empty((cfg.B, cfg.Hq, cfg.d), device="cuda") for _ in range(3)] + \
           [torch.empty((cfg.B, cfg.Hq, 64), device="cuda")]

    def step():
        kv.decode_attn(joint["desc"], q, joint["pk"], joint["pj"], joint["lk"], joint["lv"], lens, out=outs[0],
                       workspace=ws[0])
        kv.decode_attn(q43["desc"], q, q43["pk"], q43["pv"], q43["lk"], q43["lv"], lens, out=outs[1], workspace=ws[1])
        kv.decode_partials(per_head.desc, q, per_head.pk, per_head.lat_k, per_head.lat_v, lens, ws[3], split_tokens=128)
        kv.decode_combine(per_head.desc, per_head.pv, ws[3], outs[2], split_tokens=128)
        kv.decode_attn_latent(per_head.desc, q_lat, per_head.lat_k, per_head.lat_v, lens, o_lat=outs[3],
                              workspace=ws[2])

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = _capture(step)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), (rep, k)
    say("[graph] joint, 4/3-bit, two-stage and folded calls: 3 replays equal the eager calls")
