"""GPU checks of the fused decode step (kvlr_append_decode_attn): the output and the caches equal
those of kvlr_append followed by kvlr_decode_attn bit for bit, and the output matches the oracle
over the grown cache."""
from __future__ import annotations

import numpy as np
import pytest

from synth import LLAMA3_LAYER_32K, SINGLE_HEAD_F32, WORKLOADS, host
from tests.gpu_cases import build_case, say, tolerance

pytestmark = pytest.mark.gpu


def _kv():
    import rank_compressed_kv_kvlr_amd as kv
    return kv


def _run_steps(cfg, steps, split, pos_shift=None):
    """`steps` decode steps on two identical caches, one with append + decode_attn, one with the
    fused call; asserts bit equality every step and returns (case, q, lens, out) of the last step."""
    import torch
    kv = _kv()
    from synth.device import KVGenerator
    T = cfg.T
    ref_case = build_case(cfg, n_rows=T)
    fused_case = build_case(cfg, n_rows=T)
    gen = KVGenerator(cfg, 0)
    for s in range(steps):
        k_new = gen.make("k", cfg.B, 1, t0=T + s)[:, 0].contiguous()
        v_new = gen.make("v", cfg.B, 1, t0=T + s)[:, 0].contiguous()
        pos_h = np.full(cfg.B, T + s, np.int32)
        if pos_shift is not None:
            pos_h = pos_h + np.asarray(pos_shift, np.int32)
        pos = torch.from_numpy(pos_h).cuda()
        # attend through the new row; a row outside the cache is not written, so attend the prefill rows
        lens = torch.from_numpy(np.where(pos_h < cfg.capacity, pos_h + 1, T).astype(np.int32)).cuda()
        q = torch.from_numpy(host.queries(cfg, 0, 1 + s)).cuda()
        say(f"[fused step] {cfg.name} step={s} pos={pos_h.tolist()} split={split}")
        kv.append(ref_case.desc, k_new, v_new, pos, ref_case.pk, ref_case.pv, ref_case.lat_k, ref_case.lat_v)
        ref = kv.decode_attn(ref_case.desc, q, ref_case.pk, ref_case.pv, ref_case.lat_k, ref_case.lat_v, lens,
                             split_tokens=split)
        got = kv.append_decode_attn(fused_case.desc, k_new, v_new, pos, q, fused_case.pk, fused_case.pv,
                                    fused_case.lat_k, fused_case.lat_v, lens, split_tokens=split)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), s
    # written rows of both caches agree (rows never written hold whatever the allocation held)
    shift = np.zeros(cfg.B, np.int32) if pos_shift is None else np.asarray(pos_shift, np.int32)
    for b in range(cfg.B):
        n = T + steps if shift[b] == 0 else T
        for h in range(cfg.Hkv):
            for which in ("k", "v"):
                a = kv.latent_rows(fused_case.lat_k if which == "k" else fused_case.lat_v, fused_case.desc, which, b, h)
                r = kv.latent_rows(ref_case.lat_k if which == "k" else ref_case.lat_v, ref_case.desc, which, b, h)
                assert torch.equal(a[:n], r[:n]), (b, h, which)
    return fused_case, q.cpu().numpy(), lens.cpu().numpy(), got.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("wl,extra,steps,split", [
    ("long_context_128k", dict(B=2, T=1000, decode_steps=6), 6, 128),        # r 48/80 (key and value tails), row mid-split
    ("llama3_8b_layer_32k", dict(B=2, T=255, decode_steps=4), 4, 0),           # rows cross a split boundary (library plan)
    ("llama3_8b_layer_32k", dict(B=2, Hq=32, Hkv=2, T=300, decode_steps=3), 3, 64),   # G = 16: four head groups write the row
    ("llama3_8b_layer_32k", dict(B=1, d=64, T=90, decode_steps=3), 3, 64),     # head_dim 64
])
def test_fused_step_equals_append_then_decode(gpu, wl, extra, steps, split):
    cfg = WORKLOADS[wl].scaled(**extra)
    case, q, lens, got = _run_steps(cfg, steps, split)
    metric, tol = tolerance(cfg)
    worst = 0.0
    for b in range(cfg.B):
        for h in range(cfg.Hkv):
            ref = case.reference(q, b, h, int(lens[b]))
            worst = max(worst, float(metric(got[b, h * cfg.G:(h + 1) * cfg.G], ref).max()))
    say(f"[fused step] oracle worst {worst:.3e} (bound {tol})")
    assert worst <= tol


def test_fused_step_other_rows_and_caches(gpu):
    """Rows written inside the cache (overwrites), a row outside it (nothing written), and the
    caches that take the two-launch form (fp32 latents) give the separate calls' result."""
    cfg = LLAMA3_LAYER_32K.scaled(B=3, T=200, decode_steps=2)
    _run_steps(cfg, 2, 64, pos_shift=[0, -77, 2 - 200 + cfg.capacity])   # row T+s, T+s-77, capacity+s
    _run_steps(SINGLE_HEAD_F32.scaled(T=300, decode_steps=2), 2, 64)
