"""kvlr_decode_attn_noalloc: decode attention with the library's static device
scratch as the workspace, for callers that cannot allocate.

It runs the kernels and plans of kvlr_decode_attn, so its output must equal
kvlr_decode_attn's bit for bit on the same inputs; both are also checked
against the float64 oracle at the acceptance bounds. Two calls in a row, the
second on a smaller input, share the static scratch: the second must not see
anything the first left there."""
from __future__ import annotations

import numpy as np
import pytest

from synth import LLAMA3_LAYER_32K, PER_HEAD_RAGGED, host
from tests.gpu_cases import build_case, say, tolerance

pytestmark = pytest.mark.gpu


def _both(case, q, lens, split):
    import torch
    import rank_compressed_kv_kvlr_amd as kv
    qd = torch.from_numpy(q).cuda()
    lens_t = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    shape = (case.cfg.B, case.cfg.Hq, case.cfg.d)
    ref = kv.decode_attn(case.desc, qd, case.pk, case.pv, case.lat_k, case.lat_v, lens_t, split_tokens=split)
    got = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    kv.decode_attn_noalloc(case.desc, qd, case.pk, case.pv, case.lat_k, case.lat_v, lens_t, out=got,
                           split_tokens=split)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def _oracle_check(case, got, q, lens, units):
    metric, bound = tolerance(case.cfg)
    G = case.cfg.G
    worst = 0.0
    for b, h in units:
        T = int(lens[b])
        g = got[b, h * G:(h + 1) * G].astype(np.float64)
        if T == 0:
            assert np.all(g == 0)
            continue
        worst = max(worst, float(metric(g, case.reference(q, b, h, T)).max()))
    assert worst <= bound, worst
    return worst


def test_noalloc_equals_decode_attn_on_two_calls(gpu):
    import rank_compressed_kv_kvlr_amd as kv
    # first call: per-head ranks and ragged lengths (balanced plan, the larger record region)
    big = PER_HEAD_RAGGED.scaled(B=6, T_range=(700, 2600))
    # second call: a smaller input with uniform ranks (fixed plan, explicit split length)
    small = LLAMA3_LAYER_32K.scaled(B=2, Hq=16, Hkv=4, T=450)
    for cfg, split in ((big, 0), (small, 128)):
        case = build_case(cfg)
        lens = host.lengths(cfg)
        if cfg is small:
            lens = np.array([450, 0], np.int32)   # an empty row too
        q = host.queries(cfg, 0, 0)
        need = kv.decode_workspace_bytes(case.desc, split)
        say(f"[noalloc] cfg={cfg.name} B={cfg.B} lens={list(lens)} split={split} workspace={need} B")
        assert need <= kv.STATIC_SCRATCH_BYTES
        ref, got = _both(case, q, lens, split)
        assert np.array_equal(got, ref), float(np.nanmax(np.abs(got - ref)))
        units = [(b, h) for b in range(cfg.B) for h in range(cfg.Hkv)][:: max(1, cfg.B * cfg.Hkv // 8)]
        say(f"[noalloc] oracle worst={_oracle_check(case, got, q, lens, units):.3e}")


def test_noalloc_rejects_calls_beyond_the_static_scratch(gpu):
    import torch
    import rank_compressed_kv_kvlr_amd as kv
    # 64-token splits over 2^20 rows: the records alone need far more than 16 MiB
    desc = kv.Desc(64, 32, 8, 128, 1 << 20, 64, 64)
    assert kv.decode_workspace_bytes(desc, 64) > kv.STATIC_SCRATCH_BYTES
    dummy = torch.zeros(64, dtype=torch.float32, device="cuda")
    rc = kv.lib.kvlr_decode_attn_noalloc(desc.ptr, dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(),
                                         dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(), 0.1,
                                         dummy.data_ptr(), 64, None)
    assert rc == -8, rc
