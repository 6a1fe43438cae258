"""GPU parity: every kernel through the C-ABI against the float64 oracle on
the same seeded inputs (small shapes that span several tiles and ragged
tails; the full-size workloads are in test_gpu_full.py)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import LLAMA3_LAYER_32K, LONG_CONTEXT_128K, PER_HEAD_RAGGED, SINGLE_HEAD_F32, WORKLOADS, host
from tests.gpu_cases import assert_latents_close, build_case, rel_inf_rows, rel_l2_rows, say, tolerance

pytestmark = pytest.mark.gpu


def _kv():
    import rank_compressed_kv_kvlr_amd as kv
    return kv


def _decode(case, q, lens, split=0, out=None, workspace=None):
    import torch
    kv = _kv()
    lens_t = torch.as_tensor(np.asarray(lens, np.int32)).cuda()
    say(f"[decode] lens={list(np.asarray(lens))[:8]} split={split}")
    o = kv.decode_attn(case.desc, torch.from_numpy(q).cuda(), case.pk, case.pv, case.lat_k, case.lat_v,
                       lens_t, out=out, workspace=workspace, split_tokens=split)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64)


def _check_rows(case, got, q, lens, heads=None, bs=None, diag_bound=None):
    cfg = case.cfg
    metric, bound = tolerance(cfg)
    G = cfg.G
    worst, worst_diag = 0.0, 0.0
    for b in (range(cfg.B) if bs is None else bs):
        for h in (range(cfg.Hkv) if heads is None else heads):
            T = int(lens[b])
            ref = case.reference(q, b, h, T)
            g = got[b, h * G:(h + 1) * G]
            if T == 0:
                assert np.all(g == 0), "empty row must be zero"
                continue
            worst = max(worst, float(metric(g, ref).max()))
            if diag_bound is not None:
                worst_diag = max(worst_diag, float(rel_l2_rows(g, case.reference_storage_aware(q, b, h, T)).max()))
    say(f"[check] worst={worst:.3e} (bound {bound}) storage-aware={worst_diag:.3e}")
    assert worst <= bound, worst
    if diag_bound is not None:
        assert worst_diag <= diag_bound, worst_diag
    return worst


# ---------------------------------------------------------------------------
def test_device_generator_matches_host(gpu):
    import torch
    from synth.device import KVGenerator
    for cfg, B, n, t0 in ((SINGLE_HEAD_F32, 1, 300, 0), (LLAMA3_LAYER_32K, 3, 77, 1000), (LONG_CONTEXT_128K, 2, 50, 131072)):
        gen = KVGenerator(cfg, 2)
        for kind in ("k", "v"):
            dev = gen.make(kind, B, n, t0=t0)
            torch.cuda.synchronize()
            got = dev.cpu()
            got = got.view(torch.int16).numpy().view(np.uint16) if cfg.in_dtype == "bf16" else got.numpy()
            for b in range(B):
                ref = host.kv_rows(cfg, 2, kind, b, t0, n, stats=gen.stats)
                assert np.array_equal(got[b], ref), (cfg.name, kind, b)


@pytest.mark.parametrize("wl,extra", [
    ("single_head_f32", {}),
    ("llama3_8b_layer_32k", dict(B=2, T=1000)),
    ("per_head_ranks_ragged", dict(B=3, T_range=(100, 700))),
    ("long_context_128k", dict(B=2, T=2100, decode_steps=0)),
])
def test_prefill_compress_matches_oracle(gpu, wl, extra):
    import torch
    kv = _kv()
    cfg = WORKLOADS[wl].scaled(**extra)
    case = build_case(cfg)
    torch.cuda.synchronize()
    rk, rv = host.ranks(cfg)
    for b in range(cfg.B):
        for h in range(cfg.Hkv):
            n = case.n_rows
            for which, P, r in (("k", case.P32K[h], rk[h]), ("v", case.P32V[h], rv[h])):
                X = case.host_rows(which, b, h, n)
                lat = kv.latent_rows(case.lat_k if which == "k" else case.lat_v, case.desc, which, b, h)[:n]
                got = lat.float().cpu().numpy().astype(np.float64)
                assert_latents_close(got, X, P, cfg.latent_dtype)


@pytest.mark.parametrize("wl,extra,diag", [
    ("single_head_f32", {}, None),
    ("single_head_f32", dict(T=2047), None),
    ("llama3_8b_layer_32k", dict(B=2, T=1000), 2e-3),
    ("per_head_ranks_ragged", dict(B=4, T_range=(1, 700)), 2e-3),
    ("long_context_128k", dict(B=2, T=1500, decode_steps=0), 2e-3),
])
def test_decode_matches_oracle(gpu, wl, extra, diag):
    cfg = WORKLOADS[wl].scaled(**extra)
    case = build_case(cfg)
    lens = host.lengths(cfg)
    q = host.queries(cfg, 0, 0)
    got = _decode(case, q, lens)
    _check_rows(case, got, q, lens, diag_bound=diag)


@pytest.mark.parametrize("rk,rv", [(16, 16), (32, 128), (48, 80), (64, 64), (80, 48), (96, 112), (112, 96),
                                   (128, 32), (128, 128)])
def test_decode_rank_sweep_bf16(gpu, rk, rv):
    cfg = LLAMA3_LAYER_32K.scaled(B=2, Hq=8, Hkv=2, T=333, r_k=rk, r_v=rv)
    case = build_case(cfg)
    lens = np.array([333, 190], np.int32)
    q = host.queries(cfg, 0, 0)
    _check_rows(case, _decode(case, q, lens), q, lens, diag_bound=2e-3)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rk,rv", [(4, 4), (12, 32), (32, 8), (96, 128), (128, 64), (60, 20)])
def test_decode_rank_sweep_f32(gpu, rk, rv, in_dtype):
    """fp32 latents take any rank that is a multiple of 4, from fp32 or bf16 rows (ranks that
    are not whole 16-channel tiles are compressed on VALU)."""
    cfg = SINGLE_HEAD_F32.scaled(B=2, Hq=3, Hkv=3, T=300, r_k=rk, r_v=rv, in_dtype=in_dtype)
    case = build_case(cfg)
    lens = np.array([300, 129], np.int32)
    q = host.queries(cfg, 0, 0)
    _check_rows(case, _decode(case, q, lens), q, lens)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 8, 16])
def test_decode_query_groups(gpu, G):
    cfg = LLAMA3_LAYER_32K.scaled(B=2, Hq=2 * G, Hkv=2, T=200, r_k=32, r_v=48)
    case = build_case(cfg)
    lens = np.array([200, 77], np.int32)
    q = host.queries(cfg, 0, 0)
    _check_rows(case, _decode(case, q, lens), q, lens)


@pytest.mark.parametrize("lens", [[0, 5], [1, 2], [17, 64], [65, 129], [257, 256], [300, 1]])
def test_decode_edge_lengths(gpu, lens):
    cfg = LLAMA3_LAYER_32K.scaled(B=2, Hq=8, Hkv=2, T=300)
    case = build_case(cfg)
    q = host.queries(cfg, 0, 0)
    lens = np.array(lens, np.int32)
    got = _decode(case, q, lens, split=64)
    _check_rows(case, got, q, lens)
    assert np.isfinite(got).all()


def test_decode_lengths_clamped_to_capacity(gpu):
    cfg = LLAMA3_LAYER_32K.scaled(B=2, Hq=8, Hkv=2, T=128)
    case = build_case(cfg)
    q = host.queries(cfg, 0, 0)
    over = _decode(case, q, np.array([10 ** 6, -5], np.int32))
    exact = _decode(case, q, np.array([128, 0], np.int32))
    assert np.array_equal(over, exact)


@pytest.mark.parametrize("wl", ["single_head_f32", "llama3_8b_layer_32k"])
def test_split_count_invariance(gpu, wl):
    extra = dict(B=1, T=4096) if wl == "single_head_f32" else dict(B=1, Hq=8, Hkv=2, T=4096)
    cfg = WORKLOADS[wl].scaled(**extra)
    case = build_case(cfg)
    lens = np.array([4096], np.int32)
    q = host.queries(cfg, 0, 0)
    base = _decode(case, q, lens, split=4096)          # one split
    tol = 1e-6 if cfg.latent_dtype == "f32" else 1e-3
    for split in (64, 128, 192, 256, 1024, 2048):      # 64 .. 2 splits
        got = _decode(case, q, lens, split=split)
        assert rel_inf_rows(got[0], base[0]).max() <= tol, split
    _check_rows(case, base, q, lens)


def test_gqa_equals_mha_with_repeated_heads(gpu):
    """G query heads over one KV head == G KV heads holding copies of that head's latents."""
    import torch
    kv = _kv()
    cfg = LLAMA3_LAYER_32K.scaled(B=2, Hq=8, Hkv=2, T=250, r_k=48, r_v=32)
    case = build_case(cfg)
    lens = np.array([250, 111], np.int32)
    q = host.queries(cfg, 0, 0)
    gqa = _decode(case, q, lens)
    # MHA layout: 8 KV heads, head i repeats KV head i // 4
    desc = kv.Desc(cfg.B, 8, 8, cfg.d, cfg.capacity, 48, 32, kv.BF16, kv.BF16)
    lk, lv = kv.alloc_cache(desc)
    for b in range(cfg.B):
        for i in range(8):
            kv.block_view(lk, desc, "k", b, i).copy_(kv.block_view(case.lat_k, case.desc, "k", b, i // 4))
            kv.block_view(lv, desc, "v", b, i).copy_(kv.block_view(case.lat_v, case.desc, "v", b, i // 4))
    pk = kv.pack_bases([case.PK[i // 4] for i in range(8)])
    pv = kv.pack_bases([case.PV[i // 4] for i in range(8)])
    o = kv.decode_attn(desc, torch.from_numpy(q).cuda(), pk, pv, lk, lv, torch.from_numpy(lens).cuda())
    mha = o.cpu().numpy().astype(np.float64)
    assert rel_inf_rows(mha, gqa).max() <= 1e-6


def test_ragged_equals_dense_truncated(gpu):
    import torch
    cfg = LLAMA3_LAYER_32K.scaled(B=3, Hq=8, Hkv=2, T=500)
    case = build_case(cfg)
    q = host.queries(cfg, 0, 0)
    ragged = _decode(case, q, np.array([500, 123, 321], np.int32))
    for b, T in enumerate((500, 123, 321)):
        dense = _decode(case, q, np.full(3, T, np.int32))
        assert rel_inf_rows(ragged[b], dense[b]).max() <= 1e-6
    torch.cuda.synchronize()


def test_per_head_ranks_equal_single_head_calls(gpu):
    import torch
    kv = _kv()
    cfg = PER_HEAD_RAGGED.scaled(B=2, T_range=(300, 300))
    case = build_case(cfg)
    lens = np.array([300, 180], np.int32)
    q = host.queries(cfg, 0, 0)
    full = _decode(case, q, lens)
    rk, rv = host.ranks(cfg)
    G = cfg.G
    for h in (0, 3, 6):
        desc = kv.Desc(cfg.B, G, 1, cfg.d, cfg.capacity, rk[h], rv[h], kv.BF16, kv.BF16)
        lk, lv = kv.alloc_cache(desc)
        for b in range(cfg.B):
            kv.block_view(lk, desc, "k", b, 0).copy_(kv.block_view(case.lat_k, case.desc, "k", b, h))
            kv.block_view(lv, desc, "v", b, 0).copy_(kv.block_view(case.lat_v, case.desc, "v", b, h))
        qh = np.ascontiguousarray(q[:, h * G:(h + 1) * G])
        o = kv.decode_attn(desc, torch.from_numpy(qh).cuda(), kv.pack_bases([case.PK[h]]),
                           kv.pack_bases([case.PV[h]]), lk, lv, torch.from_numpy(lens).cuda())
        single = o.cpu().numpy().astype(np.float64)
        assert rel_inf_rows(single, full[:, h * G:(h + 1) * G]).max() <= 1e-6, h


@pytest.mark.parametrize("wl", ["single_head_f32", "llama3_8b_layer_32k", "long_context_128k"])
def test_append_matches_oracle_and_prefill(gpu, wl):
    """append of token T at row T == prefill of T+1 tokens (to one storage rounding), and == oracle."""
    import torch
    kv = _kv()
    extra = dict(B=2, T=200, decode_steps=3) if wl != "single_head_f32" else dict(T=200, decode_steps=3)
    cfg = WORKLOADS[wl].scaled(**extra)
    T = cfg.T
    case = build_case(cfg, n_rows=T)
    full = build_case(cfg, n_rows=T + 3)
    from synth.device import KVGenerator
    gen = KVGenerator(cfg, 0)
    for s in range(3):
        k_new = gen.make("k", cfg.B, 1, t0=T + s)[:, 0].contiguous()
        v_new = gen.make("v", cfg.B, 1, t0=T + s)[:, 0].contiguous()
        pos = torch.full((cfg.B,), T + s, dtype=torch.int32, device="cuda")
        say(f"[append] step={s}")
        kv.append(case.desc, k_new, v_new, pos, case.pk, case.pv, case.lat_k, case.lat_v)
    # a position outside the cache writes nothing
    before = case.lat_k.clone()
    kv.append(case.desc, k_new, v_new, torch.full((cfg.B,), cfg.capacity, dtype=torch.int32, device="cuda"),
              case.pk, case.pv, case.lat_k, case.lat_v)
    torch.cuda.synchronize()
    assert torch.equal(before, case.lat_k)
    for which in ("k", "v"):
        a = case.lat_k if which == "k" else case.lat_v
        f = full.lat_k if which == "k" else full.lat_v
        for b in range(cfg.B):
            for h in range(cfg.Hkv):
                got = kv.latent_rows(a, case.desc, which, b, h)[:T + 3].float().cpu().numpy().astype(np.float64)
                ref = kv.latent_rows(f, full.desc, which, b, h)[:T + 3].float().cpu().numpy().astype(np.float64)
                P = (case.P32K if which == "k" else case.P32V)[h]
                X = case.host_rows(which, b, h, 3, t0=T)
                assert_latents_close(got[T:], X, P, cfg.latent_dtype, exact_frac=0.9)
                assert_latents_close(ref[T:], X, P, cfg.latent_dtype, exact_frac=0.9)
                assert np.array_equal(got[:T], ref[:T])
    q = host.queries(cfg, 0, 1)
    lens = np.full(cfg.B, T + 3, np.int32)
    _check_rows(case, _decode(case, q, lens), q, lens)


def test_outputs_fully_written_and_deterministic(gpu):
    """NaN-poisoned outputs and workspace are fully overwritten; guard bands stay intact; runs are bitwise equal."""
    import torch
    kv = _kv()
    cfg = PER_HEAD_RAGGED.scaled(B=3, T_range=(50, 900))
    case = build_case(cfg)
    lens = host.lengths(cfg)
    q = torch.from_numpy(host.queries(cfg, 0, 0)).cuda()
    lens_t = torch.from_numpy(lens).cuda()
    guard = 4096
    nout = cfg.B * cfg.Hq * cfg.d
    big = torch.full((nout + 2 * guard,), float("nan"), device="cuda")
    big[:guard] = 7.0
    big[-guard:] = 7.0
    out = big[guard:guard + nout]
    ws = kv.alloc_workspace(case.desc)
    nc = kv.decode_counter_bytes(case.desc) // 4
    ws[nc:].fill_(float("nan"))   # records poisoned; counters start at zero as the ABI requires
    kv.decode_attn(case.desc, q, case.pk, case.pv, case.lat_k, case.lat_v, lens_t, out=out, workspace=ws)
    torch.cuda.synchronize()
    first = out.clone()
    assert torch.isfinite(first).all()
    assert (big[:guard] == 7).all() and (big[-guard:] == 7).all()
    for _ in range(3):
        kv.decode_attn(case.desc, q, case.pk, case.pv, case.lat_k, case.lat_v, lens_t, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert (ws[:nc].view(torch.int32) == 0).all(), "every call must leave the arrival counters at zero"


@pytest.mark.parametrize("wl,split", [("llama3_8b_layer_32k", 0), ("llama3_8b_layer_32k", 128), ("single_head_f32", 256), ("per_head_ranks_ragged", 0)])
def test_decode_attn_equals_two_stages(gpu, wl, split):
    """kvlr_decode_attn (one launch, merge in the last workgroup) matches partials + combine.

    With the fixed plan the split records are the same and the merges sum them in different
    orders, so fp32 rounding may differ; the balanced plan cuts the sequences elsewhere.
    """
    import torch
    kv = _kv()
    extra = {"single_head_f32": dict(T=1000), "llama3_8b_layer_32k": dict(B=2, Hq=16, Hkv=2, T=700), "per_head_ranks_ragged": dict(B=3, T_range=(10, 900))}[wl]
    cfg = WORKLOADS[wl].scaled(**extra)
    case = build_case(cfg)
    lens_t = torch.from_numpy(host.lengths(cfg)).cuda()
    q = torch.from_numpy(host.queries(cfg, 0, 0)).cuda()
    fused = kv.decode_attn(case.desc, q, case.pk, case.pv, case.lat_k, case.lat_v, lens_t, split_tokens=split)
    ws = kv.alloc_workspace(case.desc, split)
    kv.decode_partials(case.desc, q, case.pk, case.lat_k, case.lat_v, lens_t, ws, split_tokens=split)
    out = torch.empty_like(fused)
    kv.decode_combine(case.desc, case.pv, ws, out, split_tokens=split)
    torch.cuda.synchronize()
    a, b = fused.cpu().numpy().astype(np.float64), out.cpu().numpy().astype(np.float64)
    # with per-head ranks and split 0 the one-launch call takes the balanced plan while the two
    # stages keep the fixed one: other cuts, so softmax weights rounded differently (~2^-17)
    balanced = kv.decode_plan(case.desc, split)[1] == 0
    assert rel_inf_rows(a, b).max() <= (2e-5 if balanced else 1e-6)


def test_latent_guard_bands(gpu):
    """Compression and append write only their rows: canaries around the caches survive."""
    import torch
    kv = _kv()
    from synth.device import KVGenerator
    cfg = PER_HEAD_RAGGED.scaled(B=2, T_range=(100, 100), decode_steps=2)
    rk, rv = host.ranks(cfg)
    PK, PV = host.bases(cfg)
    desc = kv.Desc(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.capacity, rk, rv, kv.BF16, kv.BF16)
    nk, nv = kv.cache_elems(desc)
    guard = 2048
    canary = torch.tensor(12345.0, dtype=torch.bfloat16)
    bk = torch.full((nk + 2 * guard,), float(canary), dtype=torch.bfloat16, device="cuda")
    bv = torch.full((nv + 2 * guard,), float(canary), dtype=torch.bfloat16, device="cuda")
    lk, lv = bk[guard:guard + nk], bv[guard:guard + nv]
    gen = KVGenerator(cfg, 0)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    kv.prefill_compress(desc, gen.make("k", cfg.B, 60, 40), gen.make("v", cfg.B, 60, 40), 40, pk, pv, lk, lv)
    pos = torch.tensor([101, 5], dtype=torch.int32, device="cuda")
    kv.append(desc, gen.make("k", cfg.B, 1)[:, 0].contiguous(), gen.make("v", cfg.B, 1)[:, 0].contiguous(), pos,
              pk, pv, lk, lv)
    torch.cuda.synchronize()
    for big, n in ((bk, nk), (bv, nv)):
        assert (big[:guard] == canary).all() and (big[guard + n:] == canary).all()
    # untouched rows keep the canary too: rows 0..39 (except row 5 of batch 1), 100, 101 of batch 1
    for b in range(cfg.B):
        for h in range(cfg.Hkv):
            rows = kv.latent_rows(lk, desc, "k", b, h)
            written = set(range(40, 100)) | {int(pos[b])}
            for t in (0, 39, 100, 101):
                expect_canary = t not in written
                assert bool((rows[t] == canary).all()) == expect_canary, (b, h, t)


@pytest.mark.parametrize("lens", [[0, 1, 2999, 17, 1500, 3000], [3000, 0, 0, 0, 0, 1], [0, 0, 0, 0, 0, 0]])
def test_ragged_lengths_with_empty_rows(gpu, lens):
    """Per-head ranks with very uneven lengths (empty rows, one long row): oracle parity under the
    library's plan, and the same result with a shorter fixed split (to fp32 rounding)."""
    cfg = PER_HEAD_RAGGED.scaled(B=6, T_range=(1, 3000))
    case = build_case(cfg)
    q = host.queries(cfg, 0, 0)
    got = _decode(case, q, lens)
    _check_rows(case, got, q, lens, diag_bound=2e-3)
    other = _decode(case, q, lens, split=256)
    nz = [b for b in range(cfg.B) if lens[b] > 0]
    if nz:
        assert rel_inf_rows(got[nz], other[nz]).max() <= 1e-5
    assert np.all(got[[b for b in range(cfg.B) if lens[b] == 0]] == 0)


def test_single_unit_long_and_many_units(gpu):
    """One (batch row, KV head) over 20000 rows; and 640 (batch row, KV head, head group) units."""
    cfg = SINGLE_HEAD_F32.scaled(T=20000)
    case = build_case(cfg)
    q = host.queries(cfg, 0, 0)
    lens = [20000]
    _check_rows(case, _decode(case, q, lens), q, lens)
    cfg = LLAMA3_LAYER_32K.scaled(B=40, Hq=64, Hkv=4, T=300)   # 40 x 4 KV heads x 4 head groups
    case = build_case(cfg)
    q = host.queries(cfg, 0, 0)
    lens = host.lengths(cfg)
    _check_rows(case, _decode(case, q, lens), q, lens, heads=[0, 3], bs=[0, 17, 39])


# ---------------------------------------------------------------------------
# balanced plan (split_tokens = -1; the library's default when the KV heads' ranks differ)
@pytest.mark.parametrize("wl,extra,lens,diag", [
    ("per_head_ranks_ragged", dict(B=6, T_range=(1, 3000)), None, 2e-3),              # per-head ranks, ragged
    ("llama3_8b_layer_32k", dict(B=3, Hq=8, Hkv=2, T=2000), [2000, 17, 0], 2e-3),     # a tiny and an empty row
    ("llama3_8b_layer_32k", dict(B=1, Hq=4, Hkv=1, T=1, r_k=16, r_v=16), [1], 2e-3),  # less work than workgroups
    ("long_context_128k", dict(B=2, T=3000, decode_steps=0), [3000, 2999], 2e-3),     # ranks 48/80: tails
    ("llama3_8b_layer_32k", dict(B=5, Hq=64, Hkv=4, T=700), None, 2e-3),              # 4 head groups per KV head
    ("per_head_ranks_ragged", dict(B=40, T_range=(0, 400)), None, 2e-3),              # many short rows, some empty
    # 2000 rows (the input generator's limit): 32 chunks of the length scan
    ("llama3_8b_layer_32k", dict(B=2000, Hq=4, Hkv=2, T=16, r_k=16, r_v=16), [(7 * i) % 17 for i in range(2000)], 6e-3),
])
def test_balanced_plan_matches_oracle_and_fixed_plan(gpu, wl, extra, lens, diag):
    """Equal shares of the work per workgroup, cut across (batch row, KV head) units: the oracle's
    result, the fixed plan's to the rounding of the softmax weights, and the same bits on every run.
    The storage-aware diagnostic is looser for rank 16 over at most 16 tokens: compression rounds
    its fp32 latents to bf16, and an element on a rounding boundary can come out one ulp (2^-8)
    from the float64 oracle's rounding; with 16 channels and a few tokens one such element moves
    an output by a few 1e-3."""
    import torch
    cfg = WORKLOADS[wl].scaled(**extra)
    case = build_case(cfg)
    lens = host.lengths(cfg) if lens is None else np.array(lens, np.int32)
    q = host.queries(cfg, 0, 0)
    kv = _kv()
    say(f"[balanced] plan {kv.decode_plan(case.desc, -1)} lens={lens.tolist()[:8]}")
    bal = _decode(case, q, lens, split=-1)
    _check_rows(case, bal, q, lens, diag_bound=diag)
    assert np.array_equal(_decode(case, q, lens, split=-1), bal)
    fixed = _decode(case, q, lens, split=256)
    live = lens > 0
    # The plans cut the sequence differently, so each split's running maximum and with it the
    # rounding of the softmax weights differ: the value product keeps about 16 bits of a weight
    # (a high and a low bf16 part), i.e. 2^-17 relative, and the outputs agree to ~1e-5.
    assert rel_inf_rows(bal[live], fixed[live]).max() <= 2e-5
    # the folded entry point takes the same plan
    ql = torch.from_numpy(case.folded_queries(q)).cuda()
    lens_t = torch.from_numpy(lens).cuda()
    ob = kv.decode_attn_latent(case.desc, ql, case.lat_k, case.lat_v, lens_t, split_tokens=-1)
    of = kv.decode_attn_latent(case.desc, ql, case.lat_k, case.lat_v, lens_t, split_tokens=256)
    torch.cuda.synchronize()
    ob, of = ob.cpu().numpy().astype(np.float64), of.cpu().numpy().astype(np.float64)
    assert np.all(ob[~live] == 0)
    assert rel_inf_rows(ob[live], of[live]).max() <= 2e-5
