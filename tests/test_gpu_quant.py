"""GPU parity of the mixed 4/3-bit latent storage (block-wise Hadamard folded into
the bases, 4-bit outlier and 3-bit inlier blocks per token) against oracle/quant.py."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import quant as qo
from synth import LLAMA3_LAYER_32K, PER_HEAD_RAGGED, WORKLOADS, host
from synth.device import KVGenerator
from tests.gpu_cases import bases32, say

pytestmark = pytest.mark.gpu


def _kv():
    import rank_compressed_kv_kvlr_amd as kv
    return kv


def _block_bytes(kv, desc, lat, which, b, h):
    """The raw bytes of the (b, h) block of a 4/3-bit cache (tiles of 32 tokens)."""
    return kv.latent_rows(lat, desc, which, b, h).cpu().numpy()


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
    """Integer inputs and bases with entries +-1/16 make every fp32 latent exact, so the stored
    tiles must equal the oracle's byte for byte. Rows are written by three prefill calls that start
    and end inside tiles (so compression must keep the rows of a shared tile it does not write) and
    one append."""
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
    for a, e in ((0, 45), (45, 77), (77, T - 1)):   # 45 and 77 fall inside tiles
        kv.prefill_compress(desc, Kd[:, a:e].contiguous(), Vd[:, a:e].contiguous(), a, pk, pv, lk, lv)
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    kv.append(desc, Kd[:, T - 1].contiguous(), Vd[:, T - 1].contiguous(), pos, pk, pv, lk, lv)
    torch.cuda.synchronize()
    full_tiles = T // qo.TILE
    for which, X, P, ranks in (("k", K, PK, rk), ("v", V, PV, rv)):
        for b in range(B):
            for h in range(Hkv):
                r = ranks[h]
                lat = (X[b, :, h, :].astype(np.float64) @ P[h]).astype(np.float32)
                assert np.array_equal(lat.astype(np.float64), X[b, :, h, :].astype(np.float64) @ P[h])
                codes, meta = qo.quantize_rows(lat)
                raw = _block_bytes(kv, desc, lk if which == "k" else lv, which, b, h)
                want = qo.pack_block(codes[:full_tiles * qo.TILE], meta[:full_tiles * qo.TILE], r, which)
                bad = np.argwhere(raw[:len(want)] != want)
                assert bad.size == 0, f"{which} b={b} h={h} r={r} first mismatching bytes {bad[:5].ravel()}"
                gc, gm = qo.unpack_block(raw, T, r, which)   # the partly written last tile, row by row
                assert np.array_equal(gc, codes) and np.array_equal(gm.view(np.uint16), meta.view(np.uint16)), \
                    (which, b, h, r)
    say(f"[q43] bit-exact tiles ({in_dtype} inputs)")


def test_quantised_compression_matches_oracle(gpu):
    """Realistic rows (llama-shaped workload, folded QR bases): every stored value is within
    one quantisation step of the oracle's, and almost every code is identical."""
    import torch
    kv = _kv()
    cfg = PER_HEAD_RAGGED.scaled(B=2, T_range=(300, 300))
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
                r = int(ranks[h])
                gcs, gms = qo.unpack_block(_block_bytes(kv, desc, lat, which, b, h), T, r, which)
                for t in range(T):
                    gc, gm = gcs[t], tuple(gms[t])
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


# ---------------------------------------------------------------------------
# decode over 4/3-bit caches
# ---------------------------------------------------------------------------
def _q43_case(cfg, n_rows=None, ranks=None, chunk=None):
    """Device caches of cfg's rows stored as 4/3-bit latents with Hadamard-folded bases."""
    import torch
    kv = _kv()
    rk, rv = host.ranks(cfg) if ranks is None else ranks
    PK, PV = host.bases(cfg)
    if ranks is not None:
        PK = [P[:, :int(r)] for P, r in zip(PK, rk)] if PK[0].shape[1] >= max(rk) else PK
    n_rows = cfg.capacity if n_rows is None else n_rows
    desc = kv.Desc(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.capacity, rk, rv, kv.BF16, kv.Q43)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    kv.hadamard_bases(desc, pk, pv)
    lk, lv = kv.alloc_cache(desc)
    gen = KVGenerator(cfg, 0)
    chunk = chunk or n_rows
    for t0 in range(0, n_rows, chunk):
        n = min(chunk, n_rows - t0)
        kv.prefill_compress(desc, gen.make("k", cfg.B, n, t0=t0), gen.make("v", cfg.B, n, t0=t0), t0, pk, pv, lk, lv)
    torch.cuda.synchronize()
    say(f"[q43 case] {cfg.name} B={cfg.B} T={n_rows} rk={list(rk)} rv={list(rv)}")
    return dict(cfg=cfg, desc=desc, pk=pk, pv=pv, lk=lk, lv=lv, PK=PK, PV=PV, stats=host.kv_stats(cfg, 0))


def _q43_reference(case, q, b, h, T):
    cfg = case["cfg"]
    G = cfg.G
    K = host.decode_to_f64(host.kv_rows(cfg, 0, "k", b, 0, T, heads=[h], stats=case["stats"]), cfg.in_dtype)[:, 0]
    V = host.decode_to_f64(host.kv_rows(cfg, 0, "v", b, 0, T, heads=[h], stats=case["stats"]), cfg.in_dtype)[:, 0]
    return qo.decode_head_quantized(q[b, h * G:(h + 1) * G].astype(np.float64), K, V, bases32([case["PK"][h]])[0],
                                    bases32([case["PV"][h]])[0], 1 / np.sqrt(cfg.d))


def _q43_decode(case, q, lens, split=0):
    import torch
    kv = _kv()
    out = kv.decode_attn(case["desc"], torch.from_numpy(q).cuda(), case["pk"], case["pv"], case["lk"], case["lv"],
                         torch.as_tensor(np.asarray(lens, np.int32)).cuda(), split_tokens=split)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _q43_check(case, got, q, lens, units=None, bound=2e-2, long_bound=2e-3, long_T=256):
    """Rows against the oracle's decode over its own quantised latents.

    The two sides quantise fp32 latents that differ in the last bit (MFMA with a
    split basis vs a float64 product rounded once), so a code lying on a rounding
    boundary can come out one step apart (about 6 in a million codes). For a short
    sequence one such code moves the output by up to a step, so the bound is the
    bf16-latent bound 2e-2; with long_T rows or more the weights spread over many
    tokens and the outputs must agree to long_bound."""
    from tests.gpu_cases import rel_l2_rows
    cfg = case["cfg"]
    G = cfg.G
    worst = worst_long = 0.0
    units = [(b, h) for b in range(cfg.B) for h in range(cfg.Hkv)] if units is None else units
    for b, h in units:
        T = int(lens[b])
        g = got[b, h * G:(h + 1) * G]
        if T == 0:
            assert np.all(g == 0)
            continue
        err = float(rel_l2_rows(g, _q43_reference(case, q, b, h, T)).max())
        worst = max(worst, err)
        if T >= long_T:
            worst_long = max(worst_long, err)
    say(f"[q43 check] worst rel L2 {worst:.3e} (rows >= {long_T}: {worst_long:.3e})")
    assert worst <= bound, worst
    assert worst_long <= long_bound, worst_long
    return worst


@pytest.mark.parametrize("wl,extra", [
    ("llama3_8b_layer_32k", dict(B=2, T=1000)),
    ("per_head_ranks_ragged", dict(B=3, T_range=(1, 700))),
    ("llama3_8b_layer_32k", dict(B=2, Hq=10, Hkv=2, T=333, r_k=128, r_v=16)),
    ("llama3_8b_layer_32k", dict(B=2, Hq=8, Hkv=2, T=300, r_k=16, r_v=128)),
    ("llama3_8b_layer_32k", dict(B=2, Hq=6, Hkv=2, T=257, r_k=112, r_v=48)),
])
def test_q43_decode_matches_oracle(gpu, wl, extra):
    cfg = WORKLOADS[wl].scaled(**extra)
    case = _q43_case(cfg)
    lens = host.lengths(cfg)
    q = host.queries(cfg, 0, 0)
    _q43_check(case, _q43_decode(case, q, lens), q, lens)


def test_q43_full_llama3_layer_32k(gpu):
    """The 4/3-bit decode at the benchmark's size and launch configuration: 8 sequences of
    32768 tokens, rank 64, the library's plan (12 splits of 2752 tokens, 3 workgroups per
    CU). Seeded (batch row, KV head) units against the oracle's decode over its own
    quantised latents."""
    kv = _kv()
    cfg = LLAMA3_LAYER_32K
    case = _q43_case(cfg, chunk=8192)
    assert kv.decode_plan(case["desc"], 0) == (12, 2752)
    q = host.queries(cfg)
    lens = host.lengths(cfg)
    got = _q43_decode(case, q, lens)
    assert np.isfinite(got).all()
    g = np.random.default_rng(np.random.SeedSequence([7100, cfg.cid]))
    units = sorted({(int(g.integers(cfg.B)), int(g.integers(cfg.Hkv))) for _ in range(3)})
    _q43_check(case, got, q, lens, units=units)


@pytest.mark.parametrize("lens,split", [([0, 5], 64), ([1, 300], 64), ([257, 256], 0), ([300, 129], 128)])
def test_q43_decode_edge_lengths(gpu, lens, split):
    cfg = LLAMA3_LAYER_32K.scaled(B=2, Hq=8, Hkv=2, T=300)
    case = _q43_case(cfg)
    q = host.queries(cfg, 0, 0)
    lens = np.array(lens, np.int32)
    got = _q43_decode(case, q, lens, split)
    assert np.isfinite(got).all()
    _q43_check(case, got, q, lens)


def test_q43_decode_exact_storage(gpu):
    """Integer rows and +-1/16 bases: the GPU stores exactly the oracle's codes, so decode
    differs from the oracle only by the kernel's arithmetic: fp32, except that the value
    weights p step and p base enter the value product as half floats. Each such weight is
    p rounded to half, times a half parameter, rounded again: relative error at most
    2u + u^2 (u = 2^-11), plus 2^-25 absolute per rounding below half's normal range.
    The bound per output element is that error carried through sum_t p_t (|step_t| c_t +
    |base_t|) / l and |P_V|, plus 1e-4 max|ref| for the fp32 sums."""
    import torch
    kv = _kv()
    from oracle import kvlr_oracle as ko
    rng = np.random.default_rng(43)
    B, Hq, Hkv, d, T = 2, 8, 2, 128, 200
    rk, rv = [64, 128], [80, 48]
    PKf = [rng.choice([-1 / 16, 1 / 16], size=(d, r)) for r in rk]
    PVf = [rng.choice([-1 / 16, 1 / 16], size=(d, r)) for r in rv]
    K = rng.integers(-8, 9, size=(B, T, Hkv, d)).astype(np.float32)
    V = rng.integers(-8, 9, size=(B, T, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    desc = kv.Desc(B, Hq, Hkv, d, T, rk, rv, kv.F32, kv.Q43)
    pk, pv = kv.pack_bases(PKf), kv.pack_bases(PVf)
    lk, lv = kv.alloc_cache(desc)
    kv.prefill_compress(desc, torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), 0, pk, pv, lk, lv)
    lens = np.array([T, 137], np.int32)
    out = kv.decode_attn(desc, torch.from_numpy(q).cuda(), pk, pv, lk, lv, torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    G = Hq // Hkv
    worst = 0.0
    for b in range(B):
        for h in range(Hkv):
            n = int(lens[b])
            Kl = qo.dequantize_rows(*qo.quantize_rows((K[b, :n, h].astype(np.float64) @ PKf[h]).astype(np.float32)))
            vc, vm = qo.quantize_rows((V[b, :n, h].astype(np.float64) @ PVf[h]).astype(np.float32))
            Vl = qo.dequantize_rows(vc, vm)
            qh = q[b, h * G:(h + 1) * G].astype(np.float64)
            ref = ko.decode_head_latent(qh, Kl, Vl, PKf[h], PVf[h], 1 / np.sqrt(d))
            # envelope of the half-float value weights (a tolerance, not a second reference)
            s_ = (qh @ PKf[h]) @ Kl.T / np.sqrt(d)
            w = np.exp(s_ - s_.max(1, keepdims=True))
            w /= w.sum(1, keepdims=True)
            mag = qo.dequantize_rows(vc, np.abs(vm))          # |step| c + |base| per row and channel
            u = 2.0 ** -11
            e_lat = (2 * u + u * u) * (w @ mag) + 2 * n * 2.0 ** -25 * mag.max()
            bound = e_lat @ np.abs(PVf[h]).T + 1e-4 * np.abs(ref).max()
            diff = np.abs(got[b, h * G:(h + 1) * G] - ref)
            assert (diff <= bound).all(), (b, h, float((diff / bound).max()))
            worst = max(worst, float((diff / bound).max()))
    say(f"[q43 exact storage] worst error / bound {worst:.3f}")


def test_q43_folded_and_two_stage(gpu):
    """The folded entry point and partials + combine run the same kernel on 4/3-bit caches."""
    import torch
    kv = _kv()
    cfg = LLAMA3_LAYER_32K.scaled(B=2, Hq=16, Hkv=2, T=700)
    case = _q43_case(cfg)
    lens = host.lengths(cfg)
    q = host.queries(cfg, 0, 0)
    lt = torch.from_numpy(lens).cuda()
    qd = torch.from_numpy(q).cuda()
    full = kv.decode_attn(case["desc"], qd, case["pk"], case["pv"], case["lk"], case["lv"], lt)
    ws = kv.alloc_workspace(case["desc"])
    kv.decode_partials(case["desc"], qd, case["pk"], case["lk"], case["lv"], lt, ws)
    two = torch.empty_like(full)
    kv.decode_combine(case["desc"], case["pv"], ws, two)
    # folded: q_lat = q P'_K (folded bases, fp32 on the device), o = o_lat P'_V^T
    rk = int(case["desc"].r_k[0])
    d = cfg.d
    PKf = case["pk"].view(cfg.Hkv, d, rk)
    q_lat = torch.stack([qd[:, i] @ PKf[i // cfg.G] for i in range(cfg.Hq)], 1).contiguous()
    o_lat = kv.decode_attn_latent(case["desc"], q_lat, case["lk"], case["lv"], lt)
    torch.cuda.synchronize()
    rv = int(case["desc"].r_v[0])
    PVf = case["pv"].view(cfg.Hkv, d, rv)
    back = torch.stack([o_lat[:, i, :rv] @ PVf[i // cfg.G].T for i in range(cfg.Hq)], 1)
    f, t2, bk = (x.cpu().numpy().astype(np.float64) for x in (full, two, back))
    assert np.abs(f - t2).max() <= 1e-6 * np.abs(f).max()
    assert np.abs(f - bk).max() <= 2e-4 * np.abs(f).max()
    _q43_check(case, f, q, lens)


def test_q43_rows_past_the_end_may_hold_nan_parameters(gpu):
    """Every byte of the caches starts as 0xFF (half-float parameters 0xFFFF are NaN), then
    300 of 320 rows are written: decode over lengths that end inside a tile must ignore the
    unwritten rows' parameters and codes."""
    import torch
    kv = _kv()
    cfg = LLAMA3_LAYER_32K.scaled(B=3, Hq=8, Hkv=2, T=320)
    rk, rv = host.ranks(cfg)
    PK, PV = host.bases(cfg)
    desc = kv.Desc(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.capacity, rk, rv, kv.BF16, kv.Q43)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    kv.hadamard_bases(desc, pk, pv)
    lk, lv = kv.alloc_cache(desc)
    lk.fill_(255)
    lv.fill_(255)
    gen = KVGenerator(cfg, 0)
    kv.prefill_compress(desc, gen.make("k", cfg.B, 300), gen.make("v", cfg.B, 300), 0, pk, pv, lk, lv)
    case = dict(cfg=cfg, desc=desc, pk=pk, pv=pv, lk=lk, lv=lv, PK=PK, PV=PV, stats=host.kv_stats(cfg, 0))
    q = host.queries(cfg, 0, 0)
    lens = np.array([300, 290, 37], np.int32)
    for split in (0, 64):
        got = _q43_decode(case, q, lens, split)
        assert np.isfinite(got).all(), split
        _q43_check(case, got, q, lens)
