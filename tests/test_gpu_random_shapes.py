"""GPU parity on seeded random shapes: head dims 32 to 256, per-head ranks, GQA groups of 1 to
16 query heads, ragged lengths with empty rows, explicit split lengths, fp32 / bf16 / 4/3-bit
latents, per-head and joint values. Every case is checked against the float64 oracle with the
same acceptance bounds as the fixed cases. On the same caches the one-launch, two-stage and folded
entry points must agree; caches grown by kvlr_append decode like prefilled ones; and bf16 per-head
caches take fused decode steps that must equal append followed by decode bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import joint as jo
from oracle import quant as qo
from synth import LLAMA3_LAYER_32K, host
from tests.gpu_cases import bases32, build_case, rel_inf_rows, say
from tests.test_gpu_fused_step import _run_steps
from tests.test_gpu_joint import _check as joint_check
from tests.test_gpu_joint import _decode as joint_decode
from tests.test_gpu_joint import _joint_case
from tests.test_gpu_parity import _check_rows, _decode
from tests.test_gpu_quant import _q43_case, _q43_check, _q43_decode

pytestmark = pytest.mark.gpu


def _kv():
    import rank_compressed_kv_kvlr_amd as kv
    return kv

# storage of each case: latent dtype, and "joint" for one value latent shared by every KV head
KINDS = ["bf16", "f32", "q43", "joint_bf16", "bf16", "f32", "bf16", "joint_bf16", "q43", "bf16",
         "joint_q43", "bf16", "f32", "joint_bf16", "bf16", "q43", "joint_f32", "bf16", "f32", "joint_bf16",
         "bf16", "q43", "joint_bf16", "bf16"]
HEAD_DIMS = [32, 64, 96, 128, 160, 192, 256]
GROUPS = [1, 2, 3, 4, 5, 6, 8, 16]
SPLITS = [0, 64, 128, 256, 512]


def draw(i: int):
    """Shape of case i: (kind, cfg, lens, split, joint rank or None), from its own seed."""
    g = np.random.default_rng(np.random.SeedSequence([9100, i]))
    kind = KINDS[i]
    joint = kind.startswith("joint")
    lat = kind.split("_")[-1]
    d = int(g.choice(HEAD_DIMS))
    Hkv = int(g.integers(1, 7))
    G = int(g.choice(GROUPS))
    if joint and lat == "bf16":   # the joint bf16 kernel holds at most 32 query heads of 8 KV heads
        G = min(G, 32 // Hkv)
    B = int(g.integers(1, 5))
    T = int(g.integers(1, 700))
    gran = 4 if lat == "f32" else 16
    rmax = min(d, 128)
    choices = tuple(sorted({int(x) for x in g.choice(np.arange(gran, rmax + 1, gran), size=3)}))
    in_dtype = str(g.choice(["bf16", "f32"])) if kind != "q43" else "bf16"   # the 4/3-bit builder takes bf16 rows
    cfg = LLAMA3_LAYER_32K.scaled(B=B, Hq=Hkv * G, Hkv=Hkv, d=d, T=T, rank_mode="per_head", rank_choices=choices,
                                  n_outliers=min(4, d), in_dtype=in_dtype,
                                  latent_dtype="f32" if lat == "f32" else "bf16")
    lens = g.integers(0, T + 1, size=B).astype(np.int32)
    lens[g.integers(0, B)] = T
    if B > 1:
        lens[g.integers(0, B)] = 0
    split = int(g.choice(SPLITS))
    rj = None
    if joint:
        jmax = min(Hkv * d, 128)
        rj = int(g.choice(np.arange(gran, jmax + 1, gran)))
    return kind, cfg, lens, split, rj


@pytest.mark.parametrize("i", range(len(KINDS)))
def test_random_shape_matches_oracle(gpu, i):
    kind, cfg, lens, split, rj = draw(i)
    say(f"[random {i}] {kind} B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} T={cfg.T} ranks={cfg.rank_choices} "
        f"in={cfg.in_dtype} lens={lens.tolist()} split={split} r_joint={rj}")
    q = host.queries(cfg, 0, 0)
    if kind.startswith("joint"):
        case = _joint_case(cfg, rj, latent=kind.split("_")[1])
        joint_check(case, joint_decode(case, q, lens, split), q, lens, diag_bound=1e-2)
    elif kind == "q43":
        case = _q43_case(cfg)
        _q43_check(case, _q43_decode(case, q, lens, split), q, lens)
    else:
        case = build_case(cfg, layer=1 + i)
        q = host.queries(cfg, 1 + i, 0)
        _check_rows(case, _decode(case, q, lens, split=split), q, lens,
                    diag_bound=5e-3 if cfg.latent_dtype == "bf16" else None)


# shapes at the limits of the descriptor: 64 KV heads, 16 query heads per KV head at
# head_dim 256 and rank 128, a one-row cache, the joint bf16 kernel's 32 x 8 heads
EXTREMES = [
    ("bf16", dict(B=1, Hq=64, Hkv=64, d=32, T=70, rank_choices=(16, 32)), [70]),
    ("f32", dict(B=1, Hq=64, Hkv=64, d=32, T=70, rank_choices=(4, 32), in_dtype="f32", latent_dtype="f32"), [70]),
    ("q43", dict(B=1, Hq=64, Hkv=64, d=64, T=70, rank_choices=(16, 64)), [70]),
    ("bf16", dict(B=1, Hq=64, Hkv=4, d=256, T=130, rank_choices=(128,)), [130]),
    ("f32", dict(B=1, Hq=64, Hkv=4, d=256, T=130, rank_choices=(128,), latent_dtype="f32"), [130]),
    ("bf16", dict(B=2, Hq=8, Hkv=2, d=128, T=1, rank_choices=(64,)), [1, 0]),
    ("q43", dict(B=2, Hq=8, Hkv=2, d=128, T=1, rank_choices=(64,)), [1, 0]),
    ("joint_bf16", dict(B=2, Hq=32, Hkv=8, d=256, T=150, rank_choices=(128,)), [150, 77]),
    ("joint_bf16", dict(B=1, Hq=8, Hkv=8, d=128, T=1, rank_choices=(16,)), [1]),
]


@pytest.mark.parametrize("n", range(len(EXTREMES)))
def test_extreme_shapes_match_oracle(gpu, n):
    kind, extra, lens = EXTREMES[n]
    lens = np.asarray(lens, np.int32)
    cfg = LLAMA3_LAYER_32K.scaled(rank_mode="per_head", n_outliers=4, **extra)
    say(f"[extreme {n}] {kind} {extra} lens={lens.tolist()}")
    q = host.queries(cfg, 0, 0)
    if kind.startswith("joint"):
        case = _joint_case(cfg, 128 if cfg.T > 1 else 16, latent=kind.split("_")[1])
        joint_check(case, joint_decode(case, q, lens), q, lens, diag_bound=1e-2)
    elif kind == "q43":
        case = _q43_case(cfg)
        _q43_check(case, _q43_decode(case, q, lens), q, lens)
    else:
        case = build_case(cfg)
        _check_rows(case, _decode(case, q, lens), q, lens, diag_bound=5e-3 if cfg.latent_dtype == "bf16" else None)


def _handles(kind, cfg, case):
    """(desc, P_K, P_V, lat_k, lat_v, host P_K per head as the kernels apply it, host value basis
    rows per head) of a case of any storage."""
    if kind.startswith("joint"):
        PV = [jo.joint_slice(case["PJ"], h, cfg.d) for h in range(cfg.Hkv)]
        return case["desc"], case["pk"], case["pj"], case["lk"], case["lv"], case["PK"], PV
    if kind == "q43":
        PK = [qo.fuse_bases(P) for P in bases32(case["PK"])]
        PV = [qo.fuse_bases(P) for P in bases32(case["PV"])]
        return case["desc"], case["pk"], case["pv"], case["lk"], case["lv"], PK, PV
    return case.desc, case.pk, case.pv, case.lat_k, case.lat_v, case.P32K, case.P32V


@pytest.mark.parametrize("i", range(len(KINDS)))
def test_random_shape_entry_points_agree(gpu, i):
    """On the same caches: decode_attn writes every output element (NaN-poisoned buffer) and
    zero rows for empty sequences; decode_partials + decode_combine give its result; the folded
    entry point, back-projected on the host, gives it too."""
    import torch
    kv = _kv()
    kind, cfg, lens, split, rj = draw(i)
    say(f"[random entry points {i}] {kind} B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} split={split}")
    if kind.startswith("joint"):
        case = _joint_case(cfg, rj, latent=kind.split("_")[1])
    elif kind == "q43":
        case = _q43_case(cfg)
    else:
        case = build_case(cfg)
    desc, pk, pv, lk, lv, PK, PV = _handles(kind, cfg, case)
    q = host.queries(cfg, 0, 0)
    qd = torch.from_numpy(q).cuda()
    lens_t = torch.from_numpy(lens).cuda()
    out = torch.full((cfg.B, cfg.Hq, cfg.d), float("nan"), device="cuda")
    kv.decode_attn(desc, qd, pk, pv, lk, lv, lens_t, out=out, split_tokens=split)
    ws = kv.alloc_workspace(desc, split)
    kv.decode_partials(desc, qd, pk, lk, lv, lens_t, ws, split_tokens=split)
    two = kv.decode_combine(desc, pv, ws, torch.full_like(out, float("nan")), split_tokens=split)
    rk_max = max(P.shape[1] for P in PK)
    q_lat = np.zeros((cfg.B, cfg.Hq, rk_max), np.float32)
    for qh in range(cfg.Hq):
        P = PK[qh // cfg.G]
        q_lat[:, qh, :P.shape[1]] = (q[:, qh].astype(np.float64) @ P).astype(np.float32)
    o_lat = kv.decode_attn_latent(desc, torch.from_numpy(q_lat).cuda(), lk, lv, lens_t, split_tokens=split)
    torch.cuda.synchronize()
    a = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(a).all(), "every output element is written"
    assert np.all(a[lens == 0] == 0), "empty sequences give zero rows"
    live = lens > 0
    err_two = float(rel_inf_rows(two.cpu().numpy().astype(np.float64)[live], a[live]).max()) if live.any() else 0.0
    ol = o_lat.cpu().numpy().astype(np.float64)
    folded = np.stack([ol[:, qh, :PV[qh // cfg.G].shape[1]] @ PV[qh // cfg.G].T for qh in range(cfg.Hq)], axis=1)
    err_fold = float(rel_inf_rows(folded[live], a[live]).max()) if live.any() else 0.0
    say(f"[random entry points {i}] two-stage {err_two:.2e} folded {err_fold:.2e}")
    # the two stages keep the fixed plan; where the one-launch call takes the balanced plan
    # (per-head ranks that differ) the sequences are cut elsewhere: weights round differently
    balanced = kv.decode_plan(desc, split)[1] == 0
    assert err_two <= (2e-5 if balanced else 1e-6), err_two
    # 4/3-bit values enter the value product with half-float weights: the two entry points
    # form q~ apart in its last bits, so a weight can round to the neighbouring half float,
    # up to 2^-10 of it, and in a short row one token can carry most of the output
    fold_bound = 1e-5 if kind.endswith("f32") else (2.0 ** -10 if kind.endswith("q43") else 1e-4)
    assert err_fold <= fold_bound, err_fold


@pytest.mark.parametrize("i", range(len(KINDS)))
def test_random_shape_append(gpu, i):
    """Prefill all but the last two rows, append those two (kvlr_append, one call per row), then
    decode over the whole cache against the oracle, which regenerates every row."""
    import torch
    kv = _kv()
    kind, cfg, lens, split, rj = draw(i)
    T = cfg.T
    n_pre = max(T - 2, 0)
    say(f"[random append {i}] {kind} B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} rows {n_pre} + {T - n_pre}")
    if kind.startswith("joint"):
        case = _joint_case(cfg, rj, latent=kind.split("_")[1], n_rows=n_pre, chunk=1024)
    elif kind == "q43":
        case = _q43_case(cfg, n_rows=n_pre, chunk=1024)
    else:
        case = build_case(cfg, n_rows=n_pre, chunk=1024)
    desc, pk, pv, lk, lv, _, _ = _handles(kind, cfg, case)
    from synth.device import KVGenerator
    gen = KVGenerator(cfg, 0)
    for t in range(n_pre, T):
        pos = torch.full((cfg.B,), t, dtype=torch.int32, device="cuda")
        kv.append(desc, gen.make("k", cfg.B, 1, t0=t)[:, 0].contiguous(), gen.make("v", cfg.B, 1, t0=t)[:, 0].contiguous(),
                  pos, pk, pv, lk, lv)
    q = host.queries(cfg, 0, 0)
    if kind.startswith("joint"):
        joint_check(case, joint_decode(case, q, lens, split), q, lens, diag_bound=1e-2)
    elif kind == "q43":
        _q43_check(case, _q43_decode(case, q, lens, split), q, lens)
    else:
        _check_rows(case, _decode(case, q, lens, split=split), q, lens,
                    diag_bound=5e-3 if cfg.latent_dtype == "bf16" else None)


@pytest.mark.parametrize("i", [i for i, k in enumerate(KINDS) if k == "bf16"][:4])
def test_random_shape_fused_step(gpu, i):
    """Two fused steps (append + attend in one launch) equal the two-call form bit for bit."""
    _, cfg, _, split, _ = draw(i)
    _run_steps(cfg.scaled(decode_steps=2), 2, split)
