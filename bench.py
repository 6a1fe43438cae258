#!/usr/bin/env python3
"""Decode-attention benchmark over a rank-compressed KV cache on one MI355X.

Workload (default): one Llama-3-8B-shaped attention layer at decode, batch 8,
32 query / 8 KV heads, head_dim 128, 32768 cached tokens per sequence,
ranks r_k = r_v = 64 per KV head, bf16 latents (synthetic seeded inputs,
4 key channels per head scaled x8). A step is one decode call: query
projection, latent scores, online softmax, value mix, split merge and P_V^T
back-projection for all 8 sequences, i.e. 8 new tokens.

Inputs are resident in HBM before timing. Steps alternate between two
independent cache replicas (1 GiB of latents) so that no step finds the
previous step's bytes in the 256 MB last-level cache.

Prints one JSON line with the throughput, the split kernel's roofline
(algorithmic bytes per launch over its average duration, from one HIP event
pair on the launch stream around the timed launches, against the 8 TB/s HBM
peak) and the float64 oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_traffic.json")
# sources of the dominant kernel (decode_split_bf16): the traffic counters belong to these
DECODE_SRC = [os.path.join(ROOT, "rank_compressed_kv_kvlr_amd", "csrc", f)
              for f in ("decode.hip", "decode_common.hpp", "kvlr_internal.hpp")]
METRIC = "compressed-KV decode attn: tokens/sec + achieved HBM GB/s (% of peak), 1 GPU"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--split-tokens", type=int, default=0, help="tokens per split (0: library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle CPU time")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-compression measurement")
    ap.add_argument("--no-q43", action="store_true", help="skip the 4/3-bit latent measurement")
    ap.add_argument("--no-joint", action="store_true", help="skip the joint-value measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads (ragged per-head ranks, 128K steps, 32 layers)")
    ap.add_argument("--traffic-reference", action="store_true",
                    help="also run a plain 1 GiB device copy (a known-size reference for HBM traffic counters)")
    return ap.parse_args()


def source_hash(paths):
    """sha256 (first 16 hex digits) over the concatenated sources of a kernel."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch from rocprofv3 counters, valid only for the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("decode_src_sha256_16") != source_hash(DECODE_SRC):
        return None
    return t.get("bytes_per_launch")


def _build(kv, torch, cfg, layer=0, n_rows=None, chunk=8192):
    """Device caches of one layer of a workload (seeded synthetic rows, prefill-compressed)."""
    from synth import host
    from synth.device import KVGenerator
    rk, rv = host.ranks(cfg, layer)
    PK, PV = host.bases(cfg, layer)
    desc = kv.Desc(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.capacity, rk, rv, kv.BF16, kv.BF16)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    lk, lv = kv.alloc_cache(desc)
    gen = KVGenerator(cfg, layer)
    n_rows = cfg.capacity if n_rows is None else n_rows
    for t0 in range(0, n_rows, chunk):
        n = min(chunk, n_rows - t0)
        kv.prefill_compress(desc, gen.make("k", cfg.B, n, t0=t0), gen.make("v", cfg.B, n, t0=t0), t0, pk, pv, lk, lv)
    return dict(desc=desc, pk=pk, pv=pv, lk=lk, lv=lv, rk=rk, rv=rv, gen=gen)


def _timed(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    return min(times)


def _graph_of(torch, fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def measure_workloads(kv, torch, np):
    """The other workloads, each with its own algorithmic bytes: one decode over ragged
    sequences with per-head ranks; 64 x (append + decode) over 128K rows; a 32-layer decode
    step. The last two also as one captured HIP graph replayed (launch gaps removed)."""
    from synth import LLAMA3_32_LAYERS, LONG_CONTEXT_128K, PER_HEAD_RAGGED, host
    out = {}
    print("[bench] workload per_head_ranks_ragged", file=sys.stderr, flush=True)
    cfg = PER_HEAD_RAGGED
    c = _build(kv, torch, cfg, chunk=4096)
    lens_np = host.lengths(cfg)
    lens = torch.from_numpy(lens_np).cuda()
    q = torch.from_numpy(host.queries(cfg)).cuda()
    ws = kv.alloc_workspace(c["desc"])
    o = torch.empty((cfg.B, cfg.Hq, cfg.d), device="cuda")
    nbytes = int(lens_np.astype(np.int64).sum()) * int((c["rk"] + c["rv"]).sum()) * 2
    call = lambda: kv.decode_attn(c["desc"], q, c["pk"], c["pv"], c["lk"], c["lv"], lens, out=o, workspace=ws)  # noqa: E731
    t = _timed(torch, lambda: [call() for _ in range(20)], 3) / 20
    fixed = lambda: kv.decode_attn(c["desc"], q, c["pk"], c["pv"], c["lk"], c["lv"], lens, out=o,  # noqa: E731
                                   workspace=ws, split_tokens=4096)
    t_fixed = _timed(torch, lambda: [fixed() for _ in range(20)], 3) / 20
    out[cfg.name] = {"us_per_call": t * 1e6, "bytes": nbytes, "GBps": nbytes / t / 1e9,
                     "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBPS, "tokens_per_s": cfg.B / t,
                     "plan": "balanced (the library's choice: the KV heads' ranks differ)",
                     "fixed_plan_4096_us_per_call": t_fixed * 1e6}
    del c, ws
    torch.cuda.empty_cache()

    print("[bench] workload long_context_128k", file=sys.stderr, flush=True)
    cfg = LONG_CONTEXT_128K
    T, S = cfg.T, cfg.decode_steps
    c = _build(kv, torch, cfg, n_rows=T, chunk=16384)
    ks = [c["gen"].make("k", cfg.B, 1, t0=T + s)[:, 0].contiguous() for s in range(S)]
    vs = [c["gen"].make("v", cfg.B, 1, t0=T + s)[:, 0].contiguous() for s in range(S)]
    qs = [torch.from_numpy(host.queries(cfg, 0, s)).cuda() for s in range(S)]
    pos = [torch.full((cfg.B,), T + s, dtype=torch.int32, device="cuda") for s in range(S)]
    lns = [torch.full((cfg.B,), T + s + 1, dtype=torch.int32, device="cuda") for s in range(S)]
    ws = kv.alloc_workspace(c["desc"])
    o = torch.empty((cfg.B, cfg.Hq, cfg.d), device="cuda")

    def loop():
        for s in range(S):
            kv.append(c["desc"], ks[s], vs[s], pos[s], c["pk"], c["pv"], c["lk"], c["lv"])
            kv.decode_attn(c["desc"], qs[s], c["pk"], c["pv"], c["lk"], c["lv"], lns[s], out=o, workspace=ws)
    def fused_loop():   # the same steps through kvlr_append_decode_attn (one launch per step)
        for s in range(S):
            kv.append_decode_attn(c["desc"], ks[s], vs[s], pos[s], qs[s], c["pk"], c["pv"], c["lk"], c["lv"], lns[s],
                                  out=o, workspace=ws)
    t_e = _timed(torch, loop, 3)
    g = _graph_of(torch, loop)
    t_g = _timed(torch, g.replay, 3)
    t_f = _timed(torch, fused_loop, 3)
    gf = _graph_of(torch, fused_loop)
    t_fg = _timed(torch, gf.replay, 3)
    rk, rv = int(c["rk"][0]), int(c["rv"][0])
    nbytes = sum(T + s + 1 for s in range(S)) * cfg.B * cfg.Hkv * (rk + rv) * 2
    out[cfg.name] = {"steps": S, "eager_us_per_step": t_e / S * 1e6, "graph_us_per_step": t_g / S * 1e6,
                     "fused_eager_us_per_step": t_f / S * 1e6, "fused_graph_us_per_step": t_fg / S * 1e6,
                     "bytes": nbytes, "graph_GBps": nbytes / t_g / 1e9, "graph_hbm_frac": nbytes / t_g / 1e9 / HBM_PEAK_GBPS,
                     "graph_tokens_per_s": cfg.B * S / t_g, "fused_graph_tokens_per_s": cfg.B * S / t_fg}
    del c, ws, g, gf
    torch.cuda.empty_cache()

    print("[bench] workload llama3_8b_32_layers", file=sys.stderr, flush=True)
    cfg = LLAMA3_32_LAYERS
    layers = []
    for layer in range(cfg.n_layers):
        c = _build(kv, torch, cfg, layer=layer)
        c["q"] = torch.from_numpy(host.queries(cfg, layer)).cuda()
        c["ws"] = kv.alloc_workspace(c["desc"])
        c["o"] = torch.empty((cfg.B, cfg.Hq, cfg.d), device="cuda")
        del c["gen"]
        layers.append(c)
    lens = torch.from_numpy(host.lengths(cfg)).cuda()

    def step():
        for c in layers:
            kv.decode_attn(c["desc"], c["q"], c["pk"], c["pv"], c["lk"], c["lv"], lens, out=c["o"], workspace=c["ws"])
    t_e = _timed(torch, step, 5)
    g = _graph_of(torch, step)
    t_g = _timed(torch, g.replay, 5)
    nbytes = sum(cfg.B * cfg.T * int((c["rk"] + c["rv"]).sum()) * 2 for c in layers)
    out[cfg.name] = {"layers": cfg.n_layers, "eager_ms_per_step": t_e * 1e3, "graph_ms_per_step": t_g * 1e3,
                     "bytes": nbytes, "graph_GBps": nbytes / t_g / 1e9, "graph_hbm_frac": nbytes / t_g / 1e9 / HBM_PEAK_GBPS,
                     "graph_tokens_per_s": cfg.B / t_g}
    del layers, g
    torch.cuda.empty_cache()
    return out


def measure_joint(kv, torch, np, cfg, gen, q, lens, steps, warmup, r_joint=128):
    """The same workload with STAR-KV's hybrid decomposition: keys per head (r_k = 64),
    values of all 8 heads in one joint latent of rank 128 per token (0.625x the bytes)."""
    from synth import host
    B, T, Hkv, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    rk, _ = host.ranks(cfg)
    PK, _ = host.bases(cfg)
    desc = kv.Desc(B, cfg.Hq, Hkv, d, cfg.capacity, rk, [r_joint] * Hkv, kv.BF16, kv.BF16, kv.VALUES_JOINT)
    pk, pj = kv.pack_bases(PK), kv.pack_bases([host.joint_value_basis(cfg, r_joint)])
    print("[bench] building 2 replicas with joint values", file=sys.stderr, flush=True)
    reps = []
    for _ in range(2):
        lk, lv = kv.alloc_cache(desc)
        for t0 in range(0, T, 8192):
            n = min(8192, T - t0)
            kv.prefill_compress(desc, gen.make("k", B, n, t0=t0), gen.make("v", B, n, t0=t0), t0, pk, pj, lk, lv)
        reps.append((lk, lv))
    ws = kv.alloc_workspace(desc)
    out = torch.empty((B, cfg.Hq, d), dtype=torch.float32, device="cuda")
    for k in range(warmup):
        lk, lv = reps[k % 2]
        kv.decode_attn(desc, q, pk, pj, lk, lv, lens, out=out, workspace=ws)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t_start = time.perf_counter()
    for k in range(steps):
        lk, lv = reps[k % 2]
        evs[k][0].record()
        kv.decode_attn(desc, q, pk, pj, lk, lv, lens, out=out, workspace=ws)
        evs[k][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    us = float(np.mean([e[0].elapsed_time(e[1]) * 1e3 for e in evs]))
    nbytes = B * T * (int(rk.sum()) + r_joint) * 2
    return {"entry": "kvlr_decode_attn, value_mode KVLR_VALUES_JOINT", "r_k": int(rk[0]), "r_joint": r_joint,
            "bytes_per_launch": nbytes, "launch_us_mean": us, "GBps": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, "tokens_per_s": B * steps / elapsed,
            "note": "three launches: query projection, one split kernel per (split, batch row) that streams every head's keys and the shared value latent once, and a merge per (query head, batch row)"}


def measure_stream_ceiling(torch, np):
    """Achievable HBM read bandwidth on this device: a non-temporal streaming read of a 1 GiB
    buffer (above the 256 MB last-level cache) in 1, 2, 4 or 8 contiguous chunks per compute
    unit; the best launch shape's median over 7 event-timed passes."""
    from synth.device import stream_read
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    src.fill_(1.0)
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    best = 0.0
    for wgs in (256, 512, 1024, 2048):
        for _ in range(2):
            stream_read(src, sink, wgs)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(7)]
        for e in evs:
            e[0].record()
            stream_read(src, sink, wgs)
            e[1].record()
        torch.cuda.synchronize()
        us = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in evs]))
        best = max(best, (1 << 30) / (us * 1e-6) / 1e9)
    del src, sink
    return best


def measure_q43(kv, torch, np, cfg, gen, q, lens, steps, warmup):
    """The same workload with mixed 4/3-bit latents (4-bit outlier, 3-bit inlier block per
    token, block-wise Hadamard folded into the bases): kvlr_decode_attn launches timed with
    HIP events, two cache replicas alternating."""
    from synth import host
    B, T, Hkv, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    rk, rv = host.ranks(cfg)
    PK, PV = host.bases(cfg)
    desc = kv.Desc(B, cfg.Hq, Hkv, d, cfg.capacity, rk, rv, kv.BF16, kv.Q43)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    kv.hadamard_bases(desc, pk, pv)
    print("[bench] building 2 replicas with 4/3-bit latents", file=sys.stderr, flush=True)
    reps = []
    for _ in range(2):
        lk, lv = kv.alloc_cache(desc)
        for t0 in range(0, T, 8192):
            n = min(8192, T - t0)
            kv.prefill_compress(desc, gen.make("k", B, n, t0=t0), gen.make("v", B, n, t0=t0), t0, pk, pv, lk, lv)
        reps.append((lk, lv))
    ws = kv.alloc_workspace(desc)
    out = torch.empty((B, cfg.Hq, d), dtype=torch.float32, device="cuda")
    for k in range(warmup):
        lk, lv = reps[k % 2]
        kv.decode_attn(desc, q, pk, pv, lk, lv, lens, out=out, workspace=ws)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t_start = time.perf_counter()
    for k in range(steps):
        lk, lv = reps[k % 2]
        evs[k][0].record()
        kv.decode_attn(desc, q, pk, pv, lk, lv, lens, out=out, workspace=ws)
        evs[k][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    us = float(np.mean([e[0].elapsed_time(e[1]) * 1e3 for e in evs]))
    row_k = sum(kv.q43_row_bytes(int(r)) for r in rk)
    row_v = sum(kv.q43_row_bytes(int(r)) for r in rv)
    nbytes = B * T * (row_k + row_v)
    return {"entry": "kvlr_decode_attn on KVLR_Q43 caches", "kernel": "decode_split_q43<64>",
            "bytes_per_launch": nbytes, "launch_us_mean": us, "GBps": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, "tokens_per_s": B * steps / elapsed,
            "bytes_vs_bf16": nbytes / (B * T * int((rk + rv).sum()) * 2)}


def cpu_baseline(cfg, seconds):
    """The float64 oracle's latent-order decode on a bounded sample of the workload."""
    import numpy as np
    import oracle
    from synth import host
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:  # pragma: no cover
        blas = []
    threads = max([n for _, n in blas if n] or [1])
    b, h = 0, 0
    T, G = cfg.T, cfg.G
    PK, PV = host.bases(cfg, 0)
    P32K, P32V = [p.astype(np.float32).astype(np.float64) for p in PK], [p.astype(np.float32).astype(np.float64) for p in PV]
    stats = host.kv_stats(cfg, 0)
    K = host.decode_to_f64(host.kv_rows(cfg, 0, "k", b, 0, T, heads=[h], stats=stats), cfg.in_dtype)[:, 0]
    V = host.decode_to_f64(host.kv_rows(cfg, 0, "v", b, 0, T, heads=[h], stats=stats), cfg.in_dtype)[:, 0]
    lat_k = oracle.bf16_round(oracle.compress(K, P32K[h]))
    lat_v = oracle.bf16_round(oracle.compress(V, P32V[h]))
    q = host.queries(cfg, 0, 0)[b, h * G:(h + 1) * G].astype(np.float64)
    scale = 1 / np.sqrt(cfg.d)
    oracle.decode_head_latent(q, lat_k, lat_v, P32K[h], P32V[h], scale)   # warm-up
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_head_latent(q, lat_k, lat_v, P32K[h], P32V[h], scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_head = el / reps
    # definition order (reconstruct K~, V~ then attend), once, for context
    t1 = time.perf_counter()
    oracle.decode_head_reconstructed(q, K, V, P32K[h], P32V[h], scale)
    per_head_def = time.perf_counter() - t1
    per_token = per_head * cfg.Hkv           # one token = one batch row over all KV heads
    return {
        "value": 1.0 / per_token, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"oracle latent-order decode (float64 numpy) of batch row 0, KV head 0 "
                   f"({G} query heads) over {T} bf16-rounded latents, {reps} repetitions in {el:.1f} s; "
                   f"scaled x{cfg.Hkv} KV heads to one token"),
        "definition_order_tokens_per_s": 1.0 / (per_head_def * cfg.Hkv),
        "blas": blas,
        "cpu_model": _cpu_model(),
        "host_threads_available": len(os.sched_getaffinity(0)),
    }


def _cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import rank_compressed_kv_kvlr_amd as kv
    from synth import LLAMA3_LAYER_32K, host
    from synth.device import KVGenerator

    cfg = LLAMA3_LAYER_32K
    B, T, Hkv, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    rk, rv = host.ranks(cfg)
    PK, PV = host.bases(cfg)
    desc = kv.Desc(B, cfg.Hq, Hkv, d, cfg.capacity, rk, rv, kv.BF16, kv.BF16)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    gen = KVGenerator(cfg, 0)
    print(f"[bench] building 2 cache replicas of {cfg.name}", file=sys.stderr, flush=True)

    replicas = []
    prefill = None
    for rep in range(2):
        lat_k, lat_v = kv.alloc_cache(desc)
        K = gen.make("k", B, T)
        V = gen.make("v", B, T)
        kv.prefill_compress(desc, K, V, 0, pk, pv, lat_k, lat_v)
        if rep == 0 and not args.no_prefill:
            # prefill compression of all 32768 tokens (both K and V), timed with HIP events
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            times = []
            for _ in range(5):
                ev[0].record()
                kv.prefill_compress(desc, K, V, 0, pk, pv, lat_k, lat_v)
                ev[1].record()
                torch.cuda.synchronize()
                times.append(ev[0].elapsed_time(ev[1]) * 1e-3)
            t = float(np.median(times))
            nbytes = B * T * Hkv * (2 * d * 2 + (int(rk[0]) + int(rv[0])) * 2)
            flops = 2.0 * B * T * Hkv * d * (int(rk[0]) + int(rv[0]))
            prefill = {"tokens": B * T, "us": t * 1e6, "GBps": nbytes / t / 1e9,
                       "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBPS,
                       "mfma_util": flops / t / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                       "note": "MFMA utilisation counts useful flops; the kernel issues 2x (basis high/low parts)"}
        del K, V
        replicas.append((lat_k, lat_v))
    torch.cuda.synchronize()

    q = torch.from_numpy(host.queries(cfg, 0, 0)).cuda()
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    split = args.split_tokens
    ws = kv.alloc_workspace(desc, split)
    out = torch.empty((B, cfg.Hq, d), dtype=torch.float32, device="cuda")
    n_splits, split_len = kv.decode_plan(desc, split)

    def step(k, evs=None):
        # one kvlr_decode_attn call = one kernel launch (split workgroups merge in the last arrival)
        lk, lv = replicas[k % 2]
        if evs is not None:
            evs[0].record()
        kv.decode_attn(desc, q, pk, pv, lk, lv, lens, out=out, workspace=ws, split_tokens=split)
        if evs is not None:
            evs[1].record()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # headline: exactly K steps, nothing between the launches; a HIP event pair on the launch
    # stream around the same region gives the kernel's average duration (region / K)
    region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    region[0].record()
    for k in range(args.steps):
        step(k)
    region[1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region_us = region[0].elapsed_time(region[1]) * 1e3
    # spread: the same K steps again, each launch bracketed by its own event pair (which adds the
    # events' own overhead to every launch, so these durations run a few microseconds long)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(k, evs[k])
    torch.cuda.synchronize()

    # folded form (q_lat = q P_K in, o_lat out, P_V^T left to the caller's output projection)
    q_lat = torch.zeros((B, cfg.Hq, int(rk.max())), dtype=torch.float32, device="cuda")
    rk_pre = np.concatenate([[0], np.cumsum(rk)])
    for i in range(cfg.Hq):
        h = i // cfg.G
        q_lat[:, i, :int(rk[h])] = q[:, i] @ pk[d * int(rk_pre[h]): d * int(rk_pre[h + 1])].view(d, int(rk[h]))
    o_lat = torch.empty((B, cfg.Hq, int(rv.max())), dtype=torch.float32, device="cuda")
    fevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        lk, lv = replicas[k % 2]
        fevs[k][0].record()
        kv.decode_attn_latent(desc, q_lat, lk, lv, lens, o_lat=o_lat, workspace=ws, split_tokens=split)
        fevs[k][1].record()
    torch.cuda.synchronize()
    folded_us = float(np.mean([e[0].elapsed_time(e[1]) * 1e3 for e in fevs]))

    workloads = None
    if not args.no_workloads:
        workloads = measure_workloads(kv, torch, np)
    joint = None
    if not args.no_joint:
        joint = measure_joint(kv, torch, np, cfg, gen, q, lens, args.steps, args.warmup)
    q43 = None
    if not args.no_q43:
        q43 = measure_q43(kv, torch, np, cfg, gen, q, lens, args.steps, args.warmup)

    stream_ceiling = measure_stream_ceiling(torch, np)

    if args.traffic_reference:
        from synth.device import copy as device_copy
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            device_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst

    split_us = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
    alg_bytes = B * T * int((rk + rv).sum()) * 2     # latent bytes read per launch
    launch_us = region_us / args.steps               # average launch duration over the timed region
    split_mean_s = launch_us * 1e-6
    achieved = alg_bytes / split_mean_s / 1e9
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = B * args.steps / elapsed
    traffic = load_traffic()

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "cached_tokens": T, "q_heads": cfg.Hq, "kv_heads": Hkv,
                   "head_dim": d, "r_k": int(rk[0]), "r_v": int(rv[0]), "latents": "bf16",
                   "splits": n_splits, "split_tokens": split_len},
        "step_hbm_GBps": alg_bytes / (elapsed / args.steps) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "stream_read_ceiling_GBps": stream_ceiling, "frac_of_stream_read": achieved / stream_ceiling,
                     "kernel": "decode_split_bf16<64, 32> (kvlr_decode_attn, fixed split plan, merge fused)", "bytes_per_launch": alg_bytes,
                     "launch_us_mean": launch_us,
                     "timing": "one HIP event pair on the launch stream around the K timed launches",
                     "bracketed_launch_us_mean": float(split_us.mean()),
                     "bracketed_launch_us_p10": float(np.percentile(split_us, 10)),
                     "bracketed_launch_us_p90": float(np.percentile(split_us, 90))},
    }
    result["folded"] = {"entry": "kvlr_decode_attn_latent", "launch_us_mean": folded_us,
                        "GBps": alg_bytes / (folded_us * 1e-6) / 1e9}
    if q43 is not None:
        result["q43"] = q43
    if joint is not None:
        result["joint_values"] = joint
    if workloads is not None:
        result["workloads"] = workloads
    if prefill is not None:
        result["prefill"] = prefill
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
