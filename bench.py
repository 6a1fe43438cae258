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
COMPRESS_COUNTERS = os.path.join(ROOT, "profiles", "compress_counters.json")
COMPRESS_SRC = [os.path.join(ROOT, "rank_compressed_kv_kvlr_amd", "csrc", f) for f in ("compress.hip", "kvlr_internal.hpp")]
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
                    help="skip the other workloads (single head fp32, ragged per-head ranks, 128K, 32 layers)")
    ap.add_argument("--workload", default="all",
                    choices=["all", "headline", "single_head_f32", "per_head_ranks_ragged", "long_context_128k",
                             "llama3_8b_32_layers", "q43", "joint"],
                    help="run only this part (for profiling one workload at a time); default: everything")
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


Q43_COUNTERS = os.path.join(ROOT, "profiles", "decode_split_q43_counters.json")
# VALU issue rate of the chip: 256 CUs x 4 SIMDs x 2.4 GHz / 4 cycles per wave64 instruction
VALU_ISSUE_PEAK_PER_US = 256 * 4 * 2400 / 4


def q43_alu_roofline(median_us):
    """The 4/3-bit decode against the VALU issue rate: VALU instructions per launch from the
    rocprofv3 counters (valid only for the current decode source) over the measured time."""
    try:
        with open(Q43_COUNTERS) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("decode_src_sha256_16") != source_hash(DECODE_SRC):
        return None
    achieved = t["valu_instr_per_launch"] / median_us
    return {"bound": "alu", "achieved": achieved, "peak": VALU_ISSUE_PEAK_PER_US,
            "unit": "VALU wave64 instructions per us", "frac": achieved / VALU_ISSUE_PEAK_PER_US,
            "valu_instr_per_launch": t["valu_instr_per_launch"], "source": "profiles/decode_split_q43_counters.json"}


def compress_counters(workload):
    """MFMA busy share and HBM bytes of prefill compression on `workload` from rocprofv3 counters
    (profiles/), valid only for the current compression source."""
    try:
        with open(COMPRESS_COUNTERS) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("compress_src_sha256_16") != source_hash(COMPRESS_SRC):
        return None
    return t.get("workloads", {}).get(workload)


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


def event_times(torch, np, fn, n, warmup=3):
    """n calls fn(k), each bracketed by its own HIP event pair on the current stream (the stream
    the library launches on); returns the durations in microseconds."""
    for k in range(warmup):
        fn(k)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for k in range(n):
        evs[k][0].record()
        fn(k)
        evs[k][1].record()
    torch.cuda.synchronize()
    return np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evs])


def region_us(torch, fn, n):
    """One event pair around n back-to-back calls fn(k): the average duration per call (us)."""
    fn(0)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for k in range(n):
        fn(k)
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) * 1e3 / n


def spread(np, us):
    """Median, p10, p90 and mean of event-pair durations (us)."""
    return {"median_us": float(np.median(us)), "p10_us": float(np.percentile(us, 10)),
            "p90_us": float(np.percentile(us, 90)), "mean_us": float(np.mean(us)), "calls": int(len(us))}


def with_rates(np, st, nbytes, tokens):
    """Add GB/s, fraction of the HBM peak and tokens/s at the median duration."""
    t = st["median_us"] * 1e-6
    st.update({"bytes": int(nbytes), "GBps": nbytes / t / 1e9, "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBPS,
               "tokens_per_s": tokens / t})
    return st


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


def measure_single_head(kv, torch, np):
    """single_head_f32: B=1, one head, T=2048, r=32/32, fp32 latents (0.5 MiB, cache-resident):
    decode latency per call."""
    from synth import SINGLE_HEAD_F32, host
    from synth.device import KVGenerator
    cfg = SINGLE_HEAD_F32
    print("[bench] workload single_head_f32", file=sys.stderr, flush=True)
    rk, rv = host.ranks(cfg)
    PK, PV = host.bases(cfg)
    desc = kv.Desc(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.capacity, rk, rv, kv.F32, kv.F32)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    lk, lv = kv.alloc_cache(desc)
    gen = KVGenerator(cfg, 0)
    K, V = gen.make("k", cfg.B, cfg.T), gen.make("v", cfg.B, cfg.T)
    comp = event_times(torch, np, lambda k: kv.prefill_compress(desc, K, V, 0, pk, pv, lk, lv), 50)
    q = torch.from_numpy(host.queries(cfg)).cuda()
    lens = torch.from_numpy(host.lengths(cfg)).cuda()
    ws = kv.alloc_workspace(desc)
    o = torch.empty((cfg.B, cfg.Hq, cfg.d), device="cuda")
    us = event_times(torch, np, lambda k: kv.decode_attn(desc, q, pk, pv, lk, lv, lens, out=o, workspace=ws), 200)
    st = with_rates(np, spread(np, us), cfg.T * (int(rk[0]) + int(rv[0])) * 4, cfg.B)
    st["note"] = "latency-bound (0.5 MiB of latents, cache-resident): reported in us, not as a share of HBM"
    st["prefill_compress_median_us"] = float(np.median(comp))
    return st


def measure_ragged(kv, torch, np, n_rep=3):
    """per_head_ranks_ragged: one decode over ragged sequences with per-head ranks, the library's
    plan (balanced), rotating n_rep cache replicas (n_rep x 290 MB, above the 256 MB last-level
    cache) so that no call finds its bytes in cache; the fixed plan beside it."""
    from synth import PER_HEAD_RAGGED, host
    print("[bench] workload per_head_ranks_ragged", file=sys.stderr, flush=True)
    cfg = PER_HEAD_RAGGED
    c = _build(kv, torch, cfg, chunk=4096)
    reps = [(c["lk"], c["lv"])] + [(c["lk"].clone(), c["lv"].clone()) for _ in range(n_rep - 1)]
    lens_np = host.lengths(cfg)
    lens = torch.from_numpy(lens_np).cuda()
    q = torch.from_numpy(host.queries(cfg)).cuda()
    ws = kv.alloc_workspace(c["desc"])
    o = torch.empty((cfg.B, cfg.Hq, cfg.d), device="cuda")
    nbytes = int(lens_np.astype(np.int64).sum()) * int((c["rk"] + c["rv"]).sum()) * 2

    def call(k, split=0):
        lk, lv = reps[k % n_rep]
        kv.decode_attn(c["desc"], q, c["pk"], c["pv"], lk, lv, lens, out=o, workspace=ws, split_tokens=split)
    st = with_rates(np, spread(np, event_times(torch, np, call, 60)), nbytes, cfg.B)
    st["region_us_per_call"] = region_us(torch, call, 60)
    st["plan"] = "balanced (the library's choice: the KV heads' ranks differ)"
    st["replicas"] = n_rep
    st["fixed_plan_4096"] = spread(np, event_times(torch, np, lambda k: call(k, 4096), 60))
    del c, reps, ws
    torch.cuda.empty_cache()
    return st


def measure_long_context(kv, torch, np):
    """long_context_128k: prefill compression of 2 x 131072 tokens (r_k = 48, r_v = 80), then
    64 x (append one token + decode over all rows), eager as two calls and as the fused step, and
    each loop also as one captured HIP graph."""
    from synth import LONG_CONTEXT_128K, host
    from synth.device import KVGenerator
    print("[bench] workload long_context_128k", file=sys.stderr, flush=True)
    cfg = LONG_CONTEXT_128K
    T, S, B, Hkv, d = cfg.T, cfg.decode_steps, cfg.B, cfg.Hkv, cfg.d
    rk, rv = host.ranks(cfg)
    PK, PV = host.bases(cfg)
    desc = kv.Desc(B, cfg.Hq, Hkv, d, cfg.capacity, rk, rv, kv.BF16, kv.BF16)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    lk, lv = kv.alloc_cache(desc)
    gen = KVGenerator(cfg, 0)
    K, V = gen.make("k", B, T), gen.make("v", B, T)
    out = {}
    pre = event_times(torch, np, lambda k: kv.prefill_compress(desc, K, V, 0, pk, pv, lk, lv), 20, warmup=2)
    r_sum = int(rk[0]) + int(rv[0])
    pbytes = B * T * Hkv * (2 * d * 2 + r_sum * 2)
    flops = 2.0 * B * T * Hkv * d * r_sum
    st = with_rates(np, spread(np, pre), pbytes, B * T)
    st["useful_TFLOPs"] = flops / (st["median_us"] * 1e-6) / 1e12
    st["mfma_useful_frac"] = st["useful_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS
    st["kernel"] = "compress_bf16_mfma"
    st["counters"] = compress_counters("long_context_128k")
    st["note"] = ("bytes: K and V read (bf16) plus latents written; flops 2 d (r_k + r_v) per token and head; "
                  "counters: rocprofv3 MFMA busy share and raw EA bytes per call (profiles/)")
    out["prefill"] = st
    del K, V
    ks = [gen.make("k", B, 1, t0=T + s)[:, 0].contiguous() for s in range(S)]
    vs = [gen.make("v", B, 1, t0=T + s)[:, 0].contiguous() for s in range(S)]
    qs = [torch.from_numpy(host.queries(cfg, 0, s)).cuda() for s in range(S)]
    pos = [torch.full((B,), T + s, dtype=torch.int32, device="cuda") for s in range(S)]
    lns = [torch.full((B,), T + s + 1, dtype=torch.int32, device="cuda") for s in range(S)]
    ws = kv.alloc_workspace(desc)
    o = torch.empty((B, cfg.Hq, d), device="cuda")

    def two_calls(s):
        kv.append(desc, ks[s], vs[s], pos[s], pk, pv, lk, lv)
        kv.decode_attn(desc, qs[s], pk, pv, lk, lv, lns[s], out=o, workspace=ws)

    def fused(s):
        kv.append_decode_attn(desc, ks[s], vs[s], pos[s], qs[s], pk, pv, lk, lv, lns[s], out=o, workspace=ws)
    step_bytes = np.array([(T + s + 1) * B * Hkv * r_sum * 2 for s in range(S)])
    nbytes = int(step_bytes.mean())
    for name, fn in (("two_calls", two_calls), ("fused", fused)):
        st = with_rates(np, spread(np, event_times(torch, np, lambda k: fn(k % S), S, warmup=2)), nbytes, B)
        g = _graph_of(torch, lambda: [fn(s) for s in range(S)])
        gt = event_times(torch, np, lambda k: g.replay(), 5, warmup=1)
        st["graph_us_per_step"] = float(np.median(gt)) / S
        st["graph_tokens_per_s"] = B * S / (float(np.median(gt)) * 1e-6)
        out[name] = st
        del g
    out["steps"] = S
    out["bytes_per_step_mean"] = nbytes
    del lk, lv, ws
    torch.cuda.empty_cache()
    return out


def measure_32_layers(kv, torch, np):
    """llama3_8b_32_layers: 32 independent decodes (one per layer, each with its own bases and
    ranks), timed per whole step: as one kvlr_decode_attn_layers call (2 lanes; also 4) and as
    one kvlr_decode_attn per layer, each eager and as one captured HIP graph."""
    from synth import LLAMA3_32_LAYERS, host
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

    def step(k=0):
        for c in layers:
            kv.decode_attn(c["desc"], c["q"], c["pk"], c["pv"], c["lk"], c["lv"], lens, out=c["o"], workspace=c["ws"])
    entries = [dict(desc=c["desc"], q=c["q"], P_K=c["pk"], P_V=c["pv"], lat_k=c["lk"], lat_v=c["lv"],
                    seq_lens=lens, out=c["o"], workspace=c["ws"]) for c in layers]

    def one_call(lanes):
        return lambda k=0: kv.decode_attn_layers(entries, lanes=lanes)
    nbytes = sum(cfg.B * cfg.T * int((c["rk"] + c["rv"]).sum()) * 2 for c in layers)
    # the step as one kvlr_decode_attn_layers call over 2 lanes (layers overlap), eager and as a graph
    st = with_rates(np, spread(np, event_times(torch, np, one_call(2), 7, warmup=2)), nbytes, cfg.B)
    st["entry"] = "kvlr_decode_attn_layers, 2 lanes"
    g = _graph_of(torch, one_call(2))
    st["graph"] = with_rates(np, spread(np, event_times(torch, np, lambda k: g.replay(), 7, warmup=2)), nbytes, cfg.B)
    st["lanes_4"] = with_rates(np, spread(np, event_times(torch, np, one_call(4), 7, warmup=2)), nbytes, cfg.B)
    # one kvlr_decode_attn per layer on one stream, eager and as a graph
    st["per_layer_calls"] = with_rates(np, spread(np, event_times(torch, np, step, 7, warmup=2)), nbytes, cfg.B)
    g2 = _graph_of(torch, step)
    st["per_layer_calls"]["graph"] = with_rates(np, spread(np, event_times(torch, np, lambda k: g2.replay(), 7,
                                                                           warmup=2)), nbytes, cfg.B)
    st["layers"] = cfg.n_layers
    del layers, entries, g, g2
    torch.cuda.empty_cache()
    return st


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

    def call(k):
        lk, lv = reps[k % 2]
        kv.decode_attn(desc, q, pk, pj, lk, lv, lens, out=out, workspace=ws)
    nbytes = B * T * (int(rk.sum()) + r_joint) * 2
    st = with_rates(np, spread(np, event_times(torch, np, call, steps, warmup)), nbytes, B)
    st.update({"entry": "kvlr_decode_attn, value_mode KVLR_VALUES_JOINT", "r_k": int(rk[0]), "r_joint": r_joint,
               "region_us_per_call": region_us(torch, call, steps)})
    return st


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

    def call(k):
        lk, lv = reps[k % 2]
        kv.decode_attn(desc, q, pk, pv, lk, lv, lens, out=out, workspace=ws)
    row_k = sum(kv.q43_row_bytes(int(r)) for r in rk)
    row_v = sum(kv.q43_row_bytes(int(r)) for r in rv)
    nbytes = B * T * (row_k + row_v)
    st = with_rates(np, spread(np, event_times(torch, np, call, steps, warmup)), nbytes, B)
    st.update({"entry": "kvlr_decode_attn on KVLR_Q43 caches", "kernel": "decode_split_q43",
               "region_us_per_call": region_us(torch, call, steps),
               "bytes_vs_bf16": nbytes / (B * T * int((rk + rv).sum()) * 2),
               "alu_roofline": q43_alu_roofline(st["median_us"])})
    return st


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

    want = args.workload
    run = lambda part: want == "all" or want == part   # noqa: E731
    cfg = LLAMA3_LAYER_32K
    B, T, Hkv, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    rk, rv = host.ranks(cfg)
    PK, PV = host.bases(cfg)
    desc = kv.Desc(B, cfg.Hq, Hkv, d, cfg.capacity, rk, rv, kv.BF16, kv.BF16)
    pk, pv = kv.pack_bases(PK), kv.pack_bases(PV)
    gen = KVGenerator(cfg, 0)
    q = torch.from_numpy(host.queries(cfg, 0, 0)).cuda()
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    alg_bytes = B * T * int((rk + rv).sum()) * 2     # latent bytes read per launch
    result = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
              "config": {"workload": cfg.name, "batch": B, "cached_tokens": T, "q_heads": cfg.Hq, "kv_heads": Hkv,
                         "head_dim": d, "r_k": int(rk[0]), "r_v": int(rv[0]), "latents": "bf16"}}

    if run("headline"):
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
                pre = event_times(torch, np, lambda k: kv.prefill_compress(desc, K, V, 0, pk, pv, lat_k, lat_v), 10, 1)
                nbytes = B * T * Hkv * (2 * d * 2 + (int(rk[0]) + int(rv[0])) * 2)
                flops = 2.0 * B * T * Hkv * d * (int(rk[0]) + int(rv[0]))
                prefill = with_rates(np, spread(np, pre), nbytes, B * T)
                prefill["useful_TFLOPs"] = flops / (prefill["median_us"] * 1e-6) / 1e12
                prefill["mfma_useful_frac"] = prefill["useful_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS
                prefill["counters"] = compress_counters("llama3_8b_layer_32k")
            del K, V
            replicas.append((lat_k, lat_v))
        torch.cuda.synchronize()
        split = args.split_tokens
        ws = kv.alloc_workspace(desc, split)
        out = torch.empty((B, cfg.Hq, d), dtype=torch.float32, device="cuda")
        n_splits, split_len = kv.decode_plan(desc, split)

        def step(k):
            # one kvlr_decode_attn call = one kernel launch (split workgroups merge in the last arrival)
            lk, lv = replicas[k % 2]
            kv.decode_attn(desc, q, pk, pv, lk, lv, lens, out=out, workspace=ws, split_tokens=split)

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
        launch_us = region[0].elapsed_time(region[1]) * 1e3 / args.steps
        # spread: the same K steps again, each launch bracketed by its own event pair (which adds the
        # events' own overhead to every launch, so these durations run a few microseconds long)
        split_us = event_times(torch, np, step, args.steps, 0)

        # folded form (q_lat = q P_K in, o_lat out, P_V^T left to the caller's output projection)
        q_lat = torch.zeros((B, cfg.Hq, int(rk.max())), dtype=torch.float32, device="cuda")
        rk_pre = np.concatenate([[0], np.cumsum(rk)])
        for i in range(cfg.Hq):
            h = i // cfg.G
            q_lat[:, i, :int(rk[h])] = q[:, i] @ pk[d * int(rk_pre[h]): d * int(rk_pre[h + 1])].view(d, int(rk[h]))
        o_lat = torch.empty((B, cfg.Hq, int(rv.max())), dtype=torch.float32, device="cuda")

        def folded(k):
            lk, lv = replicas[k % 2]
            kv.decode_attn_latent(desc, q_lat, lk, lv, lens, o_lat=o_lat, workspace=ws, split_tokens=split)
        fst = with_rates(np, spread(np, event_times(torch, np, folded, args.steps, 0)), alg_bytes, B)
        fst["entry"] = "kvlr_decode_attn_latent"
        fst["region_us_per_call"] = region_us(torch, folded, args.steps)
        del replicas, ws
        torch.cuda.empty_cache()

        achieved = alg_bytes / (launch_us * 1e-6) / 1e9
        result.update({"value": B * args.steps / elapsed, "ms_per_step": elapsed / args.steps * 1e3})
        result["config"].update({"splits": n_splits, "split_tokens": split_len})
        result["step_hbm_GBps"] = alg_bytes / (elapsed / args.steps) / 1e9
        result["roofline"] = {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": load_traffic(),
            "kernel": "decode_split_bf16<64, 32> (kvlr_decode_attn, fixed split plan, merge fused)",
            "bytes_per_launch": alg_bytes, "launch_us_mean": launch_us,
            "timing": "one HIP event pair on the launch stream around the K timed launches",
            "bracketed_launch": spread(np, split_us)}
        result["folded"] = fst
        if prefill is not None:
            result["prefill"] = prefill

    workloads = {}
    if not args.no_workloads:
        if run("single_head_f32"):
            workloads["single_head_f32"] = measure_single_head(kv, torch, np)
        if run("per_head_ranks_ragged"):
            workloads["per_head_ranks_ragged"] = measure_ragged(kv, torch, np)
        if run("long_context_128k"):
            workloads["long_context_128k"] = measure_long_context(kv, torch, np)
        if run("llama3_8b_32_layers"):
            workloads["llama3_8b_32_layers"] = measure_32_layers(kv, torch, np)
    if workloads:
        result["workloads"] = workloads
    if run("joint") and not args.no_joint:
        result["joint_values"] = measure_joint(kv, torch, np, cfg, gen, q, lens, args.steps, args.warmup)
    if run("q43") and not args.no_q43:
        result["q43"] = measure_q43(kv, torch, np, cfg, gen, q, lens, args.steps, args.warmup)

    if run("headline"):
        ceiling = measure_stream_ceiling(torch, np)
        result["roofline"]["stream_read_ceiling_GBps"] = ceiling
        result["roofline"]["frac_of_stream_read"] = result["roofline"]["achieved"] / ceiling

    if args.traffic_reference:
        from synth.device import copy as device_copy
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            device_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst

    if run("headline") and not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
