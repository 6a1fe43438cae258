"""C-ABI checks that need no GPU: the library loads, exports every function
that include/kvlr.h declares, and rejects bad arguments on the host before
any HIP call (so these calls are safe without a device)."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import rank_compressed_kv_kvlr_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvlr.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KVLR_API\s+[\w\s\*]+?\b(kvlr_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kvlr_prefill_compress", "kvlr_append", "kvlr_decode_attn", "kvlr_cache_elems",
              "kvlr_decode_workspace_bytes", "kvlr_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kv.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    assert kv.status_string(0) == "ok"
    for code in range(-8, 0):
        assert kv.status_string(code) not in ("ok", "unknown status")
    assert kv.status_string(-99) == "unknown status"


def _desc(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, capacity=1000, r_k=64, r_v=32,
                in_dtype=kv.BF16, latent_dtype=kv.BF16)
    base.update(kw)
    return kv.Desc(**base)


def _ws(desc, split=0):
    n = ctypes.c_size_t()
    return kv.lib.kvlr_decode_workspace_bytes(desc.ptr, split, ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=7), -2), (dict(n_q_heads=2 * 17), -2), (dict(head_dim=100), -2), (dict(head_dim=512), -2),
    (dict(capacity=0), -2), (dict(batch=0), -2), (dict(n_kv_heads=65, n_q_heads=65), -2),
    (dict(r_k=8), -3), (dict(r_v=0), -3), (dict(r_k=144), -3), (dict(r_k=[16, 24]), -3),
    (dict(head_dim=64, r_k=96), -3), (dict(latent_dtype=kv.F32, r_k=6), -3),
    (dict(in_dtype=3), -4), (dict(latent_dtype=-1), -4),
])
def test_descriptor_validation(kw, code):
    assert _ws(_desc(**kw))[0] == code


def test_fp32_latents_allow_rank_multiple_of_four():
    assert _ws(_desc(latent_dtype=kv.F32, r_k=12, r_v=4))[0] == 0


def test_cache_elems_and_layout():
    d = _desc(r_k=[16, 48], r_v=[32, 80], capacity=100)
    nk, nv = kv.cache_elems(d)
    assert nk == 2 * 112 * 64 and nv == 2 * 112 * 112     # capacity rounded up to 16 rows
    assert list(d.rank_offsets("v")) == [0, 32, 112]


@pytest.mark.parametrize("r", [16, 32, 48, 64, 80, 96, 112, 128])
def test_key_tile_order_is_a_permutation_of_each_block(r):
    """The MFMA-order key layout maps every (t, j) of a 16-row block to a distinct slot of that block."""
    idx = kv.k_tiled_index(64, r)
    for blk in range(4):
        sub = idx[16 * blk:16 * blk + 16]
        assert sub.min() == 16 * r * blk and sub.max() == 16 * r * (blk + 1) - 1
        assert len(np.unique(sub)) == 16 * r
    # lane l = 16 q + n of pair p reads 16 contiguous bytes: token n, channels 32 p + 8 q .. + 7
    for p in range(r // 32):
        for lane in range(64):
            q, n = lane // 16, lane % 16
            assert list(idx[n, 32 * p + 8 * q:32 * p + 8 * q + 8]) == list(range(512 * p + 8 * lane, 512 * p + 8 * lane + 8))


def test_workspace_and_plan():
    d = _desc(capacity=32768)
    ns, length = kv.decode_plan(d, 1024)
    assert (ns, length) == (32, 1024)
    rc, n = _ws(d, 1024)
    assert rc == 0 and n == 256 + 2 * 8 * 32 * 36 * 4   # counters (padded to 256 B) + records, stride round_up(32 + 2, 4)
    assert kv.decode_counter_bytes(d) == 256
    big = _desc(batch=64, n_kv_heads=8, n_q_heads=96)   # G = 12: 3 head groups
    assert kv.decode_counter_bytes(big) == (4 * 64 * 8 * 3 + 255) // 256 * 256
    assert kv.lib.kvlr_decode_workspace_bytes(d.ptr, 100, ctypes.byref(ctypes.c_size_t())) == -7
    assert kv.lib.kvlr_decode_workspace_bytes(d.ptr, -64, ctypes.byref(ctypes.c_size_t())) == -7
    ns, length = kv.decode_plan(d, 0)
    assert length % 256 == 0 and ns * length >= 32768


def test_null_pointers_rejected():
    d = _desc()
    assert kv.lib.kvlr_cache_elems(None, ctypes.byref(ctypes.c_size_t()), ctypes.byref(ctypes.c_size_t())) == -1
    assert kv.lib.kvlr_decode_attn(d.ptr, None, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                                   1 << 30, 0, None) == -1
    assert kv.lib.kvlr_append(d.ptr, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert kv.lib.kvlr_prefill_compress(d.ptr, None, FAKE, 0, 10, FAKE, FAKE, FAKE, FAKE, None) == -1
    for k in range(5):
        a = [FAKE] * 5
        a[k] = None
        q, lk, lv, lens, o = a
        assert kv.lib.kvlr_decode_attn_latent(d.ptr, q, lk, lv, lens, ctypes.c_float(0.1), o, FAKE, 1 << 30, 0,
                                              None) == -1


def test_prefill_bounds_and_noop():
    d = _desc(capacity=100)
    # start + n_tok beyond capacity
    assert kv.lib.kvlr_prefill_compress(d.ptr, FAKE, FAKE, 90, 11, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert kv.lib.kvlr_prefill_compress(d.ptr, FAKE, FAKE, -1, 5, FAKE, FAKE, FAKE, FAKE, None) == -7
    # zero tokens: nothing to do, no launch, even with NULL buffers
    assert kv.lib.kvlr_prefill_compress(d.ptr, None, None, 5, 0, None, None, None, None, None) == 0


def test_decode_workspace_and_scale_checks():
    d = _desc()
    rc, need = _ws(d)
    assert rc == 0
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert kv.lib.kvlr_decode_attn(d.ptr, *args, ctypes.c_float(0.1), FAKE, FAKE, need - 1, 0, None) == -5
    assert kv.lib.kvlr_decode_attn(d.ptr, *args, ctypes.c_float(0.1), FAKE, None, need, 0, None) == -5
    assert kv.lib.kvlr_decode_attn(d.ptr, *args, ctypes.c_float(float("nan")), FAKE, FAKE, need, 0, None) == -7
    assert kv.lib.kvlr_decode_attn(d.ptr, *args, ctypes.c_float(float("inf")), FAKE, FAKE, need, 0, None) == -7
    assert kv.lib.kvlr_decode_attn(d.ptr, *args, ctypes.c_float(0.1), FAKE, FAKE, need, 65, None) == -7
    lat = [FAKE] * 4
    assert kv.lib.kvlr_decode_attn_latent(d.ptr, *lat, ctypes.c_float(0.1), FAKE, FAKE, need - 1, 0, None) == -5
    assert kv.lib.kvlr_decode_attn_latent(d.ptr, *lat, ctypes.c_float(float("nan")), FAKE, FAKE, need, 0,
                                          None) == -7


def test_python_wrapper_raises_on_bad_desc():
    with pytest.raises(kv.KvlrError) as e:
        kv.cache_elems(_desc(n_q_heads=3))
    assert e.value.code == -2


def test_oracle_is_not_imported_by_the_product_path():
    import sys
    src = open(os.path.join(ROOT, "rank_compressed_kv_kvlr_amd", "__init__.py")).read()
    assert "oracle" not in re.sub(r'""".*?"""', "", src, flags=re.S)
    for f in os.listdir(os.path.join(ROOT, "rank_compressed_kv_kvlr_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "rank_compressed_kv_kvlr_amd", "csrc", f)).read()
    imports = re.compile(r"^\s*(?:import|from)\s+(\S+)", re.M)
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            mods = imports.findall(open(os.path.join(ROOT, "oracle", f)).read())
            assert not [m for m in mods if m.startswith(("rank_compressed_kv_kvlr_amd", "synth"))], (f, mods)


def test_single_hip_runtime_whatever_the_import_order():
    """Importing the binding before torch must not map a second HIP runtime."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import rank_compressed_kv_kvlr_amd, torch; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'amdhip64' in l}))" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300).stdout
    assert out.count("amdhip64") == 1, out


def test_joint_value_mode_validation():
    # joint values: one rank for every head, up to min(Hkv d, 128); storage is one block per batch row
    d = kv.Desc(2, 8, 4, 32, 100, 32, [96, 96, 96, 96], kv.BF16, kv.BF16, kv.VALUES_JOINT)
    nk, nv = kv.cache_elems(d)
    assert nk == 2 * 112 * 4 * 32 and nv == 2 * 112 * 96
    bad = kv.Desc(2, 8, 4, 32, 100, 32, [96, 96, 64, 96], kv.BF16, kv.BF16, kv.VALUES_JOINT)
    with pytest.raises(kv.KvlrError) as e:
        kv.cache_elems(bad)
    assert e.value.code == -3
    per_head = kv.Desc(2, 8, 4, 32, 100, 32, [96] * 4, kv.BF16, kv.BF16)   # 96 > head_dim per head
    with pytest.raises(kv.KvlrError):
        kv.cache_elems(per_head)
    odd = kv.Desc(2, 8, 4, 32, 100, 32, 32, kv.BF16, kv.BF16, 7)
    with pytest.raises(kv.KvlrError) as e:
        kv.cache_elems(odd)
    assert e.value.code == -7


def test_joint_bf16_shape_limits_and_workspace():
    # the joint bf16 kernel holds at most 32 query heads and 8 KV heads
    for hq, hkv in [(64, 8), (32, 16), (48, 16)]:
        d = kv.Desc(1, hq, hkv, 64, 100, 32, [64] * hkv, kv.BF16, kv.BF16, kv.VALUES_JOINT)
        with pytest.raises(kv.KvlrError) as e:
            kv.cache_elems(d)
        assert e.value.code == -2, (hq, hkv)
    # joint values with fp32 latents run the per-head kernels: no such limit
    kv.cache_elems(kv.Desc(1, 64, 16, 64, 100, 32, [64] * 16, kv.BF16, kv.F32, kv.VALUES_JOINT))
    # workspace: counters, records, then the projected queries [B][Hq][max r_k]
    d = kv.Desc(2, 32, 8, 128, 4096, [64] * 7 + [48], [128] * 8, kv.BF16, kv.BF16, kv.VALUES_JOINT)
    rc, n = _ws(d, 512)
    assert rc == 0
    assert n == 256 + 2 * 32 * 8 * 132 * 4 + 2 * 32 * 64 * 4
    ns, length = kv.decode_plan(d, 512)
    assert (ns, length) == (8, 512)


@pytest.mark.parametrize("r", [16, 32, 48, 64, 80, 96, 112, 128])
def test_joint_value_tile_order(r):
    """bf16 joint value layout: a permutation of each 16-row block, and lane 16 q + n of
    pair p reads 16 contiguous bytes holding tokens 4 q .. 4 q + 3 of channels 32 p + n
    and 32 p + 16 + n (the tail: 8 bytes, channel 32 np + n)."""
    idx = kv.v_joint_index(64, r)
    for blk in range(4):
        sub = idx[16 * blk:16 * blk + 16]
        assert sub.min() == 16 * r * blk and sub.max() == 16 * r * (blk + 1) - 1
        assert len(np.unique(sub)) == 16 * r
    np_ = r // 32
    for lane in range(64):
        q, n = lane // 16, lane % 16
        for p in range(np_):
            got = [idx[4 * q + e, 32 * p + n] for e in range(4)] + [idx[4 * q + e, 32 * p + 16 + n] for e in range(4)]
            assert got == list(range(512 * p + 8 * lane, 512 * p + 8 * lane + 8))
        if r % 32:
            got = [idx[4 * q + e, 32 * np_ + n] for e in range(4)]
            assert got == list(range(512 * np_ + 4 * lane, 512 * np_ + 4 * lane + 4))


def test_fused_step_arguments():
    """kvlr_append_decode_attn checks every pointer, the workspace and the scale before any launch."""
    d = _desc()
    rc, need = _ws(d)
    assert rc == 0
    for k in range(10):   # k_new, v_new, pos, q, P_K, P_V, lat_k, lat_v, seq_lens, out
        a = [FAKE] * 10
        a[k] = None
        assert kv.lib.kvlr_append_decode_attn(d.ptr, *a[:9], ctypes.c_float(0.1), a[9], FAKE, need, 0, None) == -1, k
    a = [FAKE] * 9
    assert kv.lib.kvlr_append_decode_attn(d.ptr, *a, ctypes.c_float(0.1), FAKE, FAKE, need - 1, 0, None) == -5
    assert kv.lib.kvlr_append_decode_attn(d.ptr, *a, ctypes.c_float(float("nan")), FAKE, FAKE, need, 0, None) == -7


def test_misaligned_buffers_rejected():
    """Buffers read or written with 16-byte vector accesses must be 16-byte aligned, for every
    latent dtype: the entry points return KVLR_ERR_ARG before any launch."""
    odd = ctypes.c_void_p(0x1008)
    for lat in (kv.BF16, kv.F32, kv.Q43):
        d = _desc(latent_dtype=lat)
        rc, need = _ws(d)
        assert rc == 0
        for k in range(6):   # K, V, P_K, P_V, lat_k, lat_v
            a = [FAKE] * 6
            a[k] = odd
            K, V, pk, pv, lk, lv = a
            assert kv.lib.kvlr_prefill_compress(d.ptr, K, V, 0, 10, pk, pv, lk, lv, None) == -7, (lat, k)
        for k in range(4):   # P_K, P_V, lat_k, lat_v
            a = [FAKE] * 4
            a[k] = odd
            pk, pv, lk, lv = a
            assert kv.lib.kvlr_append(d.ptr, FAKE, FAKE, FAKE, pk, pv, lk, lv, None) == -7, (lat, k)
        for k in range(5):   # P_K, P_V, lat_k, lat_v, workspace
            a = [FAKE] * 5
            a[k] = odd
            pk, pv, lk, lv, ws = a
            assert kv.lib.kvlr_decode_attn(d.ptr, FAKE, pk, pv, lk, lv, FAKE, ctypes.c_float(0.1), FAKE, ws, need, 0,
                                           None) == -7, (lat, k)
        # q, out and seq_lens need only element alignment: those calls get past the check
        # (and are stopped by the workspace size instead, still before any launch)
        assert kv.lib.kvlr_decode_attn(d.ptr, ctypes.c_void_p(0x1004), FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x1004),
                                       ctypes.c_float(0.1), ctypes.c_void_p(0x1004), FAKE, need - 1, 0, None) == -5


def test_balanced_plan_queries():
    """split_tokens = -1 (KVLR_SPLIT_BALANCED): the balanced plan for bf16 per-head caches (one round of
    workgroups, no fixed split length), the library's fixed plan elsewhere; its default when the KV
    heads' ranks differ; one workspace size serves both plans."""
    uniform = _desc(batch=8, n_q_heads=32, n_kv_heads=8, capacity=32768, r_k=64, r_v=64)
    ns, length = kv.decode_plan(uniform, -1)
    assert length == 0 and ns >= 256
    assert kv.decode_plan(uniform, 0)[1] > 0            # fixed plan by default: uniform ranks
    ragged = kv.Desc(16, 32, 8, 128, 16384, [16, 32, 48, 64, 80, 96, 16, 32], [96, 80, 64, 48, 32, 16, 96, 80],
                     kv.BF16, kv.BF16)
    assert kv.decode_plan(ragged, 0)[1] == 0            # balanced by default: ranks differ
    assert kv.decode_plan(ragged, 256) == (64, 256)     # an explicit length stays fixed
    assert kv.decode_workspace_bytes(ragged, 0) == kv.decode_workspace_bytes(ragged, -1)
    assert kv.decode_workspace_bytes(ragged, 0) >= kv.decode_workspace_bytes(ragged, 4096)
    for other in (_desc(latent_dtype=kv.F32), _desc(latent_dtype=kv.Q43),
                  _desc(n_q_heads=8, n_kv_heads=8, value_mode=kv.VALUES_JOINT)):
        assert kv.decode_plan(other, -1) == kv.decode_plan(other, 0)   # the fixed choice
    assert kv.decode_plan(_desc(batch=5000, capacity=64), -1)[1] > 0   # too many rows for the balanced plan
    with pytest.raises(kv.KvlrError):
        kv.decode_plan(uniform, -2)


def test_noalloc_entry_checks_on_the_host():
    """kvlr_decode_attn_noalloc rejects a call whose workspace would exceed the static scratch
    (KVLR_ERR_SCRATCH) and bad arguments, before any device work."""
    big = kv.Desc(64, 32, 8, 128, 1 << 20, 64, 64)
    assert kv.decode_workspace_bytes(big, 64) > kv.STATIC_SCRATCH_BYTES
    f = kv.lib.kvlr_decode_attn_noalloc
    assert f(big.ptr, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, 64, None) == -8
    small = _desc()
    assert f(small.ptr, None, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, 0, None) == -1
    assert f(small.ptr, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, float("nan"), FAKE, 0, None) == -7
    assert f(small.ptr, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, 100, None) == -7   # split not a multiple of 64



def test_layers_entry_checks_on_the_host():
    """kvlr_decode_attn_layers checks every layer, the lane count and (with more than one lane)
    that the workspaces are disjoint before anything is enqueued."""
    f = kv.lib.kvlr_decode_attn_layers
    d = _desc()
    ws = kv.decode_workspace_bytes(d, 0)

    def layer(desc=d, q=FAKE, workspace=FAKE, workspace_bytes=ws, scale=0.1):
        return kv._CLayer(desc.pointer, q, FAKE, FAKE, FAKE, FAKE, FAKE, scale, FAKE, workspace, workspace_bytes, 0)

    two = (kv._CLayer * 2)(layer(), layer(workspace=FAKE.value + (1 << 24)))
    assert f(two, 0, 2, None) == kv.OK                      # nothing to do
    assert f(None, 0, 2, None) == kv.OK
    assert f(None, 2, 2, None) == kv.ERR_NULL
    assert f(two, -1, 2, None) == kv.ERR_ARG
    assert f(two, 2, 0, None) == kv.ERR_ARG
    assert f(two, 2, kv.MAX_LANES + 1, None) == kv.ERR_ARG
    bad = (kv._CLayer * 2)(layer(), layer(q=None))
    assert f(bad, 2, 2, None) == kv.ERR_NULL                # the failing layer's status
    nan = (kv._CLayer * 2)(layer(), layer(scale=float("nan")))
    assert f(nan, 2, 1, None) == kv.ERR_ARG
    small = (kv._CLayer * 2)(layer(), layer(workspace_bytes=ws - 16))
    assert f(small, 2, 2, None) == kv.ERR_WORKSPACE
    shared = (kv._CLayer * 2)(layer(), layer(workspace=FAKE.value + ws // 2 // 256 * 256))
    assert f(shared, 2, 2, None) == kv.ERR_ARG              # overlapping workspaces on two lanes
