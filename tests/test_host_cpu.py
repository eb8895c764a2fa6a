"""Host-side logic of the C-ABI library, run without a GPU.

* the library loads and exports every function include/varlen_attn.h declares;
* argument / cu_seqlens validation returns the documented status before any
  device work (the packed op's execute() rules on the page
  src/kernels/packed_varlen_attention.rs);
* the scheduler covers every visible (row, key) pair of every head exactly
  once, writes every output row exactly once, and never schedules a tile that
  lies wholly above the causal frontier;
* the valid-pair count matches a brute-force count of the tail-aligned mask.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import packed_varlen_scaled_amd as pva

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "varlen_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(varlen_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = pva.load_library()
    names = _declared_functions()
    assert "varlen_attn_fwd" in names and len(names) >= 6
    for name in names:
        assert hasattr(lib, name), f"{name} declared in the header but not exported"
    assert pva.version().count(".") == 2


def test_library_defines_every_kernel_launch_stub():
    """A kernel whose host stub is missing would link (undefined symbols are
    allowed in a shared library) and fail only when launched."""
    from packed_varlen_scaled_amd import build as b
    assert b.undefined_kernel_stubs(pva.library_path()) == []


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _fwd_status(cu_q, cu_kv, hq=4, hkv=2, d=64, dv=0, dtype=2, scale=0.0, causal=0, softcap=0.0,
                total_q=None, total_kv=None, batch=None, ptr=1):
    """Call varlen_attn_fwd with host mirrors and dummy (never dereferenced)
    device pointers: every case here must fail validation first."""
    lib = pva.load_library()
    cq = np.ascontiguousarray(cu_q, dtype=np.int32)
    ck = np.ascontiguousarray(cu_kv, dtype=np.int32)
    b = len(cq) - 1 if batch is None else batch
    tq = int(cq[-1]) if total_q is None else total_q
    tk = int(ck[-1]) if total_kv is None else total_kv
    fake = ctypes.c_void_p(ptr) if ptr else None
    st = lib.varlen_attn_fwd(fake, fake, fake, None, None, cq.ctypes.data, ck.ctypes.data, b, tq, tk,
                             hq, hkv, d, dv, dtype, scale, causal, softcap, fake, None)
    return st, lib.varlen_attn_last_error().decode()


@pytest.mark.parametrize("kwargs,status,fragment", [
    (dict(hq=8, hkv=3), 1, "multiple of kv_num_heads"),
    (dict(hq=0), 1, "num_heads must be positive"),
    (dict(d=0), 1, "head_dim must be positive"),
    (dict(dtype=7), 1, "dtype code"),
    (dict(scale=-1.0), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(softcap=float("inf")), 1, "softcap"),
    (dict(batch=0), 2, "batch must be >= 1"),
    (dict(total_q=11), 2, "must equal the packed token count"),
    (dict(d=96), 3, "f16/bf16 support head_dim"),
    (dict(d=128, dv=96), 3, "f16/bf16 support head_dim"),
    (dict(d=32, dv=64), 3, "f16/bf16 support head_dim"),
    (dict(dtype=0, d=256), 3, "f32 supports"),
    (dict(ptr=0), 1, "must be non-null"),
    (dict(ptr=8), 1, "16-byte aligned"),
])
def test_validation_rejects_before_any_device_work(kwargs, status, fragment):
    st, msg = _fwd_status(_cu([3, 4]), _cu([5, 2]), **kwargs)
    assert st == status, msg
    assert msg.startswith("varlen_attn_fwd: ") and fragment in msg, msg


@pytest.mark.parametrize("cu_q,cu_kv,fragment", [
    ([1, 3, 7], [0, 5, 7], "cu_seqlens_q[0] must be 0"),
    ([0, 5, 4], [0, 5, 7], "non-decreasing"),
    ([0, 3, 7], [0, 6, 5], "non-decreasing"),
])
def test_bad_cu_seqlens(cu_q, cu_kv, fragment):
    st, msg = _fwd_status(np.array(cu_q), np.array(cu_kv), total_q=cu_q[-1] if cu_q[-1] > 0 else 7)
    assert st == 2 and fragment in msg, msg


def test_empty_query_batch_is_ok_without_device_work():
    st, msg = _fwd_status(_cu([0, 0]), _cu([3, 0]))
    assert st == 0, msg


# --------------------------------------------------------------------------
# Valid-pair count.
# --------------------------------------------------------------------------
def _brute_pairs(lq, lkv, causal, window=0):
    n = 0
    for a, b in zip(lq, lkv):
        for i in range(a):
            for j in range(b):
                if (not causal or j <= i + b - a) and (window <= 0 or j >= i + b - a + 1 - window):
                    n += 1
    return n


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [1, 3, 17])
def test_valid_pairs_with_window_matches_brute_force(causal, window):
    rng = np.random.default_rng(6 + window)
    for _ in range(40):
        bsz = int(rng.integers(1, 6))
        lq = rng.integers(0, 40, size=bsz).tolist()
        lkv = rng.integers(0, 40, size=bsz).tolist()
        assert pva.valid_pairs(_cu(lq), _cu(lkv), causal, local_window=window) == \
            _brute_pairs(lq, lkv, causal, window)


def test_window_argument_validation():
    lib = pva.load_library()
    cq, ck = _cu([3, 4]), _cu([5, 2])
    for w, ok in [(-2, False), (-100, False), (-1, True), (0, True), (1, True), (1 << 20, True)]:
        opts = pva.Options()
        opts.local_window = w
        st = lib.varlen_attn_plan(cq.ctypes.data, ck.ctypes.data, 2, 7, 7, 4, 2, 64, 0, 2, 0.0, 1, 0.0,
                                  ctypes.byref(opts), ctypes.byref(pva.PlanStats()), None, 0)
        msg = lib.varlen_attn_last_error().decode()
        assert (st == 0) == ok, (w, st, msg)
        if not ok:
            assert st == 1 and "local_window" in msg, msg
        fake = ctypes.c_void_p(1)
        st = lib.varlen_attn_fwd_ex(fake, fake, fake, None, None, cq.ctypes.data, ck.ctypes.data, 2, 7, 7, 4, 2,
                                    64, 0, 2, 0.0, 1, 0.0, None if ok else fake, None, ctypes.byref(opts))
        if not ok:
            assert st == 1 and "local_window" in lib.varlen_attn_last_error().decode()


@pytest.mark.parametrize("causal", [False, True])
def test_valid_pairs_matches_brute_force(causal):
    rng = np.random.default_rng(5)
    for _ in range(50):
        bsz = int(rng.integers(1, 6))
        lq = rng.integers(0, 40, size=bsz).tolist()
        lkv = rng.integers(0, 40, size=bsz).tolist()
        assert pva.valid_pairs(_cu(lq), _cu(lkv), causal) == _brute_pairs(lq, lkv, causal)


# --------------------------------------------------------------------------
# Scheduler coverage.
# --------------------------------------------------------------------------
KIND_PREFILL, KIND_F32, KIND_DECODE, KIND_COMBINE = 0, 1, 2, 3


def _coverage(lq, lkv, hq, hkv, causal, dtype="bf16", d=128, window=0, **opts):
    stats, items = pva.plan(_cu(lq), _cu(lkv), hq, hkv, head_dim=d, dtype=dtype, is_causal=causal,
                            with_items=True, local_window=window or None, **opts)
    cq, ck = _cu(lq), _cu(lkv)
    # visits[(token, head)] -> list of key index arrays
    visits = {}
    writes = {}
    combined = {}
    for it in items:
        kind, seq, r0, rows, h0, nh, kv0, kv1, pbase, nsplit, qt0, kt0, Lq, Lkv, split, _ = it.tolist()
        assert qt0 == cq[seq] and kt0 == ck[seq] and Lq == lq[seq] and Lkv == lkv[seq]
        assert 0 <= r0 and r0 + rows <= Lq and 0 <= kv0 <= kv1 <= Lkv
        assert h0 % nh == 0 and (h0 // (hq // hkv)) == ((h0 + nh - 1) // (hq // hkv)), "item spans kv groups"
        for r in range(r0, r0 + rows):
            for h in range(h0, h0 + nh):
                key = (qt0 + r, h)
                if kind == KIND_COMBINE:
                    combined[key] = combined.get(key, 0) + 1
                    continue
                visits.setdefault(key, []).append(np.arange(kv0, kv1))
                if pbase < 0:
                    writes[key] = writes.get(key, 0) + 1
    for b in range(len(lq)):
        off = lkv[b] - lq[b]
        for i in range(lq[b]):
            for h in range(hq):
                key = (cq[b] + i, h)
                got = np.concatenate(visits.get(key, [np.zeros(0, int)]))
                # every visible key visited exactly once
                hi = lkv[b] if not causal else max(0, min(lkv[b], i + off + 1))
                lo = max(0, i + off + 1 - window) if window > 0 else 0
                visible = np.arange(lo, max(lo, hi))
                cnt = np.bincount(got, minlength=max(lkv[b], 1)) if got.size else np.zeros(max(lkv[b], 1), int)
                assert np.all(cnt[visible] == 1), (b, i, h)
                assert cnt.sum() - cnt[visible].sum() >= 0
                # each output row written exactly once, directly or by one combine
                assert writes.get(key, 0) + combined.get(key, 0) == 1, (b, i, h)
    return stats, items


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (32, 8), (64, 8), (6, 2), (16, 1)])
def test_scheduler_covers_each_visible_pair_once(causal, hq, hkv):
    lq = [1, 33, 70, 0, 5, 129, 1]
    lkv = [7, 33, 150, 4, 0, 100, 0]
    stats, _ = _coverage(lq, lkv, hq, hkv, causal)
    assert stats["valid_pairs"] == _brute_pairs(lq, lkv, causal)
    assert stats["visited_pairs"] >= stats["valid_pairs"]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [1, 40, 150])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (64, 8), (4, 2), (3, 3)])
def test_scheduler_with_window_covers_each_visible_pair_once(causal, window, hq, hkv):
    lq = [1, 33, 70, 0, 5, 129, 1, 300]
    lkv = [700, 33, 150, 4, 0, 100, 90, 300]
    stats, items = _coverage(lq, lkv, hq, hkv, causal, window=window)
    assert stats["valid_pairs"] == _brute_pairs(lq, lkv, causal, window)
    # window-aware tile skipping: no item starts before the first key its first row can see
    for it in items:
        kind, seq, r0 = it[0], it[1], it[2]
        if kind == KIND_COMBINE:
            continue
        off = lkv[seq] - lq[seq]
        assert it[6] >= min(lkv[seq], max(0, r0 + off + 1 - window))
    assert stats["visited_pairs"] <= 2 * stats["valid_pairs"] + 64 * 32 * len(items)


@pytest.mark.parametrize("opts", [dict(decode_chunk=128), dict(prefill_kv_chunk=64)])
def test_scheduler_splits_with_window_keep_coverage(opts):
    _coverage([1, 40, 200, 1, 3], [700, 300, 200, 65, 1000], 32, 8, True, window=100, **opts)


@pytest.mark.parametrize("opts", [dict(decode_path=1), dict(decode_chunk=128), dict(prefill_kv_chunk=64),
                                  dict(prefill_kv_chunk=100, decode_chunk=300)])
def test_scheduler_split_options_keep_coverage(opts):
    lq = [1, 40, 200, 1, 3]
    lkv = [700, 300, 200, 65, 1000]
    stats, items = _coverage(lq, lkv, 32, 8, True, **opts)
    if opts.get("decode_path") == 1:
        assert stats["n_decode_items"] == 0
    if opts.get("prefill_kv_chunk") or opts.get("decode_chunk"):
        assert stats["n_combine_items"] > 0 and stats["n_partials"] > 0


def test_scheduler_f32_items():
    stats, items = _coverage([5, 17, 32, 64], [5, 17, 32, 64], 4, 4, False, dtype="f32", d=64)
    assert set(items[:, 0].tolist()) == {KIND_F32}
    assert stats["n_decode_items"] == 0


def test_causal_tiles_never_start_above_the_frontier():
    lq, lkv = [300, 64], [300, 500]
    _, items = pva.plan(_cu(lq), _cu(lkv), 32, 8, is_causal=True, with_items=True)
    for it in items:
        kind, seq, r0, rows, *_ = it.tolist()
        kv1, Lq, Lkv = it[7], it[12], it[13]
        last = r0 + rows - 1
        assert kv1 == min(Lkv, last + Lkv - Lq + 1)


def test_prefill_item_order():
    """Sequences by their longest item first; within a sequence the row blocks
    from the last to the first, the head groups of a row block adjacent (so
    items i and i + 8 share a kv head's K/V on one XCD)."""
    lq = [900, 2048, 130, 2048]
    _, items = pva.plan(_cu(lq), _cu(lq), 32, 8, is_causal=True, with_items=True)
    pre = items[items[:, 0] == KIND_PREFILL]
    seqs = [int(b) for b in pre[:, 1]]
    order = [b for i, b in enumerate(seqs) if i == 0 or seqs[i - 1] != b]
    assert order == [1, 3, 0, 2]  # each sequence once, longest first, ties by index
    for b in set(seqs):
        mine = pre[pre[:, 1] == b]
        r0 = mine[:, 2]
        assert np.all(np.diff(r0) <= 0)
        groups = len(set(mine[:, 4].tolist()))
        assert groups == 8 and np.all(mine[:groups, 2] == mine[0, 2])
    cost = (pre[:, 7] - pre[:, 6]) * pre[:, 3]
    assert cost[0] == cost.max()
    assert pre[-1, 1] == 2 and pre[-1, 2] == 0  # the shortest sequence's first row block ends the list


def test_workload_plans_fit():
    """The five workload shapes plan without error and report sane sizes."""
    import synth
    for name, w in synth.WORKLOADS.items():
        lq, lkv = synth.draw_lengths(name)
        stats, _ = pva.plan(_cu(lq), _cu(lkv), w.num_heads, w.kv_num_heads, head_dim=w.head_dim,
                            dtype=w.dtype, is_causal=w.is_causal, softcap=w.softcap)
        assert stats["valid_pairs"] > 0
        assert stats["workspace_bytes"] < 512 << 20
        if name == "packed_decode":
            assert stats["n_decode_items"] >= 1024


def test_kernels_keep_their_working_set_in_registers():
    """No kernel of the last build uses scratch memory or spills registers (the
    compiler's own kernel-resource report, recorded by the build): a private
    array demoted to scratch in a tile loop costs an order of magnitude."""
    import json
    from packed_varlen_scaled_amd import build as b
    with open(b.RESOURCES_PATH) as f:
        recs = json.load(f)
    kernels = [r for r in recs if r["kernel"].startswith("_ZN3pva")]
    assert len(kernels) >= 20, kernels
    for r in kernels:
        assert r.get("scratch_bytes_per_lane", 0) == 0, r
        assert r.get("vgpr_spill", 0) == 0, r
        assert r.get("waves_per_simd", 0) >= 1, r


# --------------------------------------------------------------------------
# The device-scheduled (capture-safe) entry point: host-side checks only.
# --------------------------------------------------------------------------
def test_device_workspace_size():
    small = pva.device_workspace_bytes(4, 1000, 1000, 32, 8)
    assert small > 0 and small % 256 == 0
    assert pva.device_workspace_bytes(64, 1000, 1000, 32, 8) > small      # more sequences
    assert pva.device_workspace_bytes(4, 100000, 1000, 32, 8) > small     # more query rows
    assert pva.device_workspace_bytes(4, 1000, 4_000_000, 32, 8) > small  # more decode splits
    with pytest.raises(ValueError):
        pva.device_workspace_bytes(4, 1000, 1000, 32, 5)  # 5 does not divide 32


@pytest.mark.parametrize("case,fragment", [
    ("null_latch", "error latch"),
    ("small_workspace", "workspace holds"),
    ("misaligned", "256-byte aligned"),
    ("bad_window", "local_window"),
    ("bad_heads", "multiple of kv_num_heads"),
    ("misaligned_out", "16-byte aligned"),
])
def test_device_entry_rejects_before_any_device_work(case, fragment):
    lib = pva.load_library()
    need = lib.varlen_attn_device_workspace_bytes(2, 64, 64, 8, 2, 128, 0, 2)
    fake = ctypes.c_void_p(1 << 20)
    ws, ws_bytes, latch, window, hkv = ctypes.c_void_p(1 << 20), need, fake, -1, 2
    if case == "null_latch":
        latch = None
    elif case == "small_workspace":
        ws_bytes = need - 256
    elif case == "misaligned":
        ws = ctypes.c_void_p((1 << 20) + 16)
    elif case == "bad_window":
        window = -3
    elif case == "bad_heads":
        hkv = 3
    out = ctypes.c_void_p((1 << 20) + 8) if case == "misaligned_out" else fake
    st = lib.varlen_attn_fwd_device(fake, fake, fake, fake, fake, 2, 64, 64, 8, hkv, 128, 0, 2, 0.0, 1, 0.0,
                                    window, out, ws, ws_bytes, latch, None)
    msg = lib.varlen_attn_last_error().decode()
    assert st == 1 and fragment in msg, (st, msg)


# ---- the cache step and the attention over a cache: host-side validation ------
def _rope_status(batch=2, total_q=3, hq=4, hkv=2, d=64, dv=0, dtype=2, cap=16, rdim=64, rows=32, inter=0,
                 q=1, q_out=1, qs=0, ks=0, vs=0, latch=1, cos=1, kv=1):
    """varlen_kv_append_rope with dummy (never dereferenced) device pointers:
    every case here must fail validation before anything is enqueued."""
    lib = pva.load_library()
    p = lambda x: ctypes.c_void_p(x) if x else None  # noqa: E731
    st = lib.varlen_kv_append_rope(p(q), p(q_out), p(kv), p(kv), qs, ks, vs, p(1), p(1), p(1), p(1), None,
                                   p(cos), p(cos), None, batch, total_q, hq, hkv, d, dv, dtype, cap, rdim, rows,
                                   inter, p(latch), None)
    return st, lib.varlen_attn_last_error().decode()


@pytest.mark.parametrize("kwargs,status,fragment", [
    (dict(d=63), 3, "must be even"),
    (dict(dv=5), 3, "must be even"),
    (dict(cap=0), 1, "cache_capacity must be >= 1"),
    (dict(batch=70000, cap=40000), 1, "below 2^31"),
    (dict(rdim=3), 1, "rotary_dim must be 0 or even"),
    (dict(rdim=66), 1, "rotary_dim must be 0 or even"),
    (dict(rows=0), 1, "rotary_rows >= 1"),
    (dict(cos=0), 1, "rotary_rows >= 1"),
    (dict(q_out=0), 1, "q and q_out"),
    (dict(qs=100), 1, "row strides"),
    (dict(ks=64), 1, "row strides"),
    (dict(q=1, q_out=1, qs=300), 1, "in-place rotation"),
    (dict(latch=0), 1, "must be non-null"),
    (dict(kv=0), 1, "k and v must be non-null when there are new rows"),
    (dict(hq=6, hkv=4), 1, "multiple of kv_num_heads"),
    (dict(dtype=5), 1, "dtype code"),
])
def test_cache_step_rejects_before_any_device_work(kwargs, status, fragment):
    st, msg = _rope_status(**kwargs)
    assert st == status, msg
    assert msg.startswith("varlen_kv_append_rope: ") and fragment in msg, msg


def test_cache_attention_rejects_before_any_device_work():
    lib = pva.load_library()
    one = ctypes.c_void_p(1)

    def call(cap=16, kvlen=one, batch=2, latch=one):
        st = lib.varlen_attn_fwd_kvcache(one, one, one, one, kvlen, batch, 3, cap, 4, 2, 64, 0, 2, 0.0, 1, 0.0, -1,
                                         one, one, 1 << 30, latch, None)
        return st, lib.varlen_attn_last_error().decode()

    for kw, frag in [(dict(cap=0), "cache_capacity must be >= 1"), (dict(kvlen=None), "kv_seqlens"),
                     (dict(batch=70000, cap=40000), "below 2^31"), (dict(latch=None), "must be non-null")]:
        st, msg = call(**kw)
        assert st == 1 and msg.startswith("varlen_attn_fwd_kvcache: ") and frag in msg, (kw, msg)


def test_entry_name_is_restored_after_a_cache_call():
    _rope_status(cap=0)
    st, msg = _fwd_status(_cu([3, 4]), _cu([5, 2]), hq=0)
    assert msg.startswith("varlen_attn_fwd: "), msg


def _device_caps(batch, total_q, total_kv, hq, hkv, f32=False):
    """The launch-grid bounds the device path sizes its lists with."""
    group = hq // hkv

    def pow2_div(g, cap):
        p = 1
        while p * 2 <= cap and g % (p * 2) == 0:
            p *= 2
        return p
    if f32:
        nh, rows, use_dec, nh_dec = 1, 32, False, 1
    else:
        nh = pow2_div(group, 8)
        rows = 32 * (1 if nh >= 4 else 4 // nh)
        use_dec, nh_dec = True, pow2_div(group, 16)
    n_pre_seq = min(batch, total_q // 2 if use_dec else total_q)
    cap_pre = (-(-total_q // rows) + n_pre_seq) * (hq // nh)
    if not use_dec:
        return cap_pre, 0, 0, 0, nh, rows
    g = hq // nh_dec
    n_dec_seq = min(batch, total_q)
    per_chunk = min(-(-total_kv // 512), max(-(-2048 // g), -(-total_kv // 8192)))
    cap_dec = g * (per_chunk + 1 + n_dec_seq)
    return cap_pre, cap_dec, g * n_dec_seq, cap_dec * nh_dec, nh, rows


@pytest.mark.parametrize("seed", range(12))
def test_device_list_bounds_hold(seed):
    """The device path's list bounds size its launch grids; a list that
    outgrew one would latch an error, so they must hold for every batch. The
    host scheduler emits the same decode items (same chunk rule) and the
    prefill items are counted directly."""
    rng = np.random.default_rng(seed)
    for _ in range(20):
        b = int(rng.integers(1, 300))
        hkv = int(rng.choice([1, 2, 4, 8]))
        hq = hkv * int(rng.choice([1, 2, 4, 8, 16]))
        kind = rng.integers(0, 4)
        if kind == 0:    # all decode, short and empty caches
            lq = np.ones(b, dtype=np.int64)
            lkv = rng.integers(0, 40, size=b)
        elif kind == 1:  # all decode, long caches
            lq = np.ones(b, dtype=np.int64)
            lkv = rng.integers(1, 70000, size=b)
        elif kind == 2:  # mixed
            lq = rng.choice([1, 1, 1, 2, 7, 300], size=b)
            lkv = lq + rng.integers(0, 5000, size=b)
        else:            # prefill
            lq = rng.integers(0, 900, size=b)
            lkv = lq + rng.integers(0, 50, size=b)
        cq, ckv = _cu(lq), _cu(lkv)
        tq, tkv = int(cq[-1]), int(ckv[-1])
        cap_pre, cap_dec, cap_cmb, cap_part, nh, rows = _device_caps(b, tq, tkv, hq, hkv)
        stats, _ = pva.plan(cq, ckv, hq, hkv, head_dim=128, dtype="bf16", is_causal=True)
        n_pre = sum(-(-int(x) // rows) for x in lq if x >= 2) * (hq // nh)
        assert n_pre <= cap_pre, (b, hq, hkv, n_pre, cap_pre)
        assert stats["n_decode_items"] <= cap_dec, (b, hq, hkv, kind, stats, cap_dec)
        assert stats["n_combine_items"] <= cap_cmb, (stats, cap_cmb)
        assert stats["n_partials"] <= cap_part, (stats, cap_part)


# --------------------------------------------------------------------------
# The randomized parity sweep's configurations (tests/random_cases.py).
# --------------------------------------------------------------------------
def test_random_cases_cover_every_option():
    """The seeds the GPU sweep runs draw every element type, both masks,
    softcap of either sign, a custom scale, a window, D != Dv, GQA groups
    from 1 to 8+, and every kind of sequence."""
    from random_cases import KINDS, random_case
    from test_gpu_random import SEEDS
    cases = [random_case(s) for s in SEEDS]
    assert {c.dtype for c in cases} == {"bf16", "f16", "f32"}
    assert {c.causal for c in cases} == {False, True}
    assert any(c.softcap > 0 for c in cases) and any(c.softcap < 0 for c in cases)
    assert any(c.scale > 0 for c in cases) and any(c.window > 0 for c in cases)
    assert any(c.d != c.dv for c in cases if c.dtype != "f32") and any(c.d != c.dv for c in cases if c.dtype == "f32")
    assert any(c.d == 128 for c in cases if c.dtype != "f32")
    assert {c.hq // c.hkv for c in cases} >= {1, 2, 4, 8}
    assert {k for c in cases for k in c.kinds} == set(KINDS)
    assert any(a > b for c in cases for a, b in zip(c.lq, c.lkv)), "no sequence with L_q > L_kv"


@pytest.mark.parametrize("seed", list(range(0, 48, 3)))
@pytest.mark.parametrize("split", [False, True])
def test_random_cases_scheduler_covers_each_visible_pair_once(seed, split):
    from random_cases import random_case, split_options
    c = random_case(seed)
    opts = split_options(seed) if split else {}
    stats, _ = _coverage(list(c.lq), list(c.lkv), c.hq, c.hkv, c.causal, dtype=c.dtype, d=c.d,
                         window=c.window, **opts)
    assert stats["valid_pairs"] == _brute_pairs(list(c.lq), list(c.lkv), c.causal, c.window)


def test_device_ex_rejects_host_only_options_before_any_device_work():
    lib = pva.load_library()
    one = ctypes.c_void_p(1)
    for kw, frag in [(dict(decode_chunk=128), "takes only decode_path"), (dict(prefill_kv_chunk=64), "takes only decode_path"),
                     (dict(local_window=32), "takes only decode_path"), (dict(decode_path=3), "decode_path must be 0, 1 or 2")]:
        opts = pva.Options()
        for name, val in kw.items():
            setattr(opts, name, val)
        st = lib.varlen_attn_fwd_device_ex(one, one, one, one, one, 2, 16, 16, 4, 2, 64, 64, 2, 0.0, 1, 0.0, -1,
                                           one, one, 1 << 20, one, None, ctypes.byref(opts))
        msg = lib.varlen_attn_last_error().decode()
        assert st == 1 and msg.startswith("varlen_attn_fwd_device_ex: ") and frag in msg, (kw, msg)

