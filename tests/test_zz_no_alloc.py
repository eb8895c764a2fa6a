"""The allocation-free call (varlen_attn_fwd_device_noalloc) against the
device-scheduled call with a caller workspace (varlen_attn_fwd_device).

Both run the same kernels on the same items, so the outputs must be bitwise
equal; each is also checked against the fp64 oracle. Calls come in pairs, the
second smaller than the first, because every allocation-free call on a GPU
reuses the one static scratch array and keeps the previous call's contents.
"""
from __future__ import annotations

import ctypes
import sys

import pytest

import synth
from parity import compare, oracle_all


def _say(*a):
    print("[noalloc-case]", *a, flush=True)
    sys.stdout.flush()


def _workload(dtype="bf16", hq=8, hkv=2, d=128, causal=True, softcap=0.0, seed=21):
    return synth.Workload("noalloc", 0, hq, hkv, d, dtype, causal, softcap, 0.0, 1.0, seed)


def _both(batch, window=None):
    """(allocation-free output, workspace output, latch values)."""
    import torch
    import packed_varlen_scaled_amd as pva
    w = batch.workload
    cu_q = torch.from_numpy(batch.cu_q).cuda()
    cu_kv = torch.from_numpy(batch.cu_kv).cuda()
    n = pva.device_workspace_bytes(len(batch.lq), batch.total_q, batch.total_kv, w.num_heads, w.kv_num_heads,
                                   w.head_dim, w.dv, w.dtype)
    assert n <= pva.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    latch_a = torch.zeros(1, dtype=torch.int32, device="cuda")
    latch_b = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = torch.full((batch.total_q, w.num_heads, w.dv), 5.0, dtype=batch.q.dtype, device="cuda")
    want = torch.full_like(got, 6.0)
    kw = dict(scale=w.scale or None, is_causal=w.is_causal, softcap=w.softcap, local_window=window)
    pva.varlen_attn_fwd_device_noalloc(batch.q, batch.k, batch.v, cu_q, cu_kv, w.num_heads, w.kv_num_heads,
                                       out=got, error_latch=latch_a, **kw)
    pva.varlen_attn_fwd_device(batch.q, batch.k, batch.v, cu_q, cu_kv, w.num_heads, w.kv_num_heads, out=want,
                               workspace=ws, error_latch=latch_b, **kw)
    torch.cuda.synchronize()
    return got, want, int(latch_a.item()), int(latch_b.item())


# (name, workload kwargs, first call (lq, lkv), second, smaller call (lq, lkv), window)
PAIRS = [
    ("bf16_gqa_decode_mix", dict(hq=16, hkv=2),
     ([300, 1, 129, 1, 70, 0], [300, 2600, 129, 900, 500, 5]), ([40, 1, 9], [40, 700, 9]), None),
    ("bf16_softcap_gqa8", dict(hq=16, hkv=2, softcap=30.0),
     ([200, 97, 1], [1000, 97, 3000]), ([33, 1], [33, 100]), None),
    ("f16_window", dict(dtype="f16", hq=8, hkv=2),
     ([128, 64, 1], [700, 64, 1200]), ([20], [260]), 48),
    # decode-dominated (no more rows than sequences): the workspace call
    # forks decode onto a side stream, the allocation-free one stays on one
    ("bf16_decode_dominated", dict(hq=16, hkv=2),
     ([1, 1, 1, 2, 0, 1], [900, 3000, 5, 7, 1, 64]), ([1, 1], [130, 20]), None),
    ("f32_gqa", dict(dtype="f32", hq=8, hkv=2, d=64), ([70, 1, 33], [70, 200, 40]), ([5, 17], [5, 30]), None),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,kw,first,second,window", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_equals_workspace_call_on_two_calls(name, kw, first, second, window):
    w = _workload(**kw)
    for i, (lq, lkv) in enumerate((first, second)):
        _say(name, "call", i, lq, lkv, window)
        batch = synth.make_batch(w, lq, lkv, device="cuda")
        got, want, la, lb = _both(batch, window)
        assert la == 0 and lb == 0
        assert bool((got == want).all()), f"{name} call {i}: allocation-free output differs from the workspace call"
        ma, rel = compare(got.double().cpu().numpy(), oracle_all(batch, local_window=window or 0), w.dtype)
        _say(name, "call", i, "max_abs", ma, "rel_l2", rel)


@pytest.mark.gpu
def test_noalloc_latches_bad_cu_and_computes_nothing():
    import torch
    import packed_varlen_scaled_amd as pva
    w = _workload()
    batch = synth.make_batch(w, [40, 30], [40, 30], device="cuda")
    latch = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((batch.total_q, 8, 128), 3.0, dtype=batch.q.dtype, device="cuda")
    sentinel = out.clone()
    bad_q = torch.tensor([0, 40, 30], dtype=torch.int32, device="cuda")
    cu_kv = torch.from_numpy(batch.cu_kv).cuda()
    _say("latch", [0, 40, 30])
    pva.varlen_attn_fwd_device_noalloc(batch.q, batch.k, batch.v, bad_q, cu_kv, 8, 2, is_causal=True, out=out,
                                       error_latch=latch)
    torch.cuda.synchronize()
    assert int(latch.item()) == 2 and torch.equal(out, sentinel)


def test_noalloc_rejects_a_batch_larger_than_its_scratch_before_any_device_work():
    """The size check runs on the host before any HIP call (the pointers are
    never touched), so this runs without a GPU."""
    import packed_varlen_scaled_amd as pva
    lib = pva.load_library()
    fake = ctypes.c_void_p(16)
    latch = ctypes.c_void_p(16)
    # 256 decode rows against 64 M keys of capacity: the split-KV partials alone exceed the array
    st = lib.varlen_attn_fwd_device_noalloc(fake, fake, fake, fake, fake, 256, 256, 64 << 20, 64, 8, 128, 128,
                                            2, 0.0, 1, 0.0, -1, fake, latch, None)
    assert st == 1  # VARLEN_ERR_INVALID_ARGUMENT
    msg = lib.varlen_attn_last_error().decode()
    assert msg.startswith("varlen_attn_fwd_device_noalloc:") and "VARLEN_NOALLOC_SCRATCH_BYTES" in msg
    need = pva.device_workspace_bytes(256, 256, 64 << 20, 64, 8, 128, 128, "bf16")
    assert need > pva.NOALLOC_SCRATCH_BYTES
    # the header's limit and the binding's constant agree
    import os
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                            "varlen_attn.h")).read()
    assert "#define VARLEN_NOALLOC_SCRATCH_BYTES (32u << 20)" in hdr
    assert pva.NOALLOC_SCRATCH_BYTES == 32 << 20
