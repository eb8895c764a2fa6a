"""GPU parity of the decode-side input step and of attention over a
fixed-capacity KV cache, through the C ABI, against the fp64 oracles.

The cache step rounds each rotated element once from fp32 into the storage
type, where the oracle holds the exact fp64 value: an element passes when it
lies within one storage ulp of the exact value plus the fp32 evaluation
error (two products and a sum of terms no larger than the pair's inputs:
at most 2^-22 of the head row's largest input). Copied elements (values,
dims past the rotary ones, and every cache row the step does not own) must
be bit-identical.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
from oracle import rope_append as ra
from parity import compare

pytestmark = pytest.mark.gpu

ULP_BITS = {"bf16": 7, "f16": 10, "f32": 23}
MIN_EXP = {"bf16": -126, "f16": -14, "f32": -126}


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def _host_bits(t):
    """Stored values of a tensor on the host in the oracle's input form."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _as_f64(t, dtype):
    return ra.to_f64(_host_bits(t), dtype)


def _ulp(x, dtype):
    e = np.frexp(np.abs(x))[1].astype(np.int64) - 1
    e = np.maximum(e, MIN_EXP[dtype])
    return np.ldexp(1.0, e - ULP_BITS[dtype])


def _within_rounding(got, want, inputs, dtype):
    """got, want: [..., heads, dim]; inputs: the pre-rotation head rows."""
    scale = np.max(np.abs(inputs), axis=-1, keepdims=True)
    bound = _ulp(want, dtype) + 2.0 ** -22 * scale
    bad = np.abs(got - want) > bound
    return int(bad.sum()), float(np.max(np.abs(got - want))) if got.size else 0.0


def _tables(rows, rdim, device):
    if rdim == 0:
        return None, None
    return synth.rotary_tables(rows, rdim, device=device)


def _run_step(step, rdim, interleaved, pos_ids=None, packed_qkv=False, in_place=False, rows=None):
    import torch
    import packed_varlen_scaled_amd as pva
    w = step.workload
    dev = step.q.device
    cu = torch.from_numpy(step.cu_q).to(dev)
    past = torch.tensor(step.past, dtype=torch.int32, device=dev)
    kv_len = torch.full((len(step.lq),), -7, dtype=torch.int32, device=dev)
    latch = torch.zeros(1, dtype=torch.int32, device=dev)
    rows = rows or (max(step.kv_len) + 5)
    cos, sin = _tables(rows, rdim, dev)
    q, k, v = step.q, step.k, step.v
    if packed_qkv:
        # one buffer [T, (Hq + 2 Hkv) * D] with q, k, v as row views
        hq, hkv, d = w.num_heads, w.kv_num_heads, w.head_dim
        buf = torch.cat([q.reshape(q.shape[0], -1), k.reshape(k.shape[0], -1), v.reshape(v.shape[0], -1)], dim=1)
        q = buf[:, :hq * d].view(-1, hq, d)
        k = buf[:, hq * d:(hq + hkv) * d].view(-1, hkv, d)
        v = buf[:, (hq + hkv) * d:].view(-1, hkv, w.dv)
    q_in = q.clone() if in_place else q
    q_out = q_in if in_place else torch.empty(step.total_q, w.num_heads, w.head_dim, dtype=q.dtype, device=dev)
    pos_t = None if pos_ids is None else torch.from_numpy(np.asarray(pos_ids, dtype=np.int64)).to(dev)
    pva.kv_append_rope(q_in, k, v, step.k_cache, step.v_cache, cu, past, w.num_heads, w.kv_num_heads, cos=cos,
                       sin=sin, position_ids=pos_t, rotary_interleaved=interleaved, q_out=q_out,
                       kv_seqlens_out=kv_len, error_latch=latch)
    torch.cuda.synchronize()
    return q_out, kv_len, latch, (cos, sin)


STEP_CASES = [
    # (name, dtype, hq, hkv, d, dv, lq, past, capacity, rotary_dim, interleaved, options)
    ("bf16_decode_half", "bf16", 8, 2, 128, None, [1, 1, 1, 1], [0, 5, 63, 200], 256, 128, False, {}),
    ("bf16_decode_interleaved", "bf16", 8, 2, 128, None, [1, 1, 1], [7, 0, 99], 128, 128, True, {}),
    ("bf16_partial_rotary", "bf16", 4, 4, 128, None, [1, 3, 1], [10, 2, 0], 64, 64, False, {}),
    ("bf16_chunk_rows_pos_ids", "bf16", 8, 2, 64, None, [5, 0, 17, 1], [3, 9, 0, 40], 64, 64, False,
     dict(pos_ids=True)),
    ("f16_interleaved_partial", "f16", 8, 1, 64, None, [2, 1, 9], [0, 30, 5], 48, 32, True, {}),
    ("f32_half", "f32", 4, 2, 64, None, [3, 1], [4, 0], 16, 64, False, {}),
    ("bf16_no_rotation", "bf16", 4, 2, 128, None, [2, 1], [6, 1], 32, 0, False, {}),
    ("bf16_dv64", "bf16", 8, 2, 128, 64, [1, 4, 1], [11, 3, 0], 32, 128, False, {}),
    ("bf16_packed_qkv", "bf16", 8, 2, 128, None, [1, 2, 1], [3, 0, 9], 16, 128, True, dict(packed_qkv=True)),
    ("bf16_in_place", "bf16", 8, 2, 64, None, [1, 1, 5], [0, 2, 3], 16, 64, False, dict(in_place=True)),
    ("bf16_fills_capacity", "bf16", 4, 2, 64, None, [3, 1], [13, 15], 16, 64, False, {}),
    # shapes the 16-byte kernel does not take: one pair per thread
    ("f32_rotary12_pairs", "f32", 4, 2, 40, None, [2, 1], [3, 0], 16, 12, False, {}),
    ("bf16_d66_pairs", "bf16", 4, 2, 66, None, [1, 2], [0, 5], 16, 66, False, {}),
    ("bf16_rotary24_half_pairs", "bf16", 8, 2, 64, None, [1, 3], [4, 9], 16, 24, False, {}),
    ("bf16_rotary24_interleaved", "bf16", 8, 2, 64, None, [1, 3], [4, 9], 16, 24, True, {}),
    ("f16_dv72", "f16", 4, 2, 64, 72, [2, 1], [1, 1], 8, 32, False, {}),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_cache_step_matches_oracle(case):
    _check_step(*case)


@pytest.mark.parametrize("seed", list(range(64)))
def test_random_cache_step_matches_oracle(seed):
    """Seeded random steps (tests/random_cases.py) to the same bar."""
    from random_cases import random_step_case
    c = random_step_case(seed)
    _check_step(f"random_step{seed}", c.dtype, c.hq, c.hkv, c.d, c.dv, list(c.lq), list(c.past), c.capacity,
                c.rotary_dim, c.interleaved, c.opts, seed=300 + seed)


def _check_step(name, dtype, hq, hkv, d, dv, lq, past, cap, rdim, inter, opts, seed=21):
    import torch
    w = synth.Workload("custom", 0, hq, hkv, d, dtype, True, 0.0, 0.0, 1.0, seed, dv)
    _say(name, dtype, hq, hkv, d, dv, lq, past, cap, rdim, inter, opts)
    step = synth.make_cache_step(w, lq, past, cap, device="cuda")
    kc_before = _host_bits(step.k_cache).copy()
    vc_before = _host_bits(step.v_cache).copy()
    pos_ids = None
    if opts.get("pos_ids"):
        pos_ids = (np.arange(step.total_q) * 7 + 3) % (max(step.kv_len) + 5)
    q_out, kv_len, latch, (cos, sin) = _run_step(step, rdim, inter, pos_ids=pos_ids,
                                                 packed_qkv=opts.get("packed_qkv", False),
                                                 in_place=opts.get("in_place", False))
    assert int(latch.item()) == 0
    want = ra.kv_append_rope(_host_bits(step.q), _host_bits(step.k), _host_bits(step.v), kc_before, vc_before,
                             step.cu_q, step.past, cap, None if cos is None else cos.cpu().numpy(),
                             None if sin is None else sin.cpu().numpy(), position_ids=pos_ids,
                             interleaved=inter, dtype=dtype)
    assert want["err"] == 0
    assert kv_len.cpu().numpy().tolist() == want["kv_len"].tolist()
    # rotated queries
    qin = _as_f64(step.q, dtype)
    nbad, worst = _within_rounding(_as_f64(q_out, dtype), want["q"], qin, dtype)
    _say(name, "q max diff", worst, "outside bound", nbad)
    assert nbad == 0
    # written key rows within the rounding bound, value rows bit-exact
    slots = want["slots"]
    kc_after = _host_bits(step.k_cache)
    vc_after = _host_bits(step.v_cache)
    kin = _as_f64(step.k, dtype)
    nbad, worst = _within_rounding(ra.to_f64(kc_after[slots], dtype), want["k_cache"][slots], kin, dtype)
    _say(name, "k max diff", worst, "outside bound", nbad)
    assert nbad == 0
    assert np.array_equal(vc_after[slots].view(np.uint8), _host_bits(step.v).view(np.uint8))
    if rdim < d:  # dims past the rotary ones are copied bit for bit
        assert np.array_equal(kc_after[slots][..., rdim:].view(np.uint8), _host_bits(step.k)[..., rdim:].view(np.uint8))
    # no other cache row changed (NaN rows compared by their bits)
    others = np.setdiff1d(np.arange(kc_before.shape[0]), slots)
    assert np.array_equal(kc_after[others].view(np.uint8), kc_before[others].view(np.uint8))
    assert np.array_equal(vc_after[others].view(np.uint8), vc_before[others].view(np.uint8))
    if rdim == 0:
        assert np.array_equal(_host_bits(q_out).view(np.uint8), _host_bits(step.q).view(np.uint8))
    del step
    torch.cuda.empty_cache()


ERR_CASES = [
    # (name, lq, past, capacity, rows, position ids)
    ("negative_past", [1, 2], [-1, 3], 8, 64, None),
    ("overflow", [1, 3], [2, 6], 8, 64, None),
    ("position_beyond_table", [1, 2], [2, 3], 8, 4, None),
    ("negative_position_id", [2, 1], [0, 0], 8, 64, [0, -3, 1]),
]


@pytest.mark.parametrize("case", ERR_CASES, ids=[c[0] for c in ERR_CASES])
def test_cache_step_latches_invalid_input(case):
    """The conditions are forced from the host; every access stays inside the
    buffers, and the offending sequence's cache rows keep their contents."""
    import torch
    name, lq, past, cap, rows, pos_ids = case
    w = synth.Workload("custom", 0, 4, 2, 64, "bf16", True, 0.0, 0.0, 1.0, 22)
    _say("latch", name, lq, past, cap, rows, pos_ids)
    safe_past = [max(0, min(p, cap)) for p in past]
    step = synth.make_cache_step(w, lq, safe_past, cap, device="cuda")
    step.past = list(past)
    kc_before = _host_bits(step.k_cache).copy()
    _, _, latch, (cos, sin) = _run_step(step, 64, False, pos_ids=pos_ids, rows=rows)
    want = ra.kv_append_rope(_host_bits(step.q), _host_bits(step.k), _host_bits(step.v), kc_before,
                             _host_bits(step.v_cache), step.cu_q, past, cap, cos.cpu().numpy(), sin.cpu().numpy(),
                             position_ids=pos_ids, dtype="bf16")
    got = int(latch.item())
    _say("latch", name, "got", got, "want", want["err"])
    assert got == want["err"] != 0
    kc_after = _host_bits(step.k_cache)
    for b, (p, n) in enumerate(zip(past, lq)):
        if p < 0 or p + n > cap:
            region = slice(b * cap, (b + 1) * cap)
            assert np.array_equal(kc_after[region].view(np.uint8), kc_before[region].view(np.uint8))


# --------------------------------------------------------------------------
# Attention over the cache.
# --------------------------------------------------------------------------
def _attention_over_cache(q, kc, vc, cu_q, kv_len, w, out=None, ws=None, latch=None, window=None):
    import torch
    import packed_varlen_scaled_amd as pva
    bsz = cu_q.numel() - 1
    cap = kc.shape[0] // bsz
    if ws is None:
        n = pva.device_workspace_bytes(bsz, q.shape[0], bsz * cap, w.num_heads, w.kv_num_heads, w.head_dim, w.dv,
                                       w.dtype)
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    if latch is None:
        latch = torch.zeros(1, dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty(q.shape[0], w.num_heads, w.dv, dtype=q.dtype, device=q.device)
    pva.varlen_attn_fwd_kvcache(q, kc, vc, cu_q, kv_len, w.num_heads, w.kv_num_heads, scale=w.scale or None,
                                is_causal=w.is_causal, softcap=w.softcap, local_window=window, out=out,
                                workspace=ws, error_latch=latch)
    return out, latch


def _gather(cache_host, kv_len, cap):
    """Packed rows [sum kv_len, H, D] of a cache held on the host, and cu_kv."""
    parts = [cache_host[b * cap:b * cap + n] for b, n in enumerate(kv_len)]
    return np.concatenate(parts, axis=0), synth.cu_seqlens(kv_len)


ATTN_CASES = [
    # (name, dtype, hq, hkv, d, dv, softcap, lq, past, capacity, window)
    ("bf16_decode", "bf16", 16, 2, 128, None, 0.0, [1, 1, 1, 1, 1], [0, 700, 3000, 129, 5], 3072, None),
    ("bf16_chunked", "bf16", 8, 2, 128, None, 20.0, [40, 1, 129, 0], [260, 900, 0, 12], 1024, None),
    ("f16_d64_window", "f16", 8, 2, 64, None, 0.0, [1, 33, 1], [1999, 100, 64], 2048, 96),
    ("bf16_dv64", "bf16", 8, 2, 128, 64, 0.0, [1, 70, 1], [500, 30, 0], 512, None),
    ("f32_small", "f32", 4, 2, 64, None, 0.0, [3, 1, 9], [5, 40, 0], 64, None),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_over_cache_matches_oracle(case):
    """The new rows are copied into their slots (plain data movement), the
    attention reads the cache, and the packed call on the same rows gives the
    same bits; the unused slots hold NaN, so any read of one would show."""
    _check_cache_attention(*case)


@pytest.mark.parametrize("seed", list(range(48)))
def test_random_attention_over_cache_matches_oracle(seed):
    """Seeded random batches over caches (tests/random_cases.py), causal or
    not, to the same bar."""
    from random_cases import random_cache_attn_case
    c = random_cache_attn_case(seed)
    _check_cache_attention(f"random_cache{seed}", c.dtype, c.hq, c.hkv, c.d, c.dv, c.softcap, list(c.lq),
                           list(c.past), c.capacity, c.window or None, causal=c.causal, seed=600 + seed)


def _check_cache_attention(name, dtype, hq, hkv, d, dv, softcap, lq, past, cap, window, causal=True, seed=23):
    import torch
    import packed_varlen_scaled_amd as pva
    w = synth.Workload("custom", 0, hq, hkv, d, dtype, causal, softcap, 0.0, 1.0, seed, dv)
    _say("cache attention", name, dtype, hq, hkv, d, dv, causal, softcap, lq, past, cap, window)
    step = synth.make_cache_step(w, lq, past, cap, device="cuda")
    for b in range(len(lq)):
        s0, n = b * cap + past[b], lq[b]
        step.k_cache[s0:s0 + n] = step.k[step.cu_q[b]:step.cu_q[b] + n]
        step.v_cache[s0:s0 + n] = step.v[step.cu_q[b]:step.cu_q[b] + n]
    kv_len = torch.tensor(step.kv_len, dtype=torch.int32, device="cuda")
    cu_q = torch.from_numpy(step.cu_q).cuda()
    out, latch = _attention_over_cache(step.q, step.k_cache, step.v_cache, cu_q, kv_len, w, window=window)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0
    kp, cu_kv = _gather(_host_bits(step.k_cache), step.kv_len, cap)
    vp, _ = _gather(_host_bits(step.v_cache), step.kv_len, cap)
    want = oracle.attention(_host_bits(step.q), kp, vp, step.cu_q, cu_kv, hq, hkv, is_causal=causal, softcap=softcap,
                            dtype=dtype, local_window=window or 0).reshape(step.total_q, hq, w.dv)
    got = out.double().cpu().numpy().reshape(step.total_q, hq, w.dv)
    ma, rel = compare(got, want, dtype)
    _say("cache attention", name, "max_abs", ma, "rel_l2", rel)
    # the packed device call over the same rows: the same kernels, the same bits
    kpt = torch.from_numpy(kp.view(np.int16) if dtype == "bf16" else kp).cuda()
    vpt = torch.from_numpy(vp.view(np.int16) if dtype == "bf16" else vp).cuda()
    if dtype == "bf16":
        kpt, vpt = kpt.view(torch.bfloat16), vpt.view(torch.bfloat16)
    ws = torch.empty(pva.device_workspace_bytes(len(lq), step.total_q, int(cu_kv[-1]), hq, hkv, d, w.dv, dtype),
                     dtype=torch.uint8, device="cuda")
    latch2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    out2 = torch.empty_like(out)
    pva.varlen_attn_fwd_device(step.q, kpt, vpt, cu_q, torch.from_numpy(cu_kv).cuda(), hq, hkv,
                               is_causal=causal, softcap=softcap, local_window=window, out=out2, workspace=ws,
                               error_latch=latch2)
    torch.cuda.synchronize()
    assert int(latch2.item()) == 0
    assert torch.equal(out, out2)


def test_cache_attention_latches_lengths_beyond_capacity():
    import torch
    w = synth.Workload("custom", 0, 4, 2, 64, "bf16", True, 0.0, 0.0, 1.0, 24)
    step = synth.make_cache_step(w, [1, 1], [3, 5], 8, device="cuda")
    cu_q = torch.from_numpy(step.cu_q).cuda()
    for lens in ([4, 9], [-1, 2]):
        _say("cache attention latch", lens)
        out = torch.full((step.total_q, 4, 64), 3.0, dtype=torch.bfloat16, device="cuda")
        kv_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
        out, latch = _attention_over_cache(step.q, step.k_cache, step.v_cache, cu_q, kv_len, w, out=out)
        torch.cuda.synchronize()
        assert int(latch.item()) == 1024
        assert bool((out == 3.0).all())


def test_decode_step_in_a_graph():
    """Cache step + attention over the cache captured once and replayed for
    several steps of a growing decode; every replay matches the eager calls
    and the oracle."""
    import torch
    import packed_varlen_scaled_amd as pva
    w = synth.Workload("custom", 0, 16, 2, 128, "bf16", True, 0.0, 0.0, 1.0, 25)
    lq, past0, cap = [1, 1, 1], [100, 1000, 7], 2048
    bsz = len(lq)
    step = synth.make_cache_step(w, lq, past0, cap, device="cuda")
    cos, sin = synth.rotary_tables(cap, 128, device="cuda")
    dev = "cuda"
    cu_q = torch.from_numpy(step.cu_q).to(dev)
    past = torch.tensor(past0, dtype=torch.int32, device=dev)
    kv_len = torch.zeros(bsz, dtype=torch.int32, device=dev)
    latch = torch.zeros(1, dtype=torch.int32, device=dev)
    q_new = step.q.clone()
    k_new, v_new = step.k.clone(), step.v.clone()
    q_rot = torch.empty_like(q_new)
    out = torch.empty(bsz, 16, 128, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(pva.device_workspace_bytes(bsz, bsz, bsz * cap, 16, 2, 128, 0, "bf16"), dtype=torch.uint8,
                     device=dev)
    kc_ref = step.k_cache.clone()
    vc_ref = step.v_cache.clone()

    def decode_step(kc, vc, o):
        pva.kv_append_rope(q_new, k_new, v_new, kc, vc, cu_q, past, 16, 2, cos=cos, sin=sin, q_out=q_rot,
                           kv_seqlens_out=kv_len, error_latch=latch)
        pva.varlen_attn_fwd_kvcache(q_rot, kc, vc, cu_q, kv_len, 16, 2, is_causal=True, out=o, workspace=ws,
                                    error_latch=latch)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        decode_step(step.k_cache, step.v_cache, out)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        decode_step(step.k_cache, step.v_cache, out)
    gen = torch.Generator(device=dev)
    # the oracle's own cache, evolved from the seeded cache by the oracle step
    ora_k = _as_f64(kc_ref, "bf16").astype(np.float32)
    ora_v = _as_f64(vc_ref, "bf16").astype(np.float32)
    cs, sn = cos.cpu().numpy(), sin.cpu().numpy()
    for it in range(3):
        gen.manual_seed(100 + it)
        q_new.copy_(torch.randn(q_new.shape, generator=gen, device=dev).to(torch.bfloat16))
        k_new.copy_(torch.randn(k_new.shape, generator=gen, device=dev).to(torch.bfloat16))
        v_new.copy_(torch.randn(v_new.shape, generator=gen, device=dev).to(torch.bfloat16))
        now = [p + it for p in past0]
        past.copy_(torch.tensor(now, dtype=torch.int32))
        _say("graph decode step", it, now)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = torch.empty_like(out)
        decode_step(kc_ref, vc_ref, eager)
        torch.cuda.synchronize()
        assert int(latch.item()) == 0
        assert torch.equal(got, eager)
        assert torch.equal(step.k_cache.view(torch.int16), kc_ref.view(torch.int16))
        assert torch.equal(step.v_cache.view(torch.int16), vc_ref.view(torch.int16))
        res = ra.kv_append_rope(_as_f64(q_new, "bf16").astype(np.float32), _as_f64(k_new, "bf16").astype(np.float32),
                                _as_f64(v_new, "bf16").astype(np.float32), ora_k, ora_v, step.cu_q, now, cap, cs, sn,
                                dtype="f32")
        assert res["err"] == 0
        ora_k, ora_v = res["k_cache"].astype(np.float32), res["v_cache"].astype(np.float32)
        lens = res["kv_len"].tolist()
        kp, cu_kv = _gather(ora_k, lens, cap)
        vp, _ = _gather(ora_v, lens, cap)
        want = oracle.attention(res["q"].astype(np.float32), kp, vp, step.cu_q, cu_kv, 16, 2, is_causal=True,
                                dtype="f32").reshape(bsz, 16, 128)
        compare(got.double().cpu().numpy(), want, "bf16")


@pytest.mark.parametrize("name", ["packed_decode", "chunked_prefill_cache"])
def test_full_size_cache_path_sampled(name):
    """The full-size workload as the benchmark's --cache run launches it: the
    packed K/V rows fill the cache, the last L_q rows of each sequence are the
    new rows (turned by the cache step), and sampled sequences are checked
    against the oracle on the oracle's own rotation of those rows."""
    import torch
    import packed_varlen_scaled_amd as pva
    w = synth.WORKLOADS[name]
    _say("full cache", name)
    batch = synth.workload_batch(name, device="cuda")
    bsz = len(batch.lq)
    cap = (max(batch.lkv) + 255) // 256 * 256
    kc = torch.empty(bsz * cap, w.kv_num_heads, w.head_dim, dtype=batch.k.dtype, device="cuda")
    vc = torch.empty(bsz * cap, w.kv_num_heads, w.dv, dtype=batch.v.dtype, device="cuda")
    idx, past = [], []
    for b, (nq, nkv) in enumerate(zip(batch.lq, batch.lkv)):
        k0 = int(batch.cu_kv[b])
        kc[b * cap:b * cap + nkv - nq] = batch.k[k0:k0 + nkv - nq]
        vc[b * cap:b * cap + nkv - nq] = batch.v[k0:k0 + nkv - nq]
        idx.append(torch.arange(k0 + nkv - nq, k0 + nkv, device="cuda"))
        past.append(nkv - nq)
    idx = torch.cat(idx)
    k_new, v_new = batch.k[idx].contiguous(), batch.v[idx].contiguous()
    cu_q = torch.from_numpy(batch.cu_q).cuda()
    past_t = torch.tensor(past, dtype=torch.int32, device="cuda")
    kv_len = torch.empty(bsz, dtype=torch.int32, device="cuda")
    latch = torch.zeros(1, dtype=torch.int32, device="cuda")
    cos, sin = synth.rotary_tables(cap, w.head_dim, device="cuda")
    q_rot = torch.empty_like(batch.q)
    out = torch.empty(batch.total_q, w.num_heads, w.dv, dtype=batch.q.dtype, device="cuda")
    ws = torch.empty(pva.device_workspace_bytes(bsz, batch.total_q, bsz * cap, w.num_heads, w.kv_num_heads,
                                                w.head_dim, w.dv, w.dtype), dtype=torch.uint8, device="cuda")
    pva.kv_append_rope(batch.q, k_new, v_new, kc, vc, cu_q, past_t, w.num_heads, w.kv_num_heads, cos=cos, sin=sin,
                       q_out=q_rot, kv_seqlens_out=kv_len, error_latch=latch)
    pva.varlen_attn_fwd_kvcache(q_rot, kc, vc, cu_q, kv_len, w.num_heads, w.kv_num_heads, scale=w.scale or None,
                                is_causal=w.is_causal, softcap=w.softcap, out=out, workspace=ws, error_latch=latch)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0
    assert kv_len.cpu().tolist() == list(batch.lkv)
    cs, sn = cos.cpu().numpy().astype(np.float64), sin.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(1)
    longest = int(np.argmax(np.asarray(batch.lkv)))
    seqs = sorted({longest, *rng.choice(bsz, size=3, replace=False).tolist()})
    for b in seqs:
        q0, q1 = int(batch.cu_q[b]), int(batch.cu_q[b + 1])
        k0, k1 = int(batch.cu_kv[b]), int(batch.cu_kv[b + 1])
        nq = q1 - q0
        qd = _as_f64(batch.q[q0:q1], w.dtype)
        kd = _as_f64(batch.k[k0:k1], w.dtype)
        vd = _as_f64(batch.v[k0:k1], w.dtype)
        pos = past[b] + np.arange(nq)
        qr = ra.rotate(qd, cs[pos][:, None, :], sn[pos][:, None, :], w.head_dim, False)
        kd[k1 - k0 - nq:] = ra.rotate(kd[k1 - k0 - nq:], cs[pos][:, None, :], sn[pos][:, None, :], w.head_dim, False)
        want = oracle.attention(qr.astype(np.float32), kd.astype(np.float32), vd.astype(np.float32), [0, nq],
                                [0, k1 - k0], w.num_heads, w.kv_num_heads, scale=w.scale or None,
                                is_causal=w.is_causal, softcap=w.softcap, dtype="f32").reshape(nq, w.num_heads, w.dv)
        ma, rel = compare(out[q0:q1].double().cpu().numpy(), want, w.dtype)
        _say("full cache", name, "seq", b, "L_q", nq, "L_kv", k1 - k0, "max_abs", ma, "rel_l2", rel)
    del batch, kc, vc, out
    torch.cuda.empty_cache()
