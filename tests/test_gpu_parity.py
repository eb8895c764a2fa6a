"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small shapes compare every output element; the full-size workloads compare
sampled rows (the oracle computes them one by one on a sub-batch of the
sampled sequences). Every case prints what it runs before it runs it.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest

import synth
from parity import compare, gather_gpu, oracle_all, oracle_sampled, run_gpu, sample_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def _workload(dtype="bf16", hq=8, hkv=2, d=128, causal=True, softcap=0.0, scale=0.0, sigma=1.0, seed=11, dv=None):
    return synth.Workload("custom", 0, hq, hkv, d, dtype, causal, softcap, scale, sigma, seed, dv)


def _batch(w, lq, lkv):
    return synth.make_batch(w, lq, lkv, device="cuda")


SMALL = [
    # (name, workload kwargs, lq, lkv)
    ("bf16_gqa4_causal", dict(hq=8, hkv=2), [70, 1, 129, 33, 0, 200], [70, 1, 129, 33, 5, 200]),
    ("bf16_gqa4_tail_aligned", dict(hq=8, hkv=2), [40, 3, 100, 1], [300, 90, 100, 17]),
    ("bf16_lq_gt_lkv", dict(hq=4, hkv=1), [50, 65], [10, 64]),
    ("bf16_noncausal_mha", dict(hq=4, hkv=4, causal=False), [77, 128, 5], [31, 128, 200]),
    ("bf16_gqa8_softcap", dict(hq=16, hkv=2, softcap=30.0, sigma=1.5), [150, 64, 1], [150, 64, 900]),
    ("bf16_mqa", dict(hq=6, hkv=1), [90, 2], [90, 70]),
    ("bf16_gqa16", dict(hq=32, hkv=2), [45, 1], [45, 600]),
    ("bf16_d64", dict(hq=8, hkv=2, d=64), [100, 1, 37], [100, 513, 37]),
    ("f16_gqa4_causal", dict(dtype="f16", hq=8, hkv=2), [70, 1, 129], [70, 700, 129]),
    ("f16_d64_softcap", dict(dtype="f16", hq=4, hkv=2, d=64, softcap=5.0), [33, 1], [60, 300]),
    ("bf16_scale", dict(hq=4, hkv=2, scale=0.3, causal=False), [64, 20], [64, 96]),
    ("bf16_negative_softcap", dict(hq=4, hkv=2, softcap=-8.0), [80], [80]),
    ("f32_gqa_causal", dict(dtype="f32", hq=8, hkv=2, d=64), [70, 1, 33], [70, 200, 40]),
    ("f32_d128_softcap", dict(dtype="f32", hq=4, hkv=4, d=128, softcap=5.0, causal=False), [40, 3], [17, 90]),
    ("f32_odd_dim", dict(dtype="f32", hq=2, hkv=1, d=40, causal=True), [9, 30], [12, 30]),
    # Softcap ranges for the MFMA kernel's two tanh forms: every tile inside the
    # short-series range, tiles on both sides of it, and a very large cap whose
    # range bound is the f16 clamp.
    ("bf16_softcap_series_only", dict(hq=8, hkv=2, softcap=50.0, sigma=0.5), [200, 1, 77], [200, 300, 77]),
    ("bf16_softcap_series_edge", dict(hq=8, hkv=2, softcap=10.0, sigma=1.0), [150, 33], [150, 400]),
    ("f16_softcap_wide_cap", dict(dtype="f16", hq=8, hkv=2, softcap=1000.0, sigma=3.0), [130, 5], [130, 260]),
]


@pytest.mark.parametrize("name,kw,lq,lkv", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes_match_oracle(name, kw, lq, lkv):
    w = _workload(**kw)
    _say(name, w, lq, lkv)
    batch = _batch(w, lq, lkv)
    got = run_gpu(batch).double().cpu().numpy().reshape(batch.total_q, w.num_heads, w.dv)
    want = oracle_all(batch)
    ma, rel = compare(got, want, w.dtype)
    _say(name, "max_abs", ma, "rel_l2", rel)


@pytest.mark.parametrize("opts", [dict(decode_path=1), dict(decode_chunk=128), dict(prefill_kv_chunk=64),
                                  dict(prefill_kv_chunk=192, decode_chunk=256)])
def test_split_paths_match_oracle(opts):
    w = _workload(hq=16, hkv=2, softcap=20.0)
    lq, lkv = [1, 100, 1, 257, 1], [1000, 700, 129, 300, 5]
    _say("split paths", opts, lq, lkv)
    batch = _batch(w, lq, lkv)
    got = run_gpu(batch, **opts).double().cpu().numpy().reshape(batch.total_q, w.num_heads, w.dv)
    compare(got, oracle_all(batch), w.dtype)


def test_fully_masked_and_empty_rows_are_exactly_zero():
    w = _workload(hq=8, hkv=2)
    lq, lkv = [70, 5, 40, 1], [3, 0, 0, 0]
    _say("masked rows", lq, lkv)
    batch = _batch(w, lq, lkv)
    got = run_gpu(batch).float().cpu().numpy().reshape(batch.total_q, w.num_heads, w.dv)
    # sequence 0: L_q=70, L_kv=3, offset -67: rows 0..66 see nothing
    assert np.all(got[:67] == 0) and np.any(got[67:70] != 0)
    assert np.all(got[70:] == 0)  # sequences without keys


def test_single_key_returns_value_row():
    import torch
    w = _workload(hq=8, hkv=2, causal=False, softcap=3.0)
    lq, lkv = [5, 1, 40], [1, 1, 1]
    batch = _batch(w, lq, lkv)
    got = run_gpu(batch).view(batch.total_q, 8, 128)
    seq = np.repeat(np.arange(3), lq)
    for t in range(batch.total_q):
        for h in range(8):
            assert torch.equal(got[t, h], batch.v[seq[t], h // 4])


def test_gqa_exact_head_mapping_on_gpu():
    import torch
    w = _workload(hq=8, hkv=2, causal=False)
    batch = _batch(w, [40, 1], [70, 300])
    batch.k[:] = 1.0  # identical keys: output = mean of V of the head's kv group
    for g in range(2):
        batch.v[:, g, :] = g + 1
    got = run_gpu(batch).view(batch.total_q, 8, 128).float()
    for h in range(8):
        assert torch.all(got[:, h] == h // 4 + 1)


def test_neighbour_sequence_cannot_leak():
    """Poisoning the next sequence's K/V with inf/nan must not change a single
    bit of the previous sequence's output (block-diagonal attention; key tiles
    past a sequence end are zero-filled, never just masked)."""
    import torch
    w = _workload(hq=8, hkv=2)
    lq, lkv = [77, 1, 50], [77, 130, 50]
    batch = _batch(w, lq, lkv)
    a = run_gpu(batch).clone()
    k0 = int(batch.cu_kv[1])
    batch.k[k0:] = float("inf")
    batch.v[k0:] = float("nan")
    b = run_gpu(batch)
    assert torch.equal(a[:77], b[:77])


def test_rerun_is_bitwise_deterministic():
    import torch
    w = _workload(hq=16, hkv=2, softcap=10.0)
    batch = _batch(w, [300, 1, 129], [300, 5000, 200])
    outs = [run_gpu(batch).clone() for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_sequence_alone_equals_sequence_in_batch():
    """Prefill tiles start at each sequence's own row 0, so a sequence gives
    the same bits alone as inside a batch."""
    import torch
    w = _workload(hq=8, hkv=2)
    lq = [100, 257, 64]
    full = _batch(w, lq, lq)
    a = run_gpu(full)
    q0, q1 = int(full.cu_q[1]), int(full.cu_q[2])
    alone = synth.Batch(w, [257], [257], synth.cu_seqlens([257]), synth.cu_seqlens([257]),
                        full.q[q0:q1].contiguous(), full.k[q0:q1].contiguous(), full.v[q0:q1].contiguous())
    b = run_gpu(alone)
    assert torch.equal(a[q0:q1], b)


def test_rank2_layout_and_device_cu_read():
    """Rank-2 [T, H*D] tensors and cu arrays read from the device (no host
    mirrors) give the same result as rank-3 with host mirrors."""
    import torch
    import packed_varlen_scaled_amd as pva
    w = _workload(hq=8, hkv=2)
    batch = _batch(w, [30, 1, 90], [60, 100, 90])
    a = run_gpu(batch)
    cu_q = torch.from_numpy(batch.cu_q).cuda()
    cu_kv = torch.from_numpy(batch.cu_kv).cuda()
    b = pva.varlen_attn_fwd(batch.q.view(batch.total_q, -1), batch.k.view(batch.total_kv, -1),
                            batch.v.view(batch.total_kv, -1), cu_q, cu_kv, 8, 2, is_causal=True)
    torch.cuda.synchronize()
    assert b.shape == (batch.total_q, 8 * 128)
    assert torch.equal(a.view(batch.total_q, -1), b)


def test_tiny_fp32_workload_full():
    batch = synth.workload_batch("tiny_fp32", device="cuda")
    _say("tiny_fp32", batch.lq)
    got = run_gpu(batch).double().cpu().numpy().reshape(batch.total_q, 4, 64)
    ma, _ = compare(got, oracle_all(batch), "f32")
    _say("tiny_fp32 max_abs", ma)


# Reduced versions of the four large workloads (same heads, types, masks and
# value scales; a handful of sequences the oracle finishes in seconds).
REDUCED = {
    "ragged_causal_prefill": ([233, 1000, 130], None),
    "long_causal_softcap": ([700, 1500], None),
    "chunked_prefill_cache": ([3, 100, 512, 1], [3 + 2000, 100, 512 + 800, 1 + 8192]),
    "packed_decode": ([1] * 6, [256, 300, 4097, 1000, 32768, 777]),
}


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_reduced_workloads_full_compare(name):
    w = synth.WORKLOADS[name]
    lq, lkv = REDUCED[name]
    lkv = lkv or lq
    _say("reduced", name, lq, lkv)
    batch = synth.make_batch(w, lq, lkv, device="cuda")
    got = run_gpu(batch).double().cpu().numpy().reshape(batch.total_q, w.num_heads, w.dv)
    ma, rel = compare(got, oracle_all(batch), w.dtype)
    _say("reduced", name, "max_abs", ma, "rel_l2", rel)


@pytest.mark.parametrize("name", ["ragged_causal_prefill", "long_causal_softcap", "chunked_prefill_cache",
                                  "packed_decode"])
def test_full_size_workloads_sampled(name):
    """Full-size batch, launched exactly as the benchmark launches it; the
    oracle checks sampled rows of a few sequences (including the longest)."""
    import torch
    w = synth.WORKLOADS[name]
    _say("full", name)
    batch = synth.workload_batch(name, device="cuda")
    out = run_gpu(batch)
    longest = int(np.argmax(np.asarray(batch.lkv)))
    seqs = sorted({0, longest, len(batch.lq) - 1, len(batch.lq) // 2})
    picks = sample_rows(batch, seqs, rows_per_seq=6 if name != "packed_decode" else 1)
    want = oracle_sampled(batch, picks)
    got = gather_gpu(batch, out, picks)
    ma, rel = compare(got, want, w.dtype)
    _say("full", name, len(picks), "rows max_abs", ma, "rel_l2", rel)
    assert torch.isfinite(out.float()).all()
    del batch, out
    torch.cuda.empty_cache()


def test_one_16384_key_causal_softcap_sequence_sampled():
    """A single sequence at the longest length of the long softcap workload
    (16384 queries and keys, 64 query heads over 8 KV heads, softcap 50,
    inputs N(0, 1.5)): rows spread over the whole range, at the tile edges
    and at the end, on every head for some of them, against the oracle."""
    import torch
    w = synth.WORKLOADS["long_causal_softcap"]
    L = 16384
    _say("single 16384-key sequence", w)
    batch = synth.make_batch(w, [L], [L], device="cuda")
    out = run_gpu(batch)
    rng = np.random.default_rng(5)
    all_heads = [0, 127, 128, 8191, 16383]
    rows = sorted(set(all_heads) | {1, 63, 64, 255, 256, 4095, 4096, 12288, 16256, 16320}
                  | set(rng.integers(0, L, size=24).tolist()))
    picks = []
    for r in rows:
        heads = range(w.num_heads) if r in all_heads else rng.integers(0, w.num_heads, size=4).tolist()
        picks += [(0, int(r), int(h)) for h in heads]
    ma, rel = compare(gather_gpu(batch, out, picks), oracle_sampled(batch, picks), w.dtype)
    _say("single 16384-key sequence", len(picks), "rows max_abs", ma, "rel_l2", rel)
    assert torch.isfinite(out.float()).all()
    del batch, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["ragged_causal_prefill", "long_causal_softcap", "chunked_prefill_cache",
                                  "packed_decode"])
def test_benchmark_graph_replay_equals_host_call_full_size(name):
    """The call the benchmark times: varlen_attn_fwd_device on the full-size
    batch, captured once into a HIP graph after a warm-up on a side stream
    (decode-only batches fork decode and combine onto the library's side
    stream inside the capture). Three replays, with eager host-planned calls
    in between, each equal the host-planned call bit for bit."""
    import torch
    import packed_varlen_scaled_amd as pva
    w = synth.WORKLOADS[name]
    _say("bench graph", name)
    batch = synth.workload_batch(name, device="cuda")
    want = run_gpu(batch).clone()
    cu_q = torch.from_numpy(batch.cu_q).cuda()
    cu_kv = torch.from_numpy(batch.cu_kv).cuda()
    out = torch.empty_like(want)
    ws, latch = _device_buffers(batch)

    def call():
        pva.varlen_attn_fwd_device(batch.q, batch.k, batch.v, cu_q, cu_kv, w.num_heads, w.kv_num_heads,
                                   scale=w.scale or None, is_causal=w.is_causal, softcap=w.softcap, out=out,
                                   workspace=ws, error_latch=latch)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(latch.item()) == 0
        assert torch.equal(out, want), (name, rep)
        assert torch.equal(run_gpu(batch), want), (name, rep)
    _say("bench graph", name, "3 replays bitwise equal")
    del g, batch, out, want, ws
    torch.cuda.empty_cache()


def test_offsets_past_2_31_elements():
    """Sequences whose Q/O and K/V element offsets lie past 2^31: a filler of
    530000 query rows with no keys (its rows must be exactly zero) and one of
    2.2 M keys with no queries come first, then a prefill, a tail-aligned and
    a decode sequence, which the oracle checks. The device-scheduled call
    must give bitwise the same output."""
    import torch
    w = _workload(hq=32, hkv=8, d=128)
    lq = [530000, 0, 300, 100, 1]
    lkv = [0, 2200000, 300, 2000, 5000]
    _say("offsets past 2^31", lq, lkv)
    batch = _batch(w, lq, lkv)
    assert int(batch.cu_q[2]) * w.num_heads * w.head_dim > 2 ** 31
    assert int(batch.cu_kv[2]) * w.kv_num_heads * w.head_dim > 2 ** 31
    out = run_gpu(batch)
    assert int(torch.count_nonzero(out[:lq[0]]).item()) == 0
    picks = sample_rows(batch, [2, 3, 4], rows_per_seq=6)
    want = oracle_sampled(batch, picks)
    got = gather_gpu(batch, out, picks)
    ma, rel = compare(got, want, w.dtype)
    _say("offsets past 2^31", len(picks), "rows max_abs", ma, "rel_l2", rel)
    ws, latch = _device_buffers(batch)
    out2 = torch.full_like(out, 7.0)
    _device_call(batch, out2, ws, latch)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0
    assert torch.equal(out2, out)
    del batch, out, out2, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_scores_rising_after_first_tile(dtype):
    """Keys after the first 64 score far higher (by ~40 in natural-log units)
    than the first tile's: the prefill kernel must redo such items with the
    running-max softmax, and the result must still match the oracle."""
    import torch
    w = _workload(dtype=dtype, hq=8, hkv=2, causal=False)
    lq, lkv = [40, 70], [300, 200]
    batch = _batch(w, lq, lkv)
    tdt = batch.q.dtype
    batch.q[:] = 0.5
    batch.k[:] = 0.01
    k1 = int(batch.cu_kv[1])
    batch.k[64:k1] = (torch.arange(64, k1, device="cuda").float() / k1 * 2.0).view(-1, 1, 1).to(tdt)
    batch.k[k1 + 64:] = 1.5
    _say("rising scores", dtype)
    got = run_gpu(batch).double().cpu().numpy().reshape(batch.total_q, w.num_heads, w.dv)
    compare(got, oracle_all(batch), w.dtype)


def test_back_to_back_calls_on_two_streams():
    """Calls issued without synchronising, alternating two streams and three
    problem sizes (with split-KV partials): the work-list slots and the
    partials buffer are reused while earlier calls may still run, and every
    result must equal the same call made alone."""
    import torch
    import packed_varlen_scaled_amd as pva
    w = _workload(hq=16, hkv=2, softcap=20.0)
    shapes = [([1, 100, 1, 257, 1], [1000, 700, 129, 300, 5]), ([64, 1, 300], [64, 4000, 300]),
              ([1] * 9, [300 + 500 * i for i in range(9)])]
    batches = [_batch(w, lq, lkv) for lq, lkv in shapes]
    alone = [run_gpu(b).clone() for b in batches]

    def call(b, out):
        cu_q = torch.from_numpy(b.cu_q).cuda()
        cu_kv = torch.from_numpy(b.cu_kv).cuda()
        pva.varlen_attn_fwd(b.q, b.k, b.v, cu_q, cu_kv, w.num_heads, w.kv_num_heads, is_causal=True,
                            softcap=w.softcap, out=out, cu_seqlens_q_host=b.cu_q, cu_seqlens_kv_host=b.cu_kv)

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(a) for a in alone] for _ in range(4)]
    torch.cuda.synchronize()
    _say("two streams, 12 calls")
    for r in range(4):
        for i, b in enumerate(batches):
            with torch.cuda.stream(streams[(r * 3 + i) % 2]):
                call(b, outs[r][i])
    torch.cuda.synchronize()
    for r in range(4):
        for i in range(3):
            assert torch.equal(outs[r][i], alone[i]), (r, i)


# Value head size different from the query/key head size (v_head_size is
# its own input dimension: packed_varlen_attention.rs page, "Schema (v1)").
DV_CASES = [
    # (name, workload kwargs, lq, lkv, local window, options)
    ("bf16_d128_dv64_causal", dict(hq=8, hkv=2, dv=64), [70, 1, 129, 33, 0, 200], [70, 1, 129, 33, 5, 200], None, {}),
    ("bf16_d64_dv128_causal", dict(hq=8, hkv=2, d=64, dv=128), [70, 1, 129, 33], [70, 900, 129, 40], None, {}),
    ("bf16_d128_dv64_noncausal_mha", dict(hq=4, hkv=4, causal=False, dv=64), [77, 128, 5], [31, 128, 200], None, {}),
    ("f16_d64_dv128_softcap", dict(dtype="f16", hq=16, hkv=2, d=64, dv=128, softcap=20.0, sigma=1.5),
     [150, 64, 1], [150, 64, 900], None, {}),
    ("f16_d128_dv64_tail_aligned", dict(dtype="f16", hq=8, hkv=2, dv=64), [40, 3, 100, 1], [300, 90, 100, 17],
     None, {}),
    ("bf16_d128_dv64_decode_split", dict(hq=16, hkv=2, dv=64, softcap=20.0), [1, 100, 1, 257, 1],
     [1000, 700, 129, 300, 5], None, dict(decode_chunk=128)),
    ("bf16_d64_dv128_decode_split", dict(hq=16, hkv=2, d=64, dv=128), [1, 1, 1, 100], [3000, 500, 800, 1000],
     None, dict(decode_chunk=256)),
    ("bf16_d64_dv128_prefill_split", dict(hq=8, hkv=2, d=64, dv=128), [257, 100], [900, 1000], None,
     dict(prefill_kv_chunk=128)),
    ("bf16_d128_dv64_window", dict(hq=8, hkv=2, dv=64), [40, 3, 100, 1], [300, 90, 100, 1700], 64, {}),
    ("bf16_d64_dv128_prefill_only", dict(hq=8, hkv=2, d=64, dv=128), [1, 64, 1], [500, 64, 91], None,
     dict(decode_path=1)),
]


@pytest.mark.parametrize("name,kw,lq,lkv,window,opts", DV_CASES, ids=[c[0] for c in DV_CASES])
def test_value_head_size_differs(name, kw, lq, lkv, window, opts):
    w = _workload(**kw)
    _say(name, w, lq, lkv, "window", window, opts)
    batch = _batch(w, lq, lkv)
    got = run_gpu(batch, local_window=window, **opts).double().cpu().numpy().reshape(
        batch.total_q, w.num_heads, w.dv)
    ma, rel = compare(got, oracle_all(batch, local_window=window or 0), w.dtype)
    _say(name, "max_abs", ma, "rel_l2", rel)


# Local window (page src/kernels/attention.rs, softmax kernel local_min; page
# src/kernels/group_query_attention.rs, local_window_size): each case against
# the oracle with the same window.
WINDOW = [
    # (name, workload kwargs, lq, lkv, window, options)
    ("bf16_gqa4_causal_w48", dict(hq=8, hkv=2), [70, 1, 129, 33, 0, 200], [70, 1, 129, 33, 5, 200], 48, {}),
    ("bf16_gqa4_causal_w1", dict(hq=8, hkv=2), [70, 9], [70, 40], 1, {}),
    ("bf16_gqa4_tail_aligned_w100", dict(hq=8, hkv=2), [40, 3, 100, 1], [300, 90, 100, 17], 100, {}),
    ("bf16_noncausal_w70", dict(hq=4, hkv=4, causal=False), [77, 128, 5], [31, 128, 200], 70, {}),
    ("bf16_mha_rows4_w20", dict(hq=2, hkv=2), [300, 77], [300, 77], 20, {}),
    ("bf16_gqa2_rows2_w150", dict(hq=4, hkv=2), [257, 64], [257, 400], 150, {}),
    ("bf16_gqa8_softcap_w64", dict(hq=16, hkv=2, softcap=30.0, sigma=1.5), [150, 64, 1], [150, 64, 900], 64, {}),
    ("f16_gqa4_w33", dict(dtype="f16", hq=8, hkv=2), [70, 1, 129], [70, 700, 129], 33, {}),
    ("bf16_d64_w10", dict(hq=8, hkv=2, d=64), [100, 1, 37], [100, 513, 37], 10, {}),
    ("bf16_lq_gt_lkv_w5", dict(hq=4, hkv=1), [50, 65], [10, 64], 5, {}),
    ("bf16_window_covers_all", dict(hq=8, hkv=2), [90, 2], [90, 70], 100000, {}),
    ("bf16_decode_split_w700", dict(hq=16, hkv=2), [1, 1, 1, 100], [3000, 500, 800, 1000], 700,
     dict(decode_chunk=256)),
    ("bf16_prefill_split_w300", dict(hq=8, hkv=2, softcap=20.0), [257, 100], [900, 1000], 300,
     dict(prefill_kv_chunk=128)),
    ("bf16_prefill_only_w90", dict(hq=8, hkv=2), [1, 64, 1], [500, 64, 91], 90, dict(decode_path=1)),
    ("f32_gqa_w7", dict(dtype="f32", hq=8, hkv=2, d=64), [70, 1, 33], [70, 200, 40], 7, {}),
    ("f32_noncausal_w12", dict(dtype="f32", hq=4, hkv=4, d=128, softcap=5.0, causal=False), [40, 3], [17, 90], 12, {}),
]


@pytest.mark.parametrize("name,kw,lq,lkv,window,opts", WINDOW, ids=[c[0] for c in WINDOW])
def test_local_window_matches_oracle(name, kw, lq, lkv, window, opts):
    w = _workload(**kw)
    _say(name, w, lq, lkv, "window", window, opts)
    batch = _batch(w, lq, lkv)
    got = run_gpu(batch, local_window=window, **opts).double().cpu().numpy().reshape(
        batch.total_q, w.num_heads, w.dv)
    ma, rel = compare(got, oracle_all(batch, local_window=window), w.dtype)
    _say(name, "max_abs", ma, "rel_l2", rel)


def test_local_window_full_size_sampled():
    """The long causal softcap workload with a 4096-key window, launched as the
    benchmark's --window run launches it; sampled rows against the oracle."""
    import torch
    name, window = "long_causal_softcap", 4096
    w = synth.WORKLOADS[name]
    _say("full window", name, window)
    batch = synth.workload_batch(name, device="cuda")
    out = run_gpu(batch, local_window=window)
    longest = int(np.argmax(np.asarray(batch.lkv)))
    seqs = sorted({0, longest, len(batch.lq) - 1})
    picks = sample_rows(batch, seqs, rows_per_seq=6)
    ma, rel = compare(gather_gpu(batch, out, picks), oracle_sampled(batch, picks, local_window=window), w.dtype)
    _say("full window", name, len(picks), "rows max_abs", ma, "rel_l2", rel)
    assert torch.isfinite(out.float()).all()
    del batch, out
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# Device-scheduled, capture-safe calls (varlen_attn_fwd_device).
# --------------------------------------------------------------------------
def _device_call(batch, out, ws, latch, local_window=None, cu_q=None, cu_kv=None):
    import torch
    import packed_varlen_scaled_amd as pva
    w = batch.workload
    cu_q = torch.from_numpy(batch.cu_q).cuda() if cu_q is None else cu_q
    cu_kv = torch.from_numpy(batch.cu_kv).cuda() if cu_kv is None else cu_kv
    return pva.varlen_attn_fwd_device(batch.q, batch.k, batch.v, cu_q, cu_kv, w.num_heads, w.kv_num_heads,
                                      scale=w.scale or None, is_causal=w.is_causal, softcap=w.softcap,
                                      local_window=local_window, out=out, workspace=ws, error_latch=latch)


def _device_buffers(batch):
    import torch
    import packed_varlen_scaled_amd as pva
    w = batch.workload
    n = pva.device_workspace_bytes(len(batch.lq), batch.total_q, batch.total_kv, w.num_heads, w.kv_num_heads,
                                   w.head_dim, w.dv, w.dtype)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    latch = torch.zeros(1, dtype=torch.int32, device="cuda")
    return ws, latch


DEVICE = [
    ("bf16_gqa4_causal", dict(hq=8, hkv=2), [70, 1, 129, 33, 0, 200], [70, 1, 129, 33, 5, 200], None),
    ("bf16_decode_mix_softcap", dict(hq=16, hkv=2, softcap=20.0), [1, 100, 1, 257, 1], [3000, 700, 129, 300, 5], None),
    ("bf16_window", dict(hq=8, hkv=2), [40, 3, 100, 1], [300, 90, 100, 1700], 64),
    ("bf16_mha_rows4", dict(hq=2, hkv=2, causal=False), [300, 77], [300, 900], None),
    ("f16_gqa8", dict(dtype="f16", hq=16, hkv=2), [150, 64, 1], [150, 64, 900], None),
    ("bf16_d64", dict(hq=8, hkv=2, d=64), [100, 1, 37], [100, 513, 37], None),
    ("bf16_d128_dv64", dict(hq=8, hkv=2, dv=64), [1, 100, 1, 257], [3000, 700, 129, 300], None),
    ("f16_d64_dv128_window", dict(dtype="f16", hq=8, hkv=2, d=64, dv=128), [40, 1, 100], [300, 2000, 100], 48),
    ("f32_gqa", dict(dtype="f32", hq=8, hkv=2, d=64), [70, 1, 33], [70, 200, 40], None),
    # no more rows than sequences: decode + combine run on a side stream
    ("bf16_decode_dominated_mixed", dict(hq=16, hkv=2), [1, 2, 1, 0, 1, 0], [900, 3, 5000, 7, 1, 300], None),
]


@pytest.mark.parametrize("name,kw,lq,lkv,window", DEVICE, ids=[c[0] for c in DEVICE])
def test_device_scheduled_call_equals_host_planned_call(name, kw, lq, lkv, window):
    """The device scheduler emits the host scheduler's items, so the same
    kernels give the same bits."""
    import torch
    w = _workload(**kw)
    _say("device", name, lq, lkv, window)
    batch = _batch(w, lq, lkv)
    want = run_gpu(batch, local_window=window).clone()
    ws, latch = _device_buffers(batch)
    out = torch.full_like(want, 7.0)
    _device_call(batch, out, ws, latch, local_window=window)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0
    assert torch.equal(out, want)
    # and against the oracle
    compare(out.double().cpu().numpy().reshape(batch.total_q, w.num_heads, w.dv),
            oracle_all(batch, local_window=window or 0), w.dtype)


def test_device_scheduler_latches_bad_cu_seqlens():
    import torch
    w = _workload(hq=8, hkv=2)
    batch = _batch(w, [40, 30], [40, 30])
    ws, latch = _device_buffers(batch)
    sentinel = torch.full((batch.total_q, 8, 128), 3.0, dtype=batch.q.dtype, device="cuda")
    cases = [([1, 40, 70], [0, 40, 70], 1), ([0, 40, 30], [0, 40, 70], 2), ([0, 40, 71], [0, 40, 70], 4),
             ([0, 40, 70], [2, 40, 70], 8), ([0, 40, 70], [0, 50, 45], 16), ([0, 40, 70], [0, 40, 80], 32)]
    for cq, ckv, bit in cases:
        _say("latch", cq, ckv, bit)
        latch.zero_()
        out = sentinel.clone()
        _device_call(batch, out, ws, latch, cu_q=torch.tensor(cq, dtype=torch.int32, device="cuda"),
                     cu_kv=torch.tensor(ckv, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert int(latch.item()) == bit
        assert torch.equal(out, sentinel)
    # latch first: a valid call while the latch is set computes nothing
    out = sentinel.clone()
    _device_call(batch, out, ws, latch)
    torch.cuda.synchronize()
    assert int(latch.item()) == 32 and torch.equal(out, sentinel)
    latch.zero_()
    _device_call(batch, out, ws, latch)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0 and torch.equal(out, run_gpu(batch))


def test_device_scheduler_latches_cu_arrays_whose_differences_wrap():
    """A decreasing cu array whose int32 differences wrap to non-negative
    values (INT32_MIN - INT32_MAX == 1) is latched as out of order and nothing
    is computed."""
    import torch
    w = _workload(hq=8, hkv=2)
    batch = _batch(w, [20, 20, 20, 10], [20, 20, 20, 10])
    ws, latch = _device_buffers(batch)
    sentinel = torch.full((batch.total_q, 8, 128), 3.0, dtype=batch.q.dtype, device="cuda")
    imax, imin = 2**31 - 1, -2**31
    good = [0, 20, 40, 60, 70]
    for cq, ckv, bit in [([0, imax, imin, -1, 70], good, 2), (good, [0, imax, imin, -1, 70], 16),
                         ([0, imax, imin, imin + 1, 70], good, 2), ([0, imax, imin, -1, 70], [0, imax, imin, -1, 70], 18)]:
        _say("wrap latch", cq, ckv, bit)
        latch.zero_()
        out = sentinel.clone()
        _device_call(batch, out, ws, latch, cu_q=torch.tensor(cq, dtype=torch.int32, device="cuda"),
                     cu_kv=torch.tensor(ckv, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert int(latch.item()) == bit
        assert torch.equal(out, sentinel)
    latch.zero_()
    _device_call(batch, out, ws, latch)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0 and torch.equal(out, run_gpu(batch))


def test_graph_capture_replays_with_new_lengths():
    """Capture one call into a HIP graph, then replay it with new cu_seqlens
    (fewer or more rows inside the same buffers) and new data: every replay
    equals the eager host-planned call on the same inputs, bit for bit."""
    import torch
    import packed_varlen_scaled_amd as pva
    w = _workload(hq=16, hkv=2, softcap=20.0)
    cap_q, cap_kv, B = 700, 6000, 5
    big = _batch(w, [100, 1, 257, 1, 340], [700, 3000, 300, 1500, 500])
    assert big.total_q <= cap_q and big.total_kv <= cap_kv
    q = torch.zeros(cap_q, 16, 128, dtype=big.q.dtype, device="cuda")
    k = torch.zeros(cap_kv, 2, 128, dtype=big.q.dtype, device="cuda")
    v = torch.zeros(cap_kv, 2, 128, dtype=big.q.dtype, device="cuda")
    out = torch.zeros(cap_q, 16, 128, dtype=big.q.dtype, device="cuda")
    cu_q = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    cu_kv = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    n = pva.device_workspace_bytes(B, cap_q, cap_kv, 16, 2, 128)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    latch = torch.zeros(1, dtype=torch.int32, device="cuda")

    def load(bt):
        q.zero_(), k.zero_(), v.zero_()
        q[:bt.total_q].copy_(bt.q)
        k[:bt.total_kv].copy_(bt.k)
        v[:bt.total_kv].copy_(bt.v)
        cu_q.copy_(torch.from_numpy(bt.cu_q))
        cu_kv.copy_(torch.from_numpy(bt.cu_kv))

    def call():
        pva.varlen_attn_fwd_device(q, k, v, cu_q, cu_kv, 16, 2, is_causal=True, softcap=20.0, out=out,
                                   workspace=ws, error_latch=latch)

    load(big)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say("capturing")
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    shapes = [([100, 1, 257, 1, 340], [700, 3000, 300, 1500, 500]), ([5, 60, 1, 1, 200], [5, 4000, 800, 1, 900]),
              ([300, 1, 0, 200, 150], [300, 2, 0, 700, 2000]), ([1, 1, 1, 1, 1], [5000, 100, 1, 1, 300])]
    for rep, (lq, lkv) in enumerate(shapes):
        bt = _batch(_workload(hq=16, hkv=2, softcap=20.0, seed=40 + rep), lq, lkv)
        want = run_gpu(bt).clone()  # eager host-planned call
        load(bt)
        out.fill_(5.0)
        torch.cuda.synchronize()
        _say("replay", rep, lq, lkv)
        g.replay()
        torch.cuda.synchronize()
        assert int(latch.item()) == 0
        assert torch.equal(out[:bt.total_q], want), rep
        assert bool((out[bt.total_q:] == 5.0).all()), rep  # rows past cu_seqlens_q[-1] untouched


def test_graph_capture_decode_dominated_batch():
    """The side-stream form (a batch with no more rows than sequences: decode
    + combine beside prefill) captured once and replayed with new lengths,
    including prefill rows; every replay equals the eager host-planned call."""
    import torch
    import packed_varlen_scaled_amd as pva
    w = _workload(hq=16, hkv=2)
    B, cap_q, cap_kv = 6, 6, 9000
    q = torch.zeros(cap_q, 16, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(cap_kv, 2, 128, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(cap_kv, 2, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(cap_q, 16, 128, dtype=torch.bfloat16, device="cuda")
    cu_q = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    cu_kv = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(pva.device_workspace_bytes(B, cap_q, cap_kv, 16, 2, 128), dtype=torch.uint8, device="cuda")
    latch = torch.zeros(1, dtype=torch.int32, device="cuda")

    def load(bt):
        q.zero_(), k.zero_(), v.zero_()
        q[:bt.total_q].copy_(bt.q)
        k[:bt.total_kv].copy_(bt.k)
        v[:bt.total_kv].copy_(bt.v)
        cu_q.copy_(torch.from_numpy(bt.cu_q))
        cu_kv.copy_(torch.from_numpy(bt.cu_kv))

    def call():
        pva.varlen_attn_fwd_device(q, k, v, cu_q, cu_kv, 16, 2, is_causal=True, out=out, workspace=ws,
                                   error_latch=latch)

    shapes = [([1, 1, 1, 1, 1, 1], [3000, 20, 1, 900, 2500, 7]), ([1, 2, 1, 0, 1, 0], [900, 3, 5000, 7, 1, 300]),
              ([3, 0, 1, 1, 0, 1], [3, 0, 4000, 2, 0, 1000]), ([1, 1, 0, 1, 1, 1], [1, 1, 0, 6000, 100, 1800])]
    load(_batch(w, *shapes[0]))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the graph (creates the side stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say("capturing decode-dominated")
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep, (lq, lkv) in enumerate(shapes):
        bt = _batch(_workload(hq=16, hkv=2, seed=60 + rep), lq, lkv)
        want = run_gpu(bt).clone()
        load(bt)
        out.fill_(5.0)
        torch.cuda.synchronize()
        _say("replay", rep, lq, lkv)
        g.replay()
        torch.cuda.synchronize()
        assert int(latch.item()) == 0
        assert torch.equal(out[:bt.total_q], want), rep
        assert bool((out[bt.total_q:] == 5.0).all()), rep


def test_device_scheduler_large_batch():
    """3000 short sequences (prefill and decode mixed): the scheduler keeps its
    per-sequence offsets in the workspace instead of LDS."""
    import torch
    w = _workload(hq=8, hkv=2, softcap=10.0)
    rng = np.random.default_rng(9)
    lq = [int(x) if x > 1 else 1 for x in rng.integers(0, 12, size=3000)]
    lkv = [a + int(p) for a, p in zip(lq, rng.integers(0, 40, size=3000))]
    _say("device large batch", len(lq), sum(lq), sum(lkv))
    batch = _batch(w, lq, lkv)
    want = run_gpu(batch).clone()
    ws, latch = _device_buffers(batch)
    out = torch.full_like(want, 7.0)
    _device_call(batch, out, ws, latch)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0
    assert torch.equal(out, want)


def test_device_scheduler_many_items_lds_path():
    """1500 sequences keep the scheduler's offsets in LDS, so eight 1024-thread workgroups
    write the work list; with more than 16384 prefill items every
    workgroup's item loop wraps around (decode items are there too). The
    device-built list must give bitwise the host-scheduled result."""
    import torch
    import packed_varlen_scaled_amd as pva
    w = _workload(hq=8, hkv=2, d=64)
    rng = np.random.default_rng(12)
    n = 1500
    lq = [int(x) for x in rng.integers(200, 301, size=n)]
    for i in range(0, n, 5):
        lq[i] = 1  # decode sequences
    lkv = [a + int(p) for a, p in zip(lq, rng.integers(0, 3000, size=n))]
    batch = _batch(w, lq, lkv)
    stats, _ = pva.plan(batch.cu_q, batch.cu_kv, w.num_heads, w.kv_num_heads, head_dim=w.head_dim,
                        is_causal=True)
    _say("device many items", stats["n_prefill_items"], stats["n_decode_items"], stats["n_combine_items"])
    assert stats["n_prefill_items"] > 16384 and stats["n_decode_items"] > 1000
    want = run_gpu(batch).clone()
    ws, latch = _device_buffers(batch)
    out = torch.full_like(want, 7.0)
    _device_call(batch, out, ws, latch)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0
    assert torch.equal(out, want)


@pytest.mark.parametrize("n", [1, 255, 256, 2047, 2048])
def test_device_scheduler_workgroup_shape_boundaries(n):
    """Batches on both sides of each change of the scheduler's launch shape
    (256-thread workgroups below 256 sequences, 1024-thread ones up to 2047,
    one workgroup over the workspace from 2048): the device-built list gives
    bitwise the host-scheduled result."""
    import torch
    w = _workload(hq=8, hkv=2, d=64, softcap=10.0)
    rng = np.random.default_rng(100 + n)
    lq = [int(x) for x in rng.choice([0, 1, 1, 3, 17, 40], size=n)]
    lkv = [a + int(p) for a, p in zip(lq, rng.integers(0, 300, size=n))]
    _say("device shape boundary", n, sum(lq), sum(lkv))
    batch = _batch(w, lq, lkv)
    want = run_gpu(batch).clone()
    ws, latch = _device_buffers(batch)
    out = torch.full_like(want, 7.0)
    _device_call(batch, out, ws, latch)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0
    assert torch.equal(out, want)


@pytest.mark.parametrize("name,kw,lq,lkv,window", [c for c in DEVICE if c[1].get("dtype") != "f32"][:6],
                         ids=[c[0] for c in DEVICE if c[1].get("dtype") != "f32"][:6])
def test_device_call_without_decode_path(name, kw, lq, lkv, window):
    """decode_path=1 on the device-scheduled call (varlen_attn_fwd_device_ex):
    no decode or combine launch, every sequence through the prefill kernel;
    bitwise the host-planned call with the same option, and the oracle."""
    import torch
    w = _workload(**kw)
    _say("device no decode path", name, lq, lkv, window)
    batch = _batch(w, lq, lkv)
    want = run_gpu(batch, local_window=window, decode_path=1).clone()
    ws, latch = _device_buffers(batch)
    out = torch.full_like(want, 7.0)
    import packed_varlen_scaled_amd as pva
    pva.varlen_attn_fwd_device(batch.q, batch.k, batch.v, torch.from_numpy(batch.cu_q).cuda(),
                               torch.from_numpy(batch.cu_kv).cuda(), w.num_heads, w.kv_num_heads,
                               scale=w.scale or None, is_causal=w.is_causal, softcap=w.softcap, local_window=window,
                               out=out, workspace=ws, error_latch=latch, decode_path=1)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0
    assert torch.equal(out, want)
    compare(out.double().cpu().numpy().reshape(batch.total_q, w.num_heads, w.dv),
            oracle_all(batch, local_window=window or 0), w.dtype)
