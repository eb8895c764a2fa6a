"""Randomized parity sweep: seeded random configurations (tests/random_cases.py)
through the C ABI on the GPU, against the fp64 oracle element by element.

Each case runs the host-planned call and the device-scheduled call. Both must
match the oracle within the dtype's tolerance, the device call must give the
host call's bits (the device scheduler emits the same items), and its error
latch must stay clear. Every case prints its configuration before it runs.
"""
from __future__ import annotations

import sys

import pytest

import synth
from parity import compare, oracle_all, run_gpu
from random_cases import random_case

pytestmark = pytest.mark.gpu

SEEDS = list(range(96))


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("seed", SEEDS)
def test_random_case_matches_oracle(seed):
    import torch
    import packed_varlen_scaled_amd as pva
    c = random_case(seed)
    _say("random", c)
    w = synth.Workload(f"random{seed}", 0, c.hq, c.hkv, c.d, c.dtype, c.causal, c.softcap, c.scale, 1.0,
                       500 + seed, c.dv)
    batch = synth.make_batch(w, list(c.lq), list(c.lkv), device="cuda")
    window = c.window or None
    host = run_gpu(batch, local_window=window).clone()
    want = oracle_all(batch, local_window=c.window)
    ma, rel = compare(host.double().cpu().numpy().reshape(batch.total_q, c.hq, c.dv), want, c.dtype)
    _say("random", seed, "host max_abs", ma, "rel_l2", rel)

    n = pva.device_workspace_bytes(len(c.lq), batch.total_q, batch.total_kv, c.hq, c.hkv, c.d, c.dv, c.dtype)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    latch = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full_like(host, 7.0)
    pva.varlen_attn_fwd_device(batch.q, batch.k, batch.v, torch.from_numpy(batch.cu_q).cuda(),
                               torch.from_numpy(batch.cu_kv).cuda(), c.hq, c.hkv, scale=c.scale or None,
                               is_causal=c.causal, softcap=c.softcap, local_window=window, out=out,
                               workspace=ws, error_latch=latch)
    torch.cuda.synchronize()
    assert int(latch.item()) == 0
    assert torch.equal(out, host), "device-scheduled call differs from the host-planned call"


@pytest.mark.parametrize("seed", SEEDS[:48])
def test_random_case_with_split_options_matches_oracle(seed):
    """The same cases with the work split differently (host path): split-KV
    decode chunks, prefill key chunks merged by the combine pass, or no
    decode path at all."""
    from random_cases import split_options
    c = random_case(seed)
    opts = split_options(seed)
    _say("random split", c, opts)
    w = synth.Workload(f"random{seed}", 0, c.hq, c.hkv, c.d, c.dtype, c.causal, c.softcap, c.scale, 1.0,
                       500 + seed, c.dv)
    batch = synth.make_batch(w, list(c.lq), list(c.lkv), device="cuda")
    got = run_gpu(batch, local_window=c.window or None, **opts)
    ma, rel = compare(got.double().cpu().numpy().reshape(batch.total_q, c.hq, c.dv),
                      oracle_all(batch, local_window=c.window), c.dtype)
    _say("random split", seed, "max_abs", ma, "rel_l2", rel)


def _random_lengths(rng, b, cap_q, cap_kv):
    """b sequences (some empty, some single decode rows) within the buffers."""
    while True:
        lq = [int(x) for x in rng.choice([0, 1, 1, 0, 5, 40, 130, 300], size=b)]
        lq = [int(rng.integers(1, n + 1)) if n > 1 else n for n in lq]
        lkv = [n + int(rng.integers(0, 2000)) if rng.random() < 0.7 else int(rng.integers(0, n + 1)) for n in lq]
        if sum(lq) <= cap_q and sum(lkv) <= cap_kv:
            return lq, lkv


@pytest.mark.parametrize("cfg", [
    dict(dtype="bf16", hq=16, hkv=2, d=128, dv=128, causal=True, softcap=20.0, window=None),
    dict(dtype="f16", hq=8, hkv=2, d=64, dv=128, causal=False, softcap=0.0, window=100),
    dict(dtype="bf16", hq=16, hkv=2, d=128, dv=128, causal=True, softcap=0.0, window=None, decode_path=1),
], ids=["bf16_causal_softcap", "f16_noncausal_window_dv128", "bf16_causal_no_decode_path"])
def test_graph_replays_random_lengths(cfg):
    """One device-scheduled call captured into a HIP graph at fixed buffer
    sizes, replayed with eight seeded length sets and new data; every replay
    equals the eager host-planned call on the same inputs bit for bit, and
    output rows past the batch stay untouched."""
    import numpy as np
    import torch
    import packed_varlen_scaled_amd as pva
    b, cap_q, cap_kv = 6, 800, 9000
    dp = cfg.get("decode_path", 0)
    hq, hkv, d, dv = cfg["hq"], cfg["hkv"], cfg["d"], cfg["dv"]
    dt = synth.torch_dtype(cfg["dtype"])
    q = torch.zeros(cap_q, hq, d, dtype=dt, device="cuda")
    k = torch.zeros(cap_kv, hkv, d, dtype=dt, device="cuda")
    v = torch.zeros(cap_kv, hkv, dv, dtype=dt, device="cuda")
    out = torch.zeros(cap_q, hq, dv, dtype=dt, device="cuda")
    cu_q = torch.zeros(b + 1, dtype=torch.int32, device="cuda")
    cu_kv = torch.zeros(b + 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(pva.device_workspace_bytes(b, cap_q, cap_kv, hq, hkv, d, dv, cfg["dtype"]), dtype=torch.uint8,
                     device="cuda")
    latch = torch.zeros(1, dtype=torch.int32, device="cuda")

    def workload(seed):
        return synth.Workload("graph", 0, hq, hkv, d, cfg["dtype"], cfg["causal"], cfg["softcap"], 0.0, 1.0, seed, dv)

    def load(bt):
        q.zero_(), k.zero_(), v.zero_()
        q[:bt.total_q].copy_(bt.q)
        k[:bt.total_kv].copy_(bt.k)
        v[:bt.total_kv].copy_(bt.v)
        cu_q.copy_(torch.from_numpy(bt.cu_q))
        cu_kv.copy_(torch.from_numpy(bt.cu_kv))

    def call():
        pva.varlen_attn_fwd_device(q, k, v, cu_q, cu_kv, hq, hkv, is_causal=cfg["causal"], softcap=cfg["softcap"],
                                   local_window=cfg["window"], out=out, workspace=ws, error_latch=latch,
                                   decode_path=dp)

    rng = np.random.default_rng((77 if cfg["causal"] else 78) + 10 * dp)
    load(synth.make_batch(workload(90), *_random_lengths(rng, b, cap_q, cap_kv), device="cuda"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say("graph capture", cfg)
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(8):
        lq, lkv = _random_lengths(rng, b, cap_q, cap_kv)
        bt = synth.make_batch(workload(100 + rep), lq, lkv, device="cuda")
        want = run_gpu(bt, local_window=cfg["window"], decode_path=dp).clone()  # eager host-planned call
        load(bt)
        out.fill_(5.0)
        torch.cuda.synchronize()
        _say("graph replay", rep, lq, lkv)
        g.replay()
        torch.cuda.synchronize()
        assert int(latch.item()) == 0
        assert torch.equal(out[:bt.total_q], want), rep
        assert bool((out[bt.total_q:] == 5.0).all()), rep
