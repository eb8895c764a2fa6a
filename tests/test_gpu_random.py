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
