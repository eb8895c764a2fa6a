"""Seeded random attention configurations for the randomized parity sweep.

Each seed draws one configuration: element type, head sizes, GQA group,
causal or not, softcap, scale, local window and a per-sequence length mix.
The mix draws from five kinds of sequence: single decode rows against long
key ranges, self-attention prefill, chunked prefill after a cached past,
more query rows than keys (the tail-aligned causal mask then fully masks the
leading rows), and empty query ranges. The work is capped so that the fp64
oracle finishes each case in about a second. Only shapes and options are
drawn here; the tensors come from the seeded generators in ``synth``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

KINDS = ("decode", "self", "chunk", "short_kv", "empty_q")
# valid (query, key) pairs x query heads x (D + Dv), summed over the batch
MAX_WORK = 3.0e8


@dataclasses.dataclass(frozen=True)
class Case:
    seed: int
    dtype: str
    hq: int
    hkv: int
    d: int
    dv: int
    causal: bool
    softcap: float
    scale: float
    window: int
    lq: tuple
    lkv: tuple
    kinds: tuple


def _sequence(rng, kind):
    if kind == "decode":
        return 1, int(rng.integers(0, 2500))
    if kind == "self":
        n = int(rng.integers(1, 300))
        return n, n
    if kind == "chunk":
        n = int(rng.integers(1, 200))
        return n, n + int(rng.integers(0, 800))
    if kind == "short_kv":
        n = int(rng.integers(2, 150))
        return n, int(rng.integers(0, n))
    return 0, int(rng.integers(0, 100))


def random_case(seed: int) -> Case:
    rng = np.random.default_rng(1000 + seed)
    dtype = ["bf16", "bf16", "bf16", "f16", "f16", "f32"][int(rng.integers(0, 6))]
    if dtype == "f32":
        d = int(rng.choice([16, 40, 64, 96, 128]))
        dv = int(rng.choice([d, 48, 128]))
    else:
        d = int(rng.choice([64, 128]))
        dv = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    while hkv * group > 32:
        group //= 2
    causal = bool(rng.integers(0, 2))
    softcap = 0.0
    if rng.random() < 0.4:
        softcap = float(rng.uniform(2.0, 50.0)) * (1.0 if rng.random() < 0.8 else -1.0)
    scale = float(rng.uniform(0.05, 0.3)) if rng.random() < 0.3 else 0.0
    window = int(rng.integers(1, 300)) if rng.random() < 0.35 else 0
    b = int(rng.integers(1, 9))
    kinds = tuple(KINDS[int(rng.integers(0, len(KINDS)))] for _ in range(b))
    lq, lkv = [], []
    for kind in kinds:
        a, c = _sequence(rng, kind)
        lq.append(a)
        lkv.append(c)
    # halve the largest sequence's key range (and, for self-attention, its
    # query range with it) until the oracle's work fits
    hq = hkv * group
    while sum(a * c for a, c in zip(lq, lkv)) * hq * (d + dv) > MAX_WORK:
        i = int(np.argmax([a * c for a, c in zip(lq, lkv)]))
        lkv[i] //= 2
        if kinds[i] == "self":
            lq[i] = lkv[i]
    return Case(seed, dtype, hq, hkv, d, dv, causal, softcap, scale, window, tuple(lq), tuple(lkv), kinds)


def split_options(seed: int) -> dict:
    """Work-splitting options for a case (the result must not depend on them
    beyond rounding): the decode path on or off, the split-KV decode chunk,
    and the prefill key chunk."""
    rng = np.random.default_rng(5000 + seed)
    return dict(decode_path=int(rng.choice([0, 1, 2])),
                decode_chunk=int(rng.choice([0, 64, 128, 200, 1000])),
                prefill_kv_chunk=int(rng.choice([0, 0, 64, 100, 256])))


@dataclasses.dataclass(frozen=True)
class StepCase:
    """One decode-side input step: rotate and append new rows into a cache."""
    seed: int
    dtype: str
    hq: int
    hkv: int
    d: int
    dv: int
    lq: tuple
    past: tuple
    capacity: int
    rotary_dim: int
    interleaved: bool
    opts: dict


def random_step_case(seed: int) -> StepCase:
    """Head sizes include ones the 16-byte kernel form cannot take (the pair
    form runs them), rotary dims full, partial or none, position ids, packed
    QKV row views and in-place query rotation."""
    rng = np.random.default_rng(7000 + seed)
    dtype = ["bf16", "bf16", "f16", "f32"][int(rng.integers(0, 4))]
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([32, 40, 64, 66, 96, 128]))
    dv = int(rng.choice([d, 64, 72, 128]))
    r = rng.random()
    if r < 0.15:
        rdim = 0
    elif r < 0.55:
        rdim = d
    else:
        rdim = 2 * int(rng.integers(1, d // 2 + 1))
    capacity = int(rng.choice([8, 16, 64, 256]))
    b = int(rng.integers(1, 9))
    lq, past = [], []
    for _ in range(b):
        kind = int(rng.integers(0, 3))
        n = 1 if kind == 0 else (0 if kind == 1 else int(rng.integers(1, 21)))
        n = min(n, capacity)
        lq.append(n)
        past.append(int(rng.integers(0, capacity - n + 1)))
    opts = {}
    if rng.random() < 0.25:
        opts["pos_ids"] = True
    u = rng.random()
    if u < 0.15:
        opts["packed_qkv"] = True
    elif u < 0.3:
        opts["in_place"] = True
    return StepCase(seed, dtype, hq, hkv, d, dv, tuple(lq), tuple(past), capacity, rdim, bool(rng.integers(0, 2)),
                    opts)


@dataclasses.dataclass(frozen=True)
class CacheAttnCase:
    """Attention of new rows over a fixed-capacity cache."""
    seed: int
    dtype: str
    hq: int
    hkv: int
    d: int
    dv: int
    causal: bool
    softcap: float
    window: int
    lq: tuple
    past: tuple
    capacity: int


def random_cache_attn_case(seed: int) -> CacheAttnCase:
    """Decode rows, chunks after a cached past and empty query ranges over
    caches of 64 to 3072 rows per sequence."""
    rng = np.random.default_rng(9000 + seed)
    dtype = ["bf16", "bf16", "f16", "f32"][int(rng.integers(0, 4))]
    if dtype == "f32":
        d = int(rng.choice([40, 64, 128]))
        dv = int(rng.choice([d, 48]))
    else:
        d = int(rng.choice([64, 128]))
        dv = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    while hkv * group > 32:
        group //= 2
    hq = hkv * group
    causal = bool(rng.random() < 0.75)
    softcap = 0.0
    if rng.random() < 0.4:
        softcap = float(rng.uniform(2.0, 50.0)) * (1.0 if rng.random() < 0.8 else -1.0)
    window = int(rng.integers(1, 300)) if rng.random() < 0.3 else 0
    capacity = int(rng.choice([64, 256, 1024, 3072]))
    b = int(rng.integers(1, 9))
    lq, past = [], []
    for _ in range(b):
        kind = int(rng.integers(0, 3))
        n = 1 if kind == 0 else (0 if kind == 2 else int(rng.integers(1, min(200, capacity) + 1)))
        lq.append(n)
        past.append(int(rng.integers(0, capacity - n + 1)))
    while sum(a * (a + p) for a, p in zip(lq, past)) * hq * (d + dv) > MAX_WORK:
        i = int(np.argmax([a * (a + p) for a, p in zip(lq, past)]))
        if past[i] > 0:
            past[i] //= 2
        else:
            lq[i] //= 2
    return CacheAttnCase(seed, dtype, hq, hkv, d, dv, causal, softcap, window, tuple(lq), tuple(past), capacity)
