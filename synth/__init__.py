"""Seeded synthetic workloads for packed variable-length attention.

This module only draws sequence lengths and fills tensors with seeded random
values. It holds none of the attention arithmetic, so that the GPU library and
the CPU oracle can both be fed from it without sharing any of the method.

Workloads (the five shapes the library is measured and checked on):

========================  ==  ==================  ====  ===  ===  ====  ======  =======  =====
name                      B   lengths             Hq    Hkv  D    type  causal  softcap  sigma
========================  ==  ==================  ====  ===  ===  ====  ======  =======  =====
tiny_fp32                 4   {5,17,32,64}        4     4    64   f32   no      0        1.0
ragged_causal_prefill     16  L ~ U{128..2048}    32    8    128  bf16  yes     0        1.0
long_causal_softcap       8   L ~ logU[512,16384] 64    8    128  bf16  yes     50       1.5
chunked_prefill_cache     32  Lq ~ U{1..512},     32    8    128  bf16  yes     0        1.0
                              past ~ U{0..8192}
packed_decode             256 Lq = 1,             64    8    128  bf16  yes     0        1.0
                              Lkv ~ U{256..32768}
========================  ==  ==================  ====  ===  ===  ====  ======  =======  =====

Readings where the workload description is silent: "U{a..b}" is inclusive on
both ends; log-uniform draws ``floor(exp(U(ln a, ln(b+1))))`` clamped to
[a, b]; "N(0, 1.5)" means standard deviation 1.5. Lengths come from numpy's
PCG64 seeded by the workload seed; tensor values come from torch's generator on
the target device, seeded per chunk of 2^28 elements by
``(seed * 1000 + tensor_id) * 65536 + chunk`` (q=0, k=1, v=2), as fp32 normals
scaled by sigma and rounded to nearest even into the storage type. The CPU and
GPU generators differ, so a batch is made once and copied where needed.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_heads: int
    kv_num_heads: int
    head_dim: int
    dtype: str  # "f32" | "f16" | "bf16"
    is_causal: bool
    softcap: float
    scale: float  # 0 -> 1/sqrt(head_dim)
    sigma: float
    seed: int
    v_head_dim: Optional[int] = None

    @property
    def dv(self) -> int:
        return self.v_head_dim or self.head_dim


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 4, 4, 4, 64, "f32", False, 0.0, 0.125, 1.0, 1),
    "ragged_causal_prefill": Workload("ragged_causal_prefill", 16, 32, 8, 128, "bf16", True, 0.0, 0.0, 1.0, 2),
    "long_causal_softcap": Workload("long_causal_softcap", 8, 64, 8, 128, "bf16", True, 50.0, 0.0, 1.5, 3),
    "chunked_prefill_cache": Workload("chunked_prefill_cache", 32, 32, 8, 128, "bf16", True, 0.0, 0.0, 1.0, 4),
    "packed_decode": Workload("packed_decode", 256, 64, 8, 128, "bf16", True, 0.0, 0.0, 1.0, 5),
}


def draw_lengths(name: str, seed: Optional[int] = None, batch: Optional[int] = None):
    """Per-sequence (L_q list, L_kv list) for a named workload."""
    w = WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    b = w.batch if batch is None else batch
    if name == "tiny_fp32":
        lq = [5, 17, 32, 64][:b]
        return lq, list(lq)
    if name == "ragged_causal_prefill":
        lq = rng.integers(128, 2048, size=b, endpoint=True).tolist()
        return lq, list(lq)
    if name == "long_causal_softcap":
        u = rng.uniform(math.log(512), math.log(16384 + 1), size=b)
        lq = np.clip(np.floor(np.exp(u)), 512, 16384).astype(np.int64).tolist()
        return lq, list(lq)
    if name == "chunked_prefill_cache":
        lq = rng.integers(1, 512, size=b, endpoint=True)
        past = rng.integers(0, 8192, size=b, endpoint=True)
        return lq.tolist(), (lq + past).tolist()
    if name == "packed_decode":
        lkv = rng.integers(256, 32768, size=b, endpoint=True).tolist()
        return [1] * b, lkv
    raise KeyError(name)


def cu_seqlens(lengths) -> np.ndarray:
    """Exclusive prefix sum [0, L0, L0+L1, ...] as int32."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    if out[-1] > np.iinfo(np.int32).max:
        raise ValueError("packed token count exceeds int32")
    return out.astype(np.int32)


_TORCH_DTYPES = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def torch_dtype(dtype: str):
    import torch
    return getattr(torch, _TORCH_DTYPES[dtype])


def normal_tensor(shape, dtype: str, sigma: float, seed: int, tensor_id: int, device="cpu",
                  chunk_elems: int = 1 << 28):
    """Seeded N(0, sigma^2) tensor of storage type ``dtype``.

    Values are generated as fp32 normals in chunks of ``chunk_elems`` (each
    chunk with its own derived seed, so the result does not depend on how much
    memory is free) and rounded to nearest even into the storage type."""
    import torch
    tdt = torch_dtype(dtype)
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=tdt, device=device)
    gen = torch.Generator(device=device)
    for ci, start in enumerate(range(0, n, chunk_elems)):
        stop = min(n, start + chunk_elems)
        gen.manual_seed((seed * 1000 + tensor_id) * 65536 + ci)
        x = torch.randn(stop - start, generator=gen, dtype=torch.float32, device=device)
        if sigma != 1.0:
            x.mul_(sigma)
        out[start:stop] = x.to(tdt)
        del x
    return out.view(*shape)


@dataclasses.dataclass
class Batch:
    workload: Workload
    lq: list
    lkv: list
    cu_q: np.ndarray
    cu_kv: np.ndarray
    q: object  # torch tensor [total_q, Hq, D]
    k: object  # torch tensor [total_kv, Hkv, D]
    v: object  # torch tensor [total_kv, Hkv, Dv]

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def total_kv(self) -> int:
        return int(self.cu_kv[-1])


def make_batch(w: Workload, lq, lkv, device="cpu", seed: Optional[int] = None) -> Batch:
    """Q/K/V for explicit per-sequence lengths and a workload's head/type shape."""
    s = w.seed if seed is None else seed
    cu_q = cu_seqlens(lq)
    cu_kv = cu_seqlens(lkv)
    tq, tkv = int(cu_q[-1]), int(cu_kv[-1])
    q = normal_tensor((tq, w.num_heads, w.head_dim), w.dtype, w.sigma, s, 0, device)
    k = normal_tensor((tkv, w.kv_num_heads, w.head_dim), w.dtype, w.sigma, s, 1, device)
    v = normal_tensor((tkv, w.kv_num_heads, w.dv), w.dtype, w.sigma, s, 2, device)
    return Batch(w, list(lq), list(lkv), cu_q, cu_kv, q, k, v)


def workload_batch(name: str, device="cpu") -> Batch:
    """The full-size seeded batch of a named workload."""
    w = WORKLOADS[name]
    lq, lkv = draw_lengths(name)
    return make_batch(w, lq, lkv, device=device)


# ---------------------------------------------------------------------------
# Decode-side inputs: new rows for a fixed-capacity KV cache, and rotary tables.
# ---------------------------------------------------------------------------
def rotary_tables(rows: int, rotary_dim: int, base: float = 10000.0, device="cpu"):
    """cos and sin tables [rows, rotary_dim / 2] in fp32 for the usual rotary
    frequencies base^(-2m / rotary_dim) at positions 0 .. rows - 1 (an input of
    the rotary step, computed in fp64 and rounded to fp32)."""
    import torch
    m = np.arange(rotary_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * m / rotary_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    cos = torch.from_numpy(np.cos(ang).astype(np.float32))
    sin = torch.from_numpy(np.sin(ang).astype(np.float32))
    return cos.to(device), sin.to(device)


@dataclasses.dataclass
class CacheStep:
    """New rows of a packed batch and a fixed-capacity cache they append to.

    Sequence b owns cache rows [b * capacity, (b + 1) * capacity); its first
    past[b] rows hold earlier tokens (seeded normals) and the rest hold NaN,
    so that a read of a slot that holds no token shows in the result."""
    workload: Workload
    lq: list
    past: list
    capacity: int
    cu_q: np.ndarray
    q: object        # [total_q, Hq, D]
    k: object        # [total_q, Hkv, D]
    v: object        # [total_q, Hkv, Dv]
    k_cache: object  # [batch * capacity, Hkv, D]
    v_cache: object  # [batch * capacity, Hkv, Dv]

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def kv_len(self) -> list:
        return [p + n for p, n in zip(self.past, self.lq)]


def make_cache_step(w: Workload, lq, past, capacity: int, device="cpu", seed: Optional[int] = None) -> CacheStep:
    s = w.seed if seed is None else seed
    cu_q = cu_seqlens(lq)
    tq = int(cu_q[-1])
    bsz = len(lq)
    q = normal_tensor((tq, w.num_heads, w.head_dim), w.dtype, w.sigma, s, 0, device)
    k = normal_tensor((tq, w.kv_num_heads, w.head_dim), w.dtype, w.sigma, s, 1, device)
    v = normal_tensor((tq, w.kv_num_heads, w.dv), w.dtype, w.sigma, s, 2, device)
    kc = normal_tensor((bsz * capacity, w.kv_num_heads, w.head_dim), w.dtype, w.sigma, s, 3, device)
    vc = normal_tensor((bsz * capacity, w.kv_num_heads, w.dv), w.dtype, w.sigma, s, 4, device)
    for b in range(bsz):
        kc[b * capacity + past[b]:(b + 1) * capacity] = float("nan")
        vc[b * capacity + past[b]:(b + 1) * capacity] = float("nan")
    return CacheStep(w, list(lq), list(past), capacity, cu_q, q, k, v, kc, vc)


def decode_cache_step(device="cpu") -> CacheStep:
    """The packed decode workload as one decode step over a cache: each
    sequence appends its one new row after L_kv - 1 cached rows; the capacity
    is the longest L_kv rounded up to 256 rows."""
    w = WORKLOADS["packed_decode"]
    lq, lkv = draw_lengths("packed_decode")
    cap = (max(lkv) + 255) // 256 * 256
    return make_cache_step(w, lq, [n - 1 for n in lkv], cap, device=device)
