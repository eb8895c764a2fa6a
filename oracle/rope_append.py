"""fp64 oracle for the step on the input side of decode: rotary position
embedding of the new query and key rows, and the append of the new key and
value rows into a fixed-capacity KV cache.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers. The GPU library and its
Python binding never import this module, and this module never imports them.

What it computes, with the passages each step follows (crate
onnx-runtime-ep-cuda, page src/kernels/group_query_attention.rs: the rotary
kernel gqa_rope_bnsh, the cache kernels gqa_build_cache / gqa_append_cache,
the fused single-token prep gqa_fuse_decode_prep, and the op's input checks
on cos_cache, sin_cache and position_ids; page src/kernels/attention.rs, the
test of the fixed-capacity, fixed-slot append path):

* sequence b owns the new rows ``[cu_q[b], cu_q[b+1])`` of q, k and v, and the
  cache slots ``[b*C, (b+1)*C)`` (C = cache capacity); ``past[b]`` slots of it
  already hold earlier tokens;
* new row i of sequence b sits at position ``past[b] + i``, unless
  ``position_ids`` gives the position of each new row;
* rotation: the tables hold ``cos`` and ``sin`` of shape ``[rows, R/2]`` for
  rotary dimension R (the table width is R/2). Pair m < R/2 of a head vector
  is dims ``(2m, 2m+1)`` in the interleaved form and ``(m, m + R/2)`` in the
  half-split form; the pair (a, b) becomes ``(a*c - b*s, a*s + b*c)`` with c
  and s the table entries at (position, m). Dims R..D-1 pass unchanged. Every
  query head and every key head turns; values do not;
* the rotated key row and the value row of new row i go to slot
  ``b*C + past[b] + i`` of their caches; no other slot changes;
* the attention that follows reads sequence b's first ``past[b] + L_q[b]``
  slots.

Inputs are stored values (bf16 as its uint16 bit pattern, f16, f32); the
outputs here are the exact fp64 results before rounding to the storage type.
"""
from __future__ import annotations

import numpy as np

# Error bits (the same word as the attention's device scheduler): the
# conditions the GQA op's metadata check raises for a bad past length, a
# cache that would overflow, and a position outside the rotary tables.
ERR_CU_Q_START = 1
ERR_CU_Q_ORDER = 2
ERR_CU_Q_TOTAL = 4
ERR_PAST = 128        # past[b] < 0
ERR_OVERFLOW = 256    # past[b] + L_q[b] > capacity
ERR_POSITION = 512    # a rotated row's position is outside [0, rows)


def to_f64(x, dtype: str) -> np.ndarray:
    """Stored values -> fp64 (bf16 arrives as its uint16 bits)."""
    a = np.asarray(x)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def pair_dims(rotary_dim: int, interleaved: bool):
    """Indices of the two dims of each rotary pair m = 0 .. R/2 - 1."""
    m = np.arange(rotary_dim // 2)
    if interleaved:
        return 2 * m, 2 * m + 1
    return m, m + rotary_dim // 2


def rotate(x: np.ndarray, cos_row: np.ndarray, sin_row: np.ndarray, rotary_dim: int,
           interleaved: bool) -> np.ndarray:
    """Turn every rotary pair of x [..., D] by the table angle of its pair.

    cos_row, sin_row: [..., R/2] fp64, broadcast against x's leading dims."""
    y = np.array(x, dtype=np.float64, copy=True)
    if rotary_dim == 0:
        return y
    i0, i1 = pair_dims(rotary_dim, interleaved)
    a = x[..., i0]
    b = x[..., i1]
    y[..., i0] = a * cos_row - b * sin_row
    y[..., i1] = a * sin_row + b * cos_row
    return y


def check(cu_q, past, capacity: int, total_q: int, positions, rotary_rows: int, rotate_on: bool) -> int:
    """Error bits the inputs raise (0 when the step is valid)."""
    cu = np.asarray(cu_q, dtype=np.int64)
    err = 0
    if cu[0] != 0:
        err |= ERR_CU_Q_START
    if np.any(np.diff(cu) < 0):
        err |= ERR_CU_Q_ORDER
    if cu[-1] > total_q:
        err |= ERR_CU_Q_TOTAL
    if err:
        return err
    lq = np.diff(cu)
    past = np.asarray(past, dtype=np.int64)
    if np.any(past < 0):
        err |= ERR_PAST
    if np.any(past + lq > capacity):
        err |= ERR_OVERFLOW
    if rotate_on and positions is not None and len(positions):
        p = np.asarray(positions, dtype=np.int64)
        if np.any((p < 0) | (p >= rotary_rows)):
            err |= ERR_POSITION
    return err


def positions_of(cu_q, past, position_ids=None) -> np.ndarray:
    """Position of every new row: past[b] + i, or the given position ids."""
    cu = np.asarray(cu_q, dtype=np.int64)
    if position_ids is not None:
        return np.asarray(position_ids, dtype=np.int64).reshape(-1)[:cu[-1]]
    pos = np.empty(int(cu[-1]), dtype=np.int64)
    for b in range(len(cu) - 1):
        pos[cu[b]:cu[b + 1]] = past[b] + np.arange(cu[b + 1] - cu[b])
    return pos


def kv_append_rope(q, k, v, k_cache, v_cache, cu_q, past, capacity: int, cos=None, sin=None,
                   position_ids=None, interleaved: bool = False, dtype: str = "bf16"):
    """The step on fp64 copies.

    q [T, Hq, D], k [T, Hkv, D], v [T, Hkv, Dv] (stored values, T new rows);
    k_cache [B*C, Hkv, D], v_cache [B*C, Hkv, Dv]; cu_q [B+1]; past [B];
    cos, sin fp32 [rows, R/2] or None (no rotation).

    Returns dict(q=rotated q, k_cache=, v_cache=, kv_len=past + L_q, err=bits,
    slots=cache rows written); arrays are fp64. When err is non-zero nothing
    is computed and only err is meaningful.
    """
    cu = np.asarray(cu_q, dtype=np.int64)
    past = np.asarray(past, dtype=np.int64)
    qd = to_f64(q, dtype)
    kd = to_f64(k, dtype)
    vd = to_f64(v, dtype)
    kc = to_f64(k_cache, dtype)
    vc = to_f64(v_cache, dtype)
    rotate_on = cos is not None
    rows = 0 if cos is None else int(np.asarray(cos).shape[0])
    rdim = 0 if cos is None else 2 * int(np.asarray(cos).shape[1])
    pos = None
    if int(cu[0]) == 0 and np.all(np.diff(cu) >= 0):
        pos = positions_of(cu, past, position_ids)
    err = check(cu, past, capacity, qd.shape[0], pos, rows, rotate_on)
    if err:
        return dict(err=err)
    cosd = None if cos is None else np.asarray(cos, dtype=np.float32).astype(np.float64)
    sind = None if sin is None else np.asarray(sin, dtype=np.float32).astype(np.float64)
    q_out = qd.copy()
    slots = []
    for b in range(len(cu) - 1):
        for i in range(int(cu[b + 1] - cu[b])):
            t = int(cu[b] + i)
            slot = b * capacity + int(past[b]) + i
            if rotate_on:
                c, s = cosd[pos[t]], sind[pos[t]]
                q_out[t] = rotate(qd[t], c, s, rdim, interleaved)
                kc[slot] = rotate(kd[t], c, s, rdim, interleaved)
            else:
                kc[slot] = kd[t]
            vc[slot] = vd[t]
            slots.append(slot)
    return dict(q=q_out, k_cache=kc, v_cache=vc, kv_len=past + np.diff(cu), err=0,
                slots=np.asarray(slots, dtype=np.int64))
