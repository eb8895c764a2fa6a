"""Pins of the fp64 oracle against things other than itself.

Each test names what fixes the expected value: brute force on tiny inputs in a
different formulation (tests/brute.py), closed forms, or invariants the source
pages state (crate onnx-runtime-ep-cuda, page
src/kernels/packed_varlen_attention.rs "PVA", page
src/kernels/standard_attention.rs "STD"). None of them calls the GPU library.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import pytest

import oracle
from brute import padded_attention

RNG = np.random.default_rng(12345)


def _rand(shape, rng=RNG, sigma=1.0):
    return (rng.standard_normal(shape) * sigma).astype(np.float32)


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _run(q, k, v, lq, lkv, hq, hkv, scale, causal, softcap, **kw):
    return oracle.attention(q, k, v, _cu(lq), _cu(lkv), hq, hkv, scale=scale,
                            is_causal=causal, softcap=softcap, dtype="f32", **kw)


# --------------------------------------------------------------------------
# Brute force on tiny inputs (the padded + masked formulation).
# --------------------------------------------------------------------------
CASES = []
for causal, softcap, (hq, hkv), lens in itertools.product(
        [False, True], [0.0, 2.5, -1.75], [(1, 1), (2, 1), (4, 2), (4, 4), (3, 1)],
        [([3], [3]), ([2, 5, 1], [2, 5, 1]), ([4, 1, 3], [6, 2, 3]),
         ([5, 2], [3, 0]), ([0, 3, 2], [2, 4, 0]), ([7, 3], [4, 7])]):
    CASES.append((causal, softcap, hq, hkv, lens))


@pytest.mark.parametrize("causal,softcap,hq,hkv,lens", CASES)
def test_oracle_matches_padded_brute_force(causal, softcap, hq, hkv, lens):
    lq, lkv = lens
    rng = np.random.default_rng(hash((causal, softcap, hq, hkv, str(lens))) & 0xFFFF)
    d, dv = 3, 2
    tq, tkv = sum(lq), sum(lkv)
    q = _rand((tq, hq, d), rng)
    k = _rand((tkv, hkv, d), rng)
    v = _rand((tkv, hkv, dv), rng)
    scale = 0.7
    got = _run(q, k, v, lq, lkv, hq, hkv, scale, causal, softcap)
    want = padded_attention(q.astype(np.float64).tolist(), k.astype(np.float64).tolist(),
                            v.astype(np.float64).tolist(), lq, lkv, hq, hkv,
                            float(np.float32(scale)), causal, softcap)
    want = np.asarray(want, dtype=np.float64).reshape(tq * hq, dv) if tq else np.zeros((0, dv))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_half_storage_types_read_exactly(dtype):
    """bf16/f16 storage must be widened exactly: the brute force sees the same
    rounded values as fp64 and must agree to fp64 rounding."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    lq, lkv = [3, 4], [5, 4]
    hq, hkv, d = 4, 2, 5
    g = torch.Generator().manual_seed(7)
    q = torch.randn(sum(lq), hq, d, generator=g).to(tdt)
    k = torch.randn(sum(lkv), hkv, d, generator=g).to(tdt)
    v = torch.randn(sum(lkv), hkv, d, generator=g).to(tdt)
    # include values that exercise subnormals / large exponents of the type
    q[0, 0, 0] = 1e-6 if dtype == "f16" else 1e-30
    k[1, 1, 2] = -3.0e4 if dtype == "f16" else -3.0e30
    got = oracle.attention(q, k, v, _cu(lq), _cu(lkv), hq, hkv, scale=0.3, is_causal=True,
                           softcap=3.0, dtype=dtype)
    want = padded_attention(q.double().tolist(), k.double().tolist(), v.double().tolist(),
                            lq, lkv, hq, hkv, float(np.float32(0.3)), True, 3.0)
    np.testing.assert_allclose(got, np.asarray(want).reshape(-1, d), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Closed forms.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("softcap", [0.0, 1.3, 40.0, -2.0])
def test_two_keys_closed_form(softcap):
    """One query, two keys, D=1: p0 = sigmoid(z0 - z1) with z_j = softcap(scale*q*k_j)."""
    q0, k0, k1, v0, v1, scale = 1.7, 0.9, -1.4, 2.5, -0.5, 0.8
    q = np.array([[[q0]]], np.float32)
    k = np.array([[[k0]], [[k1]]], np.float32)
    v = np.array([[[v0]], [[v1]]], np.float32)
    qf, kf0, kf1, vf0, vf1, sf = (float(np.float32(x)) for x in (q0, k0, k1, v0, v1, scale))

    cf = float(np.float32(softcap))

    def z(kk):
        s = sf * qf * kk
        return cf * math.tanh(s / cf) if cf else s

    p0 = 1.0 / (1.0 + math.exp(-(z(kf0) - z(kf1))))
    want = p0 * vf0 + (1.0 - p0) * vf1
    got = _run(q, k, v, [1], [2], 1, 1, scale, False, softcap)
    assert abs(got[0, 0] - want) < 1e-14


def test_default_scale_is_inverse_sqrt_head_dim():
    d = 16
    q, k, v = _rand((3, 2, d)), _rand((5, 2, d)), _rand((5, 2, d))
    a = _run(q, k, v, [3], [5], 2, 2, 0.0, False, 0.0)
    b = _run(q, k, v, [3], [5], 2, 2, 1.0 / math.sqrt(d), False, 0.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
    c = _run(q, k, v, [3], [5], 2, 2, 0.5, False, 0.0)
    assert np.max(np.abs(a - c)) > 1e-3  # the scale actually matters


def test_single_key_returns_that_value_row():
    """L_kv = 1: the only probability is 1, so the output is that V row exactly."""
    lq, lkv = [3, 1, 2], [1, 1, 1]
    q, k, v = _rand((6, 4, 8)), _rand((3, 2, 8)), _rand((3, 2, 8))
    got = _run(q, k, v, lq, lkv, 4, 2, 0.3, False, 5.0).reshape(6, 4, 8)
    seq = [0, 0, 0, 1, 2, 2]
    for t in range(6):
        for h in range(4):
            np.testing.assert_array_equal(got[t, h], v[seq[t], h // 2].astype(np.float64))


def test_no_query_rows_give_an_empty_output_with_the_value_head_size():
    """A batch whose query ranges are all empty has no output rows; the value
    head size (here different from the key head size) still shapes them."""
    k, v = _rand((7, 2, 8)), _rand((7, 2, 12))
    q = np.zeros((0, 4, 8), dtype=np.float32)
    got = oracle.attention(q, k, v, [0, 0, 0], [0, 3, 7], 4, 2, dtype="f32")
    assert got.shape == (0, 12)


@pytest.mark.parametrize("lq,lkv", [(6, 6), (3, 9), (7, 4), (1, 5), (5, 1)])
def test_identical_keys_give_causal_prefix_mean(lq, lkv):
    """With identical keys every visible key has the same weight, so row i is the
    mean of V over keys 0..i+(L_kv-L_q) (tail-aligned causal; rows with a negative
    limit are zero): PVA "Causal alignment" and STD's negative-offset rule."""
    d = 4
    q = _rand((lq, 1, d))
    krow = _rand((1, 1, d))
    k = np.repeat(krow, lkv, axis=0)
    v = _rand((lkv, 1, d))
    got = _run(q, k, v, [lq], [lkv], 1, 1, 0.5, True, 0.0)
    off = lkv - lq
    vd = v.astype(np.float64)[:, 0, :]
    for i in range(lq):
        n = min(lkv, i + off + 1)
        want = np.zeros(d) if n <= 0 else vd[:n].sum(axis=0) / n
        np.testing.assert_allclose(got[i], want, rtol=0, atol=1e-14)


def test_zero_query_gives_mean_of_values():
    q = np.zeros((2, 2, 4), np.float32)
    k, v = _rand((5, 2, 4)), _rand((5, 2, 4))
    got = _run(q, k, v, [2], [5], 2, 2, 1.0, False, 0.0).reshape(2, 2, 4)
    np.testing.assert_allclose(got[0], v.astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_gqa_exact_head_mapping():
    """Query head h must read kv head h // (Hq/Hkv) (contiguous groups, PVA
    "Schema (v1)" kv_num_heads). V of kv head g is the constant g+1 and all keys
    are equal, so head h's output is exactly h//G + 1; an interleaved h % Hkv
    mapping would give a different constant."""
    hq, hkv, d = 8, 2, 4
    q = _rand((3, hq, d))
    k = np.ones((4, hkv, d), np.float32)
    v = np.zeros((4, hkv, d), np.float32)
    for g in range(hkv):
        v[:, g, :] = g + 1
    got = _run(q, k, v, [3], [4], hq, hkv, 1.0, False, 0.0).reshape(3, hq, d)
    for h in range(hq):
        assert np.all(got[:, h, :] == h // (hq // hkv) + 1)


def test_gqa_equals_mha_with_repeated_kv():
    hq, hkv, d = 6, 2, 5
    lq, lkv = [4, 3], [5, 6]
    q, k, v = _rand((7, hq, d)), _rand((11, hkv, d)), _rand((11, hkv, d))
    a = _run(q, k, v, lq, lkv, hq, hkv, 0.4, True, 0.0)
    kr = np.repeat(k, hq // hkv, axis=1)
    vr = np.repeat(v, hq // hkv, axis=1)
    b = _run(q, kr, vr, lq, lkv, hq, hq, 0.4, True, 0.0)
    np.testing.assert_array_equal(a, b)


# --------------------------------------------------------------------------
# Softmax invariants.
# --------------------------------------------------------------------------
def test_probabilities_sum_to_one():
    """V = 1 everywhere: each visible row's output is sum_j p_j, which must be 1."""
    lq, lkv = [5, 3, 4], [5, 6, 2]
    q, k = _rand((12, 2, 6), sigma=3.0), _rand((13, 2, 6), sigma=3.0)
    v = np.ones((13, 2, 6), np.float32)
    got = _run(q, k, v, lq, lkv, 2, 2, 1.0, True, 0.0)
    # rows of sequence 2 with i + (2-4) < 0 see no key
    rows_zero = {(5 + 3 + i) for i in range(4) if i + (2 - 4) < 0}
    for t in range(12):
        for h in range(2):
            r = got[t * 2 + h]
            if t in rows_zero:
                assert np.all(r == 0.0)
            else:
                np.testing.assert_allclose(r, 1.0, rtol=0, atol=1e-12)


def test_scale_invariance():
    """(alpha*Q) with scale/alpha gives the same scores, hence the same output."""
    q, k, v = _rand((4, 2, 8)), _rand((6, 2, 8)), _rand((6, 2, 8))
    a = _run(q, k, v, [4], [6], 2, 2, 0.5, True, 0.0)
    b = _run(q * np.float32(4.0), k, v, [4], [6], 2, 2, 0.125, True, 0.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_large_softcap_approaches_no_softcap():
    q, k, v = _rand((3, 1, 8)), _rand((5, 1, 8)), _rand((5, 1, 8))
    a = _run(q, k, v, [3], [5], 1, 1, 0.3, False, 0.0)
    b = _run(q, k, v, [3], [5], 1, 1, 0.3, False, 1e7)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-10)
    c = _run(q, k, v, [3], [5], 1, 1, 0.3, False, 0.5)
    assert np.max(np.abs(a - c)) > 1e-3


def test_negative_softcap_equals_positive():
    """tanh is odd, so c*tanh(s/c) is the same function for c and -c."""
    q, k, v = _rand((3, 2, 4)), _rand((4, 2, 4)), _rand((4, 2, 4))
    a = _run(q, k, v, [3], [4], 2, 2, 1.0, True, 2.0)
    b = _run(q, k, v, [3], [4], 2, 2, 1.0, True, -2.0)
    np.testing.assert_array_equal(a, b)


def test_softcap_applied_before_mask():
    """A masked key must stay masked after softcap (PVA row kernel stages 2-3):
    with causal L_q = L_kv, row 0 sees only key 0, so it returns V[0] even with a
    softcap; capping -inf instead would give the masked keys weight."""
    q, k, v = _rand((3, 1, 4)), _rand((3, 1, 4)), _rand((3, 1, 4))
    got = _run(q, k, v, [3], [3], 1, 1, 1.0, True, 1.5)
    np.testing.assert_array_equal(got[0], v[0, 0].astype(np.float64))


def test_empty_and_fully_masked_rows_are_zero():
    lq, lkv = [2, 3, 4], [0, 3, 1]
    q, k, v = _rand((9, 2, 4)), _rand((4, 2, 4)), _rand((4, 2, 4))
    got = _run(q, k, v, lq, lkv, 2, 2, 1.0, True, 0.0).reshape(9, 2, 4)
    assert np.all(got[0:2] == 0.0)  # no keys at all
    # sequence 2: L_q=4 > L_kv=1, offset -3: rows 0..2 fully masked, row 3 sees key 0
    assert np.all(got[5:8] == 0.0)
    np.testing.assert_array_equal(got[8, 0], v[3, 0].astype(np.float64))


# --------------------------------------------------------------------------
# Packing invariants (block-diagonality).
# --------------------------------------------------------------------------
def test_permuting_sequences_permutes_outputs():
    lq, lkv = [3, 5, 2], [4, 5, 6]
    hq, hkv, d = 2, 1, 4
    q, k, v = _rand((10, hq, d)), _rand((15, hkv, d)), _rand((15, hkv, d))
    base = _run(q, k, v, lq, lkv, hq, hkv, 0.6, True, 0.0).reshape(10, hq, d)
    order = [2, 0, 1]
    cq, ck = _cu(lq), _cu(lkv)
    qs = np.concatenate([q[cq[b]:cq[b + 1]] for b in order])
    ks = np.concatenate([k[ck[b]:ck[b + 1]] for b in order])
    vs = np.concatenate([v[ck[b]:ck[b + 1]] for b in order])
    perm = _run(qs, ks, vs, [lq[b] for b in order], [lkv[b] for b in order], hq, hkv, 0.6,
                True, 0.0).reshape(10, hq, d)
    want = np.concatenate([base[cq[b]:cq[b + 1]] for b in order])
    np.testing.assert_array_equal(perm, want)


def test_sequence_alone_equals_sequence_in_batch():
    lq, lkv = [3, 5, 2], [4, 5, 6]
    q, k, v = _rand((10, 2, 4)), _rand((15, 2, 4)), _rand((15, 2, 4))
    full = _run(q, k, v, lq, lkv, 2, 2, 0.6, False, 3.0).reshape(10, 2, 4)
    alone = _run(q[3:8], k[4:9], v[4:9], [5], [5], 2, 2, 0.6, False, 3.0).reshape(5, 2, 4)
    np.testing.assert_array_equal(full[3:8], alone)


def test_neighbour_sequences_cannot_leak():
    """Changing another sequence's K/V (even to inf/nan) leaves this one untouched."""
    lq, lkv = [3, 4], [3, 4]
    q, k, v = _rand((7, 1, 4)), _rand((7, 1, 4)), _rand((7, 1, 4))
    a = _run(q, k, v, lq, lkv, 1, 1, 1.0, True, 0.0)
    k2, v2 = k.copy(), v.copy()
    k2[3:] = np.inf
    v2[3:] = np.nan
    b = _run(q, k2, v2, lq, lkv, 1, 1, 1.0, True, 0.0)
    np.testing.assert_array_equal(a[:3], b[:3])


def test_packed_equals_padded_with_equal_lengths():
    """All-equal lengths: the packed batch is the padded batch with no padding
    (PVA "Numerics & determinism"); each sequence is an independent dense
    attention, here checked against a dense fp64 numpy softmax."""
    b, s, h, d = 3, 5, 2, 4
    q, k, v = _rand((b * s, h, d)), _rand((b * s, h, d)), _rand((b * s, h, d))
    got = _run(q, k, v, [s] * b, [s] * b, h, h, 0.5, True, 0.0).reshape(b, s, h, d)
    qd, kd, vd = (x.astype(np.float64).reshape(b, s, h, d) for x in (q, k, v))
    for bb in range(b):
        for hh in range(h):
            sc = 0.5 * qd[bb, :, hh] @ kd[bb, :, hh].T
            sc[np.triu_indices(s, 1)] = -np.inf
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            np.testing.assert_allclose(got[bb, :, hh], p @ vd[bb, :, hh], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# Log-sum-exp over key partitions (what a split-KV combine has to reproduce).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_lse_partitions_recombine_to_full(causal):
    lq, lkv = [2, 3, 1], [9, 3, 12]
    hq, hkv, d = 4, 2, 6
    q, k, v = _rand((6, hq, d)), _rand((24, hkv, d)), _rand((24, hkv, d))
    full, lse_full = _run(q, k, v, lq, lkv, hq, hkv, 0.4, causal, 0.0, with_lse=True)
    cuts = [0, 2, 5, 6, 11, 12]
    parts = [_run(q, k, v, lq, lkv, hq, hkv, 0.4, causal, 0.0, with_lse=True,
                  key_window=(a, b)) for a, b in zip(cuts[:-1], cuts[1:])]
    lses = np.stack([p[1] for p in parts])  # [S, rows]
    outs = np.stack([p[0] for p in parts])  # [S, rows, dv]
    m = np.max(lses, axis=0)
    safe = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - safe), 0.0)
    z = w.sum(axis=0)
    comb = np.where(z[:, None] > 0, (w[:, :, None] * outs).sum(axis=0) / np.where(z > 0, z, 1)[:, None], 0.0)
    np.testing.assert_allclose(comb, full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.where(np.isfinite(lse_full), lse_full, 0),
                               np.where(np.isfinite(m), safe + np.log(np.where(z > 0, z, 1)), 0),
                               rtol=0, atol=1e-12)


def test_lse_matches_direct_log_sum_exp():
    q, k, v = _rand((2, 1, 3)), _rand((4, 1, 3)), _rand((4, 1, 3))
    _, lse = _run(q, k, v, [2], [4], 1, 1, 0.9, False, 0.0, with_lse=True)
    for i in range(2):
        s = [float(np.float32(0.9)) * float(np.dot(q[i, 0].astype(np.float64), k[j, 0].astype(np.float64))) for j in range(4)]
        m = max(s)
        assert abs(lse[i] - (m + math.log(math.fsum(math.exp(x - m) for x in s)))) < 1e-13


# --------------------------------------------------------------------------
# Implementation properties of the oracle itself.
# --------------------------------------------------------------------------
def test_thread_count_does_not_change_bits():
    q, k, v = _rand((40, 4, 16)), _rand((50, 2, 16)), _rand((50, 2, 16))
    lq, lkv = [10, 30], [20, 30]
    a = _run(q, k, v, lq, lkv, 4, 2, 0.25, True, 10.0, threads=1)
    b = _run(q, k, v, lq, lkv, 4, 2, 0.25, True, 10.0, threads=7)
    np.testing.assert_array_equal(a, b)


def test_row_subset_matches_full_rows():
    q, k, v = _rand((12, 4, 8)), _rand((15, 2, 8)), _rand((15, 2, 8))
    lq, lkv = [5, 7], [6, 9]
    full = _run(q, k, v, lq, lkv, 4, 2, 0.25, True, 0.0)
    rows = np.array([47, 0, 13, 22, 5], dtype=np.int64)
    sub = _run(q, k, v, lq, lkv, 4, 2, 0.25, True, 0.0, rows=rows)
    np.testing.assert_array_equal(sub, full[rows])


def test_oracle_rejects_inconsistent_arguments():
    q, k, v = _rand((3, 4, 2)), _rand((3, 3, 2)), _rand((3, 3, 2))
    with pytest.raises(ValueError):
        _run(q, k, v, [3], [3], 4, 3, 1.0, False, 0.0)  # 3 does not divide 4
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, [0, 2], [0, 3], 4, 3, dtype="f32")  # cu_q[B] != total


# --------------------------------------------------------------------------
# Local window (page src/kernels/attention.rs, the softmax kernel source's
# local_min; page src/kernels/group_query_attention.rs, local_window_size).
# --------------------------------------------------------------------------
WINDOW_CASES = []
for causal, window, softcap, lens in itertools.product(
        [False, True], [1, 2, 3, 5], [0.0, 2.5],
        [([4], [4]), ([2, 5, 1], [2, 5, 1]), ([3, 1, 4], [6, 2, 7]), ([6, 2], [3, 0]), ([7, 3], [4, 7])]):
    WINDOW_CASES.append((causal, window, softcap, lens))


@pytest.mark.parametrize("causal,window,softcap,lens", WINDOW_CASES)
def test_window_matches_padded_brute_force(causal, window, softcap, lens):
    lq, lkv = lens
    rng = np.random.default_rng(hash((causal, window, softcap, str(lens))) & 0xFFFF)
    hq, hkv, d, dv = 4, 2, 3, 2
    tq, tkv = sum(lq), sum(lkv)
    q, k, v = _rand((tq, hq, d), rng), _rand((tkv, hkv, d), rng), _rand((tkv, hkv, dv), rng)
    got = _run(q, k, v, lq, lkv, hq, hkv, 0.7, causal, softcap, local_window=window)
    want = padded_attention(q.astype(np.float64).tolist(), k.astype(np.float64).tolist(),
                            v.astype(np.float64).tolist(), lq, lkv, hq, hkv,
                            float(np.float32(0.7)), causal, softcap, window=window)
    want = np.asarray(want, dtype=np.float64).reshape(tq * hq, dv)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lq,lkv,window", [(6, 6, 2), (3, 9, 4), (7, 4, 3), (1, 5, 2), (5, 1, 1), (8, 8, 8)])
def test_identical_keys_give_window_mean(causal, lq, lkv, window):
    """With identical keys every visible key weighs the same, so row i is the mean
    of V over keys max(0, i+off+1-W) .. i+off (causal) or .. L_kv-1 (not causal),
    off = L_kv - L_q: the window's left edge pinned exactly."""
    d = 4
    q = _rand((lq, 1, d))
    k = np.repeat(_rand((1, 1, d)), lkv, axis=0)
    v = _rand((lkv, 1, d))
    got = _run(q, k, v, [lq], [lkv], 1, 1, 0.5, causal, 0.0, local_window=window)
    off = lkv - lq
    vd = v.astype(np.float64)[:, 0, :]
    for i in range(lq):
        lo = max(0, i + off + 1 - window)
        hi = min(lkv, i + off + 1) if causal else lkv
        want = np.zeros(d) if hi <= lo else vd[lo:hi].mean(axis=0)
        np.testing.assert_allclose(got[i], want, rtol=0, atol=1e-14)


def test_window_of_one_returns_the_diagonal_value():
    """W = 1 with the causal mask leaves exactly key i + off: out = V of that key."""
    lq, lkv = [5, 3], [7, 3]
    q, k, v = _rand((8, 2, 4)), _rand((10, 1, 4)), _rand((10, 1, 4))
    got = _run(q, k, v, lq, lkv, 2, 1, 0.9, True, 3.0, local_window=1).reshape(8, 2, 4)
    rows = [(0, i, 7 - 5 + i) for i in range(5)] + [(1, i, i) for i in range(3)]
    for t, (b, i, j) in enumerate(rows):
        kt = j + (0 if b == 0 else 7)
        for h in range(2):
            np.testing.assert_array_equal(got[t, h], v[kt, 0].astype(np.float64))


@pytest.mark.parametrize("causal", [False, True])
def test_window_covering_every_key_changes_nothing(causal):
    lq, lkv = [4, 6, 1], [9, 6, 5]
    q, k, v = _rand((11, 4, 8)), _rand((20, 2, 8)), _rand((20, 2, 8))
    base = _run(q, k, v, lq, lkv, 4, 2, 0.4, causal, 0.0)
    for w in (9, 10, 1000):
        np.testing.assert_array_equal(_run(q, k, v, lq, lkv, 4, 2, 0.4, causal, 0.0, local_window=w), base)
    np.testing.assert_array_equal(_run(q, k, v, lq, lkv, 4, 2, 0.4, causal, 0.0, local_window=-1), base)
