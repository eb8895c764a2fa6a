"""Pins of the rotary + cache-append oracle against what the pages and the
mathematics fix, and mutation checks that those pins catch plausible
mistakes in it.

Rotary embedding (page src/kernels/group_query_attention.rs, rotary kernel
gqa_rope_bnsh and the op's cos_cache / sin_cache checks) turns pair m of a
head vector by the angle whose cosine and sine the tables hold; that is
multiplication of the complex number (first dim + i * second dim) by
exp(i * angle). The pins check the oracle against that complex product, the
identity at angle 0, the norm of each pair, the dependence of a query-key dot
product on the position difference only, the permutation that maps the
interleaved pairing onto the half-split one, and brute-force cache contents.
"""
from __future__ import annotations

import importlib.util
import os

import numpy as np
import pytest

import synth
from oracle import rope_append as ra

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _angles_tables(rng, rows, half):
    ang = rng.uniform(-np.pi, np.pi, size=(rows, half))
    return ang, np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# ---- pins as functions of the oracle module, so the mutants can be run through them
def pin_complex_product(mod):
    """Pair m of the output equals (a + i b) * (c + i s) for both pairings."""
    rng = np.random.default_rng(5)
    worst = 0.0
    for interleaved in (True, False):
        for d, r in [(8, 8), (12, 8), (16, 4)]:
            x = rng.standard_normal((3, d))
            _, c, s = _angles_tables(rng, 3, r // 2)
            c64, s64 = c.astype(np.float64), s.astype(np.float64)
            y = mod.rotate(x, c64, s64, r, interleaved)
            m = np.arange(r // 2)
            i0, i1 = (2 * m, 2 * m + 1) if interleaved else (m, m + r // 2)
            z = (x[:, i0] + 1j * x[:, i1]) * (c64 + 1j * s64)
            worst = max(worst, np.max(np.abs(y[:, i0] - z.real)), np.max(np.abs(y[:, i1] - z.imag)))
            worst = max(worst, np.max(np.abs(y[:, r:] - x[:, r:])) if d > r else 0.0)
    return worst


def pin_relative_position(mod):
    """<rot(q, m), rot(k, n)> depends on m - n only (standard tables)."""
    rng = np.random.default_rng(6)
    cos, sin = synth.rotary_tables(64, 16)
    cos, sin = cos.numpy().astype(np.float64), sin.numpy().astype(np.float64)
    worst = 0.0
    for interleaved in (True, False):
        q = rng.standard_normal(16)
        k = rng.standard_normal(16)
        for m, n, shift in [(5, 2, 7), (0, 9, 30), (20, 20, 11)]:
            a = mod.rotate(q, cos[m], sin[m], 16, interleaved) @ mod.rotate(k, cos[n], sin[n], 16, interleaved)
            b = (mod.rotate(q, cos[m + shift], sin[m + shift], 16, interleaved)
                 @ mod.rotate(k, cos[n + shift], sin[n + shift], 16, interleaved))
            worst = max(worst, abs(a - b) / 1e-4)  # fp32 tables: agreement to ~1e-6
    return worst if worst > 1.0 else 0.0


def pin_pairing_permutation(mod):
    """Moving dim 2m to m and 2m + 1 to m + R/2 turns the interleaved rotation
    into the half-split one."""
    rng = np.random.default_rng(7)
    r, d = 8, 10
    perm = np.concatenate([np.arange(0, r, 2), np.arange(1, r, 2), np.arange(r, d)])
    x = rng.standard_normal((4, d))
    _, c, s = _angles_tables(rng, 4, r // 2)
    c, s = c.astype(np.float64), s.astype(np.float64)
    inter = mod.rotate(x, c, s, r, True)
    half = mod.rotate(x[:, perm], c, s, r, False)
    return float(np.max(np.abs(inter[:, perm] - half)))


def pin_cache_contents(mod):
    """Brute force over tiny shapes: which slots change, and to what."""
    rng = np.random.default_rng(8)
    hq, hkv, d, dv, cap, r = 4, 2, 6, 5, 7, 4
    lq, past = [2, 0, 3], [4, 3, 0]
    cu = np.concatenate([[0], np.cumsum(lq)])
    t = int(cu[-1])
    q = rng.standard_normal((t, hq, d)).astype(np.float32)
    k = rng.standard_normal((t, hkv, d)).astype(np.float32)
    v = rng.standard_normal((t, hkv, dv)).astype(np.float32)
    kc = rng.standard_normal((3 * cap, hkv, d)).astype(np.float32)
    vc = rng.standard_normal((3 * cap, hkv, dv)).astype(np.float32)
    ang, c, s = _angles_tables(rng, 12, r // 2)
    worst = 0.0
    for pos_ids in (None, np.array([9, 1, 0, 11, 4], dtype=np.int64)):
        res = mod.kv_append_rope(q, k, v, kc, vc, cu, past, cap, c, s, position_ids=pos_ids,
                                 interleaved=False, dtype="f32")
        assert res["err"] == 0
        want_k = kc.astype(np.float64).copy()
        want_v = vc.astype(np.float64).copy()
        want_q = q.astype(np.float64).copy()
        for b in range(3):
            for i in range(lq[b]):
                row = cu[b] + i
                p = past[b] + i if pos_ids is None else pos_ids[row]
                slot = b * cap + past[b] + i
                cc, ss = c[p].astype(np.float64), s[p].astype(np.float64)
                for h in range(hq):
                    for m in range(r // 2):
                        a0, a1 = q[row, h, m], q[row, h, m + r // 2]
                        want_q[row, h, m] = a0 * cc[m] - a1 * ss[m]
                        want_q[row, h, m + r // 2] = a0 * ss[m] + a1 * cc[m]
                for h in range(hkv):
                    want_k[slot, h] = k[row, h]
                    for m in range(r // 2):
                        a0, a1 = k[row, h, m], k[row, h, m + r // 2]
                        want_k[slot, h, m] = a0 * cc[m] - a1 * ss[m]
                        want_k[slot, h, m + r // 2] = a0 * ss[m] + a1 * cc[m]
                    want_v[slot, h] = v[row, h]
        worst = max(worst, np.max(np.abs(res["q"] - want_q)), np.max(np.abs(res["k_cache"] - want_k)),
                    np.max(np.abs(res["v_cache"] - want_v)))
        if list(res["kv_len"]) != [6, 3, 3]:
            worst = max(worst, 1.0)
    return worst


def pin_error_bits(mod):
    """Each invalid input raises its own bit; valid input raises none."""
    z = np.zeros((3, 1, 2), dtype=np.float32)
    zc = np.zeros((8, 1, 2), dtype=np.float32)
    c = np.ones((6, 1), dtype=np.float32)   # positions 0..5 have table rows
    s = np.zeros((6, 1), dtype=np.float32)
    cases = [  # capacity 4 slots per sequence
        (dict(cu=[0, 1, 3], past=[1, 1]), 0),
        (dict(cu=[1, 1, 3], past=[1, 1]), mod.ERR_CU_Q_START),
        (dict(cu=[0, 2, 1], past=[1, 1]), mod.ERR_CU_Q_ORDER),
        (dict(cu=[0, 2, 4], past=[1, 1]), mod.ERR_CU_Q_TOTAL),
        (dict(cu=[0, 1, 3], past=[-1, 1]), mod.ERR_PAST | mod.ERR_POSITION),  # position -1 too
        (dict(cu=[0, 1, 3], past=[1, 3]), mod.ERR_OVERFLOW),      # 3 + 2 > capacity 4
        (dict(cu=[0, 1, 3], past=[3, 2]), 0),                     # 3 + 1 and 2 + 2 fill it exactly
        (dict(cu=[0, 1, 3], past=[1, 1], pos=[0, 3, 6]), mod.ERR_POSITION),
        (dict(cu=[0, 1, 3], past=[1, 1], pos=[0, 3, -1]), mod.ERR_POSITION),
        (dict(cu=[0, 1, 3], past=[1, 1], pos=[0, 5, 2]), 0),
        (dict(cu=[0, 1, 3], past=[1, 1], pos=[0, 5, 2], rows=5), mod.ERR_POSITION),
        (dict(cu=[0, 1, 3], past=[0, 5]), mod.ERR_OVERFLOW | mod.ERR_POSITION),  # positions 5, 6
    ]
    bad = 0
    for kw, want in cases:
        rows = kw.get("rows", 6)
        res = mod.kv_append_rope(z, z, z, zc, zc, kw["cu"], kw["past"], 4, c[:rows], s[:rows],
                                 position_ids=kw.get("pos"), dtype="f32")
        bad += res["err"] != want
    return float(bad)


def pin_bf16_widening(mod):
    """bf16 bit patterns widen to the values torch gives them."""
    import torch
    x = torch.tensor([1.5, -2.25, 3.0e-3, 65504.0], dtype=torch.bfloat16)
    got = mod.to_f64(x.view(torch.int16).numpy().view(np.uint16), "bf16")
    return float(np.max(np.abs(got - x.double().numpy())))


PINS = [pin_complex_product, pin_relative_position, pin_pairing_permutation, pin_cache_contents,
        pin_error_bits, pin_bf16_widening]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_meets_pin(pin):
    assert pin(ra) < 1e-12


def test_identity_at_angle_zero():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 12))
    for inter in (True, False):
        y = ra.rotate(x, np.ones(4), np.zeros(4), 8, inter)
        assert np.array_equal(x, y)


def test_pair_norms_preserved():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((5, 16))
    ang = rng.uniform(-3, 3, size=(5, 8))
    for inter in (True, False):
        y = ra.rotate(x, np.cos(ang), np.sin(ang), 16, inter)
        i0, i1 = ra.pair_dims(16, inter)
        assert np.allclose(x[:, i0] ** 2 + x[:, i1] ** 2, y[:, i0] ** 2 + y[:, i1] ** 2, rtol=0, atol=1e-12)


def test_no_rotation_is_a_plain_append():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 2, 4)).astype(np.float32)
    kv = rng.standard_normal((3, 1, 4)).astype(np.float32)
    kc = np.zeros((10, 1, 4), dtype=np.float32)
    res = ra.kv_append_rope(q, kv, kv, kc, kc, [0, 3], [2], 10, dtype="f32")
    assert np.array_equal(res["q"], q.astype(np.float64))
    assert np.array_equal(res["k_cache"][2:5], kv.astype(np.float64))
    assert not res["k_cache"][:2].any() and not res["k_cache"][5:].any()


# ---- mutation checks ------------------------------------------------------------
SRC = ra.__file__
MUTATIONS = {
    "sin_sign": ("y[..., i0] = a * cos_row - b * sin_row", "y[..., i0] = a * cos_row + b * sin_row"),
    "second_turns_back": ("y[..., i1] = a * sin_row + b * cos_row", "y[..., i1] = -a * sin_row + b * cos_row"),
    "half_pair_adjacent": ("return m, m + rotary_dim // 2", "return m, m + 1"),
    "interleaved_pairs_swapped": ("return 2 * m, 2 * m + 1", "return 2 * m + 1, 2 * m"),
    "position_off_by_one": ("past[b] + np.arange(cu[b + 1] - cu[b])", "past[b] + 1 + np.arange(cu[b + 1] - cu[b])"),
    "slot_ignores_past": ("slot = b * capacity + int(past[b]) + i", "slot = b * capacity + i"),
    "value_rotated": ("vc[slot] = vd[t]", "vc[slot] = rotate(vd[t], c, s, rdim, interleaved) if rotate_on else vd[t]"),
    "query_not_rotated": ("q_out[t] = rotate(qd[t], c, s, rdim, interleaved)", "q_out[t] = qd[t]"),
    "overflow_off_by_one": ("np.any(past + lq > capacity)", "np.any(past + lq >= capacity)"),
    "position_bound_inclusive": ("(p >= rotary_rows)", "(p > rotary_rows)"),
    "position_ids_ignored": ("if position_ids is not None:", "if False:"),
    "bf16_widening": ("<< 16).view(np.float32)", "<< 15).view(np.float32)"),
}


def _load_mutant(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found in the oracle"
    path = tmp_path / f"rope_mutant_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"rope_mutant_{name}", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    mod = _load_mutant(tmp_path, name)
    worst = 0.0
    for pin in PINS:
        try:
            worst = max(worst, pin(mod))
        except (AssertionError, IndexError, ValueError, KeyError):
            worst = max(worst, 1.0)
    assert worst > 1e-6, f"no pin caught mutation {name}"


def test_mutation_sources_exist():
    assert os.path.exists(SRC)
