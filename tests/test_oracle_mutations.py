"""The pins must catch plausible mistakes in the oracle.

Each case copies the oracle's C source, plants one mistake (a wrong head
mapping, a flipped causal offset, a dropped softcap, scale or normalisation,
a transposed operand, an off-by-one mask, a wrong bf16 widening, a local window
that is dropped, off by one or blind to the causal offset), builds the
copy with gcc into a temporary directory and checks that the brute-force pin
no longer agrees. The planted mistakes live only in the temporary copy.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from brute import padded_attention

SRC = os.path.join(os.path.dirname(oracle.__file__), "varlen_oracle.c")

MUTATIONS = {
    "interleaved_gqa": ("const int32_t g = h / group;", "const int32_t g = h % job->hkv;"),
    "causal_offset_sign": ("j > i + offset", "j > i - offset"),
    "causal_off_by_one": ("j > i + offset", "j >= i + offset"),
    "softcap_dropped": ("acc = job->softcap * tanh(acc / job->softcap);", "acc = acc;"),
    "scale_dropped": ("const double root = sqrt(job->scale);", "const double root = 1.0;"),
    "value_reads_keys": ("load_elem(job->v, vbase + c", "load_elem(job->k, vbase + c"),
    "no_normalisation": ("out_row[c] /= l;", "out_row[c] /= 1.0;"),
    "bf16_widening": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "wrong_sequence_owner": ("if (job->cu_q[mid] <= t) lo = mid;", "if (job->cu_q[mid] < t) lo = mid;"),
    "window_off_by_one": ("j < i + offset + 1 - job->local_window", "j <= i + offset + 1 - job->local_window"),
    "window_without_offset": ("j < i + offset + 1 - job->local_window", "j < i + 1 - job->local_window"),
    "window_dropped": ("if (job->local_window > 0 && j <", "if (0 && j <"),
}


def _build_mutant(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found in the oracle"
    path = tmp_path / f"mutant_{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"libmutant_{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", str(path), "-o",
                    str(lib), "-lm"], check=True)
    return str(lib)


def _pin_cases():
    rng = np.random.default_rng(99)
    cases = []
    for causal, softcap, (hq, hkv), (lq, lkv), window in [
        (True, 0.0, (4, 2), ([3, 4], [5, 4]), 0),
        (True, 2.0, (4, 2), ([2, 3], [2, 6]), 0),
        (False, 1.5, (6, 3), ([3, 2], [4, 3]), 0),
        (True, 0.0, (2, 2), ([4], [2]), 0),
        (True, 0.0, (2, 1), ([3, 4], [6, 4]), 2),
        (False, 1.0, (2, 2), ([4, 2], [5, 3]), 3),
    ]:
        d = 3
        q = (rng.standard_normal((sum(lq), hq, d)) * 2).astype(np.float32)
        k = (rng.standard_normal((sum(lkv), hkv, d)) * 2).astype(np.float32)
        v = rng.standard_normal((sum(lkv), hkv, d)).astype(np.float32)
        cases.append((q, k, v, lq, lkv, hq, hkv, 0.5, causal, softcap, window))
    return cases


def _max_pin_error(lib_path):
    saved = oracle._lib
    try:
        oracle._lib = None
        real = oracle._LIB_PATH
        oracle._LIB_PATH = lib_path
        oracle.build = lambda force=False: lib_path  # noqa: E731 - do not rebuild the mutant
        worst = 0.0
        for q, k, v, lq, lkv, hq, hkv, scale, causal, softcap, window in _pin_cases():
            cu = lambda x: np.concatenate([[0], np.cumsum(x)]).astype(np.int32)  # noqa: E731
            got = oracle.attention(q, k, v, cu(lq), cu(lkv), hq, hkv, scale=scale,
                                   is_causal=causal, softcap=softcap, dtype="f32", local_window=window)
            want = np.asarray(padded_attention(q.astype(float).tolist(), k.astype(float).tolist(),
                                               v.astype(float).tolist(), lq, lkv, hq, hkv, scale,
                                               causal, softcap, window=window)).reshape(got.shape)
            worst = max(worst, float(np.max(np.abs(got - want))))
        return worst
    finally:
        oracle._lib = saved
        oracle._LIB_PATH = real
        import importlib
        importlib.reload(oracle)


def _bf16_pin_error(lib_path):
    import torch
    lib = ctypes.CDLL(lib_path)
    saved, saved_path = oracle._lib, oracle._LIB_PATH
    try:
        oracle._lib = None
        oracle._LIB_PATH = lib_path
        oracle.build = lambda force=False: lib_path  # noqa: E731
        g = torch.Generator().manual_seed(3)
        q = torch.randn(3, 2, 4, generator=g).to(torch.bfloat16)
        k = torch.randn(5, 2, 4, generator=g).to(torch.bfloat16)
        v = torch.randn(5, 2, 4, generator=g).to(torch.bfloat16)
        got = oracle.attention(q, k, v, [0, 3], [0, 5], 2, 2, scale=0.5, dtype="bf16")
        want = np.asarray(padded_attention(q.double().tolist(), k.double().tolist(),
                                           v.double().tolist(), [3], [5], 2, 2, 0.5, False, 0.0))
        return float(np.max(np.abs(got - want.reshape(got.shape))))
    finally:
        del lib
        oracle._lib, oracle._LIB_PATH = saved, saved_path
        import importlib
        importlib.reload(oracle)


def test_unmutated_copy_passes(tmp_path):
    path = tmp_path / "copy.c"
    path.write_text(open(SRC).read())
    lib = tmp_path / "libcopy.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", str(path), "-o",
                    str(lib), "-lm"], check=True)
    assert _max_pin_error(str(lib)) < 1e-12
    assert _bf16_pin_error(str(lib)) < 1e-12


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    err = _bf16_pin_error(lib) if name == "bf16_widening" else _max_pin_error(lib)
    assert err > 1e-6, f"pin did not catch mutation {name} (max error {err})"
