"""Host-side logic of bench.py, on the CPU: the per-row visible-key counts
that the TFLOP/s figures are priced from, the one-GPU rule, and the shape
of the cpu_baseline record."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402
import packed_varlen_scaled_amd as pva  # noqa: E402
import synth  # noqa: E402


def _brute_keys(lq, lkv, causal, window):
    out = []
    for a, b in zip(lq, lkv):
        row = []
        for i in range(a):
            n = 0
            for j in range(b):
                if causal and j > i + b - a:
                    continue
                if window > 0 and j < i + b - a + 1 - window:
                    continue
                n += 1
            row.append(n)
        out.append(np.array(row, dtype=np.int64))
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [0, 1, 7, 100])
def test_row_keys_match_brute_force_and_the_library_pair_count(causal, window):
    lq = [1, 0, 9, 40, 3, 17, 1]
    lkv = [5, 4, 9, 25, 0, 60, 0]
    got = bench.row_keys(lq, lkv, causal, window)
    want = _brute_keys(lq, lkv, causal, window)
    for g, w in zip(got, want):
        np.testing.assert_array_equal(g, w)
    total = int(sum(x.sum() for x in got))
    assert total == pva.valid_pairs(synth.cu_seqlens(lq), synth.cu_seqlens(lkv), causal, local_window=window or None)


def test_more_than_one_gpu_is_refused_before_any_device_work(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def _tiny(decode):
    w = synth.Workload("tiny", 0, 4, 2, 64, "f32", not decode, 0.0, 0.0, 1.0, 5)
    lq = [1, 1, 1, 1, 1] if decode else [20, 33, 7]
    lkv = [90, 300, 17, 64, 5] if decode else [20, 40, 7]
    return synth.make_batch(w, lq, lkv)


@pytest.mark.parametrize("decode", [False, True])
def test_cpu_baseline_record(decode):
    rec = bench.cpu_baseline(_tiny(decode), decode, budget_s=0.2)
    assert set(rec) == {"value", "unit", "cores", "kind", "sample"}
    assert rec["kind"] == "oracle" and rec["cores"] >= 1 and rec["value"] > 0
    assert rec["unit"] == ("GB/s" if decode else "TFLOP/s")
