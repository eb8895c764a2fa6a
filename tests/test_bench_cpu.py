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


def test_step_stats_median_min_max():
    assert bench.step_stats([3.0, 1.0, 2.0]) == {"median": 2.0, "min": 1.0, "max": 3.0, "n": 3}
    assert bench.step_stats([4.0, 1.0, 2.0, 3.0])["median"] == 2.5
    assert bench.step_stats([]) is None


def test_host_cpu_info_and_oracle_threads(monkeypatch):
    info = bench.host_cpu_info()
    assert set(info) == {"model", "logical_cpus", "usable_cpus"}
    assert info["usable_cpus"] >= 1
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.oracle_threads() == 1
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.oracle_threads() == info["usable_cpus"]


@pytest.mark.parametrize("args", [["--decode-path", "1", "--path", "host"],
                                  ["--decode-path", "1", "--cache", "--workload", "packed_decode"]])
def test_decode_path_refused_where_it_would_be_ignored(args, capsys):
    assert bench.main(args) == 2
    assert "--decode-path" in capsys.readouterr().err


def test_headline_is_the_largest_workload_and_sub_records_cover_the_rest():
    sizes = {}
    for name in bench.SUB_WORKLOADS:
        w = synth.WORKLOADS[name]
        lq, lkv = synth.draw_lengths(name)
        if name == "packed_decode":
            continue
        pairs = pva.valid_pairs(synth.cu_seqlens(lq), synth.cu_seqlens(lkv), w.is_causal)
        sizes[name] = 2.0 * pairs * w.num_heads * (w.head_dim + w.dv)
    assert bench.DEFAULT_WORKLOAD == max(sizes, key=sizes.get)
    assert set(bench.SUB_WORKLOADS) == set(synth.WORKLOADS) - {"tiny_fp32"}


def test_kernel_source_hash_covers_every_local_include():
    """The traffic counters in profiles/ are used only while the hash of the
    kernel's sources matches; every header a kernel file includes from the
    package (transitively) must be part of that hash."""
    import re
    csrc = os.path.join(os.path.dirname(bench.__file__), "packed_varlen_scaled_amd", "csrc")

    def closure(name, seen):
        if name in seen:
            return seen
        seen.add(name)
        with open(os.path.join(csrc, name)) as f:
            for inc in re.findall(r'^#include "([^"]+)"', f.read(), flags=re.M):
                if os.path.exists(os.path.join(csrc, inc)):
                    closure(inc, seen)
        return seen

    for kind, files in bench.KERNEL_SOURCES.items():
        names = {os.path.basename(f) for f in files}
        main = [n for n in names if n.endswith(".hip")]
        assert len(main) == 1, (kind, names)
        assert closure(main[0], set()) <= names, (kind, closure(main[0], set()) - names)
