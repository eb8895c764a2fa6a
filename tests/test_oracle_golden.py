"""Regression check of the oracle against tests/golden/oracle_regression.json.

The fixture was written by tests/golden/make_golden.py, which calls only the
oracle; it detects unintended changes to the oracle's arithmetic. Each case
also carries a closed-form check that does not depend on the fixture."""
import json
import math
import os

import numpy as np
import pytest

import oracle

FIXTURE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_regression.json")
CASES = json.load(open(FIXTURE))["cases"]


@pytest.mark.parametrize("c", CASES, ids=[c["name"] for c in CASES])
def test_oracle_reproduces_golden(c):
    hq, hkv, d = c["num_heads"], c["kv_num_heads"], c["head_dim"]
    q = np.asarray(c["q"], np.float32).reshape(-1, hq, d)
    k = np.asarray(c["k"], np.float32).reshape(-1, hkv, d)
    v = np.asarray(c["v"], np.float32).reshape(-1, hkv, d)
    cu = lambda x: [0] + np.cumsum(x).tolist()  # noqa: E731
    for dtype in ("f32", "f16", "bf16"):
        import torch
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
        qt, kt, vt = (torch.from_numpy(x).to(tdt) for x in (q, k, v))
        out, lse = oracle.attention(qt, kt, vt, cu(c["lq"]), cu(c["lkv"]), hq, hkv, scale=c["scale"],
                                    is_causal=c["is_causal"], softcap=c["softcap"], dtype=dtype,
                                    with_lse=True)
        np.testing.assert_allclose(out.reshape(-1), np.asarray(c["out"]), rtol=0, atol=1e-14)
        want_lse = np.asarray([-math.inf if x is None else x for x in c["lse"]])
        np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-14)


def test_golden_fully_masked_rows_are_zero():
    c = next(c for c in CASES if c["name"] == "empty_and_masked_rows")
    out = np.asarray(c["out"]).reshape(-1, c["num_heads"], c["head_dim"])
    # sequence 0 has no keys; sequence 2 (L_q=3, L_kv=1) masks its first two rows
    assert np.all(out[0:2] == 0) and np.all(out[2:4] == 0)
    assert np.any(out[4] != 0)
