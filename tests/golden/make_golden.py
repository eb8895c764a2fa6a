"""Write tests/golden/oracle_regression.json.

Regression fixture for the fp64 oracle: small hand-written inputs made of
exact binary fractions (so every storage type holds them exactly) and the
oracle's outputs for them. The source pages print no worked numeric example,
so these values come from the oracle alone (this script calls nothing but
``oracle/``); they guard the oracle against unintended changes, while its
correctness is pinned by the brute-force, closed-form and invariant tests.

Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def case(name, lq, lkv, hq, hkv, d, scale, causal, softcap, seed):
    rng = np.random.default_rng(seed)
    # multiples of 1/8 in [-2, 2]: exact in f32, f16 and bf16
    q = (rng.integers(-16, 17, size=(sum(lq), hq, d)) / 8.0).astype(np.float32)
    k = (rng.integers(-16, 17, size=(sum(lkv), hkv, d)) / 8.0).astype(np.float32)
    v = (rng.integers(-16, 17, size=(sum(lkv), hkv, d)) / 8.0).astype(np.float32)
    cu = lambda x: [0] + np.cumsum(x).tolist()  # noqa: E731
    out, lse = oracle.attention(q, k, v, cu(lq), cu(lkv), hq, hkv, scale=scale, is_causal=causal,
                                softcap=softcap, dtype="f32", with_lse=True)
    return {
        "name": name, "lq": lq, "lkv": lkv, "num_heads": hq, "kv_num_heads": hkv, "head_dim": d,
        "scale": scale, "is_causal": causal, "softcap": softcap,
        "q": q.reshape(-1).tolist(), "k": k.reshape(-1).tolist(), "v": v.reshape(-1).tolist(),
        "out": out.reshape(-1).tolist(),
        "lse": [x if np.isfinite(x) else None for x in lse.tolist()],
    }


def main():
    cases = [
        case("mha_noncausal", [3, 2], [3, 2], 2, 2, 4, 0.5, False, 0.0, 1),
        case("gqa_causal_tail_aligned", [2, 4], [5, 3], 4, 2, 4, 0.0, True, 0.0, 2),
        case("mqa_causal_softcap", [3, 1], [3, 4], 3, 1, 2, 0.25, True, 2.0, 3),
        case("empty_and_masked_rows", [2, 0, 3], [0, 2, 1], 2, 1, 2, 1.0, True, 0.0, 4),
    ]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")
    with open(path, "w") as f:
        json.dump({"source": "tests/golden/make_golden.py (oracle/ only)", "cases": cases}, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
