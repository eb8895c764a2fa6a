"""Brute-force padded attention in pure Python, used only to pin the oracle.

It is deliberately formulated differently from the oracle: the packed batch
is first laid out at a common padded length, an explicit boolean mask matrix
is built per sequence (the padded + masked representation that the packed op
is stated to reproduce; packed_varlen_attention.rs page, module doc
"Relationship to ONNX Attention-24 nonpad_kv_seqlen"), scale multiplies the raw
dot product afterwards instead of being folded into the operands, sums use
math.fsum, and the per-sequence causal offset is applied through the mask
matrix. Only tiny shapes are meant to run through it.
"""
from __future__ import annotations

import math


def padded_attention(q, k, v, lq, lkv, hq, hkv, scale, causal, softcap, window=0):
    """q: packed nested lists [total_q][hq][d]; k, v: [total_kv][hkv][*].

    window > 0 keeps, for query i, only keys j with i - j < window - (lkv - lq)
    (the last `window` keys up to its tail-aligned diagonal).

    Returns packed output [total_q][hq][dv] as Python floats."""
    bsz = len(lq)
    sq = max(lq) if lq else 0
    skv = max(lkv) if lkv else 0
    d = len(q[0][0]) if q else (len(k[0][0]) if k else 1)
    dv = len(v[0][0]) if v else d
    zero_q = [[0.0] * d for _ in range(hq)]
    zero_k = [[0.0] * d for _ in range(hkv)]
    zero_v = [[0.0] * dv for _ in range(hkv)]
    # Scatter into padded [B][S][H][*] (pad rows are zeros and masked out).
    qp, kp, vp = [], [], []
    qs = ks = 0
    for b in range(bsz):
        qp.append([q[qs + i] if i < lq[b] else zero_q for i in range(sq)])
        kp.append([k[ks + j] if j < lkv[b] else zero_k for j in range(skv)])
        vp.append([v[ks + j] if j < lkv[b] else zero_v for j in range(skv)])
        qs += lq[b]
        ks += lkv[b]
    group = hq // hkv
    out = []
    for b in range(bsz):
        # mask[i][j]: query i may see key j.
        mask = [[(i < lq[b] and j < lkv[b] and
                  (not causal or j - i <= lkv[b] - lq[b]) and
                  (window <= 0 or i - j < window - (lkv[b] - lq[b])))
                 for j in range(skv)] for i in range(sq)]
        seq_out = [[None] * hq for _ in range(lq[b])]
        for h in range(hq):
            kvh = h // group
            for i in range(lq[b]):
                scores = []
                for j in range(skv):
                    raw = math.fsum(qp[b][i][h][p] * kp[b][j][kvh][p] for p in range(d)) * scale
                    if softcap:
                        raw = softcap * math.tanh(raw / softcap)
                    scores.append(raw if mask[i][j] else -math.inf)
                top = max(scores) if scores else -math.inf
                if top == -math.inf:
                    seq_out[i][h] = [0.0] * dv
                    continue
                w = [math.exp(s - top) if s != -math.inf else 0.0 for s in scores]
                z = math.fsum(w)
                seq_out[i][h] = [math.fsum(w[j] * vp[b][j][kvh][c] for j in range(skv)) / z
                                 for c in range(dv)]
        out.extend(seq_out)
    return out
