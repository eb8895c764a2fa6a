"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on
the same inputs (whole batch or sampled rows of chosen sequences), compare
with the fixed parity tolerance per dtype.

Tolerances: fp32 max|gpu - oracle| <= 1e-4; bf16 / f16 max-abs <= 2e-2 and
||gpu - oracle||_2 / ||oracle||_2 <= 5e-3, over every compared element.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL = {"f32": dict(max_abs=1e-4, rel_l2=None), "bf16": dict(max_abs=2e-2, rel_l2=5e-3),
       "f16": dict(max_abs=2e-2, rel_l2=5e-3)}


def run_gpu(batch: synth.Batch, out=None, **opts):
    import torch
    import packed_varlen_scaled_amd as pva
    w = batch.workload
    dev = batch.q.device
    cu_q = torch.from_numpy(batch.cu_q).to(dev)
    cu_kv = torch.from_numpy(batch.cu_kv).to(dev)
    o = pva.varlen_attn_fwd(batch.q, batch.k, batch.v, cu_q, cu_kv, w.num_heads, w.kv_num_heads,
                            scale=w.scale or None, is_causal=w.is_causal, softcap=w.softcap, out=out,
                            cu_seqlens_q_host=batch.cu_q, cu_seqlens_kv_host=batch.cu_kv, **opts)
    torch.cuda.synchronize()
    return o


def oracle_all(batch: synth.Batch, threads: int = 0, local_window: int = 0):
    w = batch.workload
    out = oracle.attention(batch.q.cpu(), batch.k.cpu(), batch.v.cpu(), batch.cu_q, batch.cu_kv,
                           w.num_heads, w.kv_num_heads, scale=w.scale or None, is_causal=w.is_causal,
                           softcap=w.softcap, dtype=w.dtype, threads=threads, local_window=local_window)
    return out.reshape(batch.total_q, w.num_heads, w.dv)


def sample_rows(batch: synth.Batch, seqs, rows_per_seq: int, seed: int = 0):
    """(seq, local row, head) triples: the first and last rows of each chosen
    sequence plus random ones, every head for the first row."""
    rng = np.random.default_rng(seed)
    w = batch.workload
    picks = []
    for b in seqs:
        lq = batch.lq[b]
        if lq == 0:
            continue
        rows = {0, lq - 1} | set(rng.integers(0, lq, size=rows_per_seq).tolist())
        for r in sorted(rows):
            heads = range(w.num_heads) if r == 0 else rng.integers(0, w.num_heads, size=2).tolist()
            for h in heads:
                picks.append((b, r, int(h)))
    return picks


def oracle_sampled(batch: synth.Batch, picks, threads: int = 0, local_window: int = 0):
    """Oracle values for (seq, row, head) picks, computed on a sub-batch made of
    just the picked sequences (so no full-size K/V ever goes to the host)."""
    w = batch.workload
    seqs = sorted({b for b, _, _ in picks})
    qs, ks, vs, lq, lkv = [], [], [], [], []
    for b in seqs:
        q0, q1 = int(batch.cu_q[b]), int(batch.cu_q[b + 1])
        k0, k1 = int(batch.cu_kv[b]), int(batch.cu_kv[b + 1])
        qs.append(batch.q[q0:q1].cpu())
        ks.append(batch.k[k0:k1].cpu())
        vs.append(batch.v[k0:k1].cpu())
        lq.append(q1 - q0)
        lkv.append(k1 - k0)
    import torch
    q, k, v = torch.cat(qs), torch.cat(ks), torch.cat(vs)
    cq, ckv = synth.cu_seqlens(lq), synth.cu_seqlens(lkv)
    pos = {b: i for i, b in enumerate(seqs)}
    rows = np.array([(int(cq[pos[b]]) + r) * w.num_heads + h for b, r, h in picks], dtype=np.int64)
    return oracle.attention(q, k, v, cq, ckv, w.num_heads, w.kv_num_heads, scale=w.scale or None,
                            is_causal=w.is_causal, softcap=w.softcap, dtype=w.dtype, rows=rows,
                            threads=threads, local_window=local_window)


def gather_gpu(batch: synth.Batch, out, picks):
    import torch
    idx = torch.tensor([int(batch.cu_q[b]) + r for b, r, _ in picks], dtype=torch.long, device=out.device)
    hid = torch.tensor([h for _, _, h in picks], dtype=torch.long, device=out.device)
    o = out.view(batch.total_q, batch.workload.num_heads, -1)
    return o[idx, hid].double().cpu().numpy()


def compare(got: np.ndarray, want: np.ndarray, dtype: str):
    """Returns (max_abs, rel_l2) and asserts the tolerance of dtype."""
    got = np.asarray(got, dtype=np.float64).reshape(want.shape)
    diff = got - want
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    tol = TOL[dtype]
    assert np.all(np.isfinite(got)), "non-finite output"
    assert max_abs <= tol["max_abs"], f"max-abs {max_abs:.3e} > {tol['max_abs']}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"rel-L2 {rel:.3e} > {tol['rel_l2']}"
    return max_abs, rel
