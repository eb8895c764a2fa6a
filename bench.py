#!/usr/bin/env python3
"""Benchmark of the packed varlen attention hot path on one MI355X.

A step is one attention call over the full synthetic batch of a workload,
with Q/K/V and the cu_seqlens arrays already resident in HBM. By default
(--path graph) the call is varlen_attn_fwd_device captured once into a HIP
graph, and a step is one replay: the device scheduler reads the cu arrays,
validates them and builds the work list, then every attention kernel runs.
--path device launches the same call eagerly each step; --path host times
varlen_attn_fwd (host validation and scheduling, work-list upload, kernels).

The headline workload is the largest one that fits one GPU, the long ragged
causal prefill with softcap 50 (B=8, L ~ logU[512,16384], Hq=64, Hkv=8,
D=128, bf16). The same JSON line carries sub-records, measured the same way
one after the other in this process (each batch freed before the next is
made), for the ragged causal prefill, the chunked prefill against a cache and
the packed decode (--only skips them). --cache (packed_decode,
chunked_prefill_cache) times the attention over a fixed-capacity KV cache
instead: a step is the cache step (rotary on the new q/k rows, append of k/v
into the cache) followed by the attention over the cache, both in the graph.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warmup-seconds S] [--workload NAME] [--only]
                    [--path graph|device|host] [--window W] [--cache]
    python bench.py --gemm-ceiling | --read-ceiling GIB | --copy-reference MIB

Before the K timed steps it runs at least W warm-up steps and keeps going
until S seconds (default 1) have passed: the GPU's clocks take that long to
settle under load, and the timed steps should see the steady state. The JSON
echoes W as ``warmup`` and the steps actually run as ``warmup_steps_run``.

Prints ONE JSON line. ``value`` is valid-pair TFLOP/s (2 * pairs * Hq * (D + Dv)
per step / step time) for prefill workloads and HBM GB/s (Q+K+V+O bytes per step
/ step time) for the decode workload; ``ms_per_step`` is the wall clock over
the K steps between two synchronisations divided by K, and ``step_ms`` the
median, min and max of the K steps by events on the launch stream.
``roofline`` reports the dominant kernel: its algorithmic work per launch
over its average duration, timed with HIP events recorded by the library on
the launch stream (on the graph path around K eager steps of the same call,
run after the warm-up and just before the timed replays: a graph replay
records no events). ``cpu_baseline`` times the fp64 CPU oracle on a bounded
sample of the same batch on every CPU this process may use (capped by
OMP_NUM_THREADS when set), and names the host CPU model.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "varlen attn TFLOP/s (valid pairs) + % bf16 MFMA peak; decode HBM GB/s"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# The headline is the largest configuration that fits one GPU: the long
# ragged causal prefill with softcap. The other bf16 workloads follow in the
# same line as sub-records (the tiny fp32 batch is a parity case only).
DEFAULT_WORKLOAD = "long_causal_softcap"
SUB_WORKLOADS = ("long_causal_softcap", "ragged_causal_prefill", "chunked_prefill_cache", "packed_decode")
KERNEL_SOURCES = {
    "prefill_mfma": ["packed_varlen_scaled_amd/csrc/prefill_mfma.hip", "packed_varlen_scaled_amd/csrc/prefill_tiles.h",
                     "packed_varlen_scaled_amd/csrc/combine.h", "packed_varlen_scaled_amd/csrc/common.h"],
    "decode": ["packed_varlen_scaled_amd/csrc/decode.hip", "packed_varlen_scaled_amd/csrc/combine.h",
               "packed_varlen_scaled_amd/csrc/common.h"],
    "cache_step": ["packed_varlen_scaled_amd/csrc/rope_append.hip", "packed_varlen_scaled_amd/csrc/common.h"],
}
CACHE_WORKLOADS = ("packed_decode", "chunked_prefill_cache")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def row_keys(lq, lkv, causal, window=0):
    """Visible keys of every query row, sequence by sequence (measurement only)."""
    out = []
    for a, b in zip(lq, lkv):
        i = np.arange(a, dtype=np.int64)
        hi = np.clip(i + (b - a) + 1, 0, b) if causal else np.full(a, b, dtype=np.int64)
        lo = np.clip(i + (b - a) + 1 - window, 0, b) if window > 0 else np.zeros(a, dtype=np.int64)
        out.append(np.maximum(hi - lo, 0))
    return out


def source_sha(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kind: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, or None when
    the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != source_sha(kind):
        return None
    return t.get("hbm_bytes_per_launch")


def sub_batch(batch, seqs):
    """Host copies of the chosen sequences as their own packed batch."""
    import torch
    import synth
    qs, ks, vs, lq, lkv = [], [], [], [], []
    for b in seqs:
        q0, q1 = int(batch.cu_q[b]), int(batch.cu_q[b + 1])
        k0, k1 = int(batch.cu_kv[b]), int(batch.cu_kv[b + 1])
        qs.append(batch.q[q0:q1].cpu())
        ks.append(batch.k[k0:k1].cpu())
        vs.append(batch.v[k0:k1].cpu())
        lq.append(q1 - q0)
        lkv.append(k1 - k0)
    return torch.cat(qs), torch.cat(ks), torch.cat(vs), synth.cu_seqlens(lq), synth.cu_seqlens(lkv), lq, lkv


def cpu_baseline(batch, decode: bool, budget_s: float = 12.0, window: int = 0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the batch."""
    import oracle
    w = batch.workload
    threads = oracle_threads()
    rng = np.random.default_rng(0)
    if decode:
        # whole sequences (every head), growing the sample until the budget is used
        order = rng.permutation(len(batch.lq)).tolist()
        seqs, t_used, bytes_done, n_rows = [], 0.0, 0, 0
        while order and t_used < budget_s:
            take = [order.pop() for _ in range(min(4, len(order)))]
            q, k, v, cq, ckv, lq, lkv = sub_batch(batch, take)
            t0 = time.perf_counter()
            oracle.attention(q, k, v, cq, ckv, w.num_heads, w.kv_num_heads, scale=w.scale or None,
                             is_causal=w.is_causal, softcap=w.softcap, dtype=w.dtype, threads=threads,
                             local_window=window)
            t_used += time.perf_counter() - t0
            el = 2 if w.dtype != "f32" else 4
            bytes_done += (q.numel() * 2 + k.numel() + v.numel()) * el
            seqs += take
            n_rows += sum(lq) * w.num_heads
        return {"value": bytes_done / t_used / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": f"{len(seqs)} of {len(batch.lq)} sequences, all {w.num_heads} heads "
                          f"({n_rows} rows), {t_used:.1f} s"}
    # prefill: random (token, head) rows of a few sequences, sized to the budget
    keys = row_keys(batch.lq, batch.lkv, w.is_causal, window)
    seqs = sorted(set(rng.choice(len(batch.lq), size=min(4, len(batch.lq)), replace=False).tolist()))
    q, k, v, cq, ckv, lq, lkv = sub_batch(batch, seqs)
    sub_keys = np.concatenate([keys[b] for b in seqs])
    n_all = int(cq[-1]) * w.num_heads
    perm = rng.permutation(n_all)
    flops_per_row = 2.0 * sub_keys[perm // w.num_heads] * (w.head_dim + w.dv)
    # calibrate on a growing slice (until it takes >= 1 s or covers every row),
    # then run a slice sized to the budget
    n_cal = min(n_all, 64)
    while True:
        t0 = time.perf_counter()
        oracle.attention(q, k, v, cq, ckv, w.num_heads, w.kv_num_heads, scale=w.scale or None,
                         is_causal=w.is_causal, softcap=w.softcap, dtype=w.dtype, rows=perm[:n_cal],
                         threads=threads, local_window=window)
        t_cal = max(time.perf_counter() - t0, 1e-6)
        if t_cal >= 1.0 or n_cal >= n_all:
            break
        n_cal = min(n_all, n_cal * 4)
    rate = flops_per_row[:n_cal].sum() / t_cal
    cum = np.cumsum(flops_per_row)
    n = int(min(n_all, max(n_cal, np.searchsorted(cum, rate * budget_s))))
    reps = 1
    if n == n_all:  # a small workload: time whole passes over it until the budget is used
        reps = max(1, int(budget_s / max(t_cal * flops_per_row.sum() / flops_per_row[:n_cal].sum(), 1e-6)))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.attention(q, k, v, cq, ckv, w.num_heads, w.kv_num_heads, scale=w.scale or None,
                         is_causal=w.is_causal, softcap=w.softcap, dtype=w.dtype, rows=perm[:n], threads=threads,
                         local_window=window)
    dt = (time.perf_counter() - t0) / reps
    return {"value": float(flops_per_row[:n].sum() / dt / 1e12), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} random (token, head) rows of sequences {seqs} "
                      f"({int(flops_per_row[:n].sum() / 2 / (w.head_dim + w.dv))} valid pairs), "
                      f"{reps} pass(es), {dt * reps:.1f} s"}


def gemm_ceiling(warmup_seconds: float = 1.0) -> int:
    """bf16 GEMM throughput by operand data. MFMA throughput on this chip
    depends on the operand bits (the clock drops as more bits toggle), so the
    dense spec peak is reached only on near-constant data."""
    import torch
    n = 8192
    torch.manual_seed(0)
    g = torch.Generator(device="cuda:0").manual_seed(0)
    res = {}
    for kind in ("zeros", "ones", "normal"):
        if kind == "zeros":
            a = torch.zeros(n, n, dtype=torch.bfloat16, device="cuda:0")
            b = torch.zeros(n, n, dtype=torch.bfloat16, device="cuda:0")
        elif kind == "ones":
            a = torch.ones(n, n, dtype=torch.bfloat16, device="cuda:0")
            b = torch.ones(n, n, dtype=torch.bfloat16, device="cuda:0")
        else:
            a = torch.randn(n, n, dtype=torch.float32, device="cuda:0", generator=g).to(torch.bfloat16)
            b = torch.randn(n, n, dtype=torch.float32, device="cuda:0", generator=g).to(torch.bfloat16)
        # at least 3 products, then more until warmup_seconds have passed (the
        # clocks settle under load, as for the attention steps)
        n_warm, t0 = 0, time.perf_counter()
        while n_warm < 3 or time.perf_counter() - t0 < warmup_seconds:
            torch.matmul(a, b)
            n_warm += 1
            if n_warm % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        reps = 30
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * n ** 3 / (ms / 1e3) / 1e12
        res[kind] = {"ms": ms, "tflops": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS}
        log(f"[gemm] {kind}: {ms:.3f} ms {tf:.0f} TFLOP/s")
        del a, b
    print(json.dumps({"gemm_ceiling": res, "m=n=k": n, "dtype": "bf16", "peak": PEAK_BF16_TFLOPS}), flush=True)
    return 0


class ClockSampler:
    """Graphics clock and socket power of GPU 0, polled with amdsmi from a
    thread while it runs (used over the untimed warm-up only, so the timed
    steps share the host with nothing). Every field is None when amdsmi is
    not usable."""

    def __init__(self, period_s: float = 0.02):
        import threading
        self.period_s = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._handle = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:  # no amdsmi, no device access: report nothing
            log(f"[bench] no clock samples: {e}")
            self._amdsmi = None

    def _poll(self):
        while not self._stop.is_set():
            try:
                m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
                clk, pw = m.get("current_gfxclk"), m.get("current_socket_power")
                if isinstance(clk, (int, float)) and isinstance(pw, (int, float)):
                    self.samples.append((float(clk), float(pw)))
            except Exception:
                pass
            self._stop.wait(self.period_s)

    def __enter__(self):
        if self._amdsmi is not None:
            import threading
            self._thread = threading.Thread(target=self._poll, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if self._amdsmi is not None:
            try:
                self._amdsmi.amdsmi_shut_down()
            except Exception:
                pass
            self._amdsmi = None
        return False

    def summary(self):
        """Medians over the second half of the samples (the clocks settle first)."""
        tail = self.samples[len(self.samples) // 2:]
        if not tail:
            return {"gfxclk_mhz": None, "socket_power_w": None, "samples": 0}
        clk = sorted(c for c, _ in tail)
        pw = sorted(w for _, w in tail)
        return {"gfxclk_mhz": clk[len(clk) // 2], "socket_power_w": pw[len(pw) // 2], "samples": len(tail)}


def read_ceiling(gib: float) -> int:
    """Streaming-read rate of device memory (the reference for the decode
    kernel's HBM rate). The measuring program (bench_read_ceiling.hip, beside
    this file; no part of the library) is compiled here with hipcc into a
    temporary folder and run as a child process, before this process touches
    the GPU."""
    import shutil
    import subprocess
    import tempfile
    src = os.path.join(ROOT, "bench_read_ceiling.hip")
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc") or "hipcc"
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "read_ceiling")
        cmd = [hipcc, "-O3", "-std=c++17", "-Wall", "--offload-arch=gfx950", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", src, "-o", exe]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            print(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}", file=sys.stderr)
            return 1
        res = subprocess.run([exe, str(gib)], capture_output=True, text=True)
    for line in res.stdout.splitlines():
        log(f"[read] {line}")
    if res.returncode != 0:
        print(res.stderr, file=sys.stderr)
        return res.returncode
    best = json.loads(res.stdout.strip().splitlines()[-1])
    best["peak"] = PEAK_HBM_GBS
    best["frac_of_peak"] = best["read_ceiling_GB/s"] / PEAK_HBM_GBS
    print(json.dumps(best), flush=True)
    return 0


def host_cpu_info():
    """Model name and logical CPU count of the host, and the CPUs this process
    may run on (the oracle's threads)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def oracle_threads() -> int:
    """Threads for the oracle: every CPU this process may run on, capped by
    OMP_NUM_THREADS when that is set (a job's share of a shared host)."""
    n = host_cpu_info()["usable_cpus"]
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def step_stats(ms_list):
    """Median, min and max of per-step durations (ms)."""
    xs = sorted(ms_list)
    if not xs:
        return None
    mid = len(xs) // 2
    med = xs[mid] if len(xs) % 2 else 0.5 * (xs[mid - 1] + xs[mid])
    return {"median": med, "min": xs[0], "max": xs[-1], "n": len(xs)}


def measure(name, a, cpu_budget, headline):
    """Measure one workload; returns its record (value, unit, step times,
    roofline of the dominant kernel, cpu_baseline, config). Every tensor it
    made is freed before it returns."""
    import torch
    import packed_varlen_scaled_amd as pva
    import synth

    w = synth.WORKLOADS[name]
    decode = name == "packed_decode"
    window = a.window if (headline and a.window > 0) else 0
    use_cache = headline and a.cache
    log(f"[bench] generating {name} on cuda:0")
    batch = synth.workload_batch(name, device="cuda:0")
    cu_q = torch.from_numpy(batch.cu_q).cuda()
    cu_kv = torch.from_numpy(batch.cu_kv).cuda()
    out = torch.empty(batch.total_q, w.num_heads, w.dv, dtype=batch.q.dtype, device="cuda:0")
    pairs = pva.valid_pairs(batch.cu_q, batch.cu_kv, w.is_causal, local_window=window or None)
    flops = 2.0 * pairs * w.num_heads * (w.head_dim + w.dv)
    el = 4 if w.dtype == "f32" else 2
    io_bytes = (batch.q.numel() + batch.k.numel() + batch.v.numel() + out.numel()) * el
    if window:
        # K and V rows no query row of its sequence can see are never read
        kv_rows = sum(b - max(0, b - q + 1 - window) if q else 0 for q, b in zip(batch.lq, batch.lkv))
        io_bytes = (batch.q.numel() + out.numel()) * el + kv_rows * w.kv_num_heads * (w.head_dim + w.dv) * el
    stats, _ = pva.plan(batch.cu_q, batch.cu_kv, w.num_heads, w.kv_num_heads, head_dim=w.head_dim,
                        dtype=w.dtype, is_causal=w.is_causal, softcap=w.softcap, local_window=window or None)
    log(f"[bench] total_q={batch.total_q} total_kv={batch.total_kv} valid_pairs={pairs} plan={stats}")

    def step_host():
        pva.varlen_attn_fwd(batch.q, batch.k, batch.v, cu_q, cu_kv, w.num_heads, w.kv_num_heads,
                            scale=w.scale or None, is_causal=w.is_causal, softcap=w.softcap, out=out,
                            cu_seqlens_q_host=batch.cu_q, cu_seqlens_kv_host=batch.cu_kv,
                            local_window=window or None)

    ws = latch = None
    if a.path != "host":
        ws = torch.empty(pva.device_workspace_bytes(len(batch.lq), batch.total_q, batch.total_kv, w.num_heads,
                                                    w.kv_num_heads, w.head_dim, w.dv, w.dtype),
                         dtype=torch.uint8, device="cuda:0")
        latch = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def step_device():
        pva.varlen_attn_fwd_device(batch.q, batch.k, batch.v, cu_q, cu_kv, w.num_heads, w.kv_num_heads,
                                   scale=w.scale or None, is_causal=w.is_causal, softcap=w.softcap,
                                   local_window=window or None, out=out, workspace=ws, error_latch=latch,
                                   decode_path=a.decode_path)

    step = step_host if a.path == "host" else step_device
    attn_io_bytes = io_bytes  # the attention kernels' own algorithmic bytes
    cache_bytes = 0
    cache_tensors = []
    if use_cache:
        # The cache: each sequence's first L_kv - L_q rows are its packed K/V
        # rows; its last L_q rows are the new rows the cache step appends
        # (after turning the keys). Slots past L_kv stay unwritten.
        cap = (max(batch.lkv) + 255) // 256 * 256
        bsz = len(batch.lq)
        kc = torch.empty(bsz * cap, w.kv_num_heads, w.head_dim, dtype=batch.k.dtype, device="cuda:0")
        vc = torch.empty(bsz * cap, w.kv_num_heads, w.dv, dtype=batch.v.dtype, device="cuda:0")
        new_rows = []
        past = []
        for b, (nq, nkv) in enumerate(zip(batch.lq, batch.lkv)):
            k0 = int(batch.cu_kv[b])
            kc[b * cap:b * cap + nkv - nq] = batch.k[k0:k0 + nkv - nq]
            vc[b * cap:b * cap + nkv - nq] = batch.v[k0:k0 + nkv - nq]
            new_rows.append(torch.arange(k0 + nkv - nq, k0 + nkv, device="cuda:0"))
            past.append(nkv - nq)
        idx = torch.cat(new_rows)
        k_new, v_new = batch.k[idx].contiguous(), batch.v[idx].contiguous()
        past_t = torch.tensor(past, dtype=torch.int32, device="cuda:0")
        kv_len_t = torch.empty(bsz, dtype=torch.int32, device="cuda:0")
        cos, sin = synth.rotary_tables(cap, w.head_dim, device="cuda:0")
        q_rot = torch.empty_like(batch.q)
        ws = torch.empty(pva.device_workspace_bytes(bsz, batch.total_q, bsz * cap, w.num_heads, w.kv_num_heads,
                                                    w.head_dim, w.dv, w.dtype), dtype=torch.uint8, device="cuda:0")
        cache_tensors = [kc, vc, k_new, v_new, past_t, kv_len_t, cos, sin, q_rot]
        # read q, k, v of the new rows and the two table rows; write q_out and the two cache rows
        cache_bytes = (2 * batch.total_q * (w.num_heads * w.head_dim + w.kv_num_heads * (w.head_dim + w.dv)) * el
                       + batch.total_q * w.head_dim * 4)
        io_bytes += cache_bytes
        log(f"[bench] cache: capacity {cap} rows/sequence, {kc.numel() * 2 * el / 2**30:.1f} GiB of K+V cache, "
            f"cache step moves {cache_bytes / 1e6:.1f} MB")

        def step_cache():
            pva.kv_append_rope(batch.q, k_new, v_new, kc, vc, cu_q, past_t, w.num_heads, w.kv_num_heads, cos=cos,
                               sin=sin, q_out=q_rot, kv_seqlens_out=kv_len_t, error_latch=latch)
            pva.varlen_attn_fwd_kvcache(q_rot, kc, vc, cu_q, kv_len_t, w.num_heads, w.kv_num_heads,
                                        scale=w.scale or None, is_causal=w.is_causal, softcap=w.softcap, out=out,
                                        workspace=ws, error_latch=latch)

        step = step_cache

    def warm_up(fn):
        # W untimed steps, then more until warmup_seconds have passed: the
        # GPU's clocks take a while to settle under load (the first
        # milliseconds run at lower clocks), and the timed steps should see
        # the steady state
        n, t0 = 0, time.perf_counter()
        while n < a.warmup or time.perf_counter() - t0 < a.warmup_seconds:
            fn()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return n

    sampler = ClockSampler()
    with sampler:
        warm_steps = warm_up(step)
    graph = None
    graph_warm = 0
    if a.path == "graph":
        # kernel times come from eagerly launched device-path steps (a graph
        # replay records no events); the timed steps below are replays
        pva.profile_enable(True)
        for _ in range(a.steps):
            step()
        torch.cuda.synchronize()
        prof_graph = pva.profile_read()
        pva.profile_enable(False)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        sampler = ClockSampler()
        with sampler:
            graph_warm = warm_up(graph.replay)
    log(f"[bench] warmup {warm_steps} steps (+{graph_warm} graph replays) done; timing {a.steps} steps ({a.path} path)")
    if graph is None:
        pva.profile_enable(True)
    # Per-step events on the launch stream give the median / min / max; the
    # step time itself is the wall clock over all K steps between two
    # synchronisations.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    host_s = 0.0
    evs[0].record()
    for i in range(a.steps):
        h0 = time.perf_counter()
        if graph is None:
            step()
        else:
            graph.replay()
        evs[i + 1].record()
        host_s += time.perf_counter() - h0
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(a.steps)]
    if graph is None:
        prof = pva.profile_read()
        pva.profile_enable(False)
    else:
        prof = prof_graph
    if latch is not None and int(latch.item()) != 0:
        raise RuntimeError(f"error latch set: {int(latch.item())}")
    ms = elapsed / a.steps * 1e3
    log(f"[bench] {ms:.4f} ms/step; host call {host_s / a.steps * 1e3:.4f} ms/step; kernels {prof}")

    if decode:
        value, unit = io_bytes / (ms / 1e3) / 1e9, "GB/s"
        kind = "decode"
        k_ms, k_n, _ = prof[kind]
        avg = k_ms / max(k_n, 1)
        achieved = attn_io_bytes / (avg / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        value, unit = flops / (ms / 1e3) / 1e12, "TFLOP/s"
        kind = "prefill_mfma" if w.dtype != "f32" else "prefill_f32"
        k_ms, k_n, _ = prof[kind]
        avg = k_ms / max(k_n, 1)
        achieved = flops / (avg / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    traffic = load_traffic(kind, name) if kind in KERNEL_SOURCES and not window and not use_cache else None
    roof["traffic"] = traffic
    roof["kernel"] = kind
    roof["kernel_avg_ms"] = avg
    roof["launches"] = k_n

    cache_info = None
    if use_cache:
        c_ms, c_n, _ = prof["cache_step"]
        c_avg = c_ms / max(c_n, 1)
        cache_info = {"kernel_avg_ms": c_avg, "bytes_per_launch": cache_bytes,
                      "GB/s": cache_bytes / (c_avg / 1e3) / 1e9 if c_avg else None,
                      "frac_of_hbm_peak": cache_bytes / (c_avg / 1e3) / 1e9 / PEAK_HBM_GBS if c_avg else None,
                      "traffic": load_traffic("cache_step", name), "capacity_rows": cap}
        log(f"[bench] cache step {cache_info}")

    cpu = None
    if cpu_budget > 0:
        log(f"[bench] timing the CPU oracle on a bounded sample of {name}")
        cpu = cpu_baseline(batch, decode, cpu_budget, window)
        log(f"[bench] cpu_baseline {cpu}")

    rec = {
        "value": value, "unit": unit, "ms_per_step": ms, "step_ms": step_stats(per_step),
        "warmup_steps_run": warm_steps, "dtype": w.dtype,
        "config": {"workload": name + (f" + local window {window}" if window else "")
                   + (" over a fixed-capacity KV cache (cache step + attention)" if use_cache else ""),
                   "local_window": window or None, "call": a.path,
                   "decode_path": a.decode_path if a.path != "host" and not use_cache else None,
                   "warmup_seconds": a.warmup_seconds,
                   "graph_warmup_replays": graph_warm,
                   "clock_during_warmup": sampler.summary(), "kv_cache": cache_info, "batch": w.batch,
                   "num_heads": w.num_heads, "kv_num_heads": w.kv_num_heads, "head_dim": w.head_dim,
                   "is_causal": w.is_causal, "softcap": w.softcap, "total_q": batch.total_q,
                   "total_kv": batch.total_kv, "valid_pairs": pairs, "flops_per_step": flops,
                   "io_bytes_per_step": io_bytes,
                   "pct_of_peak": 100.0 * (value / (PEAK_HBM_GBS if decode else PEAK_BF16_TFLOPS)),
                   "host_ms_per_call": host_s / a.steps * 1e3,
                   "kernel_ms_per_step": {k: v[0] / max(a.steps, 1) for k, v in prof.items() if v[1]},
                   "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu,
    }
    del graph, batch, out, ws, latch, cache_tensors
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="after the --warmup steps, keep running untimed steps until this many seconds have "
                         "passed (clocks settle under load); warmup_steps_run counts every warm-up step")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--only", action="store_true",
                    help="measure the --workload alone (no sub-records for the other workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--sub-cpu-budget", type=float, default=4.0,
                    help="seconds of oracle work for each sub-record's cpu_baseline")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB mebibytes, 5 times (the known-size "
                         "reference that HBM byte counters are calibrated against), then exit")
    ap.add_argument("--window", type=int, default=0, metavar="W",
                    help="measure the workload with a local window of W keys per row (W > 0); FLOPs count "
                         "only the pairs the window leaves visible")
    ap.add_argument("--decode-path", type=int, default=0, choices=[0, 1],
                    help="device and graph paths: 1 sends every sequence through the prefill kernel and "
                         "leaves out the decode launch (for batches known to hold no single-row sequences)")
    ap.add_argument("--path", choices=["host", "device", "graph"], default="graph",
                    help="host: varlen_attn_fwd (host scheduler, host cu mirrors); device: "
                         "varlen_attn_fwd_device (device scheduler, no host work per call); graph: one "
                         "device-path call captured in a HIP graph, the timed steps are replays")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="only time a plain library bf16 GEMM (8192^3, torch.matmul -> hipBLASLt) on "
                         "zero, constant and N(0,1) operands, then exit: the MFMA rate the chip sustains "
                         "on data like the workloads', next to the dense spec peak")
    ap.add_argument("--read-ceiling", type=float, default=0.0, metavar="GIB",
                    help="only run the streaming-read program over a GIB-gibibyte buffer (grid and loads in "
                         "flight swept), then exit: the read rate device memory sustains, next to the HBM spec")
    ap.add_argument("--cache", action="store_true",
                    help="packed_decode / chunked_prefill_cache over a fixed-capacity KV cache: each step runs "
                         "the cache step (rotary + append of the new rows) and the attention over the cache")
    a = ap.parse_args(argv)
    if a.cache and (a.workload not in CACHE_WORKLOADS or a.path == "host" or a.window):
        print(f"--cache needs one of {CACHE_WORKLOADS}, the device or graph path and no window", file=sys.stderr)
        return 2
    if a.decode_path and (a.path == "host" or a.cache):
        print("--decode-path applies to the device and graph paths without --cache (the host path and the "
              "cache call always use the automatic setting)", file=sys.stderr)
        return 2
    if a.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        return 2
    if a.gemm_ceiling:
        return gemm_ceiling(a.warmup_seconds)
    if a.read_ceiling:
        return read_ceiling(a.read_ceiling)
    if a.copy_reference:
        import torch
        n = a.copy_reference << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_reference_bytes": n, "copies": 5}), flush=True)
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the attention kernels work on one GPU's share of a batch "
              "and the library launches no multi-GPU work. Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import packed_varlen_scaled_amd as pva
    import synth

    if a.workload not in synth.WORKLOADS:
        print(f"unknown workload {a.workload}; choose from {sorted(synth.WORKLOADS)}", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    pva.load_library()
    torch.cuda.set_device(0)

    head = measure(a.workload, a, 0.0 if a.no_cpu_baseline else a.cpu_budget, headline=True)
    subs = None
    if not (a.only or a.cache or a.window):
        subs = {}
        for name in SUB_WORKLOADS:
            if name == a.workload:
                continue
            subs[name] = measure(name, a, 0.0 if a.no_cpu_baseline else a.sub_cpu_budget, headline=False)

    cpu = head["cpu_baseline"]
    if cpu is not None:
        cpu = dict(cpu, host=host_cpu_info())
    line = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "warmup_steps_run": head["warmup_steps_run"],
        "ms_per_step": head["ms_per_step"], "step_ms": head["step_ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic",
        "config": head["config"], "roofline": head["roofline"], "cpu_baseline": cpu,
        "sub_records": subs,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
