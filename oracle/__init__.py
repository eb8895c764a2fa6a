"""fp64 CPU oracle for packed variable-length scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers. The GPU library and its
Python binding never import this package, and this package never imports
them.

The arithmetic lives in ``varlen_oracle.c`` (plain C, fp64, one row at a
time). This module only builds it with gcc and marshals arguments through
ctypes. What it computes, with the passages of the source pages each step
follows (crate onnx-runtime-ep-cuda, page
src/kernels/packed_varlen_attention.rs, module doc and row kernel stages;
page src/kernels/standard_attention.rs, "Semantics"):

* sequence b owns query rows ``[cu_q[b], cu_q[b+1])`` and key/value rows
  ``[cu_kv[b], cu_kv[b+1])``; nothing attends across sequences;
* query head h reads kv head ``h // (Hq // Hkv)``;
* ``s = (q*sqrt(scale)) . (k*sqrt(scale))``, scale defaulting to
  ``1/sqrt(head_size)``;
* ``s = softcap*tanh(s/softcap)`` when softcap is non-zero, before the mask;
* with ``is_causal``, key j is visible to query i iff ``j <= i + L_kv - L_q``;
* with a local window ``W > 0`` (causal or not), key j is visible only if
  ``j >= i + L_kv - L_q + 1 - W`` (page src/kernels/attention.rs, the softmax
  kernel source's local_min; page src/kernels/group_query_attention.rs, the
  local_window_size attribute);
* stable softmax over the visible keys, rows with no visible key are zero;
* ``out = softmax . V`` in fp64.

``rope_append`` (numpy, fp64) is the oracle of the step before decode: the
rotary embedding of new query/key rows and their append to a fixed-capacity
KV cache.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "varlen_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libvarlen_oracle.so")

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no GPU, no HIP). Returns the library path."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        fn = lib.pva_oracle_attention
        fn.restype = ctypes.c_int
        fn.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_int, ctypes.c_double,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.pva_oracle_default_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    return int(_load().pva_oracle_default_threads())


def _f32(x) -> float:
    """scale and softcap are float attributes of the op (packed_varlen_attention.rs
    page, "Schema (v1)"): the oracle sees the binary32 value a caller passes."""
    return float(np.float32(x))


def _as_host_array(x, dtype: str) -> np.ndarray:
    """Contiguous host array holding the exact stored bits of ``x``.

    Accepts numpy arrays or CPU torch tensors. bf16 travels as its uint16 bit
    pattern because numpy has no bfloat16 type."""
    try:
        import torch  # noqa: F401
        is_torch = hasattr(x, "detach") and hasattr(x, "dtype") and "torch" in type(x).__module__
    except ImportError:  # pragma: no cover - torch is always present here
        is_torch = False
    if is_torch:
        import torch
        t = x.detach()
        if t.device.type != "cpu":
            raise ValueError("oracle inputs must live in host memory")
        t = t.contiguous()
        if dtype == "bf16":
            if t.dtype != torch.bfloat16:
                raise TypeError("expected a bfloat16 tensor")
            return t.view(torch.int16).numpy().view(np.uint16)
        want = {"f32": torch.float32, "f16": torch.float16}[dtype]
        if t.dtype != want:
            raise TypeError(f"expected {want}, got {t.dtype}")
        return t.numpy()
    a = np.ascontiguousarray(x)
    want = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    if a.dtype != want:
        raise TypeError(f"expected {want}, got {a.dtype}")
    return a


def attention(q, k, v, cu_q, cu_kv, num_heads: int, kv_num_heads: int | None = None,
              scale: float | None = None, is_causal: bool = False, softcap: float = 0.0,
              dtype: str = "f32", rows=None, key_window=None, with_lse: bool = False,
              threads: int = 0, local_window: int = 0):
    """Run the fp64 oracle.

    q: [total_q, Hq*D] or [total_q, Hq, D]; k: [total_kv, Hkv, D]; v: [total_kv, Hkv, Dv]
    (any shape with that many elements, contiguous, host memory, storage type ``dtype``).
    cu_q, cu_kv: int sequences of length B+1.
    scale: None or 0 -> 1/sqrt(D). rows: optional int64 row ids (token*Hq + head).
    key_window: optional (begin, end) local key window applied to every sequence.
    local_window: W > 0 limits row i to keys j >= i + L_kv - L_q + 1 - W; <= 0 no window.
    Returns out [n_rows, Dv] fp64 (and lse [n_rows] when ``with_lse``).
    """
    lib = _load()
    hq = int(num_heads)
    hkv = int(kv_num_heads) if kv_num_heads else hq
    qa = _as_host_array(q, dtype)
    ka = _as_host_array(k, dtype)
    va = _as_host_array(v, dtype)
    cuq = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int64)).astype(np.int32)
    cukv = np.ascontiguousarray(np.asarray(cu_kv, dtype=np.int64)).astype(np.int32)
    if cuq.shape != cukv.shape or cuq.ndim != 1 or cuq.size < 2:
        raise ValueError("cu_q and cu_kv must be 1-D of equal length >= 2")
    batch = cuq.size - 1
    total_q = int(cuq[-1])
    total_kv = int(cukv[-1])
    if total_q * hq == 0:  # no query rows: the head size comes from K, if any
        d = ka.size // (total_kv * hkv) if total_kv * hkv else 1
    else:
        if qa.size % (total_q * hq):
            raise ValueError("query size does not match total_q * num_heads")
        d = qa.size // (total_q * hq)
    if total_kv * hkv == 0:
        dv = d
    else:
        if ka.size != total_kv * hkv * d:
            raise ValueError("key size does not match total_kv * kv_num_heads * head_size")
        if va.size % (total_kv * hkv):
            raise ValueError("value size does not match total_kv * kv_num_heads")
        dv = va.size // (total_kv * hkv)
    if rows is None:
        n_rows = total_q * hq
        rows_arr = None
        rows_ptr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n_rows = rows_arr.size
        rows_ptr = rows_arr.ctypes.data
    out = np.zeros((n_rows, dv), dtype=np.float64)
    lse = np.zeros((n_rows,), dtype=np.float64) if with_lse else None
    kb, ke = (-1, -1) if key_window is None else (int(key_window[0]), int(key_window[1]))
    # numpy cannot hand out a pointer to an empty array's data; pass a dummy.
    dummy = np.zeros(1, dtype=np.float64)
    ptr = lambda a: a.ctypes.data if a.size else dummy.ctypes.data  # noqa: E731
    rc = lib.pva_oracle_attention(
        ptr(qa), ptr(ka), ptr(va), DTYPE_CODES[dtype],
        cuq.ctypes.data, cukv.ctypes.data, batch, total_q, total_kv, hq, hkv, d, dv,
        _f32(scale) if scale else 0.0, 1 if is_causal else 0, _f32(softcap), int(local_window),
        rows_ptr, n_rows, kb, ke,
        ptr(out), (ptr(lse) if lse is not None else None), int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (status {rc})")
    return (out, lse) if with_lse else out
