"""Packed variable-length scaled-dot-product attention on MI355X (gfx950).

A thin ctypes binding over ``libvarlen_attn.so`` (C ABI in
``include/varlen_attn.h``). This module only marshals arguments: every step
of the computation runs in the library's HIP kernels. There is no CPU or
PyTorch fallback; if the library is missing, importing the binding's entry
points raises.

Semantics follow the packed op of the crate onnx-runtime-ep-cuda (page
src/kernels/packed_varlen_attention.rs, module doc "Packed layout &
cumulative offsets", "Schema (v1)", "Causal alignment"). Q is
``[total_q, Hq, D]`` (or ``[total_q, Hq*D]``), K/V are ``[total_kv, Hkv, D]``
(or rank 2), and int32 ``cu_seqlens`` arrays of length B+1 delimit the
sequences.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "varlen_attn_fwd", "plan", "valid_pairs", "library_path", "load_library", "VarlenAttnError",
    "PlanStats", "ITEM_INTS", "DTYPE_CODES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libvarlen_attn.so")
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
ITEM_INTS = 16
STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "BAD_SEQLENS", 3: "UNSUPPORTED", 4: "DEVICE",
                5: "OUT_OF_MEMORY"}

_lib = None


class VarlenAttnError(RuntimeError):
    """A non-OK status from the library; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[{STATUS_NAMES.get(status, status)}] {message}")
        self.status = status


class Options(ctypes.Structure):
    _fields_ = [("decode_path", ctypes.c_int32), ("decode_chunk", ctypes.c_int32),
                ("prefill_kv_chunk", ctypes.c_int32), ("local_window", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 4)]


class PlanStats(ctypes.Structure):
    _fields_ = [("n_prefill_items", ctypes.c_int64), ("n_decode_items", ctypes.c_int64),
                ("n_combine_items", ctypes.c_int64), ("n_partials", ctypes.c_int64),
                ("valid_pairs", ctypes.c_int64), ("visited_pairs", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("waves_per_prefill_item", ctypes.c_int32),
                ("heads_per_item", ctypes.c_int32), ("reserved", ctypes.c_int32 * 6)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}


class ProfileTotals(ctypes.Structure):
    _fields_ = [("total_ms", ctypes.c_double * 7), ("launches", ctypes.c_int64 * 7),
                ("items", ctypes.c_int64 * 7)]


PROFILE_KINDS = ("prefill_mfma", "prefill_f32", "decode", "combine", "upload", "device_plan", "cache_step")

# Bits of the device path's error latch (include/varlen_attn.h, varlen_attn_fwd_device).
LATCH_BITS = {1: "cu_seqlens_q[0] != 0", 2: "cu_seqlens_q decreases", 4: "cu_seqlens_q[batch] > total_q",
              8: "cu_seqlens_kv[0] != 0", 16: "cu_seqlens_kv decreases", 32: "cu_seqlens_kv[batch] > total_kv",
              64: "work list overflow", 128: "cache_seqlens[b] < 0",
              256: "cache_seqlens[b] + new rows > cache_capacity", 512: "position outside the rotary tables",
              1024: "kv_seqlens[b] outside [0, cache_capacity]"}


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libvarlen_attn.so (built by ``python -m packed_varlen_scaled_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m packed_varlen_scaled_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    fwd_args = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, i32, f32, i32, f32, vp, vp]
    lib.varlen_attn_fwd.argtypes = fwd_args
    lib.varlen_attn_fwd.restype = ctypes.c_int
    lib.varlen_attn_fwd_ex.argtypes = fwd_args + [ctypes.POINTER(Options)]
    lib.varlen_attn_fwd_ex.restype = ctypes.c_int
    lib.varlen_attn_device_workspace_bytes.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32]
    lib.varlen_attn_device_workspace_bytes.restype = ctypes.c_size_t
    lib.varlen_attn_fwd_device.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, i32, f32, i32, f32,
                                           i32, vp, vp, ctypes.c_size_t, vp, vp]
    lib.varlen_attn_fwd_device.restype = ctypes.c_int
    lib.varlen_attn_fwd_device_ex.argtypes = lib.varlen_attn_fwd_device.argtypes + [ctypes.POINTER(Options)]
    lib.varlen_attn_fwd_device_ex.restype = ctypes.c_int
    lib.varlen_attn_fwd_device_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, i32, f32,
                                                   i32, f32, i32, vp, vp, vp]
    lib.varlen_attn_fwd_device_noalloc.restype = ctypes.c_int
    lib.varlen_attn_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32, i32, f32, i32,
                                            f32, i32, vp, vp, ctypes.c_size_t, vp, vp]
    lib.varlen_attn_fwd_kvcache.restype = ctypes.c_int
    lib.varlen_kv_append_rope.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64,
                                          i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.varlen_kv_append_rope.restype = ctypes.c_int
    lib.varlen_attn_plan.argtypes = [vp, vp, i32, i64, i64, i32, i32, i32, i32, i32, f32, i32, f32,
                                     ctypes.POINTER(Options), ctypes.POINTER(PlanStats), vp, i64]
    lib.varlen_attn_plan.restype = ctypes.c_int
    lib.varlen_attn_valid_pairs.argtypes = [vp, vp, i32, i32]
    lib.varlen_attn_valid_pairs.restype = ctypes.c_int64
    lib.varlen_attn_valid_pairs_window.argtypes = [vp, vp, i32, i32, i32]
    lib.varlen_attn_valid_pairs_window.restype = ctypes.c_int64
    lib.varlen_attn_last_error.argtypes = []
    lib.varlen_attn_last_error.restype = ctypes.c_char_p
    lib.varlen_attn_release.argtypes = []
    lib.varlen_attn_release.restype = ctypes.c_int
    lib.varlen_attn_profile_enable.argtypes = [i32]
    lib.varlen_attn_profile_enable.restype = ctypes.c_int
    lib.varlen_attn_profile_read.argtypes = [ctypes.POINTER(ProfileTotals)]
    lib.varlen_attn_profile_read.restype = ctypes.c_int
    lib.varlen_attn_version.argtypes = []
    lib.varlen_attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().varlen_attn_last_error().decode(errors="replace")
        raise VarlenAttnError(status, msg)


def _options(decode_path=0, decode_chunk=0, prefill_kv_chunk=0, local_window=None):
    o = Options()
    o.decode_path, o.decode_chunk, o.prefill_kv_chunk = int(decode_path), int(decode_chunk), int(prefill_kv_chunk)
    o.local_window = -1 if local_window is None else int(local_window)
    return o


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if t.dtype not in codes:
        raise TypeError(f"Q/K/V dtype {t.dtype} not supported (expected float32, float16 or bfloat16)")
    return codes[t.dtype]


def _resolve(t, heads: int, name: str):
    """[tokens, heads, dim] or [tokens, heads*dim] -> (tokens, dim), like the op's
    rank-2/rank-3 resolution (packed_varlen_attention.rs page, resolve_packed)."""
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() == 3:
        if t.shape[1] != heads:
            raise ValueError(f"{name} rank-3 head dim {t.shape[1]} must equal head count {heads}")
        return t.shape[0], t.shape[2]
    if t.dim() == 2:
        if t.shape[1] % heads:
            raise ValueError(f"{name} rank-2 hidden size {t.shape[1]} is not divisible by head count {heads}")
        return t.shape[0], t.shape[1] // heads
    raise ValueError(f"{name} must be rank 2 or 3, got rank {t.dim()}")


def _host_cu(x):
    import numpy as np
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x.cpu() if hasattr(x, "cpu") else x, dtype=np.int64))
    if a.ndim != 1:
        raise ValueError("cu_seqlens must be 1-D")
    if a.size and (a.min() < -2**31 or a.max() >= 2**31):
        raise ValueError("cu_seqlens values must fit int32")
    return a.astype(np.int32)


def varlen_attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_kv, num_heads: int, kv_num_heads=None,
                    scale=None, is_causal: bool = False, softcap: float = 0.0, out=None,
                    cu_seqlens_q_host=None, cu_seqlens_kv_host=None, stream=None,
                    decode_path: int = 0, decode_chunk: int = 0, prefill_kv_chunk: int = 0,
                    local_window=None):
    """Packed varlen attention forward on the current GPU stream.

    q, k, v: CUDA(HIP) tensors, rank 3 ``[T, H, D]`` or rank 2 ``[T, H*D]``.
    cu_seqlens_q / cu_seqlens_kv: int32 CUDA tensors ``[B+1]``; the optional
    host mirrors (any int sequence) spare the library a device->host read.
    local_window: None or -1 for no window; W > 0 keeps for row i only the
    keys j >= i + L_kv - L_q + 1 - W.
    Returns ``out`` (allocated like q with v's head size when not given)."""
    import torch
    lib = load_library()
    hq = int(num_heads)
    hkv = int(kv_num_heads) if kv_num_heads else hq
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors")
    code = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("Q, K, and V must use the same floating dtype")
    if hq <= 0 or hkv <= 0:
        raise ValueError("num_heads and kv_num_heads must be positive")
    tq, d = _resolve(q, hq, "query")
    tkv, dk = _resolve(k, hkv, "key")
    tv, dv = _resolve(v, hkv, "value")
    if dk != d:
        raise ValueError(f"query head_size {d} != key head_size {dk}")
    if tv != tkv:
        raise ValueError(f"key token count {tkv} != value token count {tv}")
    if out is None:
        shape = (tq, hq, dv) if q.dim() == 3 else (tq, hq * dv)
        out = torch.empty(shape, dtype=q.dtype, device=q.device)
    elif out.dtype != q.dtype or not out.is_contiguous() or out.numel() != tq * hq * dv or not out.is_cuda:
        raise ValueError("output must be a contiguous GPU tensor of the Q/K/V dtype with [total_q, num_heads, v_head_size] elements")
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
        if cu is not None and (not cu.is_cuda or cu.dtype != torch.int32 or not cu.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    if cu_seqlens_q is None and cu_seqlens_q_host is None:
        raise ValueError("cu_seqlens_q is required")
    n = (cu_seqlens_q.numel() if cu_seqlens_q is not None else len(cu_seqlens_q_host))
    n_kv = (cu_seqlens_kv.numel() if cu_seqlens_kv is not None else len(cu_seqlens_kv_host))
    if n != n_kv:
        raise ValueError(f"cu_seqlens_q length {n} != cu_seqlens_kv length {n_kv} (both must be batch_size + 1)")
    hq_host = _host_cu(cu_seqlens_q_host)
    hkv_host = _host_cu(cu_seqlens_kv_host)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = _options(decode_path, decode_chunk, prefill_kv_chunk, local_window)
    with torch.cuda.device(q.device):
        st = lib.varlen_attn_fwd_ex(
            q.data_ptr(), k.data_ptr(), v.data_ptr(),
            cu_seqlens_q.data_ptr() if cu_seqlens_q is not None else None,
            cu_seqlens_kv.data_ptr() if cu_seqlens_kv is not None else None,
            hq_host.ctypes.data if hq_host is not None else None,
            hkv_host.ctypes.data if hkv_host is not None else None,
            n - 1, tq, tkv, hq, hkv, d, dv, code,
            float(scale) if scale else 0.0, 1 if is_causal else 0, float(softcap),
            out.data_ptr(), stream, ctypes.byref(opts))
    _check(st)
    return out


def device_workspace_bytes(batch: int, total_q: int, total_kv: int, num_heads: int, kv_num_heads=None,
                           head_dim: int = 128, v_head_dim: int = 0, dtype: str = "bf16") -> int:
    """Bytes of workspace varlen_attn_fwd_device needs for these buffer sizes."""
    n = load_library().varlen_attn_device_workspace_bytes(int(batch), int(total_q), int(total_kv), int(num_heads),
                                                          int(kv_num_heads or 0), int(head_dim), int(v_head_dim),
                                                          DTYPE_CODES[dtype])
    if n == 0:
        raise ValueError("invalid sizes for the device workspace")
    return int(n)


def varlen_attn_fwd_device(q, k, v, cu_seqlens_q, cu_seqlens_kv, num_heads: int, kv_num_heads=None,
                           scale=None, is_causal: bool = False, softcap: float = 0.0, local_window=None,
                           out=None, workspace=None, error_latch=None, stream=None, decode_path: int = 0):
    """The capture-safe call: cu_seqlens are read only on the device, nothing is
    allocated, copied from the host or waited for. ``workspace`` is a CUDA(HIP)
    uint8 tensor of at least ``device_workspace_bytes(...)`` bytes and
    ``error_latch`` an int32 CUDA tensor of one element, zero before first use
    (see LATCH_BITS). The rows of q/out and k/v are the buffer capacities;
    cu_seqlens_*[-1] may be smaller. decode_path=1 sends every sequence through
    the prefill kernel and leaves out the decode and combine launches
    (varlen_attn_fwd_device_ex). Returns ``out``."""
    import torch
    lib = load_library()
    hq = int(num_heads)
    hkv = int(kv_num_heads) if kv_num_heads else hq
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors")
    code = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("Q, K, and V must use the same floating dtype")
    tq, d = _resolve(q, hq, "query")
    tkv, dk = _resolve(k, hkv, "key")
    tv, dv = _resolve(v, hkv, "value")
    if dk != d or tv != tkv:
        raise ValueError("key head size / token count must match query head size / value token count")
    if out is None:
        raise ValueError("out is required (the call allocates nothing)")
    if out.dtype != q.dtype or not out.is_contiguous() or out.numel() != tq * hq * dv or not out.is_cuda:
        raise ValueError("output must be a contiguous GPU tensor of the Q/K/V dtype with [total_q, num_heads, v_head_size] elements")
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
        if cu is None or not cu.is_cuda or cu.dtype != torch.int32 or not cu.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    if cu_seqlens_q.numel() != cu_seqlens_kv.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_kv lengths differ")
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    if error_latch is None or not error_latch.is_cuda or error_latch.dtype != torch.int32:
        raise ValueError("error_latch must be an int32 GPU tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_kv.data_ptr(),
            cu_seqlens_q.numel() - 1, tq, tkv, hq, hkv, d, dv, code,
            float(scale) if scale else 0.0, 1 if is_causal else 0, float(softcap),
            -1 if local_window is None else int(local_window), out.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), error_latch.data_ptr(), stream)
    with torch.cuda.device(q.device):
        if decode_path:
            opts = Options()
            opts.decode_path = int(decode_path)
            st = lib.varlen_attn_fwd_device_ex(*args, ctypes.byref(opts))
        else:
            st = lib.varlen_attn_fwd_device(*args)
    _check(st)
    return out


# Bytes of the static scratch array behind varlen_attn_fwd_device_noalloc
# (VARLEN_NOALLOC_SCRATCH_BYTES in include/varlen_attn.h).
NOALLOC_SCRATCH_BYTES = 32 << 20


def varlen_attn_fwd_device_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_kv, num_heads: int, kv_num_heads=None,
                                   scale=None, is_causal: bool = False, softcap: float = 0.0, local_window=None,
                                   out=None, error_latch=None, stream=None):
    """varlen_attn_fwd_device without a workspace argument: the library's
    static scratch array (NOALLOC_SCRATCH_BYTES per GPU) holds the work list,
    so the call allocates nothing at all. Calls that overlap on one GPU share
    that array and race. Arguments as varlen_attn_fwd_device. Returns ``out``."""
    import torch
    lib = load_library()
    hq = int(num_heads)
    hkv = int(kv_num_heads) if kv_num_heads else hq
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors")
    code = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("Q, K, and V must use the same floating dtype")
    tq, d = _resolve(q, hq, "query")
    tkv, dk = _resolve(k, hkv, "key")
    tv, dv = _resolve(v, hkv, "value")
    if dk != d or tv != tkv:
        raise ValueError("key head size / token count must match query head size / value token count")
    if out is None:
        raise ValueError("out is required (the call allocates nothing)")
    if out.dtype != q.dtype or not out.is_contiguous() or out.numel() != tq * hq * dv or not out.is_cuda:
        raise ValueError("output must be a contiguous GPU tensor of the Q/K/V dtype with [total_q, num_heads, v_head_size] elements")
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
        if cu is None or not cu.is_cuda or cu.dtype != torch.int32 or not cu.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    if cu_seqlens_q.numel() != cu_seqlens_kv.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_kv lengths differ")
    if error_latch is None or not error_latch.is_cuda or error_latch.dtype != torch.int32:
        raise ValueError("error_latch must be an int32 GPU tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib.varlen_attn_fwd_device_noalloc(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_kv.data_ptr(),
            cu_seqlens_q.numel() - 1, tq, tkv, hq, hkv, d, dv, code, float(scale) if scale else 0.0,
            1 if is_causal else 0, float(softcap), -1 if local_window is None else int(local_window),
            out.data_ptr(), error_latch.data_ptr(), stream)
    _check(st)
    return out


def _gpu_int32(x, name, n=None):
    import torch
    if x is None or not x.is_cuda or x.dtype != torch.int32 or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    if n is not None and x.numel() != n:
        raise ValueError(f"{name} must have {n} elements, got {x.numel()}")


def _rows_of(x, width: int, name: str):
    """Rows and row stride (elements) of a [rows, >= width] view with unit inner stride."""
    if x.dim() == 3:
        if x.stride(2) != 1 or x.stride(1) != x.size(2):
            raise ValueError(f"{name} rows must be dense inside")
        if x.size(1) * x.size(2) != width:
            raise ValueError(f"{name} rows must hold {width} elements, got {x.size(1) * x.size(2)}")
        return x.size(0), x.stride(0)
    if x.dim() == 2:
        if x.stride(1) != 1 or x.size(1) != width:
            raise ValueError(f"{name} must be [rows, {width}] with unit inner stride")
        return x.size(0), x.stride(0)
    raise ValueError(f"{name} must be rank 2 or 3")


def kv_append_rope(q, k, v, k_cache, v_cache, cu_seqlens_q, cache_seqlens, num_heads: int, kv_num_heads=None,
                   cos=None, sin=None, position_ids=None, rotary_interleaved: bool = False, q_out=None,
                   kv_seqlens_out=None, error_latch=None, stream=None):
    """The step before decode over a fixed-capacity cache: rotary embedding of
    the new q/k rows and the append of k/v into the caches (one kernel, capture
    safe). q may be None (no query work); q_out defaults to q (in place).
    k/v/q may be strided row views (e.g. slices of a packed QKV buffer).
    Caches are [batch * capacity, Hkv, D] / [..., Dv]. Returns q_out."""
    import torch
    lib = load_library()
    hq = int(num_heads)
    hkv = int(kv_num_heads) if kv_num_heads else hq
    if k.dim() != 3 or v.dim() != 3:
        raise ValueError("k and v must be [rows, kv_heads, head_size] views")
    d, dv = k.size(2), v.size(2)
    code = _dtype_code(k)
    for name, t in (("v", v), ("k_cache", k_cache), ("v_cache", v_cache)) + ((("q", q),) if q is not None else ()):
        if t.dtype != k.dtype or not t.is_cuda:
            raise TypeError(f"{name} must be a GPU tensor of the key dtype")
    tq, ks = _rows_of(k, hkv * d, "k")
    tv, vs = _rows_of(v, hkv * dv, "v")
    if tv != tq:
        raise ValueError("k and v row counts differ")
    qs = 0
    if q is not None:
        tqq, qs = _rows_of(q, hq * d, "q")
        if tqq != tq:
            raise ValueError("q and k row counts differ")
        if q_out is None:
            q_out = q
        if not q_out.is_contiguous() or q_out.numel() != tq * hq * d or q_out.dtype != q.dtype:
            raise ValueError("q_out must be a dense [rows, num_heads, head_size] tensor")
    for name, t, w in (("k_cache", k_cache, hkv * d), ("v_cache", v_cache, hkv * dv)):
        if not t.is_contiguous() or t.numel() % w:
            raise ValueError(f"{name} must be a contiguous [batch * capacity, kv_heads, head_size] tensor")
    batch = cu_seqlens_q.numel() - 1
    cap = k_cache.numel() // (hkv * d)
    if batch < 1 or cap % batch or v_cache.numel() // (hkv * dv) != cap:
        raise ValueError("cache rows must be batch * capacity for both caches")
    cap //= batch
    _gpu_int32(cu_seqlens_q, "cu_seqlens_q")
    _gpu_int32(cache_seqlens, "cache_seqlens", batch)
    if kv_seqlens_out is not None:
        _gpu_int32(kv_seqlens_out, "kv_seqlens_out", batch)
    if error_latch is None:
        raise ValueError("error_latch is required")
    _gpu_int32(error_latch, "error_latch", 1)
    rdim, rows = 0, 0
    if cos is not None:
        if sin is None or cos.shape != sin.shape or cos.dim() != 2:
            raise ValueError("cos and sin must be equal [rows, rotary_dim / 2] tensors")
        if cos.dtype != torch.float32 or sin.dtype != torch.float32 or not (cos.is_contiguous() and sin.is_contiguous()):
            raise TypeError("cos and sin must be contiguous float32 GPU tensors")
        rows, rdim = cos.size(0), 2 * cos.size(1)
    if position_ids is not None and (position_ids.dtype != torch.int64 or not position_ids.is_contiguous()
                                     or position_ids.numel() != tq):
        raise ValueError("position_ids must be a contiguous int64 tensor with one entry per new row")
    if stream is None:
        stream = torch.cuda.current_stream(k.device).cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    with torch.cuda.device(k.device):
        st = lib.varlen_kv_append_rope(
            ptr(q), ptr(q_out), k.data_ptr(), v.data_ptr(), qs, ks, vs, k_cache.data_ptr(), v_cache.data_ptr(),
            cu_seqlens_q.data_ptr(), cache_seqlens.data_ptr(), ptr(kv_seqlens_out), ptr(cos), ptr(sin),
            ptr(position_ids), batch, tq, hq, hkv, d, dv, code, cap, rdim, rows, 1 if rotary_interleaved else 0,
            error_latch.data_ptr(), stream)
    _check(st)
    return q_out


def varlen_attn_fwd_kvcache(q, k_cache, v_cache, cu_seqlens_q, kv_seqlens, num_heads: int, kv_num_heads=None,
                            scale=None, is_causal: bool = False, softcap: float = 0.0, local_window=None,
                            out=None, workspace=None, error_latch=None, stream=None):
    """Capture-safe attention of packed new rows over a fixed-capacity cache
    ([batch * capacity, Hkv, D]): sequence b reads cache rows
    [b * capacity, b * capacity + kv_seqlens[b]). Workspace size:
    device_workspace_bytes(batch, total_q, batch * capacity, ...)."""
    lib = load_library()
    hq = int(num_heads)
    hkv = int(kv_num_heads) if kv_num_heads else hq
    if not (q.is_cuda and k_cache.is_cuda and v_cache.is_cuda):
        raise ValueError("q and the caches must be GPU tensors")
    code = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("Q and the caches must use the same floating dtype")
    tq, d = _resolve(q, hq, "query")
    rows, dk = _resolve(k_cache, hkv, "key cache")
    rows_v, dv = _resolve(v_cache, hkv, "value cache")
    if dk != d or rows_v != rows:
        raise ValueError("cache head size / rows do not match")
    batch = cu_seqlens_q.numel() - 1
    if batch < 1 or rows % batch:
        raise ValueError("cache rows must be batch * capacity")
    _gpu_int32(cu_seqlens_q, "cu_seqlens_q")
    _gpu_int32(kv_seqlens, "kv_seqlens", batch)
    if out is None:
        raise ValueError("out is required (the call allocates nothing)")
    if out.dtype != q.dtype or not out.is_contiguous() or out.numel() != tq * hq * dv or not out.is_cuda:
        raise ValueError("output must be a contiguous GPU tensor of the Q dtype with [total_q, num_heads, v_head_size] elements")
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    if error_latch is None:
        raise ValueError("error_latch is required")
    _gpu_int32(error_latch, "error_latch", 1)
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib.varlen_attn_fwd_kvcache(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), cu_seqlens_q.data_ptr(), kv_seqlens.data_ptr(),
            batch, tq, rows // batch, hq, hkv, d, dv, code, float(scale) if scale else 0.0, 1 if is_causal else 0,
            float(softcap), -1 if local_window is None else int(local_window), out.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), error_latch.data_ptr(), stream)
    _check(st)
    return out


def plan(cu_seqlens_q, cu_seqlens_kv, num_heads: int, kv_num_heads=None, head_dim: int = 128,
         v_head_dim: int = 0, dtype: str = "bf16", scale: float = 0.0, is_causal: bool = False,
         softcap: float = 0.0, with_items: bool = False, decode_path: int = 0, decode_chunk: int = 0,
         prefill_kv_chunk: int = 0, local_window=None):
    """Run the host scheduler alone (no GPU needed). Returns (stats dict, items or None);
    items is an int32 array [n_items, 16] (see varlen_attn_plan in the header)."""
    import numpy as np
    lib = load_library()
    cq, ckv = _host_cu(cu_seqlens_q), _host_cu(cu_seqlens_kv)
    if cq.size != ckv.size:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv lengths differ")
    stats = PlanStats()
    opts = _options(decode_path, decode_chunk, prefill_kv_chunk, local_window)
    args = (cq.ctypes.data, ckv.ctypes.data, cq.size - 1, int(cq[-1]) if cq.size else 0,
            int(ckv[-1]) if ckv.size else 0, int(num_heads), int(kv_num_heads or 0), int(head_dim),
            int(v_head_dim), DTYPE_CODES[dtype], float(scale), 1 if is_causal else 0, float(softcap),
            ctypes.byref(opts), ctypes.byref(stats))
    _check(lib.varlen_attn_plan(*args, None, 0))
    items = None
    if with_items:
        n = stats.n_prefill_items + stats.n_decode_items + stats.n_combine_items
        items = np.zeros((max(n, 1), ITEM_INTS), dtype=np.int32)
        _check(lib.varlen_attn_plan(*args, items.ctypes.data, items.size))
        items = items[:n]
    return stats.as_dict(), items


def valid_pairs(cu_seqlens_q, cu_seqlens_kv, is_causal: bool, local_window=None) -> int:
    """Visible (query row, key) pairs; attention FLOPs are 2 * pairs * Hq * (D + Dv)."""
    lib = load_library()
    cq, ckv = _host_cu(cu_seqlens_q), _host_cu(cu_seqlens_kv)
    if local_window is None:
        r = lib.varlen_attn_valid_pairs(cq.ctypes.data, ckv.ctypes.data, cq.size - 1, 1 if is_causal else 0)
    else:
        r = lib.varlen_attn_valid_pairs_window(cq.ctypes.data, ckv.ctypes.data, cq.size - 1,
                                               1 if is_causal else 0, int(local_window))
    if r < 0:
        raise ValueError("invalid cu_seqlens arrays")
    return int(r)


def profile_enable(on: bool = True):
    """Start (clearing totals) or stop recording HIP events around each kernel."""
    _check(load_library().varlen_attn_profile_enable(1 if on else 0))


def profile_read():
    """Per-kernel totals since the last enable: {kind: (total_ms, launches, items)}."""
    t = ProfileTotals()
    _check(load_library().varlen_attn_profile_read(ctypes.byref(t)))
    return {k: (t.total_ms[i], t.launches[i], t.items[i]) for i, k in enumerate(PROFILE_KINDS)}


def release():
    """Free the library's per-device workspaces."""
    _check(load_library().varlen_attn_release())


def version() -> str:
    return load_library().varlen_attn_version().decode()
