// The input-side step of decode over a fixed-capacity KV cache: rotary
// embedding of the new query and key rows, and the append of the new key and
// value rows into the cache, in one launch (page
// src/kernels/group_query_attention.rs: the rotary kernel gqa_rope_bnsh, the
// cache kernels gqa_build_cache / gqa_append_cache and their fusion
// gqa_fuse_decode_prep; page src/kernels/attention.rs, the fixed-capacity,
// fixed-slot append test).
//
// Layout: the new rows are packed as the attention's rows (cu_seqlens_q);
// the cache keeps the attention's row format, [batch * capacity, Hkv, D],
// sequence b owning rows [b * capacity, (b + 1) * capacity), so the
// attention kernels read it directly.
//
// Rotation: pair m < R/2 of a head vector (dims 2m, 2m+1 interleaved, or m,
// m + R/2 half-split) turns by the table angle at the row's position:
// (a, b) -> (a*c - b*s, a*s + b*c), worked in fp32 and rounded to nearest
// even into the storage type. Dims R.. pass unchanged.
//
// Work: HBM-bound streaming. Every new row is split into "pair units" (the
// two dims of a rotary pair, or two neighbouring dims of a copied part): all
// query heads, then all key heads, then all value heads. A workgroup of 256
// threads takes 1024 consecutive units of one row, consecutive threads taking
// consecutive pairs, so every wave reads and writes contiguous runs; the
// row's sequence, position and cache slot are found once per workgroup. A
// few workgroups past the rows write kv_len_out and check every sequence.
#include "common.h"

namespace pva {

namespace {

constexpr int kThreads = 256;
constexpr int kUnitsPerThread = 4;

template <typename T>
__device__ __forceinline__ float load_f(const T* p) {
  return static_cast<float>(*p);
}

template <typename T>
__device__ __forceinline__ void store_f(T* p, float x) {
  *p = static_cast<T>(x);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_append_kernel(RopeParams p) {
  __shared__ int32_t s_ok;
  __shared__ int32_t s_pos;
  __shared__ int64_t s_slot;
  const int tid = threadIdx.x;
  const int32_t blk = blockIdx.x;

  if (blk >= p.row_blocks) {
    // per-sequence checks and the attention's key counts
    const int32_t b = (blk - p.row_blocks) * kThreads + tid;
    int32_t err = 0;
    if (b == 0) {
      if (p.cu_q[0] != 0) err |= kLatchCuQStart;
      if (p.cu_q[p.batch] > p.total_q) err |= kLatchCuQTotal;
    }
    if (b < p.batch) {
      const int64_t lq = (int64_t)p.cu_q[b + 1] - p.cu_q[b];
      const int64_t past = p.past[b];
      if (lq < 0) err |= kLatchCuQOrder;
      if (past < 0) err |= kLatchPast;
      if (past + lq > p.capacity) err |= kLatchOverflow;
      if (p.kv_len_out) p.kv_len_out[b] = (int32_t)max((int64_t)INT32_MIN, min((int64_t)INT32_MAX, past + lq));
    }
    if (err) atomicOr(p.latch, err);
    return;
  }

  const int32_t t = blk / p.blocks_per_row;
  const int32_t part = blk - t * p.blocks_per_row;
  if (tid == 0) {
    int32_t ok = __hip_atomic_load(p.latch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
    int32_t err = 0;
    // the sequence of row t: the largest b with cu_q[b] <= t
    int32_t lo = 0, hi = p.batch;
    while (hi - lo > 1) {
      const int32_t mid = lo + (hi - lo) / 2;
      if (p.cu_q[mid] <= t) lo = mid; else hi = mid;
    }
    const int32_t c0 = p.cu_q[lo], c1 = p.cu_q[lo + 1];
    int64_t pos = 0, slot = 0;
    if (t >= p.cu_q[p.batch] && p.cu_q[p.batch] >= 0) {
      ok = 0;  // a spare row of the buffers, not a new row
    } else if (!(c0 <= t && t < c1)) {
      ok = 0;
      err |= kLatchCuQOrder;
    } else {
      const int32_t i = t - c0;
      const int64_t past = p.past[lo];
      if (past < 0 || past + (c1 - c0) > p.capacity) ok = 0;  // latched by the per-sequence workgroups
      pos = p.pos_ids ? p.pos_ids[t] : past + i;
      if (p.cos && (pos < 0 || pos >= p.rows)) {
        ok = 0;
        err |= kLatchPosition;
      }
      slot = (int64_t)lo * p.capacity + past + i;
    }
    if (err) atomicOr(p.latch, err);
    s_ok = ok;
    s_pos = (int32_t)pos;
    s_slot = slot;
  }
  __syncthreads();
  if (!s_ok) return;
  const int32_t pos = s_pos;
  const int64_t slot = s_slot;
  const int32_t hd = p.d / 2;    // pair units per query/key head
  const int32_t hdv = p.dv / 2;  // pair units per value head
  const int32_t rh = p.rot_half;

#pragma unroll
  for (int r = 0; r < kUnitsPerThread; ++r) {
    int32_t u = (part * kUnitsPerThread + r) * kThreads + tid;
    if (u >= p.units_row) break;
    const T* src;
    T* dst;
    int32_t m;
    bool turn = false;
    if (u < p.units_q + p.units_k) {
      const bool is_q = u < p.units_q;
      if (!is_q) u -= p.units_q;
      const int32_t h = u / hd;
      m = u - h * hd;
      if (is_q) {
        src = static_cast<const T*>(p.q) + (int64_t)t * p.q_stride + (int64_t)h * p.d;
        dst = static_cast<T*>(p.q_out) + ((int64_t)t * p.hq + h) * p.d;
      } else {
        src = static_cast<const T*>(p.k) + (int64_t)t * p.k_stride + (int64_t)h * p.d;
        dst = static_cast<T*>(p.k_cache) + (slot * p.hkv + h) * p.d;
      }
      turn = p.cos != nullptr && m < rh;
    } else {
      u -= p.units_q + p.units_k;
      const int32_t h = u / hdv;
      m = u - h * hdv;
      src = static_cast<const T*>(p.v) + (int64_t)t * p.v_stride + (int64_t)h * p.dv;
      dst = static_cast<T*>(p.v_cache) + (slot * p.hkv + h) * p.dv;
    }
    if (turn) {
      const int32_t d0 = p.interleaved ? 2 * m : m;
      const int32_t d1 = p.interleaved ? 2 * m + 1 : m + rh;
      const float a = load_f(src + d0);
      const float b = load_f(src + d1);
      const float c = p.cos[(int64_t)pos * rh + m];
      const float s = p.sin[(int64_t)pos * rh + m];
      store_f(dst + d0, a * c - b * s);
      store_f(dst + d1, a * s + b * c);
    } else {
      // copied pair: the two dims 2m, 2m+1 (past the rotary dims for q/k)
      const int32_t d0 = 2 * m;
      const T a = src[d0];
      const T b = src[d0 + 1];
      dst[d0] = a;
      dst[d0 + 1] = b;
    }
  }
}

}  // namespace

hipError_t launch_rope_append(const RopeParams& p, int dtype, hipStream_t s) {
  const int64_t seq_blocks = (p.batch + kThreads - 1) / kThreads;
  const int64_t grid = (int64_t)p.row_blocks + seq_blocks;
  if (grid <= 0 || grid > INT32_MAX) return hipErrorInvalidValue;
  switch (dtype) {
    case kBF16:
      hipLaunchKernelGGL(rope_append_kernel<__bf16>, dim3((uint32_t)grid), dim3(kThreads), 0, s, p);
      break;
    case kF16:
      hipLaunchKernelGGL(rope_append_kernel<_Float16>, dim3((uint32_t)grid), dim3(kThreads), 0, s, p);
      break;
    case kF32:
      hipLaunchKernelGGL(rope_append_kernel<float>, dim3((uint32_t)grid), dim3(kThreads), 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int rope_units_per_block() { return kThreads * kUnitsPerThread; }

}  // namespace pva
