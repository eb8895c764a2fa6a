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
// Work: HBM-bound streaming. A new row is cut into units: all query heads,
// then all key heads, then all value heads, each head into the units of its
// dims. The 16-byte kernel (every row, stride and head size a multiple of 16
// bytes, and the rotary dims splitting into 16-byte pieces) gives each
// thread two 16-byte pieces, each a piece of copied dims, an interleaved piece
// holding whole pairs, or (half-split) a piece of the first half together
// with its partner piece R/2 dims on; the 2-element kernel handles every
// other shape one pair per thread. A workgroup covers consecutive units of
// one row; it issues its loads before it looks up the row's sequence
// (binary search over cu_seqlens_q staged in LDS), so the lookup hides under
// the load latency. A few workgroups past the rows write kv_len_out and
// check every sequence.
#include "common.h"

namespace pva {

namespace {

constexpr int kThreads = 256;
constexpr int kVecUnitsPerThread = 2;
constexpr int kScalarUnitsPerThread = 4;
constexpr int kLdsCu = 2048;  // batches of up to kLdsCu - 1 search cu_seqlens_q in LDS

// Workgroups past the row workgroups: per-sequence checks and kv_len_out.
__device__ void sequence_pass(const RopeParams& p, int32_t seq_block) {
  const int32_t b = seq_block * kThreads + (int32_t)threadIdx.x;
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
}

struct RowSlot {
  int32_t ok;   // the row is a valid new row and the latch was clear
  int32_t pos;  // its rotary position
  int64_t slot; // its cache row
};

// The sequence, position and cache slot of new row t, for the whole
// workgroup (every thread must call it). Raises the row's own latch bits.
// Every global read it needs is issued before its first barrier (cu_seqlens_q
// and the cached lengths staged in LDS, the latch, the position id), so the
// lookup costs one round trip to memory.
__device__ RowSlot row_setup(const RopeParams& p, int32_t t) {
  __shared__ int32_t s_cu[kLdsCu];
  __shared__ int32_t s_past[kLdsCu];
  __shared__ RowSlot s_row;
  const int tid = threadIdx.x;
  const bool in_lds = p.batch + 1 <= kLdsCu;
  if (in_lds) {
    for (int32_t b = tid; b <= p.batch; b += kThreads) {
      s_cu[b] = p.cu_q[b];
      if (b < p.batch) s_past[b] = p.past[b];
    }
  }
  int32_t latch0 = 0;
  int64_t pid = 0;
  if (tid == 0) {
    latch0 = __hip_atomic_load(p.latch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.pos_ids) pid = p.pos_ids[t];
  }
  __syncthreads();
  if (tid == 0) {
    const int32_t* cu = in_lds ? s_cu : p.cu_q;
    RowSlot r = {latch0 == 0, 0, 0};
    int32_t err = 0;
    // the largest b with cu[b] <= t
    int32_t lo = 0, hi = p.batch;
    while (hi - lo > 1) {
      const int32_t mid = lo + (hi - lo) / 2;
      if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    const int32_t c0 = cu[lo], c1 = cu[lo + 1], cb = cu[p.batch];
    if (t >= cb && cb >= 0) {
      r.ok = 0;  // a spare row of the buffers, not a new row
    } else if (!(c0 <= t && t < c1)) {
      r.ok = 0;
      err |= kLatchCuQOrder;
    } else {
      const int32_t i = t - c0;
      const int64_t past = in_lds ? s_past[lo] : p.past[lo];
      if (past < 0 || past + (c1 - c0) > p.capacity) r.ok = 0;  // latched by sequence_pass
      const int64_t pos = p.pos_ids ? pid : past + i;
      if (p.cos && (pos < 0 || pos >= p.rows)) {
        r.ok = 0;
        err |= kLatchPosition;
      }
      r.pos = (int32_t)pos;
      r.slot = (int64_t)lo * p.capacity + past + i;
    }
    if (err) atomicOr(p.latch, err);
    s_row = r;
  }
  __syncthreads();
  return s_row;
}

// ---- 16-byte pieces ---------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void rope_append_vec_kernel(RopeParams p) {
  constexpr int VW = 16 / sizeof(T);  // elements per piece
  typedef T tv_t __attribute__((ext_vector_type(VW)));
  typedef float fv_t __attribute__((ext_vector_type(VW)));
  const int32_t blk = blockIdx.x;
  if (blk >= p.row_blocks) {
    sequence_pass(p, blk - p.row_blocks);
    return;
  }
  const int32_t t = blk / p.blocks_per_row;
  const int32_t part = blk - t * p.blocks_per_row;

  // Decode each unit: where its piece(s) come from and go to; load them.
  struct Unit {
    int32_t region;  // 0 query, 1 key, 2 value
    int32_t h, d0;
    bool live, turn, half;
  };
  Unit un[kVecUnitsPerThread];
  tv_t a[kVecUnitsPerThread], b[kVecUnitsPerThread];
#pragma unroll
  for (int k = 0; k < kVecUnitsPerThread; ++k) {
    int32_t u = (part * kVecUnitsPerThread + k) * kThreads + (int32_t)threadIdx.x;
    Unit& x = un[k];
    x.live = u < p.units_row;
    x.region = 2;
    if (u < p.units_q) {
      x.region = 0;
    } else if (u < p.units_q + p.units_k) {
      x.region = 1;
      u -= p.units_q;
    } else {
      u -= p.units_q + p.units_k;
    }
    const int32_t per_head = x.region == 2 ? p.head_units_v : p.head_units_qk;
    x.h = u / per_head;
    const int32_t j = u - x.h * per_head;
    x.turn = x.region != 2 && j < p.rot_units;
    x.half = x.turn && !p.interleaved;
    // first dim of the (first) piece; the partner piece is rot_half dims on
    x.d0 = (x.region == 2 || x.turn) ? j * VW : 2 * p.rot_half + (j - p.rot_units) * VW;
    const T* src;
    if (x.region == 0) src = static_cast<const T*>(p.q) + (int64_t)t * p.q_stride + (int64_t)x.h * p.d;
    else if (x.region == 1) src = static_cast<const T*>(p.k) + (int64_t)t * p.k_stride + (int64_t)x.h * p.d;
    else src = static_cast<const T*>(p.v) + (int64_t)t * p.v_stride + (int64_t)x.h * p.dv;
    a[k] = tv_t{};
    b[k] = tv_t{};
    if (x.live) {
      a[k] = *reinterpret_cast<const tv_t*>(src + x.d0);
      if (x.half) b[k] = *reinterpret_cast<const tv_t*>(src + x.d0 + p.rot_half);
    }
  }

  const RowSlot r = row_setup(p, t);
  if (!r.ok) return;
  const float* cs = p.cos ? p.cos + (int64_t)r.pos * p.rot_half : nullptr;
  const float* sn = p.sin ? p.sin + (int64_t)r.pos * p.rot_half : nullptr;
#pragma unroll
  for (int k = 0; k < kVecUnitsPerThread; ++k) {
    const Unit& x = un[k];
    if (!x.live) continue;
    T* dst;
    if (x.region == 0) dst = static_cast<T*>(p.q_out) + ((int64_t)t * p.hq + x.h) * p.d;
    else if (x.region == 1) dst = static_cast<T*>(p.k_cache) + (r.slot * p.hkv + x.h) * p.d;
    else dst = static_cast<T*>(p.v_cache) + (r.slot * p.hkv + x.h) * p.dv;
    if (!x.turn) {
      *reinterpret_cast<tv_t*>(dst + x.d0) = a[k];
      continue;
    }
    const fv_t xa = __builtin_convertvector(a[k], fv_t);
    if (x.half) {
      // pair e: (a[e], b[e]) with table entry d0 + e
      const fv_t xb = __builtin_convertvector(b[k], fv_t);
      fv_t c, s;
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        c[e] = cs[x.d0 + e];
        s[e] = sn[x.d0 + e];
      }
      const fv_t oa = xa * c - xb * s;
      const fv_t ob = xa * s + xb * c;
      *reinterpret_cast<tv_t*>(dst + x.d0) = __builtin_convertvector(oa, tv_t);
      *reinterpret_cast<tv_t*>(dst + x.d0 + p.rot_half) = __builtin_convertvector(ob, tv_t);
    } else {
      // pairs (a[2e], a[2e+1]) with table entry d0/2 + e
      fv_t o;
#pragma unroll
      for (int e = 0; e < VW / 2; ++e) {
        const float c = cs[x.d0 / 2 + e];
        const float s = sn[x.d0 / 2 + e];
        o[2 * e] = xa[2 * e] * c - xa[2 * e + 1] * s;
        o[2 * e + 1] = xa[2 * e] * s + xa[2 * e + 1] * c;
      }
      *reinterpret_cast<tv_t*>(dst + x.d0) = __builtin_convertvector(o, tv_t);
    }
  }
}

// ---- one pair per thread (any even head size and rotary dim) ------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void rope_append_pair_kernel(RopeParams p) {
  const int32_t blk = blockIdx.x;
  if (blk >= p.row_blocks) {
    sequence_pass(p, blk - p.row_blocks);
    return;
  }
  const int32_t t = blk / p.blocks_per_row;
  const int32_t part = blk - t * p.blocks_per_row;
  const RowSlot r = row_setup(p, t);
  if (!r.ok) return;
  const int32_t hd = p.d / 2;    // pair units per query/key head
  const int32_t hdv = p.dv / 2;  // pair units per value head
  const int32_t rh = p.rot_half;

#pragma unroll
  for (int k = 0; k < kScalarUnitsPerThread; ++k) {
    int32_t u = (part * kScalarUnitsPerThread + k) * kThreads + (int32_t)threadIdx.x;
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
        dst = static_cast<T*>(p.k_cache) + (r.slot * p.hkv + h) * p.d;
      }
      turn = p.cos != nullptr && m < rh;
    } else {
      u -= p.units_q + p.units_k;
      const int32_t h = u / hdv;
      m = u - h * hdv;
      src = static_cast<const T*>(p.v) + (int64_t)t * p.v_stride + (int64_t)h * p.dv;
      dst = static_cast<T*>(p.v_cache) + (r.slot * p.hkv + h) * p.dv;
    }
    if (turn) {
      const int32_t d0 = p.interleaved ? 2 * m : m;
      const int32_t d1 = p.interleaved ? 2 * m + 1 : m + rh;
      const float a = static_cast<float>(src[d0]);
      const float b = static_cast<float>(src[d1]);
      const float c = p.cos[(int64_t)r.pos * rh + m];
      const float s = p.sin[(int64_t)r.pos * rh + m];
      dst[d0] = static_cast<T>(a * c - b * s);
      dst[d1] = static_cast<T>(a * s + b * c);
    } else {
      // copied pair: dims 2m, 2m+1 (past the rotary dims for q/k)
      const T a = src[2 * m];
      const T b = src[2 * m + 1];
      dst[2 * m] = a;
      dst[2 * m + 1] = b;
    }
  }
}

template <typename T>
hipError_t launch_t(const RopeParams& p, hipStream_t s, uint32_t grid) {
  if (p.vec) hipLaunchKernelGGL(rope_append_vec_kernel<T>, dim3(grid), dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(rope_append_pair_kernel<T>, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Units of one workgroup: one 16-byte piece per thread, or
// kScalarUnitsPerThread pairs per thread.
int rope_units_per_block(int vec) { return kThreads * (vec ? kVecUnitsPerThread : kScalarUnitsPerThread); }

hipError_t launch_rope_append(const RopeParams& p, int dtype, hipStream_t s) {
  const int64_t seq_blocks = (p.batch + kThreads - 1) / kThreads;
  const int64_t grid = (int64_t)p.row_blocks + seq_blocks;
  if (grid <= 0 || grid > INT32_MAX) return hipErrorInvalidValue;
  switch (dtype) {
    case kBF16: return launch_t<__bf16>(p, s, (uint32_t)grid);
    case kF16: return launch_t<_Float16>(p, s, (uint32_t)grid);
    case kF32: return launch_t<float>(p, s, (uint32_t)grid);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pva
