// Shared definitions of the gfx950 packed varlen attention kernels and their
// host launcher: the work-item format the scheduler emits, the parameter block
// every kernel receives, and small device helpers (MFMA operand types, type
// conversion, cross-lane exchange).
#pragma once

#include <utility>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pva {

// One unit of scheduled work. Every field is a plain int32 so the host can
// build the list without device help and the kernels read it with scalar
// loads. Sequence-relative indices: q_row_begin, kv_begin, kv_end.
struct WorkItem {
  int32_t kind;          // ItemKind
  int32_t seq;           // sequence b
  int32_t q_row_begin;   // first query row of the tile (local to the sequence)
  int32_t q_rows;        // rows in the tile
  int32_t head_begin;    // first query head
  int32_t heads;         // query heads (all in one kv group)
  int32_t kv_begin;      // keys [kv_begin, kv_end) (local)
  int32_t kv_end;
  int32_t partial_base;  // -1: write out directly; else first fp32 partial row
  int32_t n_splits;      // splits of this tile (combine: how many to merge)
  int32_t q_token0;      // cu_seqlens_q[seq]
  int32_t kv_token0;     // cu_seqlens_kv[seq]
  int32_t len_q;         // L_q
  int32_t len_kv;        // L_kv
  int32_t split;         // index of this split in [0, n_splits)
  int32_t kv_head;       // kv head of the item's query heads: head_begin / group
};
static_assert(sizeof(WorkItem) == 64, "work item is 16 int32");

enum ItemKind : int32_t {
  kPrefillMfma = 0,
  kPrefillF32 = 1,
  kDecode = 2,
  kCombine = 3,
};

enum DType : int32_t { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Partial rows of split work: partial index of (split s, tile row r, head hh)
// is partial_base + (s * q_rows + r) * heads + hh. part_o holds the split's
// own normalised output (dv floats), part_lse its log2-sum-exp in the
// kernels' log2 score units (-inf when the split saw no visible key).
__host__ __device__ inline int64_t partial_index(const WorkItem& it, int split, int row, int hh) {
  return (int64_t)it.partial_base + ((int64_t)split * it.q_rows + row) * it.heads + hh;
}

// Device-built work list (the device scheduler, sched.hip): where it writes
// the lists, the per-sequence list offsets, the item counts, and the bounds
// the launch grids were sized for.
enum DeviceHeader : int32_t {
  kHdrPrefill = 0,   // items in the prefill list
  kHdrDecode = 1,    // items in the split-KV decode list
  kHdrCombine = 2,   // items in the combine list
  kHdrPartials = 3,  // partial rows used
  kHdrChunk = 4,     // split-KV chunk (keys)
  kHdrInts = 64,     // header size in int32 (256 bytes)
};
// Bits of the caller's error latch.
enum LatchBits : int32_t {
  kLatchCuQStart = 1,     // cu_seqlens_q[0] != 0
  kLatchCuQOrder = 2,     // cu_seqlens_q decreases
  kLatchCuQTotal = 4,     // cu_seqlens_q[B] > the query buffer's rows
  kLatchCuKvStart = 8,    // cu_seqlens_kv[0] != 0
  kLatchCuKvOrder = 16,   // cu_seqlens_kv decreases
  kLatchCuKvTotal = 32,   // cu_seqlens_kv[B] > the key/value buffers' rows
  kLatchCapacity = 64,    // a list outgrew its bound (not expected)
  kLatchPast = 128,       // cache step: a cached length is negative
  kLatchOverflow = 256,   // cache step: cached + new rows exceed the capacity
  kLatchPosition = 512,   // cache step: a rotated row's position has no table row
  kLatchKvLen = 1024,     // attention over a cache: a length is negative or exceeds the capacity
};
struct DevicePlan {
  int32_t batch, hq, group;  // group = hq / hkv
  int32_t nh, rows_per_item, prefill_kind;  // prefill items: nh heads x rows_per_item rows
  int32_t nh_dec, use_decode;               // decode items: nh_dec heads, L_q == 1 sequences
  int32_t causal, window;
  int32_t cap_q, cap_kv;                    // rows of the q/out and k/v buffers
  // Fixed-capacity cache: non-null kv_len [batch] gives L_kv of each
  // sequence, whose keys start at row b * kv_capacity; cu_kv is not read.
  const int32_t* kv_len;
  int32_t kv_capacity;
  int64_t cap_prefill, cap_decode, cap_combine, cap_partials;
  int32_t* header;
  // [batch + 1] each, used when the batch is too large for the scheduler's LDS
  int32_t *seq_q, *seq_kv, *seq_pre, *seq_decf, *seq_decp, *seq_cmb, *seq_part;
  WorkItem *prefill, *decode, *combine;
};

// The cache step: rotary embedding of new query/key rows and their append
// into a fixed-capacity cache (one thread per rotary pair or copied pair).
struct RopeParams {
  const void* q;      // [rows, q_stride] new query rows, or null (no query work)
  void* q_out;        // [total_q, hq, d]; may equal q when q_stride == hq * d
  const void* k;      // new key rows, k_stride elements apart
  const void* v;      // new value rows, v_stride elements apart
  void* k_cache;      // [batch * capacity, hkv, d]
  void* v_cache;      // [batch * capacity, hkv, dv]
  const int32_t* cu_q;
  const int32_t* past;
  int32_t* kv_len_out;     // [batch] or null
  const float* cos;        // [rows, rot_half] or null (no rotation)
  const float* sin;
  const int64_t* pos_ids;  // [total_q] or null (position past + i)
  int32_t* latch;
  int64_t q_stride, k_stride, v_stride;
  int32_t batch, total_q, hq, hkv, d, dv, capacity, rot_half, rows, interleaved;
  int32_t vec;                          // 1: 16-byte pieces; 0: one pair per unit
  int32_t units_q, units_k, units_row;  // units of one new row (q, then k, then v)
  int32_t rot_units, head_units_qk, head_units_v;  // 16-byte pieces: turned per q/k head, all per head
  int32_t blocks_per_row, row_blocks;   // row workgroups; then the per-sequence workgroups
};

struct Params {
  // Items of the launch: with a device-built list the grid is an upper bound
  // and workgroups at or past *item_count return at once; null otherwise.
  const int32_t* item_count;
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* part_o;
  float* part_lse;
  int32_t hq, hkv, group, d, dv;
  int32_t causal;
  int32_t window;  // > 0: row i sees only keys j >= i + L_kv - L_q + 1 - window
  int32_t softcap_on;
  // Scores are worked in log2 units: y = s * score_log2 without softcap, and
  // y = cap_log2 * tanh(s * scale / |softcap|) with it, where the tanh is
  // formed as 1 - 2 / (exp2(s * tanh_log2) + 1).
  float score_log2;  // scale * log2(e)
  float cap_log2;    // |softcap| * log2(e)
  float tanh_log2;   // 2 * scale / |softcap| * log2(e)
  float scale;       // the effective scale (fp32 path)
  float softcap;     // |softcap| (fp32 path)
  // Device path: a prefill launch also carries the combine items. Its
  // workgroups from prefill_grid on run combine item blockIdx.x - prefill_grid
  // while that is below *combine_count; null combine_items: none.
  const WorkItem* combine_items;
  const int32_t* combine_count;
  int32_t prefill_grid;
};

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ninf() { return -__builtin_inff(); }

// Two fp32 values -> two 16-bit values packed in one dword, round to nearest
// even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 on gfx950).
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  f32x2_t x = {a, b};
  if constexpr (BF16) {
    bf16x2_t y = __builtin_convertvector(x, bf16x2_t);
    return __builtin_bit_cast(uint32_t, y);
  } else {
    f16x2_t y = __builtin_convertvector(x, f16x2_t);
    return __builtin_bit_cast(uint32_t, y);
  }
}

// 32x32x16 MFMA with fp32 accumulators on 8 packed 16-bit values per lane.
template <bool BF16>
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// 16x16x32 MFMA with fp32 accumulators on 8 packed 16-bit values per lane.
template <bool BF16>
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float xor_lanes(float x, int mask) { return __shfl_xor(x, mask, 64); }

// The value of lane l ^ 32 (v_permlane32_swap exchanges the two wave halves;
// each lane keeps its own value in one result and receives its partner's in
// the other).
__device__ __forceinline__ float partner32(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}

// max / sum of a lane's value and its partner's (lane l ^ 32); both lanes of
// a pair get bit-identical results.
__device__ __forceinline__ float max_with_partner32(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float sum_with_partner32(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Sum of the two 16-bit values packed in w, in fp32 (v_dot2 against 1.0).
template <bool BF16>
__device__ __forceinline__ float sum2(uint32_t w, float acc) {
  if constexpr (BF16) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
  } else {
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), one, acc, false);
  }
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4 in its scalar-base form): lane i reads
// sbase + voff_i and its bytes land at M0 + 16*i, with M0 = lds_base + OFF
// (wave-uniform; the constant is folded into the instruction that sets M0,
// so a run of loads into one buffer needs one scalar register, not one per
// load). gfx950 reads a vector memory instruction's scalar operands at
// issue, so the base may be overwritten right after.
// Issued as inline assembly, the load is not among the outstanding
// vector-memory loads the compiler counts, so it adds no vmcnt wait of its
// own before later LDS reads (it cannot tell which LDS bytes such a load
// writes and would otherwise wait after every one). Whoever issues it orders
// it explicitly: an s_waitcnt vmcnt covering the load, then a workgroup
// barrier, before any wave reads the bytes. The compiler's own vmcnt waits
// stay correct (loads retire in order, so an extra load issued in between
// only makes them wait longer).
template <uint32_t OFF>
__device__ __forceinline__ void lds_dma16_async_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base), "i"(OFF)
      : "memory", "m0", "scc");
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, each i a constant
// expression in f.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// LDS byte address of a pointer into a __shared__ array (wave-uniform when
// the pointer is).
__device__ __forceinline__ uint32_t lds_addr32(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p));
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, lane i receives element i % 4 of the 4-element rows addressed by
// lanes 4j + i/4, j = 0..3: when lanes 4j..4j+3 address consecutive
// 4-element pieces of row j of a [rows][cols] 16-bit array, lane i gets
// column i of rows 0..3.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}
#endif

}  // namespace pva
