// Device-side work scheduler: the work list of a call built on the GPU from
// device cu_seqlens, so that a call needs no host copy of the cu arrays, no
// synchronisation and no host-to-device upload, and can be captured in a
// HIP graph and replayed with new lengths.
//
// It emits the same items as the host scheduler (sequence b, a block of query
// rows, a group of query heads of one kv head, a key range) and validates the
// cu arrays on the device. A violation is OR-ed into a caller-owned error
// word (a latch: once set, every later call schedules nothing until the
// caller clears it), after the manner of the metadata-prep kernel of the GQA
// op (page src/kernels/group_query_attention.rs, gqa_prepare_metadata and
// its capture-error bit flags). The cu array rules are the packed op's
// (page src/kernels/packed_varlen_attention.rs, execute(): cumulative arrays
// start at 0 and never decrease), with the packed totals read as buffer
// capacities: cu[B] may not exceed them.
//
// One workgroup of 1024 threads:
//   1. every thread validates and counts the items of its sequences; the
//      split-KV chunk needs the total decode key count, so that is reduced
//      first;
//   2. one exclusive scan over the sequences (five counts at once) gives each
//      sequence's first item in the prefill list, in the two parts of the
//      decode list, in the combine list, and its first partial row; the
//      offsets and the cu arrays stay in LDS when the batch fits (else in the
//      workspace);
//   3. every thread writes items k = tid, tid + 1024, ..., finding the
//      sequence of item k by binary search over those offsets.
// With a fixed-capacity KV cache (the attention that follows the cache step)
// the keys of sequence b are rows [b * capacity, b * capacity + L_kv[b]) and
// L_kv comes from a device array instead of cu_seqlens_kv; each length is
// checked against the capacity.
// The prefill list takes the host scheduler's order: sequences by their
// longest item (a bitonic sort in LDS; sequence order for batches too large
// for it), each sequence's row blocks from the last to the first, head
// groups innermost. The decode list holds every full-chunk split first and
// the shorter last splits after them, longest first, so that the last items
// handed to the GPU are the short ones.
#include "common.h"

namespace pva {

namespace {

constexpr int kThreads = 1024;
constexpr int kLdsSeq = 2048;  // batches of up to kLdsSeq - 1 keep their offsets in LDS

__device__ int32_t visible_end_dev(int32_t lq, int32_t lkv, int32_t r0, int32_t rows, int32_t causal) {
  if (!causal) return lkv;
  const int64_t e = (int64_t)r0 + rows - 1 + (lkv - lq) + 1;
  return (int32_t)min((int64_t)lkv, max((int64_t)0, e));
}

__device__ int32_t visible_begin_dev(int32_t lq, int32_t lkv, int32_t r0, int32_t window) {
  if (window <= 0) return 0;
  const int64_t b = (int64_t)r0 + (lkv - lq) + 1 - window;
  return (int32_t)min((int64_t)lkv, max((int64_t)0, b));
}

struct Counts {
  int32_t pre, decf, decp, cmb, part;
};

// Exclusive scan of one Counts per thread over the workgroup; *total gets the sums.
__device__ Counts block_exclusive_scan(Counts v, Counts* buf, Counts* total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    Counts add = {0, 0, 0, 0, 0};
    if (tid >= off) add = buf[tid - off];
    __syncthreads();
    buf[tid].pre += add.pre;
    buf[tid].decf += add.decf;
    buf[tid].decp += add.decp;
    buf[tid].cmb += add.cmb;
    buf[tid].part += add.part;
    __syncthreads();
  }
  const Counts incl = buf[tid];
  *total = buf[kThreads - 1];
  __syncthreads();
  return Counts{incl.pre - v.pre, incl.decf - v.decf, incl.decp - v.decp, incl.cmb - v.cmb, incl.part - v.part};
}

// Largest b in [0, n) with off[b] <= k (off is non-decreasing, off[0] == 0).
__device__ int32_t owner(const int32_t* off, int32_t n, int32_t k) {
  int32_t lo = 0, hi = n;
  while (hi - lo > 1) {
    const int32_t mid = lo + (hi - lo) / 2;
    if (off[mid] <= k) lo = mid; else hi = mid;
  }
  return lo;
}

// Sorts key[0, n) in descending order (n a power of two <= kLdsSeq), the
// whole workgroup taking part.
__device__ void bitonic_sort_desc(int64_t* key, int32_t n) {
  const int tid = threadIdx.x;
  for (int32_t k = 2; k <= n; k <<= 1) {
    for (int32_t j = k >> 1; j > 0; j >>= 1) {
      for (int32_t i = tid; i < n; i += kThreads) {
        const int32_t ixj = i ^ j;
        if (ixj > i) {
          const int64_t a = key[i], c = key[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (a < c) : (a > c)) {
            key[i] = c;
            key[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

// The split-KV key range of the single row of a decode sequence.
struct DecRange {
  int32_t vb, ve, ns, nfull;
};
__device__ DecRange dec_range(int32_t lq, int32_t lkv, const DevicePlan& dp, int32_t dchunk) {
  DecRange r;
  r.vb = visible_begin_dev(lq, lkv, 0, dp.window);
  r.ve = max(r.vb, visible_end_dev(lq, lkv, 0, 1, dp.causal));
  const int32_t n = r.ve - r.vb;
  r.ns = max(1, (n + dchunk - 1) / dchunk);
  r.nfull = (n > 0 && n % dchunk == 0) ? r.ns : r.ns - 1;  // splits of exactly dchunk keys
  return r;
}

}  // namespace

__global__ __launch_bounds__(kThreads) void plan_kernel(DevicePlan dp, const int32_t* __restrict__ cu_q,
                                                        const int32_t* __restrict__ cu_kv, int32_t* latch) {
  __shared__ Counts scan_buf[kThreads];
  __shared__ int32_t s_q[kLdsSeq], s_kv[kLdsSeq];                    // cu arrays
  __shared__ int32_t s_pre[kLdsSeq], s_decf[kLdsSeq], s_decp[kLdsSeq];  // list offsets
  __shared__ int32_t s_cmb[kLdsSeq], s_part[kLdsSeq];
  __shared__ int64_t s_key[kLdsSeq];   // prefill order of the sequences (LDS path)
  __shared__ int64_t s_key2[kLdsSeq];  // order of the sequences' short last decode splits
  __shared__ int32_t s_err;
  __shared__ int32_t s_dchunk;
  __shared__ int64_t s_dec_keys;
  const int tid = threadIdx.x;
  const int32_t B = dp.batch;
  int32_t* header = dp.header;
  const bool in_lds = B + 1 <= kLdsSeq;
  // offsets and cu values live in LDS or (large batches) in the workspace;
  // generic pointers read either
  int32_t* aq = in_lds ? s_q : dp.seq_q;
  int32_t* akv = in_lds ? s_kv : dp.seq_kv;
  int32_t* apre = in_lds ? s_pre : dp.seq_pre;
  int32_t* adecf = in_lds ? s_decf : dp.seq_decf;
  int32_t* adecp = in_lds ? s_decp : dp.seq_decp;
  int32_t* acmb = in_lds ? s_cmb : dp.seq_cmb;
  int32_t* apart = in_lds ? s_part : dp.seq_part;
  // Keys of sequence b: packed (akv holds cu_seqlens_kv) or in a
  // fixed-capacity cache (akv[b] holds L_kv, the keys start at b * capacity).
  const bool cache = dp.kv_len != nullptr;
  auto lkv_of = [&](int32_t b) -> int32_t { return cache ? akv[b] : akv[b + 1] - akv[b]; };
  auto kv0_of = [&](int32_t b) -> int32_t { return cache ? b * dp.kv_capacity : akv[b]; };

  // ---- 1. validation (latch first), cu arrays, the decode key total ------------
  const int32_t latched = __hip_atomic_load(latch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) {
    s_err = latched != 0 ? -1 : 0;
    s_dec_keys = 0;
  }
  int32_t err = 0;
  int64_t dec_keys = 0;
  for (int32_t b = tid; b <= B; b += kThreads) {
    aq[b] = cu_q[b];
    akv[b] = cache ? (b < B ? dp.kv_len[b] : 0) : cu_kv[b];
  }
  if (!in_lds) __threadfence();
  __syncthreads();
  if (s_err == 0) {
    if (tid == 0) {
      if (aq[0] != 0) err |= kLatchCuQStart;
      if (aq[B] > dp.cap_q) err |= kLatchCuQTotal;
      if (!cache && akv[0] != 0) err |= kLatchCuKvStart;
      if (!cache && akv[B] > dp.cap_kv) err |= kLatchCuKvTotal;
    }
    for (int32_t b = tid; b < B; b += kThreads) {
      const int32_t lq = aq[b + 1] - aq[b];
      const int32_t lkv = lkv_of(b);
      if (lq < 0) err |= kLatchCuQOrder;
      if (cache ? (lkv < 0 || lkv > dp.kv_capacity) : lkv < 0) err |= cache ? kLatchKvLen : kLatchCuKvOrder;
      if (dp.use_decode && lq == 1 && lkv > 0) dec_keys += lkv;
    }
    if (err) atomicOr(&s_err, err);
    if (dec_keys) atomicAdd((unsigned long long*)&s_dec_keys, (unsigned long long)dec_keys);
  }
  __syncthreads();
  if (s_err != 0) {
    if (tid == 0) {
      if (s_err > 0) atomicOr(latch, s_err);
      header[kHdrPrefill] = 0;
      header[kHdrDecode] = 0;
      header[kHdrCombine] = 0;
      header[kHdrPartials] = 0;
      header[kHdrChunk] = 0;
    }
    return;
  }
  // split-KV chunk: the host scheduler's rule (enough items to fill the chip
  // several times, 512..8192 keys, a multiple of 128)
  if (tid == 0) {
    const int64_t groups = dp.hq / dp.nh_dec;
    int64_t c = (s_dec_keys * groups + 2047) / 2048;
    c = max((int64_t)512, min((int64_t)8192, c));
    s_dchunk = (int32_t)((c + 127) / 128 * 128);
  }
  __syncthreads();
  const int32_t dchunk = s_dchunk;
  const int32_t g_pre = dp.hq / dp.nh;      // head groups of a prefill item
  const int32_t g_dec = dp.hq / dp.nh_dec;  // head groups of a decode item

  // ---- 2a. sequence orders (LDS path; sequence order for batches too large for
  // it). Prefill: by the cost of the sequence's longest item, descending, ties
  // by index (the host scheduler's order). Short last decode splits: by length,
  // descending. key = value << 11 | (2047 - b).
  const bool sorted = in_lds;
  if (sorted) {
    int32_t n = 1;
    while (n < B) n <<= 1;
    for (int32_t b = tid; b < n; b += kThreads) {
      int64_t key = -1, key2 = -1;
      if (b < B) {
        int64_t top = 0, last = 0;
        const int32_t lq = aq[b + 1] - aq[b];
        const int32_t lkv = lkv_of(b);
        if (lq > 0 && !(dp.use_decode && lq == 1)) {
          // An item's key range never shrinks from one full row block to the
          // next (causal) or never grows (window without causal), so the
          // longest item is in the first, the second-to-last or the last
          // (possibly short) row block.
          const int32_t n_rb = (lq + dp.rows_per_item - 1) / dp.rows_per_item;
          const int32_t cand[3] = {0, max(0, n_rb - 2), n_rb - 1};
          for (int32_t ci = 0; ci < 3; ++ci) {
            const int32_t rb = cand[ci];
            const int32_t r0 = rb * dp.rows_per_item;
            const int32_t rows = min(dp.rows_per_item, lq - r0);
            const int32_t vb = visible_begin_dev(lq, lkv, r0, dp.window);
            const int32_t ve = max(vb, visible_end_dev(lq, lkv, r0, rows, dp.causal));
            top = max(top, (int64_t)(ve - vb) * rows);
          }
        } else if (lq == 1) {
          const DecRange r = dec_range(lq, lkv, dp, dchunk);
          last = (r.ve - r.vb) - (int64_t)r.nfull * dchunk;  // keys of the short last split
        }
        key = (top << 11) | (int64_t)(kLdsSeq - 1 - b);
        key2 = (last << 11) | (int64_t)(kLdsSeq - 1 - b);
      }
      s_key[b] = key;
      s_key2[b] = key2;
    }
    __syncthreads();
    bitonic_sort_desc(s_key, n);
    bitonic_sort_desc(s_key2, n);
  }
  // the sequence at position p of the prefill list order / of the decode
  // list's short-split order
  auto seq_at = [&](int32_t pos) -> int32_t {
    return sorted ? (int32_t)(kLdsSeq - 1 - (s_key[pos] & (kLdsSeq - 1))) : pos;
  };
  auto seq_at2 = [&](int32_t pos) -> int32_t {
    return sorted ? (int32_t)(kLdsSeq - 1 - (s_key2[pos] & (kLdsSeq - 1))) : pos;
  };

  // ---- 2b. per-sequence counts, one scan of all five ------------------------------
  // (prefill counts are taken in prefill order, the others in sequence order)
  Counts base = {0, 0, 0, 0, 0};
  for (int32_t b0 = 0; b0 <= B; b0 += kThreads) {
    const int32_t b = b0 + tid;
    Counts n = {0, 0, 0, 0, 0};
    if (b < B) {
      const int32_t lq = aq[b + 1] - aq[b];
      const int32_t lkv = lkv_of(b);
      if (lq > 0) {
        if (dp.use_decode && lq == 1) {
          const DecRange r = dec_range(lq, lkv, dp, dchunk);
          n.decf = g_dec * r.nfull;
          if (r.ns > 1) {
            n.cmb = g_dec;
            n.part = g_dec * r.ns * dp.nh_dec;
          }
        }
      }
      const int32_t bp = seq_at(b);  // prefill counts in prefill order
      const int32_t lqp = aq[bp + 1] - aq[bp];
      if (lqp > 0 && !(dp.use_decode && lqp == 1)) n.pre = ((lqp + dp.rows_per_item - 1) / dp.rows_per_item) * g_pre;
      const int32_t bd = seq_at2(b);  // short-split counts in their order
      const int32_t lqd = aq[bd + 1] - aq[bd];
      if (dp.use_decode && lqd == 1) {
        const DecRange r = dec_range(lqd, lkv_of(bd), dp, dchunk);
        n.decp = g_dec * (r.ns - r.nfull);
      }
    }
    Counts tot;
    const Counts o = block_exclusive_scan(n, scan_buf, &tot);
    if (b <= B) {
      apre[b] = base.pre + o.pre;
      adecf[b] = base.decf + o.decf;
      adecp[b] = base.decp + o.decp;
      acmb[b] = base.cmb + o.cmb;
      apart[b] = base.part + o.part;
    }
    base.pre += tot.pre;
    base.decf += tot.decf;
    base.decp += tot.decp;
    base.cmb += tot.cmb;
    base.part += tot.part;
  }
  const int64_t n_dec = (int64_t)base.decf + base.decp;
  // the lists must fit their bounds (they size the launch grids)
  if (base.pre > dp.cap_prefill || n_dec > dp.cap_decode || base.cmb > dp.cap_combine ||
      base.part > dp.cap_partials) {
    if (tid == 0) {
      atomicOr(latch, kLatchCapacity);
      header[kHdrPrefill] = 0;
      header[kHdrDecode] = 0;
      header[kHdrCombine] = 0;
      header[kHdrPartials] = 0;
      header[kHdrChunk] = dchunk;
    }
    return;
  }
  if (!in_lds) __threadfence();
  __syncthreads();

  // ---- 3. the items ---------------------------------------------------------------
  auto proto = [&](int32_t b, int32_t kind) {
    WorkItem it;
    it.kind = kind;
    it.seq = b;
    it.q_row_begin = 0;
    it.q_rows = 0;
    it.head_begin = 0;
    it.heads = 0;
    it.kv_begin = 0;
    it.kv_end = 0;
    it.partial_base = -1;
    it.n_splits = 1;
    it.q_token0 = aq[b];
    it.kv_token0 = kv0_of(b);
    it.len_q = aq[b + 1] - aq[b];
    it.len_kv = lkv_of(b);
    it.split = 0;
    it.pad = 0;
    return it;
  };
  for (int32_t k = tid; k < base.pre; k += kThreads) {
    const int32_t pos = owner(apre, B, k);
    const int32_t b = seq_at(pos);
    const int32_t j = k - apre[pos];
    WorkItem it = proto(b, dp.prefill_kind);
    const int32_t n_rb = (it.len_q + dp.rows_per_item - 1) / dp.rows_per_item;
    const int32_t rb = n_rb - 1 - j / g_pre;  // last row block first
    it.q_row_begin = rb * dp.rows_per_item;
    it.q_rows = min(dp.rows_per_item, it.len_q - it.q_row_begin);
    it.head_begin = (j % g_pre) * dp.nh;
    it.heads = dp.nh;
    it.kv_begin = visible_begin_dev(it.len_q, it.len_kv, it.q_row_begin, dp.window);
    it.kv_end = max(it.kv_begin, visible_end_dev(it.len_q, it.len_kv, it.q_row_begin, it.q_rows, dp.causal));
    dp.prefill[k] = it;
  }
  for (int32_t k = tid; k < n_dec; k += kThreads) {
    const bool full = k < base.decf;
    const int32_t* off = full ? adecf : adecp;
    const int32_t kk = full ? k : k - base.decf;
    const int32_t pos = owner(off, B, kk);
    const int32_t b = full ? pos : seq_at2(pos);
    const int32_t j = kk - off[pos];
    WorkItem it = proto(b, kDecode);
    const DecRange r = dec_range(it.len_q, it.len_kv, dp, dchunk);
    const int32_t gi = full ? j / r.nfull : j;
    const int32_t s = full ? j % r.nfull : r.ns - 1;
    it.q_rows = 1;
    it.head_begin = gi * dp.nh_dec;
    it.heads = dp.nh_dec;
    if (r.ns == 1) {
      it.kv_begin = r.vb;
      it.kv_end = r.ve;
    } else {
      it.partial_base = apart[b] + gi * r.ns * dp.nh_dec;
      it.n_splits = r.ns;
      it.split = s;
      it.kv_begin = r.vb + s * dchunk;
      it.kv_end = min(r.ve, r.vb + (s + 1) * dchunk);
    }
    dp.decode[k] = it;
  }
  for (int32_t k = tid; k < base.cmb; k += kThreads) {
    const int32_t b = owner(acmb, B, k);
    const int32_t gi = k - acmb[b];
    WorkItem it = proto(b, kCombine);
    const DecRange r = dec_range(it.len_q, it.len_kv, dp, dchunk);
    it.q_rows = 1;
    it.head_begin = gi * dp.nh_dec;
    it.heads = dp.nh_dec;
    it.partial_base = apart[b] + gi * r.ns * dp.nh_dec;
    it.n_splits = r.ns;
    it.kv_begin = r.vb;
    it.kv_end = r.ve;
    dp.combine[k] = it;
  }
  if (tid == 0) {
    header[kHdrPrefill] = base.pre;
    header[kHdrDecode] = (int32_t)n_dec;
    header[kHdrCombine] = base.cmb;
    header[kHdrPartials] = base.part;
    header[kHdrChunk] = dchunk;
  }
}

hipError_t launch_plan(const DevicePlan& dp, const int32_t* cu_q, const int32_t* cu_kv, int32_t* latch,
                       hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, s, dp, cu_q, cu_kv, latch);
  return hipGetLastError();
}

}  // namespace pva
