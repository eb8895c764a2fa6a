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
// Written for few barriers (each costs a few hundred cycles with 16 waves).
// When the per-sequence arrays fit in LDS, several workgroups (32 of 256
// threads for batches below 256 sequences, else 8 of 1024) each run steps 1
// and 2 on their own copy and write their share of the item chunks in step
// 3 (the first one also writes the header and the latch); a larger batch
// keeps its arrays in the workspace and runs in one 1024-thread workgroup:
//   1. every thread validates and counts the items of its sequences; the
//      split-KV chunk needs the total decode key count, so that is reduced
//      first;
//   2. the sequence orders (a rank sort: every sequence counts the sequences
//      that go before it) and one exclusive scan over the sequences (five
//      counts at once, wave prefix sums then one pass over the wave totals)
//      give each sequence's first item in the prefill list, in the two parts
//      of the decode list, in the combine list, and its first partial row;
//      the offsets and the cu arrays stay in LDS when the batch fits (else in
//      the workspace, without sorting);
//   3. each wave writes 64 consecutive items at a time, finding the sequence
//      of item k by binary search over those offsets; the items pass through
//      LDS so that the wave's stores cover whole 64-byte items back to back.
// With a fixed-capacity KV cache (the attention that follows the cache step)
// the keys of sequence b are rows [b * capacity, b * capacity + L_kv[b]) and
// L_kv comes from a device array instead of cu_seqlens_kv; each length is
// checked against the capacity.
// The prefill list takes the host scheduler's order: sequences by their
// longest item, each sequence's row blocks from the last to the first, head
// groups innermost. The decode list holds every full-chunk split first and
// the shorter last splits after them, longest first, so that the last items
// handed to the GPU are the short ones.
#include "common.h"

namespace pva {

namespace {

// Workgroup shapes. Batches of up to kSmallThreads - 1 sequences run in
// 256-thread workgroups: every phase then syncs 4 waves, not 16 (ragged
// batch of 16 sequences: 9.6 against 12.9 us). Larger ones keep 1024 threads,
// which cover more sequences per pass (256 sequences: 26.7 against 38.8 us).
constexpr int kSmallThreads = 256;
constexpr int kSmallGroups = 32;  // workgroups of the LDS path at 256 threads
constexpr int kBigThreads = 1024;
constexpr int kBigGroups = 8;     // ... at 1024 threads (the workspace path uses one)
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

__device__ Counts add(Counts a, Counts b) {
  return Counts{a.pre + b.pre, a.decf + b.decf, a.decp + b.decp, a.cmb + b.cmb, a.part + b.part};
}

// Exclusive scan of one Counts per thread over the workgroup; *total gets
// the sums. Wave prefix sums by lane shifts; then every wave scans the 16
// wave totals across its first 16 lanes (one LDS read per lane) and takes
// the prefix of the waves before its own: two barriers.
__device__ Counts shfl_counts(Counts c, int src) {
  return Counts{__shfl(c.pre, src, 64), __shfl(c.decf, src, 64), __shfl(c.decp, src, 64), __shfl(c.cmb, src, 64),
                __shfl(c.part, src, 64)};
}

template <int NT>
__device__ Counts block_exclusive_scan(Counts v, Counts* wave_tot, Counts* total) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  Counts incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const Counts o = {__shfl_up(incl.pre, off, 64), __shfl_up(incl.decf, off, 64), __shfl_up(incl.decp, off, 64),
                      __shfl_up(incl.cmb, off, 64), __shfl_up(incl.part, off, 64)};
    if (lane >= off) incl = add(incl, o);
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  Counts t = {0, 0, 0, 0, 0};
  if (lane < kWaves) t = wave_tot[lane];
#pragma unroll
  for (int off = 1; off < kWaves; off <<= 1) {
    const Counts o = {__shfl_up(t.pre, off, 64), __shfl_up(t.decf, off, 64), __shfl_up(t.decp, off, 64),
                      __shfl_up(t.cmb, off, 64), __shfl_up(t.part, off, 64)};
    if (lane >= off) t = add(t, o);
  }
  // lane w (< kWaves) now holds the totals of waves 0..w
  const Counts all = shfl_counts(t, kWaves - 1);
  const Counts prev = shfl_counts(t, wave > 0 ? wave - 1 : 0);
  const Counts before = wave > 0 ? prev : Counts{0, 0, 0, 0, 0};
  __syncthreads();  // wave_tot is reused by the next scan
  *total = all;
  return Counts{before.pre + incl.pre - v.pre, before.decf + incl.decf - v.decf, before.decp + incl.decp - v.decp,
                before.cmb + incl.cmb - v.cmb, before.part + incl.part - v.part};
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

// Writes the items of lanes with k0 + lane < n at list[k0 + lane]; every
// lane of the wave calls it together. Each lane's 64-byte item goes to LDS,
// then the wave stores the 64 items as consecutive 16-byte pieces.
__device__ void store_items(WorkItem* list, int32_t k0, int32_t n, const WorkItem& it, u32x4_t* stage) {
  const int lane = threadIdx.x & 63;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(&it);
#pragma unroll
  for (int c = 0; c < 4; ++c) stage[lane * 4 + c] = src[c];
  __builtin_amdgcn_wave_barrier();
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(list + k0);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = lane + 64 * r;  // piece c holds quarter c % 4 of item c / 4
    if (k0 + c / 4 < n) dst[c] = stage[c];
  }
  __builtin_amdgcn_wave_barrier();
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

template <int NT>
struct SchedLds {
  int32_t q[kLdsSeq], kv[kLdsSeq];                    // cu arrays (cache: kv holds L_kv)
  int32_t pre[kLdsSeq], decf[kLdsSeq], decp[kLdsSeq];  // list offsets
  int32_t cmb[kLdsSeq], part[kLdsSeq];
  int32_t ord[kLdsSeq], ord2[kLdsSeq];  // position -> sequence: prefill order, short-split order
  union {
    struct {
      int64_t cost[kLdsSeq], cost2[kLdsSeq];  // sort keys
    } sort;
    u32x4_t stage[NT / 64][256];  // item staging, 4 KB per wave
  } u;
  Counts wave_tot[NT / 64];
  int32_t err, has_pre, has_dec;
  int64_t dec_keys;
};

// The scheduler; LDS selects where the per-sequence arrays live (LDS, or the
// workspace for batches too large for it).
template <bool LDS, int NT>
__device__ void plan_body(const DevicePlan& dp, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv,
                          int32_t* latch, SchedLds<NT>& sh) {
  constexpr int kThreads = NT;
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int32_t B = dp.batch;
  // With several workgroups (LDS path only) every one of them works out the
  // same per-sequence offsets in its own LDS and writes its share of the
  // items; only the first writes the header and the latch.
  const bool lead = blockIdx.x == 0;
  int32_t* header = dp.header;
  int32_t* aq = LDS ? sh.q : dp.seq_q;
  int32_t* akv = LDS ? sh.kv : dp.seq_kv;
  int32_t* apre = LDS ? sh.pre : dp.seq_pre;
  int32_t* adecf = LDS ? sh.decf : dp.seq_decf;
  int32_t* adecp = LDS ? sh.decp : dp.seq_decp;
  int32_t* acmb = LDS ? sh.cmb : dp.seq_cmb;
  int32_t* apart = LDS ? sh.part : dp.seq_part;
  // Keys of sequence b: packed (akv holds cu_seqlens_kv) or in a
  // fixed-capacity cache (akv[b] holds L_kv, the keys start at b * capacity).
  const bool cache = dp.kv_len != nullptr;
  auto lkv_of = [&](int32_t b) -> int32_t { return cache ? akv[b] : akv[b + 1] - akv[b]; };
  auto kv0_of = [&](int32_t b) -> int32_t { return cache ? b * dp.kv_capacity : akv[b]; };

  // ---- 1. validation (latch first), cu arrays, the decode key total ------------
  const int32_t latched = __hip_atomic_load(latch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) {
    sh.err = latched != 0 ? -1 : 0;
    sh.dec_keys = 0;
    sh.has_pre = 0;
    sh.has_dec = 0;
  }
  for (int32_t b = tid; b <= B; b += kThreads) {
    aq[b] = cu_q[b];
    akv[b] = cache ? (b < B ? dp.kv_len[b] : 0) : cu_kv[b];
  }
  if (!LDS) __threadfence();
  __syncthreads();
  if (sh.err == 0) {
    int32_t err = 0, has_pre = 0, has_dec = 0;
    int64_t dec_keys = 0;
    if (tid == 0) {
      if (aq[0] != 0) err |= kLatchCuQStart;
      if (aq[B] > dp.cap_q) err |= kLatchCuQTotal;
      if (!cache && akv[0] != 0) err |= kLatchCuKvStart;
      if (!cache && akv[B] > dp.cap_kv) err |= kLatchCuKvTotal;
    }
    for (int32_t b = tid; b < B; b += kThreads) {
      // Order is tested on the elements themselves, never on a difference:
      // a difference of two int32 can wrap (e.g. INT32_MIN - INT32_MAX) and
      // look non-negative. With cu[0] == 0, no decrease and cu[B] <= the
      // buffer's rows, every element lies in [0, rows] and the differences
      // taken below cannot wrap.
      const bool q_bad = aq[b + 1] < aq[b];
      const bool kv_bad = cache ? (akv[b] < 0 || akv[b] > dp.kv_capacity) : akv[b + 1] < akv[b];
      if (q_bad) err |= kLatchCuQOrder;
      if (kv_bad) err |= cache ? kLatchKvLen : kLatchCuKvOrder;
      if (q_bad || kv_bad) continue;
      const int32_t lq = aq[b + 1] - aq[b];
      const int32_t lkv = lkv_of(b);
      const bool dec = dp.use_decode && lq == 1;
      if (dec && lkv > 0) dec_keys += lkv;
      has_dec |= dec;
      has_pre |= lq > 0 && !dec;
    }
    if (err) atomicOr(&sh.err, err);
    if (dec_keys) atomicAdd((unsigned long long*)&sh.dec_keys, (unsigned long long)dec_keys);
    if (has_pre) sh.has_pre = 1;
    if (has_dec) sh.has_dec = 1;
  }
  __syncthreads();
  if (sh.err != 0) {
    if (tid == 0 && lead) {
      if (sh.err > 0) atomicOr(latch, sh.err);
      header[kHdrPrefill] = 0;
      header[kHdrDecode] = 0;
      header[kHdrCombine] = 0;
      header[kHdrPartials] = 0;
      header[kHdrChunk] = 0;
    }
    return;
  }
  // split-KV chunk: the host scheduler's rule (enough items to fill the chip
  // several times, 512..8192 keys, a multiple of 128); every thread works it
  // out from the shared total
  int32_t dchunk;
  {
    const int64_t groups = dp.hq / dp.nh_dec;
    int64_t c = (sh.dec_keys * groups + 2047) / 2048;
    c = max((int64_t)512, min((int64_t)8192, c));
    dchunk = (int32_t)((c + 127) / 128 * 128);
  }
  const int32_t g_pre = dp.hq / dp.nh;      // head groups of a prefill item
  const int32_t g_dec = dp.hq / dp.nh_dec;  // head groups of a decode item
  const bool need_pre = sh.has_pre != 0;
  const bool need_dec = sh.has_dec != 0;

  // ---- 2a. sequence orders (LDS path). Prefill: by the cost of the sequence's
  // longest item, descending, ties by index (the host scheduler's order).
  // Short last decode splits: by length, descending, ties by index.
  if (LDS) {
    for (int32_t b = tid; b < B; b += kThreads) {
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
      sh.u.sort.cost[b] = top;
      sh.u.sort.cost2[b] = last;
    }
    __syncthreads();
    // rank of sequence b: the sequences with a larger key, or an equal key
    // and a smaller index. tpk threads (neighbouring lanes) share a key and
    // count every tpk-th other key, so all 16 waves take part for small
    // batches; their counts are summed across the lanes.
    int32_t tpk = 1;
    while (tpk < 64 && tpk * 2 * B <= kThreads) tpk *= 2;
    const int32_t part = tid & (tpk - 1);
    for (int32_t b0 = 0; b0 < B; b0 += kThreads / tpk) {
      const int32_t b = b0 + tid / tpk;
      int32_t r = 0, r2 = 0;
      if (b < B) {
        const int64_t mine = sh.u.sort.cost[b], mine2 = sh.u.sort.cost2[b];
#pragma unroll 8
        for (int32_t j = part; j < B; j += tpk) {
          const int64_t c = sh.u.sort.cost[j], c2 = sh.u.sort.cost2[j];
          r += (c > mine) | ((c == mine) & (j < b));
          r2 += (c2 > mine2) | ((c2 == mine2) & (j < b));
        }
      }
      for (int32_t m = 1; m < tpk; m <<= 1) {
        r += __shfl_xor(r, m, 64);
        r2 += __shfl_xor(r2, m, 64);
      }
      if (b < B && part == 0) {
        if (need_pre) sh.ord[r] = b;
        if (need_dec) sh.ord2[r2] = b;
      }
    }
    __syncthreads();
  }
  // the sequence at position p of the prefill list order / of the decode
  // list's short-split order
  auto seq_at = [&](int32_t pos) -> int32_t { return LDS && need_pre ? sh.ord[pos] : pos; };
  auto seq_at2 = [&](int32_t pos) -> int32_t { return LDS && need_dec ? sh.ord2[pos] : pos; };

  // ---- 2b. per-sequence counts, one scan of all five ------------------------------
  // (prefill counts are taken in prefill order, the others in sequence order)
  Counts base = {0, 0, 0, 0, 0};
  for (int32_t b0 = 0; b0 <= B; b0 += kThreads) {
    const int32_t b = b0 + tid;
    Counts n = {0, 0, 0, 0, 0};
    if (b < B) {
      const int32_t lq = aq[b + 1] - aq[b];
      if (dp.use_decode && lq == 1) {
        const DecRange r = dec_range(lq, lkv_of(b), dp, dchunk);
        n.decf = g_dec * r.nfull;
        if (r.ns > 1) {
          n.cmb = g_dec;
          n.part = g_dec * r.ns * dp.nh_dec;
        }
      }
      if (need_pre) {
        const int32_t bp = seq_at(b);  // prefill counts in prefill order
        const int32_t lqp = aq[bp + 1] - aq[bp];
        if (lqp > 0 && !(dp.use_decode && lqp == 1))
          n.pre = ((lqp + dp.rows_per_item - 1) / dp.rows_per_item) * g_pre;
      }
      if (need_dec) {
        const int32_t bd = seq_at2(b);  // short-split counts in their order
        const int32_t lqd = aq[bd + 1] - aq[bd];
        if (dp.use_decode && lqd == 1) {
          const DecRange r = dec_range(lqd, lkv_of(bd), dp, dchunk);
          n.decp = g_dec * (r.ns - r.nfull);
        }
      }
    }
    Counts tot;
    const Counts o = block_exclusive_scan<NT>(n, sh.wave_tot, &tot);
    if (b <= B) {
      apre[b] = base.pre + o.pre;
      adecf[b] = base.decf + o.decf;
      adecp[b] = base.decp + o.decp;
      acmb[b] = base.cmb + o.cmb;
      apart[b] = base.part + o.part;
    }
    base = add(base, tot);
  }
  const int64_t n_dec = (int64_t)base.decf + base.decp;
  // the lists must fit their bounds (they size the launch grids)
  if (base.pre > dp.cap_prefill || n_dec > dp.cap_decode || base.cmb > dp.cap_combine ||
      base.part > dp.cap_partials) {
    if (tid == 0 && lead) {
      atomicOr(latch, kLatchCapacity);
      header[kHdrPrefill] = 0;
      header[kHdrDecode] = 0;
      header[kHdrCombine] = 0;
      header[kHdrPartials] = 0;
      header[kHdrChunk] = dchunk;
    }
    return;
  }
  if (!LDS) __threadfence();
  __syncthreads();

  // ---- 3. the items, 64 per wave at a time ------------------------------------------
  u32x4_t* stage = sh.u.stage[wave];
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
    it.kv_head = 0;
    return it;
  };
  auto make_pre = [&](int32_t k) {
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
    it.kv_head = it.head_begin / dp.group;
    it.kv_begin = visible_begin_dev(it.len_q, it.len_kv, it.q_row_begin, dp.window);
    it.kv_end = max(it.kv_begin, visible_end_dev(it.len_q, it.len_kv, it.q_row_begin, it.q_rows, dp.causal));
    return it;
  };
  auto make_dec = [&](int32_t k) {
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
    it.kv_head = it.head_begin / dp.group;
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
    return it;
  };
  auto make_cmb = [&](int32_t k) {
    const int32_t b = owner(acmb, B, k);
    const int32_t gi = k - acmb[b];
    WorkItem it = proto(b, kCombine);
    const DecRange r = dec_range(it.len_q, it.len_kv, dp, dchunk);
    it.q_rows = 1;
    it.head_begin = gi * dp.nh_dec;
    it.heads = dp.nh_dec;
    it.kv_head = it.head_begin / dp.group;
    it.partial_base = apart[b] + gi * r.ns * dp.nh_dec;
    it.n_splits = r.ns;
    it.kv_begin = r.vb;
    it.kv_end = r.ve;
    return it;
  };
  // Two 64-item chunks per wave and pass, so that the lookups of one hide
  // under those of the other; the workgroups take interleaved chunks.
  const int32_t span = kThreads * (int32_t)gridDim.x;  // items of one chunk per wave of every workgroup
  auto emit = [&](WorkItem* list, int32_t n, auto make) {
    for (int32_t k0 = ((int32_t)blockIdx.x * kWaves + wave) * 64; k0 < n; k0 += 2 * span) {
      const int32_t k1 = k0 + span;
      const WorkItem a = make(min(k0 + lane, n - 1));
      const WorkItem c = make(min(k1 + lane, n - 1));
      store_items(list, k0, n, a, stage);
      if (k1 < n) store_items(list, k1, n, c, stage);
    }
  };
  emit(dp.prefill, base.pre, make_pre);
  emit(dp.decode, (int32_t)n_dec, make_dec);
  emit(dp.combine, base.cmb, make_cmb);
  if (tid == 0 && lead) {
    header[kHdrPrefill] = base.pre;
    header[kHdrDecode] = (int32_t)n_dec;
    header[kHdrCombine] = base.cmb;
    header[kHdrPartials] = base.part;
    header[kHdrChunk] = dchunk;
  }
}

}  // namespace

template <bool LDS, int NT>
__global__ __launch_bounds__(NT) void plan_kernel(DevicePlan dp, const int32_t* __restrict__ cu_q,
                                                  const int32_t* __restrict__ cu_kv, int32_t* latch) {
  __shared__ SchedLds<NT> sh;
  plan_body<LDS, NT>(dp, cu_q, cu_kv, latch, sh);
}

hipError_t launch_plan(const DevicePlan& dp, const int32_t* cu_q, const int32_t* cu_kv, int32_t* latch,
                       hipStream_t s) {
  if (dp.batch + 1 <= kSmallThreads)
    hipLaunchKernelGGL((plan_kernel<true, kSmallThreads>), dim3(kSmallGroups), dim3(kSmallThreads), 0, s, dp, cu_q,
                       cu_kv, latch);
  else if (dp.batch + 1 <= kLdsSeq)
    hipLaunchKernelGGL((plan_kernel<true, kBigThreads>), dim3(kBigGroups), dim3(kBigThreads), 0, s, dp, cu_q, cu_kv,
                       latch);
  else
    hipLaunchKernelGGL((plan_kernel<false, kBigThreads>), dim3(1), dim3(kBigThreads), 0, s, dp, cu_q, cu_kv, latch);
  return hipGetLastError();
}

}  // namespace pva
