// Host side of the packed varlen attention library: argument validation, the
// cu_seqlens-driven work scheduler, the per-device workspace, and the kernel
// launches behind the C ABI declared in include/varlen_attn.h.
//
// Validation follows the packed op's execute() on the source page
// src/kernels/packed_varlen_attention.rs (crate onnx-runtime-ep-cuda
// 0.1.0-dev.6): dtype equality, kv heads dividing query heads, head sizes,
// token counts, cumulative arrays that start at 0, never decrease and end at
// the packed totals, and the output extent -- all before any device work.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/varlen_attn.h"
#include "common.h"

namespace pva {
hipError_t launch_prefill_mfma(const Params& p, const WorkItem* items, int n, int dtype, int nw,
                               hipStream_t s);
hipError_t launch_decode(const Params& p, const WorkItem* items, int n, int dtype, hipStream_t s);
hipError_t launch_combine(const Params& p, const WorkItem* items, int n, int dtype, hipStream_t s);
hipError_t launch_prefill_f32(const Params& p, const WorkItem* items, int n, hipStream_t s);
hipError_t launch_plan(const DevicePlan& dp, const int32_t* cu_q, const int32_t* cu_kv, int32_t* latch,
                       hipStream_t s);
hipError_t launch_rope_append(const RopeParams& p, int dtype, hipStream_t s);
int rope_units_per_block(int vec);
}  // namespace pva

// Scratch of the allocation-free call (varlen_attn_fwd_device_noalloc): the
// device-built work list and the split-KV partials of one call, in a static
// array of which every GPU the library runs on holds its own copy until the
// process ends. In host code `scratch` names a host-side stand-in, not a
// device address: the device address of the current GPU's copy comes from
// hipGetSymbolAddress (noalloc_scratch below) and only that address is
// passed to kernels. Nothing in it has to start at zero (the scheduler writes
// the list header on every call, and partials are written before they are
// read). Every such call on one GPU shares the array, so calls that overlap
// on a GPU (other streams, other threads) race.
static __device__ __align__(256) unsigned char scratch[VARLEN_NOALLOC_SCRATCH_BYTES];

namespace {

using pva::WorkItem;

thread_local std::string g_last_error;
thread_local const char* g_entry = "varlen_attn_fwd";  // names the failing call in messages

varlen_status_t fail(varlen_status_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(g_entry) + ": " + buf;
  return code;
}

// Sets the call name of error messages for the duration of an entry point.
struct EntryName {
  const char* saved;
  explicit EntryName(const char* name) : saved(g_entry) { g_entry = name; }
  ~EntryName() { g_entry = saved; }
};

// ---------------------------------------------------------------------------
// Arguments after defaults are resolved.
// ---------------------------------------------------------------------------
struct Problem {
  int32_t batch;
  int64_t total_q, total_kv;
  int32_t hq, hkv, group, d, dv, dtype;
  float scale;  // effective scale
  int32_t causal;
  int32_t window;  // 0: none; > 0: keys j >= i + off + 1 - window
  float softcap;
  const int32_t* cu_q;   // host
  const int32_t* cu_kv;  // host
};

struct Options {
  int32_t decode_path = 0;
  int32_t decode_chunk = 0;
  int32_t prefill_kv_chunk = 0;
  int32_t local_window = 0;
};

Options resolve_options(const varlen_attn_options_t* o) {
  Options r;
  if (o) {
    r.decode_path = o->decode_path;
    r.decode_chunk = o->decode_chunk;
    r.prefill_kv_chunk = o->prefill_kv_chunk;
    r.local_window = o->local_window;
  }
  return r;
}

// The local window: -1 (the GroupQueryAttention attribute's default) and 0
// mean none; below -1 is rejected as that op rejects it (page
// src/kernels/group_query_attention.rs, local_window_size validation).
varlen_status_t check_window(int32_t w, Problem* pr) {
  if (w < -1)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "local_window must be -1 or 0 (no window) or a positive key count, got %d", w);
  pr->window = w > 0 ? w : 0;
  return VARLEN_OK;
}

// Scalar and shape checks that need no cu arrays.
varlen_status_t check_scalars(int32_t batch, int64_t total_q, int64_t total_kv, int32_t num_heads,
                              int32_t kv_num_heads, int32_t head_dim, int32_t v_head_dim,
                              int32_t dtype, float scale, float softcap, Problem* pr) {
  if (dtype != VARLEN_F32 && dtype != VARLEN_F16 && dtype != VARLEN_BF16)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "dtype code %d not supported (expected f32=0, f16=1 or bf16=2)", dtype);
  if (num_heads <= 0)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "num_heads must be positive, got %d", num_heads);
  const int32_t hkv = kv_num_heads <= 0 ? num_heads : kv_num_heads;
  if (num_heads % hkv != 0)
    return fail(VARLEN_ERR_INVALID_ARGUMENT,
                "num_heads %d must be a positive multiple of kv_num_heads %d (MHA/GQA/MQA)", num_heads, hkv);
  if (head_dim <= 0) return fail(VARLEN_ERR_INVALID_ARGUMENT, "head_dim must be positive, got %d", head_dim);
  const int32_t dv = v_head_dim <= 0 ? head_dim : v_head_dim;
  if (batch < 1)
    return fail(VARLEN_ERR_BAD_SEQLENS, "batch must be >= 1 (cu_seqlens of length batch + 1 >= 2), got %d", batch);
  if (total_q < 0 || total_kv < 0 || total_q > INT32_MAX || total_kv > INT32_MAX)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "token totals must lie in [0, 2^31), got %lld and %lld",
                (long long)total_q, (long long)total_kv);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "scale must be finite and >= 0 (0 selects 1/sqrt(head_dim)), got %g",
                (double)scale);
  if (!std::isfinite(softcap))
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "softcap must be finite, got %g", (double)softcap);
  pr->batch = batch;
  pr->total_q = total_q;
  pr->total_kv = total_kv;
  pr->hq = num_heads;
  pr->hkv = hkv;
  pr->group = num_heads / hkv;
  pr->d = head_dim;
  pr->dv = dv;
  pr->dtype = dtype;
  pr->scale = scale == 0.f ? 1.0f / std::sqrt((float)head_dim) : scale;
  pr->softcap = std::fabs(softcap);
  return VARLEN_OK;
}

// The cumulative arrays: start at 0, never decrease, end at the packed total.
varlen_status_t check_cu(const int32_t* cu, int32_t batch, int64_t total, const char* name) {
  if (cu[0] != 0) return fail(VARLEN_ERR_BAD_SEQLENS, "%s[0] must be 0, got %d", name, cu[0]);
  for (int32_t b = 0; b < batch; ++b) {
    if (cu[b + 1] < cu[b])
      return fail(VARLEN_ERR_BAD_SEQLENS, "%s must be non-decreasing, but element %d (%d) > %d (%d)", name, b,
                  cu[b], b + 1, cu[b + 1]);
  }
  if ((int64_t)cu[batch] != total)
    return fail(VARLEN_ERR_BAD_SEQLENS, "%s[%d] = %d must equal the packed token count %lld", name, batch,
                cu[batch], (long long)total);
  return VARLEN_OK;
}

// The bf16/f16 kernels move q, k, v and out in 16-byte pieces.
varlen_status_t check_aligned(const Problem& pr, const void* q, const void* k, const void* v, const void* out) {
  if (pr.dtype == VARLEN_F32) return VARLEN_OK;
  auto a16 = [](const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; };
  if (!a16(q) || !a16(k) || !a16(v) || !a16(out))
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "f16/bf16 q, k, v and out must be 16-byte aligned");
  return VARLEN_OK;
}

varlen_status_t check_supported(const Problem& pr) {
  if (pr.dtype == VARLEN_F32) {
    if (pr.d > 128 || pr.dv > 128)
      return fail(VARLEN_ERR_UNSUPPORTED, "f32 supports head_dim and v_head_dim <= 128, got %d and %d", pr.d, pr.dv);
    return VARLEN_OK;
  }
  if ((pr.d != 64 && pr.d != 128) || (pr.dv != 64 && pr.dv != 128))
    return fail(VARLEN_ERR_UNSUPPORTED, "f16/bf16 support head_dim and v_head_dim in {64, 128}, got %d and %d", pr.d,
                pr.dv);
  return VARLEN_OK;
}

// ---------------------------------------------------------------------------
// The scheduler.
// ---------------------------------------------------------------------------
struct Plan {
  std::vector<WorkItem> prefill;  // kind kPrefillMfma
  std::vector<WorkItem> f32;      // kind kPrefillF32
  std::vector<WorkItem> decode;   // kind kDecode
  std::vector<WorkItem> combine;  // kind kCombine
  int64_t n_partials = 0;
  int64_t valid_pairs = 0;
  int64_t visited_pairs_x_heads = 0;
  int32_t prefill_waves = 0;
  int32_t heads_per_item = 0;
};

int64_t valid_pairs_of(const int32_t* cu_q, const int32_t* cu_kv, int32_t batch, bool causal, int32_t window) {
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t lq = (int64_t)cu_q[b + 1] - cu_q[b];
    const int64_t lkv = (int64_t)cu_kv[b + 1] - cu_kv[b];
    const int64_t off = lkv - lq;
    if (window > 0) {
      // row i sees [clamp(i + off + 1 - W, 0, lkv), hi)
      for (int64_t i = 0; i < lq; ++i) {
        const int64_t hi = causal ? std::min(lkv, std::max<int64_t>(0, i + off + 1)) : lkv;
        const int64_t lo = std::min(lkv, std::max<int64_t>(0, i + off + 1 - window));
        total += std::max<int64_t>(0, hi - lo);
      }
      continue;
    }
    if (!causal) {
      total += lq * lkv;
      continue;
    }
    // row i sees clamp(i + off + 1, 0, lkv) keys
    const int64_t i_first = std::max<int64_t>(0, -off);          // first row seeing >= 1 key
    const int64_t i_full = std::max<int64_t>(0, lkv - off - 1);  // first row seeing all keys
    const int64_t lo = std::min(lq, i_first);
    const int64_t hi = std::min(lq, std::max(lo, i_full));
    const int64_t n = hi - lo;  // rows seeing i + off + 1 keys
    total += n * (off + 1) + (lo + hi - 1) * n / 2;
    total += (lq - hi) * lkv;
  }
  return total;
}

WorkItem make_item(int32_t kind, int32_t b, const Problem& pr) {
  WorkItem it;
  std::memset(&it, 0, sizeof it);
  it.kind = kind;
  it.seq = b;
  it.q_token0 = pr.cu_q[b];
  it.kv_token0 = pr.cu_kv[b];
  it.len_q = pr.cu_q[b + 1] - pr.cu_q[b];
  it.len_kv = pr.cu_kv[b + 1] - pr.cu_kv[b];
  it.partial_base = -1;
  it.n_splits = 1;
  it.split = 0;
  return it;
}

// Keys [visible_begin, visible_end) that rows [r0, r0 + rows) of a sequence
// can see: the union of the rows' ranges (consecutive rows see overlapping,
// shifting ranges). An empty range (begin >= end) means the rows see nothing.
int32_t visible_end(const WorkItem& it, int32_t r0, int32_t rows, bool causal) {
  if (!causal) return it.len_kv;
  const int64_t last = (int64_t)r0 + rows - 1;
  const int64_t e = last + (it.len_kv - it.len_q) + 1;
  return (int32_t)std::min<int64_t>(it.len_kv, std::max<int64_t>(0, e));
}
int32_t visible_begin(const WorkItem& it, int32_t r0, int32_t window) {
  if (window <= 0) return 0;
  const int64_t b = (int64_t)r0 + (it.len_kv - it.len_q) + 1 - window;
  return (int32_t)std::min<int64_t>(it.len_kv, std::max<int64_t>(0, b));
}

int largest_pow2_divisor_upto(int g, int cap) {
  int r = 1;
  for (int c = cap; c >= 1; c >>= 1) {
    if (g % c == 0) {
      r = c;
      break;
    }
  }
  return r;
}

// Splits tile items (all with the same rows and heads) over [kv_begin, kv_end)
// in chunks; appends them (and their combine item) to `dst`/`plan.combine`.
// An empty range gives one item with no keys (it writes zero rows).
void emit_split(Plan& plan, std::vector<WorkItem>& dst, WorkItem base, int32_t kv_begin, int32_t kv_end,
                int32_t chunk) {
  kv_end = std::max(kv_begin, kv_end);
  const int32_t n_splits = std::max<int32_t>(1, (kv_end - kv_begin + chunk - 1) / chunk);
  if (n_splits == 1) {
    base.kv_begin = kv_begin;
    base.kv_end = kv_end;
    dst.push_back(base);
    return;
  }
  base.partial_base = (int32_t)plan.n_partials;
  base.n_splits = n_splits;
  plan.n_partials += (int64_t)n_splits * base.q_rows * base.heads;
  for (int32_t s = 0; s < n_splits; ++s) {
    WorkItem it = base;
    it.split = s;
    it.kv_begin = kv_begin + s * chunk;
    it.kv_end = std::min(kv_end, kv_begin + (s + 1) * chunk);
    dst.push_back(it);
  }
  WorkItem c = base;
  c.kind = pva::kCombine;
  c.kv_begin = kv_begin;
  c.kv_end = kv_end;
  plan.combine.push_back(c);
}

varlen_status_t build_plan(const Problem& pr, const Options& opt, Plan& plan) {
  const bool causal = pr.causal != 0;
  plan.valid_pairs = valid_pairs_of(pr.cu_q, pr.cu_kv, pr.batch, causal, pr.window);
  if (pr.dtype == VARLEN_F32) {
    plan.prefill_waves = 4;
    plan.heads_per_item = 1;
    for (int32_t b = 0; b < pr.batch; ++b) {
      const WorkItem proto = make_item(pva::kPrefillF32, b, pr);
      for (int32_t r0 = 0; r0 < proto.len_q; r0 += 32) {
        const int32_t rows = std::min(32, proto.len_q - r0);
        const int32_t kv_begin = visible_begin(proto, r0, pr.window);
        const int32_t kv_end = std::max(kv_begin, visible_end(proto, r0, rows, causal));
        for (int32_t h = 0; h < pr.hq; ++h) {
          WorkItem it = proto;
          it.q_row_begin = r0;
          it.q_rows = rows;
          it.head_begin = h;
          it.heads = 1;
          it.kv_head = h / pr.group;
          it.kv_begin = kv_begin;
          it.kv_end = kv_end;
          plan.f32.push_back(it);
          plan.visited_pairs_x_heads += (int64_t)rows * (kv_end - kv_begin);
        }
      }
    }
  } else {
    // Prefill tiles: NH heads of one kv group x R blocks of 32 rows per item.
    const int nh = largest_pow2_divisor_upto(pr.group, 8);
    const int rblocks = nh >= 4 ? 1 : 4 / nh;
    const int rows_per_item = 32 * rblocks;
    plan.prefill_waves = nh * rblocks;
    plan.heads_per_item = nh;
    const int nh_dec = largest_pow2_divisor_upto(pr.group, 16);
    const bool use_decode = opt.decode_path != 1;

    // Split-KV decode chunk: aim for enough items to fill the chip several
    // times over, in multiples of 128 keys.
    int64_t decode_keys = 0;
    for (int32_t b = 0; b < pr.batch; ++b) {
      if (pr.cu_q[b + 1] - pr.cu_q[b] == 1) decode_keys += pr.cu_kv[b + 1] - pr.cu_kv[b];
    }
    int32_t dchunk = opt.decode_chunk;
    if (dchunk <= 0) {
      const int64_t groups = pr.hq / nh_dec;
      const int64_t target_items = 2048;
      int64_t c = (decode_keys * groups + target_items - 1) / target_items;
      c = std::max<int64_t>(512, std::min<int64_t>(8192, c));
      dchunk = (int32_t)c;
    }
    dchunk = (dchunk + 127) / 128 * 128;
    const int32_t pchunk = opt.prefill_kv_chunk > 0 ? ((opt.prefill_kv_chunk + 63) / 64 * 64) : 0;

    for (int32_t b = 0; b < pr.batch; ++b) {
      const WorkItem proto = make_item(pva::kPrefillMfma, b, pr);
      if (proto.len_q == 0) continue;
      if (use_decode && proto.len_q == 1) {
        for (int32_t h0 = 0; h0 < pr.hq; h0 += nh_dec) {
          WorkItem it = proto;
          it.kind = pva::kDecode;
          it.q_row_begin = 0;
          it.q_rows = 1;
          it.head_begin = h0;
          it.heads = nh_dec;
          it.kv_head = h0 / pr.group;
          const int32_t kv_begin = visible_begin(proto, 0, pr.window);
          const int32_t kv_end = std::max(kv_begin, visible_end(proto, 0, 1, causal));
          emit_split(plan, plan.decode, it, kv_begin, kv_end, dchunk);
          plan.visited_pairs_x_heads += (int64_t)(kv_end - kv_begin) * nh_dec;
        }
        continue;
      }
      for (int32_t r0 = 0; r0 < proto.len_q; r0 += rows_per_item) {
        const int32_t rows = std::min(rows_per_item, proto.len_q - r0);
        const int32_t kv_begin = visible_begin(proto, r0, pr.window);
        const int32_t kv_end = std::max(kv_begin, visible_end(proto, r0, rows, causal));
        for (int32_t h0 = 0; h0 < pr.hq; h0 += nh) {
          WorkItem it = proto;
          it.q_row_begin = r0;
          it.q_rows = rows;
          it.head_begin = h0;
          it.heads = nh;
          it.kv_head = h0 / pr.group;
          emit_split(plan, plan.prefill, it, kv_begin, kv_end,
                     pchunk > 0 ? pchunk : std::max<int32_t>(kv_end - kv_begin, 1));
          plan.visited_pairs_x_heads += (int64_t)rows * (kv_end - kv_begin) * nh;
        }
      }
    }
    // Item order. The dispatcher hands out workgroups in index order and
    // deals them to the eight XCDs round-robin (index i to XCD i % 8).
    // Prefill: sequences by their longest item first (most of the greedy
    // longest-processing-time effect), then a sequence's row blocks from the
    // last (longest key range) to the first, head groups innermost. Items i
    // and i + 8 then read the same kv head's K/V over neighbouring row blocks
    // of one sequence and run at about the same time on one XCD, so one L2
    // serves both.
    std::vector<int64_t> seq_top(pr.batch, 0);
    for (const WorkItem& it : plan.prefill)
      seq_top[it.seq] = std::max(seq_top[it.seq], (int64_t)(it.kv_end - it.kv_begin) * it.q_rows);
    std::stable_sort(plan.prefill.begin(), plan.prefill.end(), [&](const WorkItem& a, const WorkItem& b) {
      if (seq_top[a.seq] != seq_top[b.seq]) return seq_top[a.seq] > seq_top[b.seq];
      if (a.seq != b.seq) return a.seq < b.seq;
      if (a.q_row_begin != b.q_row_begin) return a.q_row_begin > b.q_row_begin;
      if (a.kv_begin != b.kv_begin) return a.kv_begin < b.kv_begin;
      return a.head_begin < b.head_begin;
    });
    // Split-KV decode: longest first (equal chunks, then the shorter last
    // splits in decreasing length).
    std::stable_sort(plan.decode.begin(), plan.decode.end(), [](const WorkItem& a, const WorkItem& b) {
      return (int64_t)(a.kv_end - a.kv_begin) * a.q_rows > (int64_t)(b.kv_end - b.kv_begin) * b.q_rows;
    });
  }
  return VARLEN_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
  size_t items_off, lse_off, po_off, total;
  size_t n_items;
};

Layout layout_of(const Plan& plan, int32_t dv) {
  Layout l;
  l.n_items = plan.prefill.size() + plan.f32.size() + plan.decode.size() + plan.combine.size();
  l.items_off = 0;
  l.lse_off = align_up(l.n_items * sizeof(WorkItem), 256);
  l.po_off = align_up(l.lse_off + (size_t)plan.n_partials * sizeof(float), 256);
  l.total = align_up(l.po_off + (size_t)plan.n_partials * (size_t)dv * sizeof(float), 256);
  return l;
}

// ---------------------------------------------------------------------------
// Device-built work list: item shapes (the host scheduler's), list bounds
// that size the launch grids, and the caller's workspace layout.
// ---------------------------------------------------------------------------
struct DeviceShape {
  int nh = 1, rows_per_item = 32, prefill_kind = pva::kPrefillMfma, waves = 4;
  int nh_dec = 1, use_decode = 0;
  int64_t cap_prefill = 0, cap_decode = 0, cap_combine = 0, cap_partials = 0;
  size_t hdr_off = 0, seq_off = 0, pre_off = 0, dec_off = 0, cmb_off = 0, lse_off = 0, po_off = 0, total = 0;
};

DeviceShape device_shape(const Problem& pr, bool allow_decode = true) {
  DeviceShape d;
  const int64_t B = pr.batch;
  if (pr.dtype == VARLEN_F32) {
    d.nh = 1;
    d.rows_per_item = 32;
    d.prefill_kind = pva::kPrefillF32;
    d.waves = 4;
    d.use_decode = 0;
  } else {
    d.nh = largest_pow2_divisor_upto(pr.group, 8);
    const int rblocks = d.nh >= 4 ? 1 : 4 / d.nh;
    d.rows_per_item = 32 * rblocks;
    d.waves = d.nh * rblocks;
    d.nh_dec = largest_pow2_divisor_upto(pr.group, 16);
    d.use_decode = allow_decode ? 1 : 0;
  }
  // These bounds size the launch grids (workgroups past the device-built
  // count return at once), so they are kept tight. Prefill: every prefill
  // sequence adds at most one partial row block, and with the decode path a
  // prefill sequence has at least two rows.
  const int64_t n_pre_seq = std::min<int64_t>(B, d.use_decode ? pr.total_q / 2 : pr.total_q);
  d.cap_prefill = ((pr.total_q + d.rows_per_item - 1) / d.rows_per_item + n_pre_seq) * (pr.hq / d.nh);
  if (d.use_decode) {
    // A decode sequence has one row, so there are at most min(B, total_q).
    // The split-KV chunk c is at least 512 and at least ceil(decode keys *
    // groups / 2048) unless clamped to 8192, so the splits of one head group
    // number at most decode keys / c + (decode sequences) with decode keys / c
    // <= min(total_kv / 512, max(2048 / groups, total_kv / 8192)).
    const int64_t g = pr.hq / d.nh_dec;
    const int64_t n_dec_seq = std::min<int64_t>(B, pr.total_q);
    const int64_t per_chunk = std::min<int64_t>((pr.total_kv + 511) / 512,
                                                std::max<int64_t>((2048 + g - 1) / g, (pr.total_kv + 8191) / 8192));
    d.cap_decode = g * (per_chunk + 1 + n_dec_seq);
    d.cap_combine = g * n_dec_seq;
    d.cap_partials = d.cap_decode * d.nh_dec;
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  d.hdr_off = take(sizeof(int32_t) * pva::kHdrInts);
  d.seq_off = take(sizeof(int32_t) * 7 * (size_t)(B + 1));
  d.pre_off = take(sizeof(WorkItem) * (size_t)d.cap_prefill);
  d.dec_off = take(sizeof(WorkItem) * (size_t)d.cap_decode);
  d.cmb_off = take(sizeof(WorkItem) * (size_t)d.cap_combine);
  d.lse_off = take(sizeof(float) * (size_t)d.cap_partials);
  d.po_off = take(sizeof(float) * (size_t)d.cap_partials * (size_t)pr.dv);
  d.total = off;
  return d;
}

// ---------------------------------------------------------------------------
// Per-device workspace.
// ---------------------------------------------------------------------------
struct DeviceState {
  std::mutex mu;
  void* dev = nullptr;
  size_t dev_cap = 0;
  void* host = nullptr;  // pinned staging of the work list
  size_t host_cap = 0;
  hipEvent_t copied = nullptr;  // after the last work-list upload
  hipEvent_t done = nullptr;    // after the last call's kernels
  bool pending = false;
  // device path, decode-dominated batches: decode + combine run on `side`
  // beside prefill (fork/join)
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // device address of this GPU's copy of `scratch` (the allocation-free
  // call), looked up once; the memory lives until the process ends
  void* scratch = nullptr;
};

// New capacity of a grow-only buffer that holds `old_cap` bytes and must
// hold `need`: at least twice the old capacity.
size_t grown_capacity(size_t old_cap, size_t need) { return std::max(need, old_cap * 2); }

constexpr int kMaxDevices = 64;
DeviceState g_dev[kMaxDevices];

// ---------------------------------------------------------------------------
// Optional kernel timing (HIP events around each launch, on its stream).
// ---------------------------------------------------------------------------
// Set for the duration of varlen_attn_fwd_device_noalloc on its thread: no
// timing events are made or recorded (an event pool may have to grow).
thread_local bool g_no_alloc_call = false;

struct ProfRecord {
  int kind;
  int64_t items;
  hipEvent_t start, end;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof_pending;
varlen_attn_profile_t g_prof_totals;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` between two recorded events when profiling is on.
template <class F>
hipError_t timed(int kind, int64_t items, hipStream_t s, F&& launch) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    on = g_prof_on;
  }
  if (!on || items <= 0 || g_no_alloc_call) return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    a = prof_event();
    b = prof_event();
  }
  if (!a || !b) return launch();
  hipError_t e = hipEventRecord(a, s);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, s);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (e == hipSuccess) {
    g_prof_pending.push_back({kind, items, a, b});
  } else {
    g_prof_pool.push_back(a);
    g_prof_pool.push_back(b);
  }
  return e;
}

varlen_status_t hip_fail(hipError_t e, const char* what) {
  return fail(e == hipErrorOutOfMemory ? VARLEN_ERR_OUT_OF_MEMORY : VARLEN_ERR_DEVICE, "%s failed: %s", what,
              hipGetErrorString(e));
}

#define PVA_HIP(call, what)                        \
  do {                                             \
    hipError_t e_ = (call);                        \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

varlen_status_t run(const void* q, const void* k, const void* v, const int32_t* cu_q_dev,
                    const int32_t* cu_kv_dev, const int32_t* cu_q_host, const int32_t* cu_kv_host,
                    int32_t batch, int64_t total_q, int64_t total_kv, int32_t num_heads,
                    int32_t kv_num_heads, int32_t head_dim, int32_t v_head_dim, int32_t dtype,
                    float scale, int32_t is_causal, float softcap, void* out, void* stream_v,
                    const varlen_attn_options_t* options) {
  g_last_error.clear();
  Problem pr;
  varlen_status_t st = check_scalars(batch, total_q, total_kv, num_heads, kv_num_heads, head_dim, v_head_dim,
                                     dtype, scale, softcap, &pr);
  if (st != VARLEN_OK) return st;
  pr.causal = is_causal != 0;
  if ((st = check_window(options ? options->local_window : 0, &pr)) != VARLEN_OK) return st;
  if (total_q > 0 && (!q || !out))
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "query and output pointers must be non-null");
  if (total_kv > 0 && (!k || !v))
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "key and value pointers must be non-null");
  hipStream_t stream = static_cast<hipStream_t>(stream_v);

  // The cu arrays on the host: the caller's mirrors, or a copy of the
  // device arrays (the one synchronising case).
  std::vector<int32_t> cuq_copy, cukv_copy;
  if (!cu_q_host || !cu_kv_host) {
    if (!cu_q_dev || !cu_kv_dev)
      return fail(VARLEN_ERR_INVALID_ARGUMENT, "cu_seqlens_q/cu_seqlens_kv: need device arrays or host mirrors");
    cuq_copy.resize(batch + 1);
    cukv_copy.resize(batch + 1);
    PVA_HIP(hipMemcpyAsync(cuq_copy.data(), cu_q_dev, sizeof(int32_t) * (batch + 1), hipMemcpyDeviceToHost, stream),
            "reading cu_seqlens_q");
    PVA_HIP(hipMemcpyAsync(cukv_copy.data(), cu_kv_dev, sizeof(int32_t) * (batch + 1), hipMemcpyDeviceToHost,
                           stream),
            "reading cu_seqlens_kv");
    PVA_HIP(hipStreamSynchronize(stream), "synchronising after reading cu_seqlens");
    cu_q_host = cuq_copy.data();
    cu_kv_host = cukv_copy.data();
  }
  if ((st = check_cu(cu_q_host, batch, total_q, "cu_seqlens_q")) != VARLEN_OK) return st;
  if ((st = check_cu(cu_kv_host, batch, total_kv, "cu_seqlens_kv")) != VARLEN_OK) return st;
  if ((st = check_supported(pr)) != VARLEN_OK) return st;
  pr.cu_q = cu_q_host;
  pr.cu_kv = cu_kv_host;
  if (total_q == 0) return VARLEN_OK;
  if ((st = check_aligned(pr, q, k, v, out)) != VARLEN_OK) return st;

  Plan plan;
  if ((st = build_plan(pr, resolve_options(options), plan)) != VARLEN_OK) return st;
  const Layout lay = layout_of(plan, pr.dv);

  int dev_id = 0;
  PVA_HIP(hipGetDevice(&dev_id), "hipGetDevice");
  if (dev_id < 0 || dev_id >= kMaxDevices) return fail(VARLEN_ERR_DEVICE, "device index %d out of range", dev_id);
  DeviceState& ds = g_dev[dev_id];
  std::lock_guard<std::mutex> lock(ds.mu);

  if (!ds.copied) {
    PVA_HIP(hipEventCreateWithFlags(&ds.copied, hipEventDisableTiming), "hipEventCreate");
    PVA_HIP(hipEventCreateWithFlags(&ds.done, hipEventDisableTiming), "hipEventCreate");
  }
  // The previous call may still be reading the staging buffer (upload) or
  // the device workspace (kernels on another stream).
  if (ds.pending) {
    PVA_HIP(hipEventSynchronize(ds.copied), "waiting for the previous work-list upload");
    PVA_HIP(hipStreamWaitEvent(stream, ds.done, 0), "ordering after the previous call");
  }
  const size_t item_bytes = lay.n_items * sizeof(WorkItem);
  // Both buffers grow to at least twice their previous size, so a run of
  // slightly larger calls reallocates O(log n) times, not once per call.
  if (lay.total > ds.dev_cap) {
    const size_t cap = grown_capacity(ds.dev_cap, lay.total);
    if (ds.dev) {
      PVA_HIP(hipEventSynchronize(ds.done), "waiting before growing the workspace");
      PVA_HIP(hipFree(ds.dev), "hipFree");
      ds.dev = nullptr;
      ds.dev_cap = 0;
    }
    PVA_HIP(hipMalloc(&ds.dev, cap), "allocating the workspace");
    ds.dev_cap = cap;
  }
  if (item_bytes > ds.host_cap) {
    const size_t cap = grown_capacity(ds.host_cap, item_bytes);
    if (ds.host) {
      PVA_HIP(hipHostFree(ds.host), "hipHostFree");
      ds.host = nullptr;
      ds.host_cap = 0;
    }
    PVA_HIP(hipHostMalloc(&ds.host, cap, hipHostMallocDefault), "allocating the pinned staging buffer");
    ds.host_cap = cap;
  }
  WorkItem* stage = static_cast<WorkItem*>(ds.host);
  size_t pos = 0;
  const size_t off_prefill = pos;
  std::memcpy(stage + pos, plan.prefill.data(), plan.prefill.size() * sizeof(WorkItem));
  pos += plan.prefill.size();
  const size_t off_decode = pos;
  std::memcpy(stage + pos, plan.decode.data(), plan.decode.size() * sizeof(WorkItem));
  pos += plan.decode.size();
  const size_t off_f32 = pos;
  std::memcpy(stage + pos, plan.f32.data(), plan.f32.size() * sizeof(WorkItem));
  pos += plan.f32.size();
  const size_t off_combine = pos;
  std::memcpy(stage + pos, plan.combine.data(), plan.combine.size() * sizeof(WorkItem));
  pos += plan.combine.size();

  char* base = static_cast<char*>(ds.dev);
  WorkItem* dev_items = reinterpret_cast<WorkItem*>(base + lay.items_off);
  PVA_HIP(timed(4, (int64_t)item_bytes, stream,
                [&] { return hipMemcpyAsync(dev_items, stage, item_bytes, hipMemcpyHostToDevice, stream); }),
          "uploading the work list");
  PVA_HIP(hipEventRecord(ds.copied, stream), "hipEventRecord");
  ds.pending = true;

  pva::Params p;
  std::memset(&p, 0, sizeof p);
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.part_lse = reinterpret_cast<float*>(base + lay.lse_off);
  p.part_o = reinterpret_cast<float*>(base + lay.po_off);
  p.hq = pr.hq;
  p.hkv = pr.hkv;
  p.group = pr.group;
  p.d = pr.d;
  p.dv = pr.dv;
  p.causal = pr.causal;
  p.window = pr.window;
  p.softcap_on = pr.softcap != 0.f;
  const float log2e = 1.4426950408889634f;
  p.scale = pr.scale;
  p.softcap = pr.softcap;
  p.score_log2 = pr.scale * log2e;
  if (p.softcap_on) {
    p.cap_log2 = pr.softcap * log2e;
    p.tanh_log2 = 2.f * pr.scale / pr.softcap * log2e;
  }

  const int n_pre = (int)plan.prefill.size(), n_dec = (int)plan.decode.size();
  const int n_f32 = (int)plan.f32.size(), n_cmb = (int)plan.combine.size();
  hipError_t e = timed(0, n_pre, stream, [&] {
    return pva::launch_prefill_mfma(p, dev_items + off_prefill, n_pre, pr.dtype, plan.prefill_waves, stream);
  });
  if (e == hipSuccess)
    e = timed(2, n_dec, stream, [&] { return pva::launch_decode(p, dev_items + off_decode, n_dec, pr.dtype, stream); });
  if (e == hipSuccess)
    e = timed(1, n_f32, stream, [&] { return pva::launch_prefill_f32(p, dev_items + off_f32, n_f32, stream); });
  if (e == hipSuccess)
    e = timed(3, n_cmb, stream, [&] { return pva::launch_combine(p, dev_items + off_combine, n_cmb, pr.dtype, stream); });
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  PVA_HIP(hipEventRecord(ds.done, stream), "hipEventRecord");
  return VARLEN_OK;
}

// The capture-safe call: no host copy of the cu arrays, no synchronisation,
// no allocation, no host-to-device copy. The work list is built on the device
// into the caller's workspace; total_q / total_kv are the rows of the q/out
// and k/v buffers.
varlen_status_t run_device(const void* q, const void* k, const void* v, const int32_t* cu_q_dev,
                           const int32_t* cu_kv_dev, int32_t batch, int64_t total_q, int64_t total_kv,
                           int32_t num_heads, int32_t kv_num_heads, int32_t head_dim, int32_t v_head_dim,
                           int32_t dtype, float scale, int32_t is_causal, float softcap, int32_t local_window,
                           void* out, void* workspace, size_t workspace_bytes, int32_t* latch, void* stream_v,
                           const int32_t* kv_len_dev = nullptr, int32_t kv_capacity = 0,
                           bool allow_decode = true, bool no_alloc = false) {
  g_last_error.clear();
  Problem pr;
  varlen_status_t st = check_scalars(batch, total_q, total_kv, num_heads, kv_num_heads, head_dim, v_head_dim,
                                     dtype, scale, softcap, &pr);
  if (st != VARLEN_OK) return st;
  pr.causal = is_causal != 0;
  if ((st = check_window(local_window, &pr)) != VARLEN_OK) return st;
  if ((st = check_supported(pr)) != VARLEN_OK) return st;
  if (!cu_q_dev || !(cu_kv_dev || kv_len_dev) || !latch)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "device cu_seqlens arrays and the error latch must be non-null");
  if (total_q > 0 && (!q || !out))
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "query and output pointers must be non-null");
  if (total_kv > 0 && (!k || !v))
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "key and value pointers must be non-null");
  if ((st = check_aligned(pr, q, k, v, out)) != VARLEN_OK) return st;
  const DeviceShape sh = device_shape(pr, allow_decode);
  if (!workspace || workspace_bytes < sh.total)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "workspace holds %zu bytes, the call needs %zu (varlen_attn_device_workspace_bytes)",
                workspace ? workspace_bytes : (size_t)0, sh.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (sh.cap_prefill + sh.cap_combine > INT32_MAX || sh.cap_decode > INT32_MAX || sh.cap_partials > INT32_MAX)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "the batch is too large for one launch");
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  char* ws = static_cast<char*>(workspace);

  pva::DevicePlan dp;
  std::memset(&dp, 0, sizeof dp);
  dp.batch = pr.batch;
  dp.hq = pr.hq;
  dp.group = pr.group;
  dp.nh = sh.nh;
  dp.rows_per_item = sh.rows_per_item;
  dp.prefill_kind = sh.prefill_kind;
  dp.nh_dec = sh.nh_dec;
  dp.use_decode = sh.use_decode;
  dp.causal = pr.causal;
  dp.window = pr.window;
  dp.cap_q = (int32_t)total_q;
  dp.cap_kv = (int32_t)total_kv;
  dp.kv_len = kv_len_dev;
  dp.kv_capacity = kv_capacity;
  dp.cap_prefill = sh.cap_prefill;
  dp.cap_decode = sh.cap_decode;
  dp.cap_combine = sh.cap_combine;
  dp.cap_partials = sh.cap_partials;
  dp.header = reinterpret_cast<int32_t*>(ws + sh.hdr_off);
  int32_t* seq = reinterpret_cast<int32_t*>(ws + sh.seq_off);
  const int64_t nb = (int64_t)pr.batch + 1;
  dp.seq_q = seq;
  dp.seq_kv = seq + nb;
  dp.seq_pre = seq + 2 * nb;
  dp.seq_decf = seq + 3 * nb;
  dp.seq_decp = seq + 4 * nb;
  dp.seq_cmb = seq + 5 * nb;
  dp.seq_part = seq + 6 * nb;
  dp.prefill = reinterpret_cast<WorkItem*>(ws + sh.pre_off);
  dp.decode = reinterpret_cast<WorkItem*>(ws + sh.dec_off);
  dp.combine = reinterpret_cast<WorkItem*>(ws + sh.cmb_off);

  pva::Params p;
  std::memset(&p, 0, sizeof p);
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.part_lse = reinterpret_cast<float*>(ws + sh.lse_off);
  p.part_o = reinterpret_cast<float*>(ws + sh.po_off);
  p.hq = pr.hq;
  p.hkv = pr.hkv;
  p.group = pr.group;
  p.d = pr.d;
  p.dv = pr.dv;
  p.causal = pr.causal;
  p.window = pr.window;
  p.softcap_on = pr.softcap != 0.f;
  const float log2e = 1.4426950408889634f;
  p.scale = pr.scale;
  p.softcap = pr.softcap;
  p.score_log2 = pr.scale * log2e;
  if (p.softcap_on) {
    p.cap_log2 = pr.softcap * log2e;
    p.tanh_log2 = 2.f * pr.scale / pr.softcap * log2e;
  }

  // Two launch forms.
  //  * Decode-dominated batches (no more query rows than sequences): decode
  //    + combine run on a side stream beside the (at most small) prefill
  //    launch, a fork after the scheduler and a join before the call
  //    returns, so decode starts right after the scheduler while the mostly
  //    empty prefill grid drains beside it (measured +2.4 % on the packed
  //    decode workload against one stream). The side stream and its two
  //    events are made once per device, outside any graph capture.
  //  * Other batches, on one stream: scheduler, decode, then the prefill
  //    launch, whose workgroups past the prefill grid run the combine items
  //    (the decode partials they merge are complete by then). That saves a
  //    launch whose list is empty in a prefill batch. (The side form would
  //    let an empty decode grid's early-exit workgroups take dispatch slots
  //    beside prefill and shift its XCD-aware item order: -2 % measured.)
  // The allocation-free call always takes the one-stream form: making the
  // side stream and its events would allocate.
  std::unique_lock<std::mutex> side_lock;
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  if (!no_alloc && sh.cap_prefill > 0 && sh.cap_decode > 0 && total_q <= batch) {
    int dev_id = 0;
    PVA_HIP(hipGetDevice(&dev_id), "hipGetDevice");
    if (dev_id >= 0 && dev_id < kMaxDevices) {
      DeviceState& ds = g_dev[dev_id];
      side_lock = std::unique_lock<std::mutex>(ds.mu);
      if (!ds.side) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) {
          hipStream_t st = nullptr;
          hipEvent_t f = nullptr, j = nullptr;
          if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&f, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&j, hipEventDisableTiming) == hipSuccess) {
            ds.side = st;
            ds.fork = f;
            ds.join = j;
          } else {  // no side stream: the one-stream form
            if (f) (void)hipEventDestroy(f);
            if (j) (void)hipEventDestroy(j);
            if (st) (void)hipStreamDestroy(st);
          }
        }
      }
      side = ds.side;
      fork_ev = ds.fork;
      join_ev = ds.join;
    }
  }

  hipError_t e = timed(5, 1, stream, [&] { return pva::launch_plan(dp, cu_q_dev, cu_kv_dev, latch, stream); });
  auto launch_decode_on = [&](hipStream_t s) {
    if (sh.cap_decode <= 0) return hipSuccess;
    pva::Params pd = p;
    pd.item_count = dp.header + pva::kHdrDecode;
    return timed(2, sh.cap_decode, s,
                 [&] { return pva::launch_decode(pd, dp.decode, (int)sh.cap_decode, pr.dtype, s); });
  };
  if (side) {
    if (e == hipSuccess) e = hipEventRecord(fork_ev, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(side, fork_ev, 0);
    if (e == hipSuccess) e = launch_decode_on(side);
    if (e == hipSuccess && sh.cap_combine > 0) {
      pva::Params pc = p;
      pc.item_count = dp.header + pva::kHdrCombine;
      e = timed(3, sh.cap_combine, side,
                [&] { return pva::launch_combine(pc, dp.combine, (int)sh.cap_combine, pr.dtype, side); });
    }
    if (e == hipSuccess) e = hipEventRecord(join_ev, side);
  } else if (e == hipSuccess) {
    e = launch_decode_on(stream);
  }
  if (e == hipSuccess && pr.dtype == VARLEN_F32) {
    // the fp32 path has no split work (no decode items, no prefill splits)
    if (sh.cap_combine > 0) return fail(VARLEN_ERR_DEVICE, "internal: fp32 work list with combine items");
    if (sh.cap_prefill > 0) {
      pva::Params pp = p;
      pp.item_count = dp.header + pva::kHdrPrefill;
      e = timed(1, sh.cap_prefill, stream,
                [&] { return pva::launch_prefill_f32(pp, dp.prefill, (int)sh.cap_prefill, stream); });
    }
  } else if (e == hipSuccess) {
    pva::Params pp = p;
    pp.item_count = dp.header + pva::kHdrPrefill;
    int64_t grid = sh.cap_prefill;
    if (!side && sh.cap_combine > 0) {
      pp.combine_items = dp.combine;
      pp.combine_count = dp.header + pva::kHdrCombine;
      pp.prefill_grid = (int32_t)sh.cap_prefill;
      grid += sh.cap_combine;
    }
    if (grid > 0)
      e = timed(0, grid, stream,
                [&] { return pva::launch_prefill_mfma(pp, dp.prefill, (int)grid, pr.dtype, sh.waves, stream); });
  }
  if (e == hipSuccess && side) e = hipStreamWaitEvent(stream, join_ev, 0);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return VARLEN_OK;
}

// Device address of the current GPU's copy of `scratch`, looked up once per
// device (the first allocation-free call on it).
varlen_status_t noalloc_scratch(void** ptr) {
  int dev_id = 0;
  PVA_HIP(hipGetDevice(&dev_id), "hipGetDevice");
  if (dev_id < 0 || dev_id >= kMaxDevices) return fail(VARLEN_ERR_DEVICE, "device index %d out of range", dev_id);
  DeviceState& ds = g_dev[dev_id];
  std::lock_guard<std::mutex> lock(ds.mu);
  if (!ds.scratch) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(VARLEN_ERR_DEVICE, "hipGetSymbolAddress(scratch) gave a null address");
    ds.scratch = p;
  }
  *ptr = ds.scratch;
  return VARLEN_OK;
}

// Clears the allocation-free flag when the call returns.
struct NoAllocCall {
  NoAllocCall() { g_no_alloc_call = true; }
  ~NoAllocCall() { g_no_alloc_call = false; }
};

}  // namespace

extern "C" {

varlen_status_t varlen_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_kv, const int32_t* cu_seqlens_q_host,
                                const int32_t* cu_seqlens_kv_host, int32_t batch, int64_t total_q,
                                int64_t total_kv, int32_t num_heads, int32_t kv_num_heads, int32_t head_dim,
                                int32_t v_head_dim, int32_t dtype, float scale, int32_t is_causal,
                                float softcap, void* out, void* stream) {
  return run(q, k, v, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_host, cu_seqlens_kv_host, batch, total_q,
             total_kv, num_heads, kv_num_heads, head_dim, v_head_dim, dtype, scale, is_causal, softcap, out, stream,
             nullptr);
}

size_t varlen_attn_device_workspace_bytes(int32_t batch, int64_t total_q, int64_t total_kv, int32_t num_heads,
                                          int32_t kv_num_heads, int32_t head_dim, int32_t v_head_dim,
                                          int32_t dtype) {
  g_last_error.clear();
  Problem pr;
  if (check_scalars(batch, total_q, total_kv, num_heads, kv_num_heads, head_dim, v_head_dim, dtype, 0.f, 0.f,
                    &pr) != VARLEN_OK)
    return 0;
  pr.causal = 0;
  pr.window = 0;
  // enough for either setting of decode_path (varlen_attn_fwd_device_ex)
  return std::max(device_shape(pr).total, device_shape(pr, false).total);
}

varlen_status_t varlen_attn_fwd_device(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_kv, int32_t batch, int64_t total_q,
                                       int64_t total_kv, int32_t num_heads, int32_t kv_num_heads,
                                       int32_t head_dim, int32_t v_head_dim, int32_t dtype, float scale,
                                       int32_t is_causal, float softcap, int32_t local_window, void* out,
                                       void* workspace, size_t workspace_bytes, int32_t* error_latch,
                                       void* stream) {
  return run_device(q, k, v, cu_seqlens_q, cu_seqlens_kv, batch, total_q, total_kv, num_heads, kv_num_heads,
                    head_dim, v_head_dim, dtype, scale, is_causal, softcap, local_window, out, workspace,
                    workspace_bytes, error_latch, stream);
}

varlen_status_t varlen_attn_fwd_device_ex(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                                          const int32_t* cu_seqlens_kv, int32_t batch, int64_t total_q,
                                          int64_t total_kv, int32_t num_heads, int32_t kv_num_heads,
                                          int32_t head_dim, int32_t v_head_dim, int32_t dtype, float scale,
                                          int32_t is_causal, float softcap, int32_t local_window, void* out,
                                          void* workspace, size_t workspace_bytes, int32_t* error_latch,
                                          void* stream, const varlen_attn_options_t* options) {
  g_last_error.clear();
  EntryName name("varlen_attn_fwd_device_ex");
  const Options o = resolve_options(options);
  if (o.decode_chunk != 0 || o.prefill_kv_chunk > 0 || (o.local_window != 0 && o.local_window != -1))
    return fail(VARLEN_ERR_INVALID_ARGUMENT,
                "the device-scheduled call takes only decode_path from the options (decode_chunk %d, "
                "prefill_kv_chunk %d and options.local_window %d must be 0, or -1 for the window; the window is "
                "an argument)",
                o.decode_chunk, o.prefill_kv_chunk, o.local_window);
  if (o.decode_path < 0 || o.decode_path > 2)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "decode_path must be 0, 1 or 2, got %d", o.decode_path);
  return run_device(q, k, v, cu_seqlens_q, cu_seqlens_kv, batch, total_q, total_kv, num_heads, kv_num_heads,
                    head_dim, v_head_dim, dtype, scale, is_causal, softcap, local_window, out, workspace,
                    workspace_bytes, error_latch, stream, nullptr, 0, o.decode_path != 1);
}

varlen_status_t varlen_attn_fwd_device_noalloc(const void* q, const void* k, const void* v,
                                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                               int32_t batch, int64_t total_q, int64_t total_kv, int32_t num_heads,
                                               int32_t kv_num_heads, int32_t head_dim, int32_t v_head_dim,
                                               int32_t dtype, float scale, int32_t is_causal, float softcap,
                                               int32_t local_window, void* out, int32_t* error_latch,
                                               void* stream) {
  g_last_error.clear();
  EntryName name("varlen_attn_fwd_device_noalloc");
  NoAllocCall no_alloc;
  Problem pr;
  varlen_status_t st = check_scalars(batch, total_q, total_kv, num_heads, kv_num_heads, head_dim, v_head_dim,
                                     dtype, scale, softcap, &pr);
  if (st != VARLEN_OK) return st;
  const size_t need = device_shape(pr).total;
  if (need > (size_t)VARLEN_NOALLOC_SCRATCH_BYTES)
    return fail(VARLEN_ERR_INVALID_ARGUMENT,
                "this batch needs %zu bytes of scratch and the allocation-free call holds %zu "
                "(VARLEN_NOALLOC_SCRATCH_BYTES); call varlen_attn_fwd_device with a workspace instead",
                need, (size_t)VARLEN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != VARLEN_OK) return st;
  return run_device(q, k, v, cu_seqlens_q, cu_seqlens_kv, batch, total_q, total_kv, num_heads, kv_num_heads,
                    head_dim, v_head_dim, dtype, scale, is_causal, softcap, local_window, out, ws,
                    (size_t)VARLEN_NOALLOC_SCRATCH_BYTES, error_latch, stream, nullptr, 0, true, true);
}

varlen_status_t varlen_attn_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* cu_seqlens_q, const int32_t* kv_seqlens, int32_t batch,
                                        int64_t total_q, int32_t cache_capacity, int32_t num_heads,
                                        int32_t kv_num_heads, int32_t head_dim, int32_t v_head_dim,
                                        int32_t dtype, float scale, int32_t is_causal, float softcap,
                                        int32_t local_window, void* out, void* workspace,
                                        size_t workspace_bytes, int32_t* error_latch, void* stream) {
  g_last_error.clear();
  EntryName name("varlen_attn_fwd_kvcache");
  if (cache_capacity < 1)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "cache_capacity must be >= 1, got %d", cache_capacity);
  if (batch >= 1 && (int64_t)batch * cache_capacity > INT32_MAX)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "batch * cache_capacity must stay below 2^31 rows, got %d * %d", batch,
                cache_capacity);
  if (!kv_seqlens) return fail(VARLEN_ERR_INVALID_ARGUMENT, "kv_seqlens must be non-null");
  const int64_t rows = batch >= 1 ? (int64_t)batch * cache_capacity : 0;
  return run_device(q, k_cache, v_cache, cu_seqlens_q, nullptr, batch, total_q, rows, num_heads, kv_num_heads,
                    head_dim, v_head_dim, dtype, scale, is_causal, softcap, local_window, out, workspace,
                    workspace_bytes, error_latch, stream, kv_seqlens, cache_capacity);
}

varlen_status_t varlen_kv_append_rope(const void* q, void* q_out, const void* k, const void* v,
                                      int64_t q_row_stride, int64_t k_row_stride, int64_t v_row_stride,
                                      void* k_cache, void* v_cache, const int32_t* cu_seqlens_q,
                                      const int32_t* cache_seqlens, int32_t* kv_seqlens_out,
                                      const float* cos_cache, const float* sin_cache,
                                      const int64_t* position_ids, int32_t batch, int64_t total_q,
                                      int32_t num_heads, int32_t kv_num_heads, int32_t head_dim,
                                      int32_t v_head_dim, int32_t dtype, int32_t cache_capacity,
                                      int32_t rotary_dim, int32_t rotary_rows, int32_t rotary_interleaved,
                                      int32_t* error_latch, void* stream) {
  g_last_error.clear();
  EntryName name("varlen_kv_append_rope");
  Problem pr;
  varlen_status_t st = check_scalars(batch, total_q, 0, num_heads, kv_num_heads, head_dim, v_head_dim, dtype, 0.f,
                                     0.f, &pr);
  if (st != VARLEN_OK) return st;
  if (pr.d % 2 || pr.dv % 2)
    return fail(VARLEN_ERR_UNSUPPORTED, "head_dim and v_head_dim must be even, got %d and %d", pr.d, pr.dv);
  if (cache_capacity < 1)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "cache_capacity must be >= 1, got %d", cache_capacity);
  if ((int64_t)batch * cache_capacity > INT32_MAX)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "batch * cache_capacity must stay below 2^31 rows, got %d * %d", batch,
                cache_capacity);
  if (rotary_dim != 0) {
    if (rotary_dim < 2 || rotary_dim % 2 || rotary_dim > pr.d)
      return fail(VARLEN_ERR_INVALID_ARGUMENT, "rotary_dim must be 0 or even in [2, head_dim=%d], got %d", pr.d,
                  rotary_dim);
    if (rotary_rows < 1 || !cos_cache || !sin_cache)
      return fail(VARLEN_ERR_INVALID_ARGUMENT, "rotation needs cos/sin tables with rotary_rows >= 1 rows");
  }
  if ((q == nullptr) != (q_out == nullptr))
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "q and q_out must both be given or both be null");
  const int64_t qs = q_row_stride ? q_row_stride : (int64_t)pr.hq * pr.d;
  const int64_t ks = k_row_stride ? k_row_stride : (int64_t)pr.hkv * pr.d;
  const int64_t vs = v_row_stride ? v_row_stride : (int64_t)pr.hkv * pr.dv;
  if (qs < (int64_t)pr.hq * pr.d || ks < (int64_t)pr.hkv * pr.d || vs < (int64_t)pr.hkv * pr.dv)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "row strides must cover a row's heads (q %lld, k %lld, v %lld)",
                (long long)qs, (long long)ks, (long long)vs);
  if (q && q_out == q && qs != (int64_t)pr.hq * pr.d)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "in-place rotation (q_out == q) needs dense query rows");
  if (total_q > 0 && (!k || !v))
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "k and v must be non-null when there are new rows");
  if (!k_cache || !v_cache || !cu_seqlens_q || !cache_seqlens || !error_latch)
    return fail(VARLEN_ERR_INVALID_ARGUMENT,
                "the caches, cu_seqlens_q, cache_seqlens and the error latch must be non-null");
  pva::RopeParams rp;
  std::memset(&rp, 0, sizeof rp);
  rp.q = q;
  rp.q_out = q_out;
  rp.k = k;
  rp.v = v;
  rp.k_cache = k_cache;
  rp.v_cache = v_cache;
  rp.cu_q = cu_seqlens_q;
  rp.past = cache_seqlens;
  rp.kv_len_out = kv_seqlens_out;
  rp.cos = rotary_dim ? cos_cache : nullptr;
  rp.sin = rotary_dim ? sin_cache : nullptr;
  rp.pos_ids = position_ids;
  rp.latch = error_latch;
  rp.q_stride = qs;
  rp.k_stride = ks;
  rp.v_stride = vs;
  rp.batch = batch;
  rp.total_q = (int32_t)total_q;
  rp.hq = pr.hq;
  rp.hkv = pr.hkv;
  rp.d = pr.d;
  rp.dv = pr.dv;
  rp.capacity = cache_capacity;
  rp.rot_half = rotary_dim / 2;
  rp.rows = rotary_dim ? rotary_rows : 0;
  rp.interleaved = rotary_interleaved != 0;
  // 16-byte pieces when every row, stride and head size is a whole number
  // of pieces and the rotary dims split into whole pieces (per half for the
  // half-split pairing); one pair per unit otherwise.
  const int el = dtype == VARLEN_F32 ? 4 : 2;
  const int vw = 16 / el;
  auto aligned16 = [](const void* ptr) { return ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % 16 == 0; };
  const bool vec = pr.d % vw == 0 && pr.dv % vw == 0 && qs % vw == 0 && ks % vw == 0 && vs % vw == 0 &&
                   (rotary_interleaved ? rotary_dim % vw == 0 : rotary_dim % (2 * vw) == 0) && aligned16(q) &&
                   aligned16(q_out) && aligned16(k) && aligned16(v) && aligned16(k_cache) && aligned16(v_cache);
  rp.vec = vec;
  if (vec) {
    rp.rot_units = rotary_interleaved ? rotary_dim / vw : rotary_dim / (2 * vw);
    rp.head_units_qk = rp.rot_units + (pr.d - rotary_dim) / vw;
    rp.head_units_v = pr.dv / vw;
    rp.units_q = q ? pr.hq * rp.head_units_qk : 0;
    rp.units_k = pr.hkv * rp.head_units_qk;
    rp.units_row = rp.units_q + rp.units_k + pr.hkv * rp.head_units_v;
  } else {
    rp.units_q = q ? pr.hq * (pr.d / 2) : 0;
    rp.units_k = pr.hkv * (pr.d / 2);
    rp.units_row = rp.units_q + rp.units_k + pr.hkv * (pr.dv / 2);
  }
  const int per_block = pva::rope_units_per_block(vec);
  rp.blocks_per_row = (rp.units_row + per_block - 1) / per_block;
  const int64_t row_blocks = total_q * rp.blocks_per_row;
  if (row_blocks + ((int64_t)batch + 255) / 256 > INT32_MAX)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "too many new rows for one launch");
  rp.row_blocks = (int32_t)row_blocks;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(6, row_blocks + (batch + 255) / 256, s, [&] { return pva::launch_rope_append(rp, dtype, s); });
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return VARLEN_OK;
}

varlen_status_t varlen_attn_fwd_ex(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_kv, const int32_t* cu_seqlens_q_host,
                                   const int32_t* cu_seqlens_kv_host, int32_t batch, int64_t total_q,
                                   int64_t total_kv, int32_t num_heads, int32_t kv_num_heads, int32_t head_dim,
                                   int32_t v_head_dim, int32_t dtype, float scale, int32_t is_causal,
                                   float softcap, void* out, void* stream, const varlen_attn_options_t* options) {
  return run(q, k, v, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_q_host, cu_seqlens_kv_host, batch, total_q,
             total_kv, num_heads, kv_num_heads, head_dim, v_head_dim, dtype, scale, is_causal, softcap, out, stream,
             options);
}

varlen_status_t varlen_attn_plan(const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_kv_host,
                                 int32_t batch, int64_t total_q, int64_t total_kv, int32_t num_heads,
                                 int32_t kv_num_heads, int32_t head_dim, int32_t v_head_dim, int32_t dtype,
                                 float scale, int32_t is_causal, float softcap,
                                 const varlen_attn_options_t* options, varlen_attn_plan_stats_t* stats,
                                 int32_t* items, int64_t items_capacity) {
  g_last_error.clear();
  if (stats) std::memset(stats, 0, sizeof *stats);
  Problem pr;
  varlen_status_t st = check_scalars(batch, total_q, total_kv, num_heads, kv_num_heads, head_dim, v_head_dim,
                                     dtype, scale, softcap, &pr);
  if (st != VARLEN_OK) return st;
  pr.causal = is_causal != 0;
  if ((st = check_window(options ? options->local_window : 0, &pr)) != VARLEN_OK) return st;
  if (!cu_seqlens_q_host || !cu_seqlens_kv_host)
    return fail(VARLEN_ERR_INVALID_ARGUMENT, "varlen_attn_plan needs host cu arrays");
  if ((st = check_cu(cu_seqlens_q_host, batch, total_q, "cu_seqlens_q")) != VARLEN_OK) return st;
  if ((st = check_cu(cu_seqlens_kv_host, batch, total_kv, "cu_seqlens_kv")) != VARLEN_OK) return st;
  if ((st = check_supported(pr)) != VARLEN_OK) return st;
  pr.cu_q = cu_seqlens_q_host;
  pr.cu_kv = cu_seqlens_kv_host;
  Plan plan;
  if (total_q > 0) {
    if ((st = build_plan(pr, resolve_options(options), plan)) != VARLEN_OK) return st;
  } else {
    plan.valid_pairs = 0;
  }
  const Layout lay = layout_of(plan, pr.dv);
  if (stats) {
    stats->n_prefill_items = (int64_t)(plan.prefill.size() + plan.f32.size());
    stats->n_decode_items = (int64_t)plan.decode.size();
    stats->n_combine_items = (int64_t)plan.combine.size();
    stats->n_partials = plan.n_partials;
    stats->valid_pairs = plan.valid_pairs;
    stats->visited_pairs = plan.visited_pairs_x_heads / pr.hq;
    stats->workspace_bytes = total_q > 0 ? (int64_t)lay.total : 0;
    stats->waves_per_prefill_item = plan.prefill_waves;
    stats->heads_per_item = plan.heads_per_item;
  }
  if (items) {
    const int64_t need = (int64_t)lay.n_items * VARLEN_PLAN_ITEM_INTS;
    if (items_capacity < need)
      return fail(VARLEN_ERR_INVALID_ARGUMENT, "item buffer holds %lld int32, the plan needs %lld",
                  (long long)items_capacity, (long long)need);
    int32_t* dst = items;
    for (const auto* vec : {&plan.prefill, &plan.decode, &plan.f32, &plan.combine}) {
      std::memcpy(dst, vec->data(), vec->size() * sizeof(WorkItem));
      dst += vec->size() * VARLEN_PLAN_ITEM_INTS;
    }
  }
  return VARLEN_OK;
}

int64_t varlen_attn_valid_pairs(const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_kv_host,
                                int32_t batch, int32_t is_causal) {
  if (!cu_seqlens_q_host || !cu_seqlens_kv_host || batch < 1) return -1;
  for (int32_t b = 0; b < batch; ++b) {
    if (cu_seqlens_q_host[b + 1] < cu_seqlens_q_host[b] || cu_seqlens_kv_host[b + 1] < cu_seqlens_kv_host[b])
      return -1;
  }
  if (cu_seqlens_q_host[0] != 0 || cu_seqlens_kv_host[0] != 0) return -1;
  return valid_pairs_of(cu_seqlens_q_host, cu_seqlens_kv_host, batch, is_causal != 0, 0);
}

int64_t varlen_attn_valid_pairs_window(const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_kv_host,
                                       int32_t batch, int32_t is_causal, int32_t local_window) {
  if (varlen_attn_valid_pairs(cu_seqlens_q_host, cu_seqlens_kv_host, batch, is_causal) < 0) return -1;
  return valid_pairs_of(cu_seqlens_q_host, cu_seqlens_kv_host, batch, is_causal != 0, local_window);
}

const char* varlen_attn_last_error(void) { return g_last_error.c_str(); }

varlen_status_t varlen_attn_release(void) {
  g_last_error.clear();
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess) n = 0;
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (int d = 0; d < kMaxDevices; ++d) {
    DeviceState& ds = g_dev[d];
    std::lock_guard<std::mutex> lock(ds.mu);
    if (!ds.dev && !ds.host && !ds.copied && !ds.side) continue;
    if (d < n) (void)hipSetDevice(d);
    if (ds.done) (void)hipEventSynchronize(ds.done);
    if (ds.dev) (void)hipFree(ds.dev);
    if (ds.host) (void)hipHostFree(ds.host);
    if (ds.copied) (void)hipEventDestroy(ds.copied);
    if (ds.done) (void)hipEventDestroy(ds.done);
    if (ds.side) {
      (void)hipStreamSynchronize(ds.side);
      (void)hipStreamDestroy(ds.side);
    }
    if (ds.fork) (void)hipEventDestroy(ds.fork);
    if (ds.join) (void)hipEventDestroy(ds.join);
    ds.dev = ds.host = nullptr;
    ds.dev_cap = ds.host_cap = 0;
    ds.copied = ds.done = nullptr;
    ds.side = nullptr;
    ds.fork = ds.join = nullptr;
    ds.pending = false;
  }
  if (n > 0) (void)hipSetDevice(cur);
  return VARLEN_OK;
}

const char* varlen_attn_version(void) { return "0.1.0"; }

varlen_status_t varlen_attn_profile_enable(int32_t enable) {
  g_last_error.clear();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (enable) {
    for (auto& r : g_prof_pending) {
      (void)hipEventSynchronize(r.end);
      g_prof_pool.push_back(r.start);
      g_prof_pool.push_back(r.end);
    }
    g_prof_pending.clear();
    std::memset(&g_prof_totals, 0, sizeof g_prof_totals);
  }
  g_prof_on = enable != 0;
  return VARLEN_OK;
}

varlen_status_t varlen_attn_profile_read(varlen_attn_profile_t* out) {
  g_last_error.clear();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_pending) {
    hipError_t e = hipEventSynchronize(r.end);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.end);
    if (e != hipSuccess) return hip_fail(e, "reading kernel timing events");
    g_prof_totals.total_ms[r.kind] += ms;
    g_prof_totals.launches[r.kind] += 1;
    g_prof_totals.items[r.kind] += r.items;
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.end);
  }
  g_prof_pending.clear();
  if (out) *out = g_prof_totals;
  return VARLEN_OK;
}

}  // extern "C"
