// Flash-style packed varlen attention prefill for gfx950 (bf16 / f16 I/O,
// fp32 accumulation), one workgroup per scheduled work item.
//
// What it computes follows the packed op of the crate onnx-runtime-ep-cuda
// (page src/kernels/packed_varlen_attention.rs: module doc "Packed layout &
// cumulative offsets", "Schema (v1)", "Causal alignment"; the row kernel's
// stages: scores, softcap, causal mask, stable softmax, P.V). The pages' own
// kernel materialises each row's scores and runs the softmax in one thread;
// here the same result is reached with an online (running max / running sum)
// softmax over key tiles, which the pages name as the intended follow-up
// (module doc "Correctness-first scope").
//
// Work item: one sequence, up to 32*R consecutive query rows, NH query heads
// of one kv head (NH * R waves of 64 lanes), keys [kv_begin, kv_end).
// Each wave owns one query head and 32 query rows. Per key tile of 64 keys:
//   * the workgroup streams K and V from HBM straight into LDS (global_load_lds,
//     no staging registers) in the blocked layout of prefill_tiles.h: loads
//     coalesce, neither the K fragment reads nor the V transpose reads
//     collide in LDS banks, and every fragment read is a per-lane base plus
//     an immediate offset; double-buffered, once for all NH heads of the
//     group (the GQA reuse); one barrier per tile;
//   * S^T = K . Q^T on 32x32x16 MFMA: lane l then holds 32 scores of query
//     row l%32, so a row's max / sum need one exchange between lane halves
//     (v_permlane32_swap);
//   * softcap c*tanh(s/c) (the row kernel's softcap stage): on a tile whose
//     scores all have |s/c| <= 1/4, as s*(1 - x^2/3 + 2x^4/15), x = s/c, in
//     packed f16 (one transcendental per score); otherwise the exact form
//     from 2^x and a reciprocal;
//   * the mask only on tiles that cross kv_end, the causal frontier or a
//     window edge for some row of the workgroup (an item's first tile, too,
//     only when some row does not see all of it);
//   * softmax in registers in log2 units (exp2 with log2(e) folded into the
//     scale). Each row's first tile fixes a reference max and every later P
//     is taken against it, so O is never rescaled and no tile max is taken
//     inside the loop: bf16 P and the fp32 accumulators have fp32's exponent
//     range. A workgroup whose l or O overflowed (scores rising ~2^127 above
//     the first tile's, or ~2^16 for f16 P) redoes its item with the textbook
//     running-max softmax. Either way the result is the same softmax up to
//     rounding;
//   * O^T += V^T . P^T on 32x32x16 MFMA, P rounded to the I/O type with the
//     score accumulator registers reused directly as the B operand (the
//     MFMA reduction order over keys is free, so V^T is read in the order
//     the score layout leaves the keys in), V^T fragments gathered from the
//     [key][d] tile with the LDS transpose read; the row sum l is taken from
//     the same rounded P (v_dot2), so numerator and denominator agree.
// The normalised output goes through LDS (each wave's 32 x DV tile, in the
// bytes the key tiles used) so that the stores cover whole rows, and is
// written with the nontemporal hint: it is never read again here. Rows of
// the tile that lie past the sequence are never stored; keys at or past
// kv_end are zero-filled in LDS (so data of the next sequence can never
// reach a product) and masked.
#include <climits>
#include <type_traits>

#include "combine.h"
#include "common.h"
#include "prefill_tiles.h"

namespace pva {

template <int D, int DV, bool BF16, int NW, bool SOFTCAP>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(Params p, const WorkItem* __restrict__ items) {
  constexpr int BN = 64;  // keys per tile
  using KL = TileLayout<D>;
  using VL = TileLayout<DV>;
  static_assert(KL::BLOCKS % NW == 0 && VL::BLOCKS % NW == 0, "tile blocks must split evenly over the waves");
  constexpr int KBPW = KL::BLOCKS / NW;  // 1 KB load blocks per wave per tile
  constexpr int VBPW = VL::BLOCKS / NW;

  // K0 K1 V0 V1 in the blocked layout of TileLayout. After the key loop the
  // same bytes stage each wave's 32 x DV output tile (OST elements per wave).
  constexpr int OST = 32 * DV;
  constexpr int LDS_ELEMS = (2 * KL::TILE + 2 * VL::TILE) > NW * OST ? (2 * KL::TILE + 2 * VL::TILE) : NW * OST;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
  constexpr int V0 = 2 * KL::TILE;  // first V buffer

  // Device path: workgroups past the prefill grid run the combine items
  // (their split-KV partials are complete: decode ran before this launch).
  if (p.combine_items && (int)blockIdx.x >= p.prefill_grid) {
    const int ci = (int)blockIdx.x - p.prefill_grid;
    if (ci < *p.combine_count) combine_item<BF16 ? kBF16 : kF16>(p, p.combine_items[ci]);
    return;
  }
  if (p.item_count && (int)blockIdx.x >= *p.item_count) return;
  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int half = lane >> 5;
  const int l32 = lane & 31;
  // it.heads is a power of two (the schedulers take the largest one that
  // divides the GQA group, up to 8): no division at item start
  const int hh = wave & (it.heads - 1);
  const int rb = wave >> __builtin_ctz(it.heads);
  const int head = it.head_begin + hh;
  const int g = it.kv_head;
  const int row0 = rb * 32;
  const int my_row = row0 + l32;
  const bool row_ok = my_row < it.q_rows;
  const int i_local = it.q_row_begin + my_row;
  const int off = it.len_kv - it.len_q;
  const bool wave_active = row0 < it.q_rows;
  const int wave_first = it.q_row_begin + row0;
  const int wave_last = it.q_row_begin + min(row0 + 31, it.q_rows - 1);
  // Keys this lane's row may see: [key_lo, key_hi] (tail-aligned causal
  // bound, local window of p.window keys ending at the diagonal, kv_end).
  const int key_hi = p.causal ? min(it.kv_end - 1, i_local + off) : it.kv_end - 1;
  const int key_lo = p.window > 0 ? i_local + off + 1 - p.window : INT_MIN;
  const int kv_begin = it.kv_begin;
  const int kv_end = it.kv_end;
  const int64_t tok = (int64_t)it.q_token0 + it.q_row_begin + my_row;
  // Short-series softcap (see the tile body): x = a * cap_k for a raw score
  // a, usable while x^2 <= 1/16. The series is even in x, so a negative cap
  // takes it too.
  const float cap_kf = SOFTCAP ? p.scale / p.softcap : 0.f;
  const f16x2_t cap_k = {(_Float16)cap_kf, (_Float16)cap_kf};
  const f16x2_t cap_c1 = {(_Float16)(-1.f / 3.f), (_Float16)(-1.f / 3.f)};
  const f16x2_t cap_c2 = {(_Float16)(2.f / 15.f), (_Float16)(2.f / 15.f)};

  // Q fragments, the B operand of S^T = K Q^T: lane l supplies query row
  // l%32 at head dims 16*kk + 8*half + 0..7.
  // (one masked region for all of them: rows past the tile load nothing)
  u32x4_t qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) qf[kk] = u32x4_t{0u, 0u, 0u, 0u};
  if (row_ok) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        static_cast<const uint16_t*>(p.q) + (tok * p.hq + head) * D);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = src[2 * kk + half];
  }

  f32x16_t oacc[DV / 32];
#pragma unroll
  for (int mb = 0; mb < DV / 32; ++mb) oacc[mb] = f32x16_t{};
  float m_ref = ninf();  // reference max of the row (log2 units)
  float l_run = 0.f;     // this lane's half of the row sum

  // ---- HBM -> LDS tile loads ------------------------------------------------
  // Wave w fills 1 KB blocks w, w + NW, ... of each tile; lane L of a block
  // lands in slot L of it and so fetches the (row, chunk) the layout puts
  // there.
  const int64_t k_stride = (int64_t)p.hkv * D;   // elements between consecutive tokens
  const int64_t v_stride = (int64_t)p.hkv * DV;
  const char* kbase = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.k) +
                                                    ((int64_t)it.kv_token0 * p.hkv + g) * D);
  const char* vbase = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.v) +
                                                    ((int64_t)it.kv_token0 * p.hkv + g) * DV);
  const int k_row = KL::load_row(wave, lane);  // row in this wave's first K block
  const int v_row = VL::load_row(wave, lane);
  const uint32_t k_off = (uint32_t)((k_row * k_stride + KL::load_chunk(lane) * 8) * 2);
  const uint32_t v_off = (uint32_t)((v_row * v_stride + VL::load_chunk(lane) * 8) * 2);
  const uint32_t k_step = (uint32_t)(NW * KL::RB * k_stride * 2);  // bytes between this wave's blocks
  const uint32_t v_step = (uint32_t)(NW * VL::RB * v_stride * 2);

  // LDS byte addresses of this wave's first K and V block in buffer 0 (the
  // generic-to-LDS pointer conversion is done once, not per load).
  const uint32_t k_lds0 = lds_addr32(lds) + wave * KL::BLOCK_ELEMS * 2;
  const uint32_t v_lds0 = lds_addr32(lds) + (V0 + wave * VL::BLOCK_ELEMS) * 2;
  const uint32_t k_row_bytes = (uint32_t)(k_stride * 2);
  const uint32_t v_row_bytes = (uint32_t)(v_stride * 2);
  // this lane's byte offset within a tile for each of the wave's blocks
  uint32_t k_voff[KBPW], v_voff[VBPW];
#pragma unroll
  for (int i = 0; i < KBPW; ++i) k_voff[i] = k_off + i * k_step;
#pragma unroll
  for (int i = 0; i < VBPW; ++i) v_voff[i] = v_off + i * v_step;

  // All 8 (or 4) waves issue a tile's loads right after the same barrier, and
  // their scalar instructions share the CU's one scalar unit, so the common
  // case - a whole tile inside kv_end, decided per workgroup - is kept to a
  // few scalar operations per load. kt >= 0, so the 32 x 32-bit product is
  // the byte offset.
  auto issue_tile = [&](int kt, int buf) {
    const char* kb = kbase + (uint64_t)(uint32_t)kt * k_row_bytes;
    const char* vb = vbase + (uint64_t)(uint32_t)kt * v_row_bytes;
    const uint32_t km0 = k_lds0 + buf * (KL::TILE * 2);
    const uint32_t vm0 = v_lds0 + buf * (VL::TILE * 2);
    const int rows = kv_end - kt;
    if (rows >= BN) {
      static_for<KBPW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        lds_dma16_async_sv<i * NW * KL::BLOCK_ELEMS * 2>(kb, k_voff[i], km0);
      });
      static_for<VBPW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        lds_dma16_async_sv<i * NW * VL::BLOCK_ELEMS * 2>(vb, v_voff[i], vm0);
      });
      return;
    }
    // The item's last tile: lanes whose row lies at or past kv_end write
    // zeros instead (never the next sequence's data).
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    uint16_t* kl = lds + buf * KL::TILE + wave * KL::BLOCK_ELEMS + 8 * lane;
    uint16_t* vl = lds + V0 + buf * VL::TILE + wave * VL::BLOCK_ELEMS + 8 * lane;
    static_for<KBPW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (k_row + i * NW * KL::RB < rows) {
        lds_dma16_async_sv<i * NW * KL::BLOCK_ELEMS * 2>(kb, k_voff[i], km0);
      } else {
        *reinterpret_cast<u32x4_t*>(kl + i * NW * KL::BLOCK_ELEMS) = zero;
      }
    });
    static_for<VBPW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (v_row + i * NW * VL::RB < rows) {
        lds_dma16_async_sv<i * NW * VL::BLOCK_ELEMS * 2>(vb, v_voff[i], vm0);
      } else {
        *reinterpret_cast<u32x4_t*>(vl + i * NW * VL::BLOCK_ELEMS) = zero;
      }
    });
  };

  // ---- per-lane LDS read bases (element offsets within a tile) ---------------
  // K fragment of S^T: key row 32*mt + l32, chunk 2*kk + half, at
  // k_lane + k_frag(kk, mt) (a constant).
  const int k_lane = KL::elem(l32, half);
  // V^T fragments via the transpose read: 16-lane group G covers head dims
  // 16*(G%2) + 0..15 of keys 4*(G/2) + 0..3 (+8) of each 16-key block, at
  // v_lane + v_frag(kb, mb, h) for key offset 16*kb + 8*h.
  const int trg = lane >> 4;
  const int tr_i = lane & 15;
  const int tr_key = 4 * (trg >> 1) + (tr_i >> 2);
  const int tr_d = 16 * (trg & 1) + 4 * (tr_i & 3);
  const int v_lane = VL::elem(tr_key, tr_d >> 3) + (tr_d & 7);

  // One key tile. MODE selects the masking and the softmax bookkeeping:
  //   kFirst  - first tile of the item: masked; sets each row's reference
  //             max m_ref, against which every later P is taken;
  //   kFirstOpen - the same for a first tile that every row of the
  //             workgroup sees whole (no key masked), without the mask;
  //   kPlain  - a tile that needs no mask for any row of the workgroup;
  //   kMasked - a tile that crosses the causal frontier, a window edge or
  //             kv_end;
  //   kSafe   - the textbook online softmax (masked, running max, O rescaled
  //             on every tile), used only to redo an item whose P, l or O
  //             overflowed against the first tile's max.
  // Outside kSafe, P = 2^(y - m_ref) with no running max: O is never
  // rescaled and no max is taken inside the loop.
  auto compute = [&](int buf, int kt, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr bool MASK = MODE != kPlain && MODE != kFirstOpen;
    const uint16_t* ks = lds + buf * KL::TILE + k_lane;
    const uint16_t* vs = lds + V0 + buf * VL::TILE + v_lane;
    // fragment offsets from the lane bases: the row steps are multiples of
    // the block height and the chunk steps keep the in-block swizzle
    constexpr auto k_frag = [](int kk, int mt) { return KL::elem(32 * mt, 2 * kk) - KL::elem(0, 0); };
    constexpr auto v_frag = [](int kb, int mb, int h) { return VL::elem(16 * kb + 8 * h, 4 * mb) - VL::elem(0, 0); };

    // ---- S^T = K Q^T -------------------------------------------------------
    // K fragments stream through a ring of KPF register slots, KPF - 1 steps
    // ahead of the MFMAs that use them, so LDS latency hides behind MFMA work.
    constexpr int KPF = 4;
    constexpr int KSTEPS = D / 16;
    f32x16_t sacc[BN / 32];
#pragma unroll
    for (int mt = 0; mt < BN / 32; ++mt) sacc[mt] = f32x16_t{};
    u32x4_t kfr[KPF][BN / 32];
    auto load_k = [&](int kk) {
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt)
        kfr[kk % KPF][mt] = *reinterpret_cast<const u32x4_t*>(ks + k_frag(kk, mt));
    };
#pragma unroll
    for (int kk = 0; kk < KPF - 1 && kk < KSTEPS; ++kk) load_k(kk);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (kk + KPF - 1 < KSTEPS) load_k(kk + KPF - 1);
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt) sacc[mt] = mfma32<BF16>(kfr[kk % KPF][mt], qf[kk], sacc[mt]);
    }
    // sacc[mt][r] is the score of query row l32 and key
    // kt + 32*mt + 8*(r/4) + 4*half + r%4.

    // ---- softcap: short-series form when every score of the tile is small ----
    // With x = s / c (s = scale * q.k, c the softcap), c tanh(x) = s (1 + t)
    // with t = -x^2/3 + 2 x^4/15 - 17 x^6/315 + ... For |x| <= 1/4 the first
    // two terms leave a relative error below 1.3e-5, and t is small enough
    // (|t| <= 0.021) to be formed in packed f16: its own f16 rounding then
    // moves the score by less than 2^-9 of a unit in log2 scale, well under
    // the bf16 rounding of P. This takes one transcendental per score instead
    // of three (2^x, reciprocal, 2^x). The form is chosen per wave and tile:
    // every raw score of the wave's tile (masked ones included, taken before
    // the mask) must give x^2 <= 1/16 in f16, else the tile takes the exact
    // form. x^2 of each register pair is formed here once, in packed f16, and
    // reused by the series; its maximum takes 8 v_pk_maximum3_f16. A score
    // outside f16's range, or a NaN, fails the test (maximum keeps NaN).
    bool short_cap = false;
    [[maybe_unused]] f16x2_t cap_u[BN / 32][8];
    if constexpr (SOFTCAP && MODE != kSafe) {
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const f16x2_t x = __builtin_convertvector(f32x2_t{sacc[mt][r], sacc[mt][r + 1]}, f16x2_t) * cap_k;
          cap_u[mt][r / 2] = x * x;
        }
      }
      f16x2_t um = cap_u[0][0];
#pragma unroll
      for (int i = 1; i < BN / 2; i += 2) {
        const f16x2_t b = cap_u[i / 8][i % 8];
        um = (i + 1 < BN / 2) ? __builtin_elementwise_maximum(__builtin_elementwise_maximum(um, b),
                                                              cap_u[(i + 1) / 8][(i + 1) % 8])
                              : __builtin_elementwise_maximum(um, b);
      }
      const float umax = (float)__builtin_elementwise_maximum(um.x, um.y);
      short_cap = !__any(!(umax <= 0.0625f));
    }

    // ---- mask and tile max ---------------------------------------------------
    if constexpr (MASK) {
      // Register r of sacc[mt] holds key kt + 4*half + c with the constant
      // c = 32*mt + 8*(r/4) + r%4, so each key test is one compare of a
      // constant against a per-lane bound (two with a window).
      const int base = kt + 4 * half;
      const int hi = key_hi - base;
      if (p.window > 0) {
        const int lo = key_lo - base;
#pragma unroll
        for (int mt = 0; mt < BN / 32; ++mt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * mt + 8 * (r >> 2) + (r & 3);
            sacc[mt][r] = (c > hi || c < lo) ? ninf() : sacc[mt][r];
          }
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < BN / 32; ++mt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * mt + 8 * (r >> 2) + (r & 3);
            sacc[mt][r] = c > hi ? ninf() : sacc[mt][r];
          }
        }
      }
    }
    if constexpr (MODE == kFirst || MODE == kFirstOpen || MODE == kSafe) {
      float mx = ninf();
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sacc[mt][r]), sacc[mt][r + 1]);
      }
      mx = max_with_partner32(mx);
      float tmax;
      if constexpr (SOFTCAP) {
        tmax = (mx == ninf()) ? ninf()
                              : p.cap_log2 * (1.f - 2.f * rcp_fast(exp2_fast(mx * p.tanh_log2) + 1.f));
      } else {
        tmax = mx * p.score_log2;
      }
      if constexpr (MODE == kFirst || MODE == kFirstOpen) {
        m_ref = tmax;
      } else {
        const float m_new = fmaxf(m_ref, tmax);
        const float alpha = (m_new == ninf()) ? 1.f : exp2_fast(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < DV / 32; ++mb) oacc[mb] *= alpha;
      }
    }
    if constexpr (MODE == kPlain || MODE == kMasked) {
      // A row whose first visible key lies past the first tile (rows of a
      // later 32-row block under a local window) still has no reference
      // max: it takes this tile's. Its O and l are still zero, so nothing
      // needs rescaling. Rows that see no key at all keep -inf.
      if (__builtin_expect(__any(m_ref == ninf()), 0)) {
        float mx = ninf();
#pragma unroll
        for (int mt = 0; mt < BN / 32; ++mt) {
#pragma unroll
          for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sacc[mt][r]), sacc[mt][r + 1]);
        }
        mx = max_with_partner32(mx);
        float tmax;
        if constexpr (SOFTCAP) {
          tmax = (mx == ninf()) ? ninf()
                                : p.cap_log2 * (1.f - 2.f * rcp_fast(exp2_fast(mx * p.tanh_log2) + 1.f));
        } else {
          tmax = mx * p.score_log2;
        }
        m_ref = (m_ref == ninf()) ? tmax : m_ref;
      }
    }
    const float m_use = (m_ref == ninf()) ? 0.f : m_ref;

    // ---- P = 2^(y - m_use) -----------------------------------------------------
    if (short_cap) {
      // y = score_log2 * a * (1 + t), a the raw score, t from u = x^2 in
      // packed f16 (a masked score is -inf and gives P = 0 either way)
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float a0 = sacc[mt][r], a1 = sacc[mt][r + 1];
          const f16x2_t u = cap_u[mt][r / 2];
          const f16x2_t t = u * (u * cap_c2 + cap_c1);
          float pr0 = exp2_fast(__builtin_fmaf(__builtin_fmaf(a0, (float)t.x, a0), p.score_log2, -m_use));
          float pr1 = exp2_fast(__builtin_fmaf(__builtin_fmaf(a1, (float)t.y, a1), p.score_log2, -m_use));
          if constexpr (MASK) {
            pr0 = (a0 == ninf()) ? 0.f : pr0;
            pr1 = (a1 == ninf()) ? 0.f : pr1;
          }
          sacc[mt][r] = pr0;
          sacc[mt][r + 1] = pr1;
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float s = sacc[mt][r];
          float pr;
          if constexpr (SOFTCAP) {
            const float t = exp2_fast(s * p.tanh_log2);
            const float rr = rcp_fast(t + 1.f);
            pr = exp2_fast(__builtin_fmaf(rr, -2.f * p.cap_log2, p.cap_log2 - m_use));
            if constexpr (MASK) pr = (s == ninf()) ? 0.f : pr;
          } else {
            pr = exp2_fast(__builtin_fmaf(s, p.score_log2, -m_use));
          }
          sacc[mt][r] = pr;
        }
      }
    }

    // ---- P (B operand) and its row sum ----------------------------------------
    // Key block kb (16 keys) takes registers 8*(kb%2) .. +7 of sacc[kb/2]:
    // lane half h holds keys 16kb + 4h + 0..3 and 16kb + 8 + 4h + 0..3.
    u32x4_t pf[BN / 16];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 16; ++kb) {
      const int mt = kb >> 1;
      const int b0 = 8 * (kb & 1);
      pf[kb] = u32x4_t{pack2<BF16>(sacc[mt][b0 + 0], sacc[mt][b0 + 1]),
                       pack2<BF16>(sacc[mt][b0 + 2], sacc[mt][b0 + 3]),
                       pack2<BF16>(sacc[mt][b0 + 4], sacc[mt][b0 + 5]),
                       pack2<BF16>(sacc[mt][b0 + 6], sacc[mt][b0 + 7])};
#pragma unroll
      for (int e = 0; e < 4; ++e) psum = sum2<BF16>(pf[kb][e], psum);
    }
    l_run += psum;

    // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
    for (int kb = 0; kb < BN / 16; ++kb) {
      u32x4_t a[DV / 32];
#pragma unroll
      for (int mb = 0; mb < DV / 32; ++mb) {
        const u32x2_t lo = lds_read_tr16(vs + v_frag(kb, mb, 0));
        const u32x2_t hi = lds_read_tr16(vs + v_frag(kb, mb, 1));
        a[mb] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
      }
#pragma unroll
      for (int mb = 0; mb < DV / 32; ++mb) oacc[mb] = mfma32<BF16>(a[mb], pf[kb], oacc[mb]);
    }
  };

  // ---- key-tile loops ----------------------------------------------------------
  // Every loop step: wait for this wave's loads of the current tile, one
  // barrier (all waves' loads landed; the other buffer is free again), start
  // loading the next tile into the other buffer, compute the current one.
  const int n_tiles = (kv_end - kv_begin + BN - 1) / BN;
  // Tiles [t_plain0, t_plain1) need no mask for any row of the workgroup:
  // they end at or before kv_end, before the first row's causal frontier and
  // start at or after the last row's window start.
  int t_plain1 = (kv_end - kv_begin) / BN;  // full tiles
  if (p.causal) {
    const int frontier = it.q_row_begin + off + 1;  // keys [0, frontier) seen by every row
    t_plain1 = min(t_plain1, max(0, (frontier - kv_begin) / BN));
  }
  int t_plain0 = 1;
  // The first tile needs no mask when it is whole, before the first row's
  // causal frontier and, with a window, not before the last row's window start.
  bool first_open = t_plain1 >= 1;
  if (p.window > 0) {
    const int lo_last = it.q_row_begin + it.q_rows - 1 + off + 1 - p.window;  // last row's window start
    t_plain0 = max(1, (lo_last - kv_begin + BN - 1) / BN);
    first_open = first_open && lo_last <= kv_begin;
  }
  // This wave's rows see none of the keys of the tile at kt.
  auto skips = [&](int kt) {
    return !wave_active || (p.causal && kt > wave_last + off) ||
           (p.window > 0 && kt + BN <= wave_first + off + 1 - p.window);
  };
  auto step = [&](int t) {
    const int kt = kv_begin + t * BN;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile t have landed
    __syncthreads();                      // ... and every wave's; the other buffer is free again
    if (t + 1 < n_tiles) issue_tile(kt + BN, (t + 1) & 1);
    return kt;
  };
  auto run_pass = [&](auto safe_tag) {
    constexpr bool SAFE = decltype(safe_tag)::value;
    if (n_tiles > 0) issue_tile(kv_begin, 0);
    if constexpr (SAFE) {
      for (int t = 0; t < n_tiles; ++t) {
        const int kt = step(t);
        if (!skips(kt)) compute(t & 1, kt, std::integral_constant<int, kSafe>{});
      }
    } else {
      // regions: first tile | plain | masked. A window whose left edge
      // reaches past tile 1 for some row (only items of 128 rows) gets no
      // plain region: a third loop instantiation of the tile body makes the
      // compiler move the accumulators to scratch memory.
      if (n_tiles > 0) {
        if (first_open) {
          compute(0, step(0), std::integral_constant<int, kFirstOpen>{});
        } else {
          compute(0, step(0), std::integral_constant<int, kFirst>{});
        }
      }
      const int p1 = t_plain0 > 1 ? 1 : max(1, min(t_plain1, n_tiles));
      for (int t = 1; t < p1; ++t) compute(t & 1, step(t), std::integral_constant<int, kPlain>{});
      for (int t = p1; t < n_tiles; ++t) {
        const int kt = step(t);
        if (!skips(kt)) compute(t & 1, kt, std::integral_constant<int, kMasked>{});
      }
    }
  };

  run_pass(std::false_type{});
  // P was taken against each row's first-tile max without any bound. If a
  // later score rose so far above it that P, l or O overflowed, the item is
  // redone with the rescaling softmax (decided for the whole workgroup: the
  // tiles are loaded by all of its waves). chk is NaN/inf iff l or an O
  // element is.
  {
    float chk = sum_with_partner32(l_run);
#pragma unroll
    for (int mb = 0; mb < DV / 32; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) chk = __builtin_fmaf(oacc[mb][r], 0.f, chk);
    }
    const bool bad = wave_active && row_ok && !__builtin_isfinite(chk);
    if (__syncthreads_or(__any(bad) ? 1 : 0)) {
#pragma unroll
      for (int mb = 0; mb < DV / 32; ++mb) oacc[mb] = f32x16_t{};
      m_ref = ninf();
      l_run = 0.f;
      run_pass(std::true_type{});
      __syncthreads();  // every wave is done with the key tiles before the output reuses the LDS
    }
  }

  // oacc[mb][r] is the output of row l32 at head dim 32*mb + 8*(r/4) + 4*half + r%4.
  const float l_tot = sum_with_partner32(l_run);
  const float inv = (l_tot == 0.f) ? 0.f : 1.f / l_tot;
  if (it.partial_base < 0) {
    // Each lane holds pieces of one row, so direct stores would write 16
    // bytes into each of 32 rows per instruction. Instead every wave stages
    // its normalised tile in its own LDS region ([row][DV], 16-byte chunk c
    // of row r at c ^ (r % CPR)) and stores whole rows: lane i writes chunk
    // i % CPR of row 64/CPR * k + i / CPR. The barrier of the overflow check
    // above has passed, so no wave reads the key tiles any more.
    constexpr int CPR = DV / 8;         // 16-byte chunks per output row
    constexpr int RPS = 64 / CPR;       // rows per store instruction
    uint16_t* ost = lds + wave * OST;
    if (wave_active) {
#pragma unroll
      for (int mb = 0; mb < DV / 32; ++mb) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = 4 * mb + u;  // chunk of head dims 32*mb + 8*u .. +7
          const u32x2_t w = {pack2<BF16>(oacc[mb][4 * u] * inv, oacc[mb][4 * u + 1] * inv),
                             pack2<BF16>(oacc[mb][4 * u + 2] * inv, oacc[mb][4 * u + 3] * inv)};
          *reinterpret_cast<u32x2_t*>(ost + l32 * DV + ((c ^ (l32 % CPR)) << 3) + 4 * half) = w;
        }
      }
    }
    __syncthreads();
    if (!wave_active) return;
    const int c = lane % CPR;
#pragma unroll
    for (int k = 0; k < 32 / RPS; ++k) {
      const int r = k * RPS + lane / CPR;
      if (row0 + r < it.q_rows) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(ost + r * DV + ((c ^ (r % CPR)) << 3));
        const int64_t t = (int64_t)it.q_token0 + it.q_row_begin + row0 + r;
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.out) + (t * p.hq + head) * DV + 8 * c));
      }
    }
  } else {
    if (!wave_active || !row_ok) return;
    const int64_t pidx = partial_index(it, it.split, my_row, hh);
    float* po = p.part_o + pidx * DV;
#pragma unroll
    for (int mb = 0; mb < DV / 32; ++mb) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = 32 * mb + 8 * u + 4 * half;
        const f32x4_t w = {oacc[mb][4 * u] * inv, oacc[mb][4 * u + 1] * inv,
                           oacc[mb][4 * u + 2] * inv, oacc[mb][4 * u + 3] * inv};
        *reinterpret_cast<f32x4_t*>(po + d) = w;
      }
    }
    if (half == 0) p.part_lse[pidx] = (l_tot == 0.f) ? ninf() : m_ref + log2_fast(l_tot);
  }
}

template <int D, int DV, bool BF16, int NW>
static hipError_t launch_nw(const Params& p, const WorkItem* items, int n, bool softcap,
                            hipStream_t s) {
  if (softcap) {
    hipLaunchKernelGGL((prefill_mfma_kernel<D, DV, BF16, NW, true>), dim3(n), dim3(NW * 64), 0, s, p, items);
  } else {
    hipLaunchKernelGGL((prefill_mfma_kernel<D, DV, BF16, NW, false>), dim3(n), dim3(NW * 64), 0, s, p, items);
  }
  return hipGetLastError();
}

template <int D, int DV, bool BF16>
static hipError_t launch_d(const Params& p, const WorkItem* items, int n, int nw, bool softcap,
                           hipStream_t s) {
  return nw == 8 ? launch_nw<D, DV, BF16, 8>(p, items, n, softcap, s)
                 : launch_nw<D, DV, BF16, 4>(p, items, n, softcap, s);
}

template <bool BF16>
static hipError_t launch_t(const Params& p, const WorkItem* items, int n, int nw, bool softcap, hipStream_t s) {
  if (p.d == 128 && p.dv == 128) return launch_d<128, 128, BF16>(p, items, n, nw, softcap, s);
  if (p.d == 64 && p.dv == 64) return launch_d<64, 64, BF16>(p, items, n, nw, softcap, s);
  if (p.d == 128 && p.dv == 64) return launch_d<128, 64, BF16>(p, items, n, nw, softcap, s);
  if (p.d == 64 && p.dv == 128) return launch_d<64, 128, BF16>(p, items, n, nw, softcap, s);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_mfma(const Params& p, const WorkItem* items, int n, int dtype, int nw,
                               hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool sc = p.softcap_on != 0;
  return dtype == kBF16 ? launch_t<true>(p, items, n, nw, sc, s) : launch_t<false>(p, items, n, nw, sc, s);
}

}  // namespace pva
