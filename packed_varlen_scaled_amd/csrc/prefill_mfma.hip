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
//   * the workgroup stages K as [key][d] and V transposed as [d][key] in LDS,
//     once for all NH heads of the group (the GQA reuse);
//   * S^T = K . Q^T on 32x32x16 MFMA: lane l then holds 32 scores of query
//     row l%32, so the row max / sum need one exchange between lane halves;
//   * online softmax in registers in log2 units (exp2 with log2(e) folded
//     into the scale);
//   * O^T += V^T . P^T on 32x32x16 MFMA, P rounded to the I/O type, with the
//     score accumulator registers reused directly as the B operand (the MFMA
//     reduction order over keys is free, so V^T is read in the order the
//     score layout leaves the keys in).
// Rows of the tile that lie past the sequence are never stored; keys at or
// past kv_end are zero-filled in LDS (so data of the next sequence can never
// reach a product) and masked.
#include "common.h"

namespace pva {

template <int D, bool BF16, int NW, bool SOFTCAP>
__global__ __launch_bounds__(NW * 64) void prefill_mfma_kernel(Params p,
                                                               const WorkItem* __restrict__ items) {
  constexpr int BN = 64;              // keys per tile
  constexpr int KS = D + 8;           // LDS K row stride (16-bit elements)
  constexpr int VS = BN + 4;          // LDS V^T row stride
  constexpr int NT = NW * 64;
  constexpr int DCH = D / 8;          // 16-byte chunks per key row
  constexpr int CHUNKS = BN * DCH;    // chunks per K (or V) tile
  constexpr int CPT = (CHUNKS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint16_t ks[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];

  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int hh = wave % it.heads;
  const int rb = wave / it.heads;
  const int head = it.head_begin + hh;
  const int g = it.head_begin / p.group;
  const int row0 = rb * 32;
  const int my_row = row0 + l32;
  const bool row_ok = my_row < it.q_rows;
  const int i_local = it.q_row_begin + my_row;
  const int off = it.len_kv - it.len_q;
  const bool wave_active = row0 < it.q_rows;
  const int wave_first = it.q_row_begin + row0;
  const int wave_last = it.q_row_begin + min(row0 + 31, it.q_rows - 1);
  const int kv_begin = it.kv_begin;
  const int kv_end = it.kv_end;
  const int64_t tok = (int64_t)it.q_token0 + it.q_row_begin + my_row;

  // Q fragments, the B operand of S^T = K Q^T: lane l supplies query row
  // l%32 at head dims 16*kk + 8*half + 0..7.
  u32x4_t qf[D / 16];
  {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        static_cast<const uint16_t*>(p.q) + (tok * p.hq + head) * D);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = row_ok ? src[2 * kk + half] : zero;
  }

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = f32x16_t{};
  float m_run = ninf();
  float l_run = 0.f;

  const int64_t tok_stride = (int64_t)p.hkv * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + ((int64_t)it.kv_token0 * p.hkv + g) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + ((int64_t)it.kv_token0 * p.hkv + g) * D;

  u32x4_t kreg[CPT], vreg[CPT];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + c * NT;
      const int key = chunk / DCH;
      const int d0 = (chunk % DCH) * 8;
      const int j = kt + key;
      const bool ok = (CHUNKS % NT == 0 || chunk < CHUNKS) && j < kv_end;
      const u32x4_t zero = {0u, 0u, 0u, 0u};
      kreg[c] = ok ? *reinterpret_cast<const u32x4_t*>(kbase + j * tok_stride + d0) : zero;
      vreg[c] = ok ? *reinterpret_cast<const u32x4_t*>(vbase + j * tok_stride + d0) : zero;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + c * NT;
      if (CHUNKS % NT != 0 && chunk >= CHUNKS) continue;
      const int key = chunk / DCH;
      const int d0 = (chunk % DCH) * 8;
      *reinterpret_cast<u32x4_t*>(&ks[key * KS + d0]) = kreg[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = vreg[c][e];
        vt[(d0 + 2 * e) * VS + key] = (uint16_t)(w & 0xffffu);
        vt[(d0 + 2 * e + 1) * VS + key] = (uint16_t)(w >> 16);
      }
    }
  };

  if (kv_begin < kv_end) load_tile(kv_begin);
  for (int kt = kv_begin; kt < kv_end; kt += BN) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + BN < kv_end) load_tile(kt + BN);
    // Whole tile beyond every row of this wave (causal), or no rows at all.
    if (!wave_active || (p.causal && kt > wave_last + off)) continue;
    const bool need_mask = (kt + BN > kv_end) || (p.causal && kt + BN - 1 > wave_first + off);

    // ---- S^T = K Q^T -------------------------------------------------------
    f32x16_t sacc[BN / 32];
#pragma unroll
    for (int mt = 0; mt < BN / 32; ++mt) sacc[mt] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt) {
        const u32x4_t a =
            *reinterpret_cast<const u32x4_t*>(&ks[(32 * mt + l32) * KS + 16 * kk + 8 * half]);
        sacc[mt] = mfma32<BF16>(a, qf[kk], sacc[mt]);
      }
    }
    // sacc[mt][r] is the score of query row l32 and key
    // kt + 32*mt + 8*(r/4) + 4*half + r%4.

    // ---- mask and tile max ---------------------------------------------------
    float mx = ninf();
#pragma unroll
    for (int mt = 0; mt < BN / 32; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = sacc[mt][r];
        if (need_mask) {
          const int key = kt + 32 * mt + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool bad = key >= kv_end || (p.causal && key > i_local + off);
          s = bad ? ninf() : s;
          sacc[mt][r] = s;
        }
        mx = fmaxf(mx, s);
      }
    }
    mx = fmaxf(mx, xor_lanes(mx, 32));

    // ---- online softmax (log2 units) ------------------------------------
    float tmax;
    if constexpr (SOFTCAP) {
      tmax = (mx == ninf()) ? ninf()
                            : p.cap_log2 * (1.f - 2.f * rcp_fast(exp2_fast(mx * p.tanh_log2) + 1.f));
    } else {
      tmax = mx * p.score_log2;
    }
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == ninf()) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float psum = 0.f;
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
          if (need_mask) pr = (s == ninf()) ? 0.f : pr;
        } else {
          pr = exp2_fast(__builtin_fmaf(s, p.score_log2, -m_use));
        }
        sacc[mt][r] = pr;
        psum += pr;
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;

    // ---- P (B operand) -------------------------------------------------------
    // Key block kb (16 keys) takes registers 8*(kb%2) .. +7 of sacc[kb/2]:
    // lane half h holds keys 16kb + 4h + 0..3 and 16kb + 8 + 4h + 0..3.
    u32x4_t pf[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 16; ++kb) {
      const int mt = kb >> 1;
      const int b0 = 8 * (kb & 1);
      pf[kb] = u32x4_t{pack2<BF16>(sacc[mt][b0 + 0], sacc[mt][b0 + 1]),
                       pack2<BF16>(sacc[mt][b0 + 2], sacc[mt][b0 + 3]),
                       pack2<BF16>(sacc[mt][b0 + 4], sacc[mt][b0 + 5]),
                       pack2<BF16>(sacc[mt][b0 + 6], sacc[mt][b0 + 7])};
    }

    // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
    for (int kb = 0; kb < BN / 16; ++kb) {
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
        const uint16_t* src = &vt[(32 * mb + l32) * VS + 16 * kb + 4 * half];
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(src);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(src + 8);
        const u32x4_t a = {lo.x, lo.y, hi.x, hi.y};
        oacc[mb] = mfma32<BF16>(a, pf[kb], oacc[mb]);
      }
    }
  }

  if (!wave_active || !row_ok) return;
  // oacc[mb][r] is the output of row l32 at head dim 32*mb + 8*(r/4) + 4*half + r%4.
  const float l_tot = l_run + xor_lanes(l_run, 32);
  if (it.partial_base < 0) {
    const float inv = (l_tot == 0.f) ? 0.f : 1.f / l_tot;
    uint16_t* dst = static_cast<uint16_t*>(p.out) + (tok * p.hq + head) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = 32 * mb + 8 * u + 4 * half;
        const u32x2_t w = {pack2<BF16>(oacc[mb][4 * u] * inv, oacc[mb][4 * u + 1] * inv),
                           pack2<BF16>(oacc[mb][4 * u + 2] * inv, oacc[mb][4 * u + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(dst + d) = w;
      }
    }
  } else {
    const float inv = (l_tot == 0.f) ? 0.f : 1.f / l_tot;
    const int64_t pidx = partial_index(it, it.split, my_row, hh);
    float* po = p.part_o + pidx * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = 32 * mb + 8 * u + 4 * half;
        const f32x4_t w = {oacc[mb][4 * u] * inv, oacc[mb][4 * u + 1] * inv,
                           oacc[mb][4 * u + 2] * inv, oacc[mb][4 * u + 3] * inv};
        *reinterpret_cast<f32x4_t*>(po + d) = w;
      }
    }
    if (half == 0) p.part_lse[pidx] = (l_tot == 0.f) ? ninf() : m_run + log2_fast(l_tot);
  }
}

template <int D, bool BF16, int NW>
static hipError_t launch_nw(const Params& p, const WorkItem* items, int n, bool softcap,
                            hipStream_t s) {
  if (softcap) {
    hipLaunchKernelGGL((prefill_mfma_kernel<D, BF16, NW, true>), dim3(n), dim3(NW * 64), 0, s, p, items);
  } else {
    hipLaunchKernelGGL((prefill_mfma_kernel<D, BF16, NW, false>), dim3(n), dim3(NW * 64), 0, s, p, items);
  }
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_d(const Params& p, const WorkItem* items, int n, int nw, bool softcap,
                           hipStream_t s) {
  return nw == 8 ? launch_nw<D, BF16, 8>(p, items, n, softcap, s)
                 : launch_nw<D, BF16, 4>(p, items, n, softcap, s);
}

hipError_t launch_prefill_mfma(const Params& p, const WorkItem* items, int n, int dtype, int nw,
                               hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool sc = p.softcap_on != 0;
  const bool bf = dtype == kBF16;
  if (p.d == 128) return bf ? launch_d<128, true>(p, items, n, nw, sc, s) : launch_d<128, false>(p, items, n, nw, sc, s);
  if (p.d == 64) return bf ? launch_d<64, true>(p, items, n, nw, sc, s) : launch_d<64, false>(p, items, n, nw, sc, s);
  return hipErrorInvalidValue;
}

}  // namespace pva
