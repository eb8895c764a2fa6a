// Split-KV decode (one query row per sequence) and the log-sum-exp combine,
// for gfx950.
//
// Decode is a streaming pass over each sequence's keys and values: it is
// bound by HBM bandwidth, not by arithmetic. Each work item is one sequence,
// the query heads of one kv head (up to 16) and a contiguous chunk of that
// sequence's keys. The four waves of the workgroup take interleaved 32-key
// blocks of the chunk; every K/V element is read from HBM exactly once and
// feeds all the query heads of its group:
//   * S^T = K . Q^T on 16x16x32 MFMA, K fragments loaded straight from HBM
//     into the A-operand registers (16 bytes per lane), the query heads in
//     the N dimension;
//   * online softmax per head in log2 units;
//   * O^T += V^T . P^T on 16x16x32 MFMA, V staged transposed through a
//     per-wave LDS block;
//   * the four waves' (max, sum, O) are merged through LDS, and the item
//     writes either the final output (a single chunk) or an fp32 partial
//     (its normalised O and log2-sum-exp).
// A combine item then merges a row's partials in split order s = 0, 1, ...:
// M = max_s lse_s, w_s = 2^(lse_s - M), out = sum_s w_s O_s / sum_s w_s, a row
// whose partials all saw no visible key gives 0.
//
// The pages this follows (crate onnx-runtime-ep-cuda): the semantics of the
// packed op (src/kernels/packed_varlen_attention.rs, module doc and row
// kernel stages) and the split-K decode with a partial pass and a merge pass
// that src/kernels/group_query_attention.rs dispatches to for single-token
// decode (backend dispatch in its run()).
#include "combine.h"
#include "common.h"

namespace pva {

// One wave per SIMD for the 128-dim kernels: fewer loads in flight per CU
// streamed faster (measured +1.5 % on the packed decode batch).
template <int D, int DV>
constexpr int decode_waves_per_eu() { return (D == 128 && DV == 128) ? 1 : 4; }

template <int D, int DV, bool BF16, bool SOFTCAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, decode_waves_per_eu<D, DV>())))
void decode_kernel(Params p, const WorkItem* __restrict__ items) {
  constexpr int NW = 4;
  constexpr int BK = 32;            // keys per wave step
  constexpr int VSD = BK + 4;       // per-wave LDS V^T row stride (16-bit elements)
  constexpr int DCH = DV / 8;       // 16-byte chunks per value row
  constexpr int VCH = BK * DCH / 64;  // V chunks per lane per step
  constexpr int OS = DV + 4;        // LDS row stride of the cross-wave O merge (floats)
  static_assert(VCH * 64 == BK * DCH, "V block must split evenly over a wave");
  constexpr int VT_BYTES = NW * DV * VSD * 2;
  constexpr int RED_BYTES = NW * 16 * OS * 4;
  constexpr int LDS_BYTES = VT_BYTES > RED_BYTES ? VT_BYTES : RED_BYTES;

  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
  __shared__ float red_m[NW][16];
  __shared__ float red_l[NW][16];

  if (p.item_count && (int)blockIdx.x >= *p.item_count) return;
  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane >> 4;   // 0..3
  const int n = lane & 15;     // query head slot within the item
  const bool slot_ok = n < it.heads;
  const int head = it.head_begin + (slot_ok ? n : 0);
  const int g = it.kv_head;
  const int i_local = it.q_row_begin;  // the single query row
  const int off = it.len_kv - it.len_q;
  const int kv_end = it.kv_end;
  const int64_t tok = (int64_t)it.q_token0 + it.q_row_begin;

  uint16_t* vt = reinterpret_cast<uint16_t*>(lds) + wave * DV * VSD;

  // Q fragments, the B operand of S^T = K Q^T: lane supplies head slot n at
  // head dims 32*kk + 8*grp + 0..7.
  u32x4_t qf[D / 32];
  {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        static_cast<const uint16_t*>(p.q) + (tok * p.hq + head) * D);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qf[kk] = slot_ok ? src[4 * kk + grp] : zero;
  }

  f32x4_t oacc[DV / 16];
#pragma unroll
  for (int mb = 0; mb < DV / 16; ++mb) oacc[mb] = f32x4_t{};
  float m_run = ninf();
  float l_run = 0.f;

  const int64_t tok_stride = (int64_t)p.hkv * D;   // between consecutive key tokens
  const int64_t v_stride = (int64_t)p.hkv * DV;    // between consecutive value tokens
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + ((int64_t)it.kv_token0 * p.hkv + g) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + ((int64_t)it.kv_token0 * p.hkv + g) * DV;

  u32x4_t kf[2][D / 32];
  u32x4_t vr[VCH];
  auto load_block = [&](int kb) {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int j = kb + 16 * mt + n;
      const bool ok = j < kv_end;
      const uint16_t* src = kbase + j * tok_stride + 8 * grp;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        kf[mt][kk] = ok ? *reinterpret_cast<const u32x4_t*>(src + 32 * kk) : zero;
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int chunk = lane + 64 * c;
      const int key = chunk / DCH;
      const int d0 = (chunk % DCH) * 8;
      const int j = kb + key;
      vr[c] = (j < kv_end) ? *reinterpret_cast<const u32x4_t*>(vbase + j * v_stride + d0) : zero;
    }
  };

  int kb = it.kv_begin + wave * BK;
  if (kb < kv_end) load_block(kb);
  for (; kb < kv_end; kb += NW * BK) {
    // Stage this block's V transposed ([d][key]) in the wave's LDS block.
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int chunk = lane + 64 * c;
      const int key = chunk / DCH;
      const int d0 = (chunk % DCH) * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = vr[c][e];
        vt[(d0 + 2 * e) * VSD + key] = (uint16_t)(w & 0xffffu);
        vt[(d0 + 2 * e + 1) * VSD + key] = (uint16_t)(w >> 16);
      }
    }
    // ---- S^T = K Q^T for 2 x 16 keys ----------------------------------------
    f32x4_t sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x4_t{};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) sacc[mt] = mfma16<BF16>(kf[mt][kk], qf[kk], sacc[mt]);
    }
    const int kcur = kb;
    if (kb + NW * BK < kv_end) load_block(kb + NW * BK);
    // sacc[mt][r]: head slot n, key kcur + 16*mt + 4*grp + r.
    const bool need_mask = (kcur + BK > kv_end) || (p.causal && kcur + BK - 1 > i_local + off) ||
                           (p.window > 0 && kcur < i_local + off + 1 - p.window);
    float mx = ninf();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = sacc[mt][r];
        if (need_mask) {
          const int key = kcur + 16 * mt + 4 * grp + r;
          const bool bad = key >= kv_end || (p.causal && key > i_local + off) ||
                           (p.window > 0 && key < i_local + off + 1 - p.window);
          s = bad ? ninf() : s;
          sacc[mt][r] = s;
        }
        mx = fmaxf(mx, s);
      }
    }
    mx = fmaxf(mx, xor_lanes(mx, 16));
    mx = fmaxf(mx, xor_lanes(mx, 32));
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
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
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
    for (int mb = 0; mb < DV / 16; ++mb) oacc[mb] *= alpha;
    // P as the B operand over 32 keys: lane group grp holds keys 4grp + 0..3
    // (from sacc[0]) and 16 + 4grp + 0..3 (from sacc[1]).
    const u32x4_t pf = {pack2<BF16>(sacc[0][0], sacc[0][1]), pack2<BF16>(sacc[0][2], sacc[0][3]),
                        pack2<BF16>(sacc[1][0], sacc[1][1]), pack2<BF16>(sacc[1][2], sacc[1][3])};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int mb = 0; mb < DV / 16; ++mb) {
      const uint16_t* src = &vt[(16 * mb + n) * VSD + 4 * grp];
      const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(src);
      const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(src + 16);
      const u32x4_t a = {lo.x, lo.y, hi.x, hi.y};
      oacc[mb] = mfma16<BF16>(a, pf, oacc[mb]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four waves ---------------------------------------------------
  // oacc[mb][r]: head slot n, head dim 16*mb + 4*grp + r (unnormalised).
  float l_w = l_run + xor_lanes(l_run, 16);
  l_w += xor_lanes(l_w, 32);
  __syncthreads();  // every wave is done with its V^T block; reuse the LDS
  float* red_o = reinterpret_cast<float*>(lds);
  if (grp == 0) {
    red_m[wave][n] = m_run;
    red_l[wave][n] = l_w;
  }
#pragma unroll
  for (int mb = 0; mb < DV / 16; ++mb) {
    *reinterpret_cast<f32x4_t*>(&red_o[(wave * 16 + n) * OS + 16 * mb + 4 * grp]) = oacc[mb];
  }
  __syncthreads();

  // thread -> (head slot, 8 or 4 consecutive head dims)
  constexpr int PER = DV / 16;  // value dims per thread (16 threads per slot)
  const int slot = tid >> 4;
  const int d0 = (tid & 15) * PER;
  if (slot >= it.heads) return;
  float M = ninf();
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w][slot]);
  const float Mu = (M == ninf()) ? 0.f : M;
  float wsum = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float wt = exp2_fast(red_m[w][slot] - Mu);
    wsum += wt * red_l[w][slot];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += wt * red_o[(w * 16 + slot) * OS + d0 + e];
  }
  const float inv = (wsum == 0.f) ? 0.f : 1.f / wsum;
  const int ohead = it.head_begin + slot;
  if (it.partial_base < 0) {
    uint16_t* dst = static_cast<uint16_t*>(p.out) + (tok * p.hq + ohead) * DV + d0;
#pragma unroll
    for (int e = 0; e < PER; e += 2) {
      *reinterpret_cast<uint32_t*>(dst + e) = pack2<BF16>(acc[e] * inv, acc[e + 1] * inv);
    }
  } else {
    const int64_t pidx = partial_index(it, it.split, 0, slot);
    float* po = p.part_o + pidx * DV + d0;
#pragma unroll
    for (int e = 0; e < PER; ++e) po[e] = acc[e] * inv;
    if ((tid & 15) == 0) p.part_lse[pidx] = (wsum == 0.f) ? ninf() : M + log2_fast(wsum);
  }
}

// One workgroup per combine item.
template <int OUT>
__global__ __launch_bounds__(256) void combine_kernel(Params p, const WorkItem* __restrict__ items) {
  if (p.item_count && (int)blockIdx.x >= *p.item_count) return;
  combine_item<OUT>(p, items[blockIdx.x]);
}

hipError_t launch_decode(const Params& p, const WorkItem* items, int n, int dtype, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool sc = p.softcap_on != 0;
  const bool bf = dtype == kBF16;
#define PVA_DECODE(DD, DVV, BB, SS) \
  hipLaunchKernelGGL((decode_kernel<DD, DVV, BB, SS>), dim3(n), dim3(256), 0, s, p, items)
#define PVA_DECODE_DV(DD, DVV)                                                  \
  do {                                                                         \
    if (bf) { if (sc) PVA_DECODE(DD, DVV, true, true); else PVA_DECODE(DD, DVV, true, false); }    \
    else { if (sc) PVA_DECODE(DD, DVV, false, true); else PVA_DECODE(DD, DVV, false, false); }     \
  } while (0)
  if (p.d == 128 && p.dv == 128) PVA_DECODE_DV(128, 128);
  else if (p.d == 64 && p.dv == 64) PVA_DECODE_DV(64, 64);
  else if (p.d == 128 && p.dv == 64) PVA_DECODE_DV(128, 64);
  else if (p.d == 64 && p.dv == 128) PVA_DECODE_DV(64, 128);
  else return hipErrorInvalidValue;
#undef PVA_DECODE_DV
#undef PVA_DECODE
  return hipGetLastError();
}

hipError_t launch_combine(const Params& p, const WorkItem* items, int n, int dtype, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == kBF16) hipLaunchKernelGGL((combine_kernel<kBF16>), dim3(n), dim3(256), 0, s, p, items);
  else if (dtype == kF16) hipLaunchKernelGGL((combine_kernel<kF16>), dim3(n), dim3(256), 0, s, p, items);
  else hipLaunchKernelGGL((combine_kernel<kF32>), dim3(n), dim3(256), 0, s, p, items);
  return hipGetLastError();
}

}  // namespace pva
