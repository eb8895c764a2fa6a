// fp32 packed varlen attention (any head_dim, v_head_dim <= 128) on the
// vector ALUs, one workgroup of 256 threads per work item of up to 32 query
// rows of one query head.
//
// gfx950 has no fp32 matrix path worth tiling this for (its fp32 MFMA rate is
// the vector rate); fp32 I/O is the small, exactness-first case of the op
// ([PVA] = crate onnx-runtime-ep-cuda, page src/kernels/packed_varlen_attention.rs,
// "Schema (v1)" dtypes and the row kernel's five stages). The result is
// reached by the same online softmax over 32-key tiles as the MFMA kernels:
// Q, K, V tiles live in LDS, eight threads share one query row (each owns
// four keys of the score tile and every eighth output channel), row max and
// sum reduce over those eight lanes.
#include "common.h"

namespace pva {

__global__ __launch_bounds__(256) void prefill_f32_kernel(Params p, const WorkItem* __restrict__ items) {
  constexpr int BM = 32, BN = 32, MAXD = 128;
  __shared__ float qs[BM][MAXD + 1];
  __shared__ float ksh[BN][MAXD + 1];
  __shared__ float vs[BN][MAXD + 1];
  __shared__ float ps[BM][BN + 1];

  if (p.item_count && (int)blockIdx.x >= *p.item_count) return;
  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x;
  const int row = tid >> 3;  // tile row owned by this group of 8 lanes
  const int sub = tid & 7;
  const int d = p.d, dv = p.dv;
  const int head = it.head_begin;
  const int g = head / p.group;
  const int off = it.len_kv - it.len_q;
  const bool row_ok = row < it.q_rows;
  const int i_local = it.q_row_begin + row;
  const float* q = static_cast<const float*>(p.q);
  const float* k = static_cast<const float*>(p.k);
  const float* v = static_cast<const float*>(p.v);

  for (int e = tid; e < BM * d; e += 256) {
    const int r = e / d, c = e % d;
    qs[r][c] = (r < it.q_rows)
                   ? q[(((int64_t)it.q_token0 + it.q_row_begin + r) * p.hq + head) * d + c]
                   : 0.f;
  }
  float o[MAXD / 8];
#pragma unroll
  for (int c = 0; c < MAXD / 8; ++c) o[c] = 0.f;
  float m_run = ninf(), l_run = 0.f;

  for (int kt = it.kv_begin; kt < it.kv_end; kt += BN) {
    __syncthreads();
    for (int e = tid; e < BN * d; e += 256) {
      const int r = e / d, c = e % d;
      const int j = kt + r;
      ksh[r][c] = (j < it.kv_end) ? k[(((int64_t)it.kv_token0 + j) * p.hkv + g) * d + c] : 0.f;
    }
    for (int e = tid; e < BN * dv; e += 256) {
      const int r = e / dv, c = e % dv;
      const int j = kt + r;
      vs[r][c] = (j < it.kv_end) ? v[(((int64_t)it.kv_token0 + j) * p.hkv + g) * dv + c] : 0.f;
    }
    __syncthreads();
    float s[4];
    float mx = ninf();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = sub + 8 * u;
      float acc = 0.f;
      for (int c = 0; c < d; ++c) acc = __builtin_fmaf(qs[row][c], ksh[key][c], acc);
      acc *= p.scale;
      if (p.softcap_on) acc = p.softcap * tanhf(acc / p.softcap);
      const int j = kt + key;
      const bool bad = j >= it.kv_end || (p.causal && j > i_local + off) ||
                       (p.window > 0 && j < i_local + off + 1 - p.window);
      s[u] = bad ? ninf() : acc;
      mx = fmaxf(mx, s[u]);
    }
    mx = fmaxf(mx, xor_lanes(mx, 1));
    mx = fmaxf(mx, xor_lanes(mx, 2));
    mx = fmaxf(mx, xor_lanes(mx, 4));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == ninf()) ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float pr = expf(s[u] - m_use);
      ps[row][sub + 8 * u] = pr;
      psum += pr;
    }
    psum += xor_lanes(psum, 1);
    psum += xor_lanes(psum, 2);
    psum += xor_lanes(psum, 4);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // the eight lanes of a row are consecutive lanes of one wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int cc = 0; cc < MAXD / 8; ++cc) {
      const int c = sub + 8 * cc;
      if (c < dv) {
        float acc = o[cc] * alpha;
        for (int j = 0; j < BN; ++j) acc = __builtin_fmaf(ps[row][j], vs[j][c], acc);
        o[cc] = acc;
      }
    }
  }
  if (!row_ok) return;
  const float inv = (l_run == 0.f) ? 0.f : 1.f / l_run;
  const int64_t tok = (int64_t)it.q_token0 + it.q_row_begin + row;
  float* dst = static_cast<float*>(p.out) + (tok * p.hq + head) * dv;
#pragma unroll
  for (int cc = 0; cc < MAXD / 8; ++cc) {
    const int c = sub + 8 * cc;
    if (c < dv) dst[c] = o[cc] * inv;
  }
}

hipError_t launch_prefill_f32(const Params& p, const WorkItem* items, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (p.d > 128 || p.dv > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_f32_kernel, dim3(n), dim3(256), 0, s, p, items);
  return hipGetLastError();
}

}  // namespace pva
