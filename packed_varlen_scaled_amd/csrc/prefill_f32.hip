// fp32 packed varlen attention (any head_dim, v_head_dim <= 128) on the
// vector ALUs, one workgroup of 256 threads per work item of up to 32 query
// rows of one query head.
//
// gfx950 has no fp32 matrix path worth tiling this for (its fp32 MFMA rate is
// the vector rate); fp32 I/O is the small, exactness-first case of the op
// ([PVA] = crate onnx-runtime-ep-cuda, page src/kernels/packed_varlen_attention.rs,
// "Schema (v1)" dtypes and the row kernel's five stages). The result is
// reached by the same online softmax over 32-key tiles as the MFMA kernels:
// Q, K, V tiles live in LDS (rows zero-padded to whole 16-byte pieces and
// read 16 bytes at a time), eight threads share one query row (each owns
// four keys of the score tile and four groups of four output channels), row
// max and sum reduce over those eight lanes.
#include "common.h"

namespace pva {

__global__ __launch_bounds__(256) void prefill_f32_kernel(Params p, const WorkItem* __restrict__ items) {
  constexpr int BM = 32, BN = 32, MAXD = 128;
  constexpr int LD = MAXD + 4;  // row stride: 16-byte aligned rows, rows 4 banks apart
  __shared__ __attribute__((aligned(16))) float qs[BM][LD];
  __shared__ __attribute__((aligned(16))) float ksh[BN][LD];
  __shared__ __attribute__((aligned(16))) float vs[BN][LD];
  __shared__ __attribute__((aligned(16))) float ps[BM][BN + 4];

  if (p.item_count && (int)blockIdx.x >= *p.item_count) return;
  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x;
  const int row = tid >> 3;  // tile row owned by this group of 8 lanes
  const int sub = tid & 7;
  const int d = p.d, dv = p.dv;
  const int d4 = (d + 3) & ~3;    // head dims rounded up to whole 16-byte pieces (zero padded)
  const int dv4 = (dv + 3) & ~3;
  const int head = it.head_begin;
  const int g = head / p.group;
  const int off = it.len_kv - it.len_q;
  const bool row_ok = row < it.q_rows;
  const int i_local = it.q_row_begin + row;
  const float* q = static_cast<const float*>(p.q);
  const float* k = static_cast<const float*>(p.k);
  const float* v = static_cast<const float*>(p.v);

  // Tile staging: every load of a tile is issued before any LDS write, so
  // the loads' latencies overlap. The 8 lanes of a row group stage one tile
  // row: lane sub takes columns sub + 8 i, i = 0..15, from one base address.
  constexpr int PER = MAXD / 8;
  auto gather = [&](float (&tmp)[PER], const float* src, bool ok, int w) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = sub + 8 * i;
      tmp[i] = (ok && c < w) ? src[c] : 0.f;
    }
  };
  auto scatter = [&](float* dst, const float (&tmp)[PER], int w4) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = sub + 8 * i;
      if (c < w4) dst[c] = tmp[i];
    }
  };
  {
    float tq[PER];
    gather(tq, q + (((int64_t)it.q_token0 + it.q_row_begin + row) * p.hq + head) * d, row_ok, d);
    scatter(qs[row], tq, d4);
  }
  // Output channels of this lane: 4 * sub + 32 * j + 0..3, j = 0..3, so that
  // the 8 lanes of a row read 32 consecutive channels of a value row.
  f32x4_t o[MAXD / 32];
#pragma unroll
  for (int j = 0; j < MAXD / 32; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = ninf(), l_run = 0.f;

  // K and V rows of the tile at kt, loaded into registers one tile ahead of
  // its use, so the loads overlap the previous tile's arithmetic
  float tk[PER], tv[PER];
  auto load_kv = [&](int kt) {
    const int j = kt + row;  // key of this row group's tile row
    const bool key_ok = j < it.kv_end;
    const int64_t tokj = (int64_t)it.kv_token0 + (key_ok ? j : 0);
    gather(tk, k + (tokj * p.hkv + g) * d, key_ok, d);
    gather(tv, v + (tokj * p.hkv + g) * dv, key_ok, dv);
  };
  if (it.kv_begin < it.kv_end) load_kv(it.kv_begin);
  for (int kt = it.kv_begin; kt < it.kv_end; kt += BN) {
    __syncthreads();  // the previous tile's K, V and P are no longer read
    scatter(ksh[row], tk, d4);
    scatter(vs[row], tv, dv4);
    __syncthreads();
    if (kt + BN < it.kv_end) load_kv(kt + BN);
    // scores of keys sub + 8u, u = 0..3: 16-byte reads, the query piece shared by the four keys
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = 0; c < d4; c += 4) {
      const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(&qs[row][c]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(&ksh[sub + 8 * u][c]);
        acc[u] = __builtin_fmaf(qv.x, kv.x, acc[u]);
        acc[u] = __builtin_fmaf(qv.y, kv.y, acc[u]);
        acc[u] = __builtin_fmaf(qv.z, kv.z, acc[u]);
        acc[u] = __builtin_fmaf(qv.w, kv.w, acc[u]);
      }
    }
    float s[4];
    float mx = ninf();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float a = acc[u] * p.scale;
      if (p.softcap_on) a = p.softcap * tanhf(a / p.softcap);
      const int key = sub + 8 * u;
      const int j = kt + key;
      const bool bad = j >= it.kv_end || (p.causal && j > i_local + off) ||
                       (p.window > 0 && j < i_local + off + 1 - p.window);
      s[u] = bad ? ninf() : a;
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
    for (int j = 0; j < MAXD / 32; ++j) o[j] *= alpha;
#pragma unroll 2
    for (int j4 = 0; j4 < BN; j4 += 4) {
      const f32x4_t pv = *reinterpret_cast<const f32x4_t*>(&ps[row][j4]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float pj = pv[jj];
#pragma unroll
        for (int j = 0; j < MAXD / 32; ++j) {
          if (32 * j + 4 * sub < dv4) {
            const f32x4_t vv = *reinterpret_cast<const f32x4_t*>(&vs[j4 + jj][32 * j + 4 * sub]);
            o[j][0] = __builtin_fmaf(pj, vv.x, o[j][0]);
            o[j][1] = __builtin_fmaf(pj, vv.y, o[j][1]);
            o[j][2] = __builtin_fmaf(pj, vv.z, o[j][2]);
            o[j][3] = __builtin_fmaf(pj, vv.w, o[j][3]);
          }
        }
      }
    }
  }
  if (!row_ok) return;
  const float inv = (l_run == 0.f) ? 0.f : 1.f / l_run;
  const int64_t tok = (int64_t)it.q_token0 + it.q_row_begin + row;
  float* dst = static_cast<float*>(p.out) + (tok * p.hq + head) * dv;
#pragma unroll
  for (int j = 0; j < MAXD / 32; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 32 * j + 4 * sub + i;
      if (c < dv) dst[c] = o[j][i] * inv;
    }
  }
}

hipError_t launch_prefill_f32(const Params& p, const WorkItem* items, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (p.d > 128 || p.dv > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_f32_kernel, dim3(n), dim3(256), 0, s, p, items);
  return hipGetLastError();
}

}  // namespace pva
