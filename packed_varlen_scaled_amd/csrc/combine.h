// The log-sum-exp combine of split work: one combine item merges, for every
// (row, head) of its tile, the n_splits partials in split order s = 0, 1,
// ...: M = max_s lse_s, w_s = 2^(lse_s - M), out = sum_s w_s O_s / sum_s w_s,
// and a row whose partials all saw no visible key gives 0 (split-K decode
// with a partial pass and a merge pass, page
// src/kernels/group_query_attention.rs, backend dispatch in its run()).
// Used by the combine kernel and by the extra workgroups of a prefill launch
// that carries the combine items; any block size works.
#pragma once

#include "common.h"

namespace pva {

template <int OUT>
__device__ __forceinline__ void combine_item(const Params& p, const WorkItem& it) {
  const int dv = p.dv;
  const int total = it.q_rows * it.heads * dv;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int c = e % dv;
    const int rh = e / dv;
    const int hh = rh % it.heads;
    const int r = rh / it.heads;
    float M = ninf();
    for (int s = 0; s < it.n_splits; ++s) M = fmaxf(M, p.part_lse[partial_index(it, s, r, hh)]);
    float val = 0.f;
    if (M != ninf()) {
      float wsum = 0.f, acc = 0.f;
      for (int s = 0; s < it.n_splits; ++s) {
        const int64_t pi = partial_index(it, s, r, hh);
        const float w = exp2_fast(p.part_lse[pi] - M);
        wsum += w;
        acc += w * p.part_o[pi * dv + c];
      }
      val = acc / wsum;
    }
    const int64_t tok = (int64_t)it.q_token0 + it.q_row_begin + r;
    const int64_t oi = (tok * p.hq + it.head_begin + hh) * dv + c;
    if constexpr (OUT == kF32) {
      static_cast<float*>(p.out)[oi] = val;
    } else {
      const uint32_t w = pack2<OUT == kBF16>(val, 0.f);
      static_cast<uint16_t*>(p.out)[oi] = (uint16_t)(w & 0xffffu);
    }
  }
}

}  // namespace pva
