// Top-k routing of one token by one wave, shared by the routing kernels
// and the fused decode kernel.
#pragma once

#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------
// Top-k of one token's logits by one wave.  Lane l holds logits l, l+64,
// ...; each of k rounds takes the lane-local best not yet chosen and a
// DPP wave arg-max with the order (value descending, index ascending).
// Gate weights: exp(l_j - l_max) over their sum (softmax over the chosen
// logits) or over all E logits (renormalize = 0).  The r-th choice (r < k)
// goes to ids_out[r] / w_out[r] (global, skipped when null) and to
// lds_ids[r] / lds_w[r] (skipped when null).
template <int NV>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E,
                                            int k, int renorm, int lane,
                                            int32_t* __restrict__ ids_out,
                                            float* __restrict__ w_out,
                                            int32_t* lds_ids, float* lds_w = nullptr) {
  float v[NV];
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? row[e] : -INFINITY;
    if (e >= E) taken |= 1u << j;
  }
  float top = 0.0f, denom = 0.0f;
  float sel_ex[NV];
  int sel_id[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) { sel_ex[j] = 0.0f; sel_id[j] = 0; }
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = lane + 64 * j;
      const bool free_j = !((taken >> j) & 1u);
      if (free_j && beats(v[j], e, bv, bi)) {
        bv = v[j];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (r == 0) top = bv;
    const float ex = expf(bv - top);
    denom += ex;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (r == lane + 64 * j) { sel_ex[j] = ex; sel_id[j] = bi; }
  }
  if (!renorm) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (lane + 64 * j < E) s += expf(v[j] - top);
    denom = wave_sum(s);
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int r = lane + 64 * j;
    if (r < k) {
      const float wr = sel_ex[j] / denom;
      if (ids_out) {
        ids_out[r] = sel_id[j];
        w_out[r] = wr;
      }
      if (lds_ids) lds_ids[r] = sel_id[j];
      if (lds_w) lds_w[r] = wr;
    }
  }
}

}  // namespace moe
