// Top-k routing of a token by a group of lanes (a whole wave, or one row of
// 16 lanes), shared by the routing kernels and the fused decode kernel.
#pragma once

#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------
// Top-k of one token's logits by LANES lanes (64: a wave; 16: a row of the
// wave, four tokens per wave).  Lane r of the group holds logits r,
// r + LANES, ...; each of k rounds takes the lane-local best not yet chosen
// and an arg-max across the group with the order (value descending, index
// ascending).  The order is carried by one 64-bit key per candidate: the
// value mapped monotonically to 32 bits (-0 taken as +0) above the inverted
// index, so one unsigned compare decides, and taken or absent candidates
// have key 0.  Gate weights: exp(l_j - l_max) over their sum (softmax over
// the chosen logits), or over all E logits (renormalize = 0); the sums are
// per-lane sums added across the group, the same in every lane.  The r-th choice
// (r < k) goes to ids_out[r] / w_out[r] (global, skipped when null) and to
// lds_ids[r] / lds_w[r] (skipped when null).
__device__ __forceinline__ uint32_t route_ord(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float route_unord(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void key_max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t ohi = (uint32_t)dpp_i<CTRL, ROW_MASK>((int)hi, (int)hi);
  const uint32_t olo = (uint32_t)dpp_i<CTRL, ROW_MASK>((int)lo, (int)lo);
  const uint64_t a = ((uint64_t)hi << 32) | lo, b = ((uint64_t)ohi << 32) | olo;
  if (b > a) {
    hi = ohi;
    lo = olo;
  }
}

template <int LANES, int NVV>
__device__ __forceinline__ void route_group_load(const float* __restrict__ row, int E, int r,
                                                 float (&v)[NVV]) {
#pragma unroll
  for (int j = 0; j < NVV; ++j) {
    const int e = r + LANES * j;
    v[j] = e < E ? row[e] : -INFINITY;
  }
}

template <int LANES, int NVV>
__device__ __forceinline__ void route_group_vals(const float (&v)[NVV], int E, int k,
                                                 int renorm, int r, bool write,
                                                 int32_t* __restrict__ ids_out,
                                                 float* __restrict__ w_out, int32_t* lds_ids,
                                                 float* lds_w) {
  uint32_t key_hi[NVV];
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < NVV; ++j) {
    key_hi[j] = route_ord(v[j]);
    if (r + LANES * j >= E) taken |= 1u << j;
  }
  float top = 0.0f;
  float sel_v[NVV];
  int sel_id[NVV];
#pragma unroll
  for (int j = 0; j < NVV; ++j) { sel_v[j] = 0.0f; sel_id[j] = 0; }
  for (int rr = 0; rr < k; ++rr) {
    // the lane's best free candidate: a pairwise tree over its NVV keys
    // (keys are unique, so the maximum is the same in any order; the tree
    // is log2(NVV) dependent steps instead of NVV)
    uint64_t cand[NVV];
#pragma unroll
    for (int j = 0; j < NVV; ++j) {
      const bool free_j = !((taken >> j) & 1u);
      cand[j] = free_j ? (((uint64_t)key_hi[j] << 32) | ~(uint32_t)(r + LANES * j)) : 0ull;
    }
#pragma unroll
    for (int wdt = 1; wdt < NVV; wdt *= 2)
#pragma unroll
      for (int j = 0; j + wdt < NVV; j += 2 * wdt)
        cand[j] = cand[j + wdt] > cand[j] ? cand[j + wdt] : cand[j];
    uint32_t hi = (uint32_t)(cand[0] >> 32), lo = (uint32_t)cand[0];
    key_max_step<kDppXor1>(hi, lo);
    key_max_step<kDppXor2>(hi, lo);
    key_max_step<kDppRowHalfMirror>(hi, lo);
    key_max_step<kDppRowMirror>(hi, lo);
    if (LANES == 64) {
      key_max_step<kDppRowBcast15, 0xA>(hi, lo);
      key_max_step<kDppRowBcast31, 0xC>(hi, lo);
      hi = __builtin_amdgcn_readlane(hi, 63);
      lo = __builtin_amdgcn_readlane(lo, 63);
    }
    const int bi = (int)~lo;
    const float bv = route_unord(hi);
    if (bi % LANES == r) taken |= 1u << (bi / LANES);
    if (rr == 0) top = bv;
#pragma unroll
    for (int j = 0; j < NVV; ++j)
      if (rr == r + LANES * j) { sel_v[j] = bv; sel_id[j] = bi; }
  }
  // gate numerators of this lane's choices, all lanes at once (not one
  // exponential per round), and their sum over the group
  float sel_ex[NVV], part = 0.0f;
#pragma unroll
  for (int j = 0; j < NVV; ++j) {
    sel_ex[j] = r + LANES * j < k ? expf(sel_v[j] - top) : 0.0f;
    part += sel_ex[j];
  }
  float denom = LANES == 64 ? wave_sum(part) : group_sum(part, 16);
  if (!renorm) {
    float sm = 0.0f;
#pragma unroll
    for (int j = 0; j < NVV; ++j)
      if (r + LANES * j < E) sm += expf(v[j] - top);
    denom = LANES == 64 ? wave_sum(sm) : group_sum(sm, 16);
  }
  if (!write) return;
#pragma unroll
  for (int j = 0; j < NVV; ++j) {
    const int rr = r + LANES * j;
    if (rr < k) {
      const float wr = sel_ex[j] / denom;
      if (ids_out) {
        ids_out[rr] = sel_id[j];
        w_out[rr] = wr;
      }
      if (lds_ids) lds_ids[rr] = sel_id[j];
      if (lds_w) lds_w[rr] = wr;
    }
  }
}

// Batches of at least this many tokens route one token per row of 16 lanes
// (when E <= 256): four tokens per wave at once; smaller batches one token
// per wave.  A workgroup's waves share its CU's four SIMDs, so from five
// tokens on (more token waves than SIMDs) the row form finishes first: at
// 12 tokens in one workgroup the last of twelve token waves ended ~9.3 k
// cycles after the start, three waves per SIMD of ~3 k each.  Every routing
// kernel applies the same rule, so their results agree bit for bit.
constexpr int kRouteRowMinT = 5;
// From this many tokens the routing of moe_route_permute / the layer call
// runs over several workgroups (16 tokens each), then the sort.
constexpr int kRouteMultiMinT = 16;

// Route tokens [0, T) with the waves w0, w0 + ws, ... of the caller (w0 =
// this wave's index among the ws routing waves).  Each wave handles up to
// 4 * MAXPER tokens; all its loads are issued before its first top-k.
template <int NV, int MAXPER>
__device__ __forceinline__ void route_tokens(const float* __restrict__ logits, int T, int E,
                                             int k, int renorm, int lane, int w0, int ws,
                                             int32_t* ids, float* w, int32_t* lds_ids,
                                             float* lds_w) {
  if (NV <= 4 && T >= kRouteRowMinT) {
    constexpr int NVL = NV <= 4 ? 4 * NV : 1;
    const int r = lane & 15, sub = lane >> 4;
    float v[MAXPER][NVL];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int t = min((w0 + ws * i) * 4 + sub, T - 1);
      if ((w0 + ws * i) * 4 < T) route_group_load<16, NVL>(logits + (size_t)t * E, E, r, v[i]);
    }
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int t0 = (w0 + ws * i) * 4;
      if (t0 < T) {
        const int t = t0 + sub;
        const bool ok = t < T;
        const int tt = ok ? t : T - 1;
        route_group_vals<16, NVL>(v[i], E, k, renorm, r, ok,
                                  ids ? ids + (size_t)tt * k : nullptr,
                                  w ? w + (size_t)tt * k : nullptr,
                                  lds_ids ? lds_ids + tt * k : nullptr,
                                  lds_w ? lds_w + tt * k : nullptr);
      }
    }
  } else {
    float v[MAXPER * 4][NV];
#pragma unroll
    for (int i = 0; i < MAXPER * 4; ++i) {
      const int t = w0 + ws * i;
      if (t < T) route_group_load<64, NV>(logits + (size_t)t * E, E, lane, v[i]);
    }
#pragma unroll
    for (int i = 0; i < MAXPER * 4; ++i) {
      const int t = w0 + ws * i;
      if (t < T)
        route_group_vals<64, NV>(v[i], E, k, renorm, lane, true,
                                 ids ? ids + (size_t)t * k : nullptr,
                                 w ? w + (size_t)t * k : nullptr,
                                 lds_ids ? lds_ids + t * k : nullptr,
                                 lds_w ? lds_w + t * k : nullptr);
    }
  }
}

}  // namespace moe
