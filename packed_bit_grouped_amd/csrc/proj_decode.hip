// Grouped expert projections for decode batches with bf16 activations: a
// latency-first form of the split-K GEMV.
//
// Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", sections
// "Keep low-bit weights packed, do the work on the NPU" (grouped
// projections straight from packed weights, fused gate/up, routing and
// tile reuse, blocked reduction) and "Remove sync and launch overhead from
// the token loop" (fewer, fused launches per step).  At a few tokens per
// expert the layer streams a few MB of packed weights, about the amount
// the chip moves in one memory latency, so the kernels are shaped around
// that latency rather than around the ALUs:
//
//  * every weight load of a workgroup is issued before anything waits:
//    one 16-byte chunk per lane and per `CPL` slot, all in flight at once,
//    and the weight rows stay in registers while every token of the tile
//    is applied to them (tile reuse);
//  * gate/up: a workgroup owns 8 units (gate row i and up row I+i) of one
//    tile, one per wave; 32 lanes share a row (split-K), DPP sums the row,
//    and the gate half of the wave fetches the up sum from the other half
//    for SiLU(g) * u - no LDS round trip and no barrier after the staging
//    of the activations;
//  * down + combine: a workgroup owns 4 output columns of every token;
//    each wave takes whole tiles (16 lanes per weight row), the weighted
//    combine of a token's k routed rows and the shared rows happens in the
//    same workgroup in the fixed order of the combine (routed j = 0..k-1,
//    then shared), so no per-pair fp32 round trip through HBM and no
//    separate combine launch;
//  * the products use the exact bf16 unpack of the codes with
//    v_dot2_f32_bf16 and the per-block activation sums (shared helpers).
#include "gemv_common.h"
#include "route_common.h"

namespace moe {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecGuLanes = 32;   // lanes per weight row, gate/up
constexpr int kDecDnLanes = 16;   // lanes per weight row, down
constexpr int kDecDnCols = 64 / kDecDnLanes;   // output columns per workgroup
constexpr int kDecDnRounds = 2;   // tiles per wave with loads in flight together
constexpr int kDecSortedLds = 2048;   // pairs whose sorted list is copied to LDS

// Tile of slot `slot`: shared slots first (tokens [ti*sh_tile, ...)), then
// the routed tiles of the permutation.  Returns false for slots past the
// device-side tile count.
__device__ __forceinline__ bool dec_tile(const ProjArgs& a, int slot, int n_tiles, bool& is_sh,
                                         int& e, int& r0, int& r1) {
  if (slot < a.n_sh_slots) {
    const int per = (a.T + a.sh_tile - 1) / a.sh_tile;
    const int s = slot / per, ti = slot - s * per;
    is_sh = true;
    e = s;
    r0 = ti * a.sh_tile;
    r1 = min(a.T, r0 + a.sh_tile);
    return true;
  }
  const int j = slot - a.n_sh_slots;
  if (j >= a.max_tiles || j >= n_tiles) return false;
  const int4 tl = reinterpret_cast<const int4*>(a.tiles)[j];
  is_sh = false;
  e = tl.x;
  r0 = tl.y;
  r1 = tl.z;
  return true;
}

// The same from a copy of the tile list in LDS.
__device__ __forceinline__ bool dec_tile_lds(const ProjArgs& a, int slot, int n_tiles,
                                             const int4* tiles, bool& is_sh, int& e, int& r0,
                                             int& r1) {
  if (slot < a.n_sh_slots) {
    const int per = (a.T + a.sh_tile - 1) / a.sh_tile;
    const int s = slot / per, ti = slot - s * per;
    is_sh = true;
    e = s;
    r0 = ti * a.sh_tile;
    r1 = min(a.T, r0 + a.sh_tile);
    return true;
  }
  const int j = slot - a.n_sh_slots;
  if (j >= a.max_tiles || j >= n_tiles) return false;
  const int4 tl = tiles[j];
  is_sh = false;
  e = tl.x;
  r0 = tl.y;
  r1 = tl.z;
  return true;
}

// Copy n 16-byte words from global memory to LDS with the whole block.
__device__ __forceinline__ void copy_words(u32x4_v* dst, const void* src, int n) {
  const u32x4_v* s = reinterpret_cast<const u32x4_v*>(src);
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = ld_global(s + i);
}
__device__ __forceinline__ void copy_ints(int* dst, const int* src, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = ld_global(src + i);
}

// Descriptor tables (routed then shared) in LDS: [E + n_shared] moe_qmat.
__device__ __forceinline__ void copy_descs(moe_qmat* dst, const ProjArgs& a) {
  constexpr int w = sizeof(moe_qmat) / 16;
  copy_words(reinterpret_cast<u32x4_v*>(dst), a.w, a.E * w);
  if (a.n_shared > 0)
    copy_words(reinterpret_cast<u32x4_v*>(dst + a.E), a.w_sh, a.n_shared * w);
}

// Scale word of code chunk c (int2 with 32-wide groups: two scales).
__device__ __forceinline__ uint32_t dec_scale(const uint16_t* sp, const RowGeom& G, int c) {
  return (G.bits == 2 && G.group == 32) ? ld_global(reinterpret_cast<const uint32_t*>(sp + 2 * c))
                                        : (uint32_t)ld_global(sp + (c * G.CK) / G.group);
}

// ---------------------------------------------------------------------
// gate/up + SiLU*mul.  Grid: (n_sh_slots + max_tiles) * n_ub workgroups;
// workgroup (slot, ub) owns units [16 ub, 16 ub + 16) of its tile's
// expert.  Wave w: units 16 ub + w and 16 ub + 8 + w, the loads of both
// issued together; lanes 0-31 hold a unit's gate row, lanes 32-63 its up
// row.  srow: the sorted pair list in LDS, or null (read from memory).
template <int MAXT, int CPL>
__device__ __forceinline__ void gateup_tile(const ProjArgs& a, bool is_sh, int e, int r_begin,
                                            int r_end, const moe_qmat& q, int ub,
                                            const int* srow, uint32_t* xs, float* xsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const int U = is_sh ? a.U_sh : a.U;
  const RowGeom G = row_geom(q, K, 0);
  const int lis = lane & (kDecGuLanes - 1);
  const bool up = lane >= kDecGuLanes;
  int unit[2], wr[2];
  bool vrow[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    unit[r] = ub * 2 * kDecWaves + r * kDecWaves + wave;
    vrow[r] = unit[r] < U;
    wr[r] = vrow[r] ? unit[r] + (up ? U : 0) : 0;
  }

  // ---- every weight load of the workgroup, then the activation rows
  uint4 wv[2][CPL];
  uint32_t sv[2][CPL];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint4* cp = reinterpret_cast<const uint4*>(q.codes + (size_t)wr[r] * G.row_bytes);
    const uint16_t* sp = q.scales + (size_t)wr[r] * G.ng;
#pragma unroll
    for (int b = 0; b < CPL; ++b) {
      const int c = lis + kDecGuLanes * b;
      if (vrow[r] && c < G.C_r) {
        const u32x4_v t4 = ld_global_nt(reinterpret_cast<const u32x4_v*>(cp + c));
        wv[r][b] = make_uint4(t4.x, t4.y, t4.z, t4.w);
        sv[r][b] = dec_scale(sp, G, c);
      } else {
        wv[r][b] = make_uint4(0u, 0u, 0u, 0u);
        sv[r][b] = 0u;
      }
    }
  }
  const int xs_row = K / 2, xsum_row = K / 32, nb32 = K / 32;
  // one pass: the launcher guarantees a tile has at most MAXT rows
  const int nt = min(MAXT, r_end - r_begin);
  for (int u = tid; u < nt * nb32; u += kDecThreads) {
    const int m = u / nb32, b = u - m * nb32;
    int row = r_begin + m;
    if (!is_sh) row = (srow ? srow[row] : ld_global(a.sorted_pair + row)) / a.k;
    stage_a16_block(a.in_bf16 + (size_t)row * a.ld_in, b, K, G.bits, xs + m * xs_row,
                    xsum + m * xsum_row);
  }
  __syncthreads();

  const int orow0 = is_sh ? a.P + e * a.T + r_begin : r_begin;
  uint16_t* h = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    float acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int b = 0; b < CPL; ++b) {
      const int c = lis + kDecGuLanes * b;
      if (c < G.C_r)
        chunk_dot<MOE_A16, MAXT, false>(a, wv[r][b], sv[r][b], c, G, nt, xs, xs_row, xsum,
                                        xsum_row, acc, lis, vrow[r], wr[r], 0);
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t >= nt) break;
      // rows of 16 lanes, then row 0 into row 1 and row 2 into row 3:
      // lane 16 ends with the gate sum, lane 48 with the up sum
      float g = group_sum(acc[t], 16);
      g += dpp_f<kDppRowBcast15, 0xA>(0.0f, g);
      const float u = __shfl_down(g, 32);
      if (lane == 16 && vrow[r])
        h[(size_t)(orow0 + t) * a.ld_out + unit[r]] = (uint16_t)f32_to_bf16(silu_mul(g, u));
    }
  }
}

// LDS carve-up shared by the gate/up kernels: activation planes, their
// block sums, then 16-byte aligned tables.
template <int MAXT>
__device__ __forceinline__ unsigned char* gateup_tables(unsigned char* smem, int K) {
  return smem + ((size_t)MAXT * (K / 2 + K / 32) * 4 + 15) / 16 * 16;
}

template <int MAXT, int CPL>
__global__ __launch_bounds__(kDecThreads) void dec_gateup_kernel(ProjArgs a, int n_ub) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int slot = blockIdx.x / n_ub, ub = blockIdx.x - slot * n_ub;
  const int K = a.K;
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem);
  float* xsum = reinterpret_cast<float*>(xs + MAXT * (K / 2));
  moe_qmat* descs = reinterpret_cast<moe_qmat*>(gateup_tables<MAXT>(smem, K));
  int* srow = reinterpret_cast<int*>(descs + a.E + a.n_shared);
  const bool srow_lds = a.P <= kDecSortedLds;

  // ---- round trip 1, all independent: tile count, this slot's tile,
  // descriptor tables, sorted pairs
  const int n_tiles = ld_global(a.n_tiles);
  const int j = slot - a.n_sh_slots;
  int4 tl = make_int4(0, 0, 0, 0);
  if (j >= 0 && j < a.max_tiles) {
    const u32x4_v t4 = ld_global(reinterpret_cast<const u32x4_v*>(a.tiles) + j);
    tl = make_int4((int)t4.x, (int)t4.y, (int)t4.z, (int)t4.w);
  }
  copy_descs(descs, a);
  if (srow_lds) copy_ints(srow, a.sorted_pair, a.P);
  __syncthreads();

  bool is_sh;
  int e, r_begin, r_end;
  if (slot < a.n_sh_slots) {
    dec_tile(a, slot, n_tiles, is_sh, e, r_begin, r_end);
  } else {
    if (j >= a.max_tiles || j >= n_tiles) return;
    is_sh = false;
    e = tl.x;
    r_begin = tl.y;
    r_end = tl.z;
  }
  const int U = is_sh ? a.U_sh : a.U;
  if (ub * 2 * kDecWaves >= U) return;
  if (!is_sh && (unsigned)e >= (unsigned)a.E) {
    if (tid == 0) atomicOr(a.err, 2);
    return;
  }
  const moe_qmat q = descs[is_sh ? a.E + e : e];
  if (!qmat_usable(q, 2 * U, K)) {
    if (tid == 0) atomicOr(a.err, 1);
    return;
  }
  gateup_tile<MAXT, CPL>(a, is_sh, e, r_begin, r_end, q, ub, srow_lds ? srow : nullptr, xs,
                         xsum);
}

// ---------------------------------------------------------------------
// Route, permute and gate/up in one launch for small batches (T * k <=
// 64).  Every workgroup routes the whole batch itself (one wave per
// token), sorts the pairs by expert with one wave, and then works on its
// (tile, unit block) exactly as dec_gateup_kernel; workgroup 0 also writes
// the routing outputs that the down projection reads.  The routing costs a
// few hundred ALU cycles per workgroup, less than the launch and the
// memory round trip of a separate routing kernel.
struct RouteOut {
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_pos;
  int32_t* tiles;
  int32_t* n_tiles;
};

constexpr int kFusedMaxP = 64;

// Stable counting sort of P <= 64 pairs by expert with one wave (lane p
// holds pair p), by direct counting over the pairs with lane reads: sorted
// position = pairs of a smaller expert + earlier pairs of the same expert;
// a pair starts a tile when its rank inside its expert is a multiple of
// tile_m, and the tile's index is the number of starts before it.  The
// same outputs as the block-wide sort of the routing kernels.
template <int NV>
__device__ void wave_permute(const int* ids, int P, int E, int tile_m, int* srt_l, int4* til_l,
                             int* ntl_l, const RouteOut* ro) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < P;
  const int ep = in ? ids[lane] : 0x7fffffff;
  int lt = 0, same = 0, before = 0;
  for (int q = 0; q < P; ++q) {
    const int eq = __builtin_amdgcn_readlane(ep, q);
    lt += eq < ep;
    same += eq == ep;
    before += (eq == ep) & (q < lane);
  }
  const int pos = lt + before;
  const bool start = in && before % tile_m == 0;
  int tidx = 0;
  for (int q = 0; q < P; ++q) {
    const int sq = __builtin_amdgcn_readlane((int)start, q);
    const int pq = __builtin_amdgcn_readlane(pos, q);
    tidx += sq & (pq < pos);
  }
  const int n_tiles = __popcll(__ballot(start));
  if (in) srt_l[pos] = lane;
  if (start) til_l[tidx] = make_int4(ep, pos, min(pos + tile_m, lt + same), 0);
  if (lane == 0) *ntl_l = n_tiles;
  if (ro) {
    if (in) {
      ro->sorted_pair[pos] = lane;
      ro->pair_pos[lane] = pos;
    }
    if (start)
      reinterpret_cast<int4*>(ro->tiles)[tidx] =
          make_int4(ep, pos, min(pos + tile_m, lt + same), 0);
    if (lane == 0) {
      *ro->n_tiles = n_tiles;
      ro->offsets[E] = P;
    }
    // counts and offsets of every expert
#pragma unroll
    for (int jv = 0; jv < NV; ++jv) {
      const int ex = lane + 64 * jv;
      int c = 0, o = 0;
      for (int q = 0; q < P; ++q) {
        const int eq = __builtin_amdgcn_readlane(ep, q);
        c += eq == ex;
        o += eq < ex;
      }
      if (ex < E) {
        ro->counts[ex] = c;
        ro->offsets[ex] = o;
      }
    }
  }
}

template <int MAXT, int CPL, int NV>
__global__ __launch_bounds__(kDecThreads) void dec_route_gateup_kernel(ProjArgs a, RouteOut ro,
                                                                       int n_ub,
                                                                       const float* logits,
                                                                       int renorm, int tile_m) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = blockIdx.x / n_ub, ub = blockIdx.x - slot * n_ub;
  const int K = a.K, E = a.E, P = a.P;
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem);
  float* xsum = reinterpret_cast<float*>(xs + MAXT * (K / 2));
  moe_qmat* descs = reinterpret_cast<moe_qmat*>(gateup_tables<MAXT>(smem, K));
  int4* til = reinterpret_cast<int4*>(descs + E + a.n_shared);         // [64]
  int* rid = reinterpret_cast<int*>(til + kFusedMaxP);                 // [64]
  float* rw = reinterpret_cast<float*>(rid + kFusedMaxP);              // [64]
  int* srt = reinterpret_cast<int*>(rw + kFusedMaxP);                  // [64]
  int* ntl = srt + kFusedMaxP;                                         // [1]

  // ---- round trip 1: descriptors and logits; routing and sorting
  copy_descs(descs, a);
  const bool writer = blockIdx.x == 0;
  static_assert(kFusedMaxP <= 8 * kDecWaves, "every token routed in two passes");
  route_tokens<NV, 2>(logits, a.T, E, a.k, renorm, lane, wave, kDecWaves,
                      writer ? ro.ids : nullptr, writer ? ro.w : nullptr, rid, rw);
  __syncthreads();
  if (wave == 0) wave_permute<NV>(rid, P, E, tile_m, srt, til, ntl, writer ? &ro : nullptr);
  __syncthreads();

  bool is_sh;
  int e, r_begin, r_end;
  if (!dec_tile_lds(a, slot, *ntl, til, is_sh, e, r_begin, r_end)) return;
  const int U = is_sh ? a.U_sh : a.U;
  if (ub * 2 * kDecWaves >= U) return;
  const moe_qmat q = descs[is_sh ? E + e : e];
  if (!qmat_usable(q, 2 * U, K)) {
    if (tid == 0) atomicOr(a.err, 1);
    return;
  }
  gateup_tile<MAXT, CPL>(a, is_sh, e, r_begin, r_end, q, ub, srt, xs, xsum);
}

// ---------------------------------------------------------------------
// down + weighted combine.  Workgroup b owns output columns [4b, 4b + 4)
// of every token.  Every h row of the layer (sorted routed rows, then the
// shared rows) is staged once into LDS, in the planes of the bits of the
// matrix that consumes it; wave w takes the tiles w, w + 8, ... with 16
// lanes per weight row (one output column per lane group); the per-row
// results meet in LDS and each token's 8 outputs are combined in the
// fixed order of the combine: routed j = 0..k-1 (weighted), then shared.
template <int MAXT, int CPL>
__global__ __launch_bounds__(kDecThreads) void dec_down_combine_kernel(ProjArgs a, int R_rows,
                                                                       uint16_t* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ld = a.ld_in;                                                // h row stride
  const int xs_row = ld / 2, xsum_row = ld / 32;
  // LDS: tile list, descriptor tables, pair positions and gate weights
  // first (16-byte aligned), then the staged rows and the results
  int4* tls = reinterpret_cast<int4*>(smem);                             // [max_tiles]
  moe_qmat* descs = reinterpret_cast<moe_qmat*>(tls + a.max_tiles);      // [E + n_shared]
  int* ppos = reinterpret_cast<int*>(descs + a.E + a.n_shared);          // [P]
  float* gw = reinterpret_cast<float*>(ppos + a.P);                      // [P]
  int* rbits = reinterpret_cast<int*>(gw + a.P);                         // [R_rows]
  uint32_t* xs = reinterpret_cast<uint32_t*>(
      smem + (((size_t)a.max_tiles * 16 + (size_t)(a.E + a.n_shared) * sizeof(moe_qmat) +
               (size_t)a.P * 8 + (size_t)R_rows * 4 + 15) / 16 * 16));   // [R_rows][ld/2]
  float* xsum = reinterpret_cast<float*>(xs + (size_t)R_rows * xs_row);  // [R_rows][ld/32]
  float* yb = xsum + (size_t)R_rows * xsum_row;                          // [R_rows][4]
  const int H = a.U;
  const int n0 = blockIdx.x * kDecDnCols;
  const int lis = lane & (kDecDnLanes - 1), col = lane / kDecDnLanes;
  const int n = n0 + col;

  // ---- round trip 1, all independent: counts and every table
  const int n_tiles = min(ld_global(a.n_tiles), a.max_tiles);
  const int total_valid = ld_global(a.offsets + a.E);
  copy_words(reinterpret_cast<u32x4_v*>(tls), a.tiles, a.max_tiles);
  copy_descs(descs, a);
  copy_ints(ppos, a.pair_pos, a.P);
  copy_ints(reinterpret_cast<int*>(gw), reinterpret_cast<const int*>(a.topk_w), a.P);
  __syncthreads();
  const int S = a.n_sh_slots + n_tiles;

  // ---- this wave's tiles, kDecDnRounds at a time: every weight load of
  // the batch (round trip 2, together with the h rows below)
  bool ok[kDecDnRounds], shr[kDecDnRounds];
  int te[kDecDnRounds], tr0[kDecDnRounds], tr1[kDecDnRounds];
  RowGeom G[kDecDnRounds];
  uint4 wv[kDecDnRounds][CPL];
  uint32_t sv[kDecDnRounds][CPL];
  auto issue = [&](int batch) {
#pragma unroll
    for (int i = 0; i < kDecDnRounds; ++i) {
      const int slot = wave + kDecWaves * (batch * kDecDnRounds + i);
      ok[i] = slot < S && dec_tile_lds(a, slot, n_tiles, tls, shr[i], te[i], tr0[i], tr1[i]);
      if (ok[i] && !shr[i] && (unsigned)te[i] >= (unsigned)a.E) {
        if (lane == 0) atomicOr(a.err, 2);
        ok[i] = false;
      }
      moe_qmat q;
      if (ok[i]) {
        q = descs[shr[i] ? a.E + te[i] : te[i]];
        const int K = shr[i] ? a.K_sh : a.K;
        if (!qmat_usable(q, H, K)) {
          if (lane == 0) atomicOr(a.err, 1);
          ok[i] = false;
        } else {
          G[i] = row_geom(q, K, 1);
        }
      }
#pragma unroll
      for (int b = 0; b < CPL; ++b) {
        const int c = lis + kDecDnLanes * b;
        if (ok[i] && c < G[i].C_r) {
          const uint4* cp = reinterpret_cast<const uint4*>(q.codes + (size_t)n * G[i].row_bytes);
          const u32x4_v t4 = ld_global_nt(reinterpret_cast<const u32x4_v*>(cp + c));
          wv[i][b] = make_uint4(t4.x, t4.y, t4.z, t4.w);
          sv[i][b] = dec_scale(q.scales + (size_t)n * G[i].ng, G[i], c);
        } else {
          wv[i][b] = make_uint4(0u, 0u, 0u, 0u);
          sv[i][b] = 0u;
        }
      }
    }
  };
  issue(0);

  // ---- bits of every staged row: routed rows from their tiles, shared
  // rows from their expert
  for (int j = tid; j < S; j += kDecThreads) {
    bool is_sh;
    int e, r0, r1;
    if (!dec_tile_lds(a, j, n_tiles, tls, is_sh, e, r0, r1)) continue;
    if (!is_sh && (unsigned)e >= (unsigned)a.E) continue;
    const int bits = descs[is_sh ? a.E + e : e].bits;
    const int base = is_sh ? a.P + e * a.T : 0;
    for (int r = r0; r < r1; ++r) rbits[base + r] = bits;
  }
  __syncthreads();
  // ---- stage the h rows (routed rows past the valid ones are never read)
  const int nbmax = ld / 32;
  for (int u = tid; u < R_rows * nbmax; u += kDecThreads) {
    const int row = u / nbmax, b = u - row * nbmax;
    const int K = row < a.P ? a.K : a.K_sh;
    if (b >= K / 32 || (row < a.P && row >= total_valid)) continue;
    stage_a16_block(a.in_bf16 + (size_t)row * ld, b, K, rbits[row], xs + (size_t)row * xs_row,
                    xsum + (size_t)row * xsum_row);
  }
  __syncthreads();

  // ---- the tiles: 4 rows (columns n0..n0+3) of each, every token
  auto run = [&](const int i) {
    // one pass: the launcher guarantees a tile has at most MAXT rows; a
    // wave without a tile in this round computes nothing and stores
    // nothing (no early exit, so both rounds stay one straight block)
    const int nt = ok[i] ? min(MAXT, tr1[i] - tr0[i]) : 0;
    const int hrow0 = ok[i] ? (shr[i] ? a.P + te[i] * a.T : 0) + tr0[i] : 0;
    const int C_r = ok[i] ? G[i].C_r : 0;
    float acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int b = 0; b < CPL; ++b) {
      const int c = lis + kDecDnLanes * b;
      if (c < C_r)
        chunk_dot<MOE_A16, MAXT, false>(a, wv[i][b], sv[i][b], c, G[i], nt,
                                        xs + (size_t)hrow0 * xs_row, xs_row,
                                        xsum + (size_t)hrow0 * xsum_row, xsum_row, acc, lis,
                                        true, n, 0);
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t >= nt) break;
      const float v = group_sum(acc[t], kDecDnLanes);
      if (lis == 0) yb[(size_t)(hrow0 + t) * kDecDnCols + col] = v;
    }
  };
  static_assert(kDecDnRounds == 2, "one run() per round below");
  const int n_batches = (S + kDecWaves * kDecDnRounds - 1) / (kDecWaves * kDecDnRounds);
  for (int batch = 0; batch < n_batches; ++batch) {
    if (batch > 0) issue(batch);
    run(0);
    run(1);
  }
  __syncthreads();

  // ---- combine: out[t][n] = sum_j w[t][j] * y[pair_pos[t*k+j]][n] + sum_s y_s[t][n]
  for (int idx = tid; idx < a.T * kDecDnCols; idx += kDecThreads) {
    const int t = idx / kDecDnCols, cc = idx - t * kDecDnCols;
    float acc = 0.0f;
    // eight pairs at a time: all LDS reads first, then the fma chain in j
    // order
    for (int j0 = 0; j0 < a.k; j0 += 8) {
      int pp[8];
      float wj[8], yv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = j0 + u < a.k;
        pp[u] = in ? ppos[t * a.k + j0 + u] : -1;
        wj[u] = in ? gw[t * a.k + j0 + u] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) yv[u] = pp[u] >= 0 ? yb[(size_t)pp[u] * kDecDnCols + cc] : 0.0f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (pp[u] >= 0) acc = fmaf(wj[u], yv[u], acc);
    }
    for (int s = 0; s < a.n_shared; ++s) acc += yb[(size_t)(a.P + s * a.T + t) * kDecDnCols + cc];
    out[(size_t)t * H + n0 + cc] = (uint16_t)f32_to_bf16(acc);
  }
}

// ---------------------------------------------------------------------
// Launchers.  Both keep every weight chunk of a lane in registers, so the
// chunks per lane (CPL) is a template parameter: K / 32 int4 chunks per
// row over 32 (gate/up) or 16 (down) lanes, rounded up to 1 or 2 (more
// would not fit the registers of two waves per SIMD; those shapes take
// the general GEMV).
static int dec_cpl(int K, int lanes) {
  const int c = (K / 32 + lanes - 1) / lanes;
  return c <= 1 ? 1 : c <= 2 ? 2 : 0;
}

// Rows staged per tile: a tile never holds more than min(T, tile_m) rows;
// the decode kernels take it in one pass of up to 16 rows.
int dec_maxt(int T, int tile_m) {
  const int r = min(T, tile_m);
  return r <= 1 ? 1 : r <= 2 ? 2 : r <= 4 ? 4 : r <= 8 ? 8 : r <= 16 ? 16 : 0;
}

bool dec_gateup_ok(int T, int H, int tile_m) {
  return dec_cpl(H, kDecGuLanes) != 0 && dec_maxt(T, tile_m) != 0;
}

size_t dec_down_lds(int T, int k, int E, int n_shared, int max_tiles, int ld) {
  const size_t P = (size_t)T * k, R_rows = P + (size_t)n_shared * T;
  const size_t meta = ((size_t)max_tiles * 16 + (size_t)(E + n_shared) * 32 + P * 8 +
                       R_rows * 4 + 15) / 16 * 16;
  return meta + R_rows * ((size_t)ld * 2 + (size_t)(ld / 32) * 4 + kDecDnCols * 4);
}

bool dec_down_ok(int T, int k, int E, int n_shared, int H, int I, int I_shared, int ld,
                 int tile_m, int max_tiles) {
  return H % kDecDnCols == 0 && dec_maxt(T, tile_m) != 0 &&
         dec_cpl(n_shared > 0 && I_shared > I ? I_shared : I, kDecDnLanes) != 0 &&
         dec_down_lds(T, k, E, n_shared, max_tiles, ld) <= 64 * 1024;
}

template <int MAXT>
static hipError_t gu_cpl(const ProjArgs& a, int cpl, dim3 grid, size_t lds, int n_ub,
                         hipStream_t st) {
  switch (cpl) {
    case 1: dec_gateup_kernel<MAXT, 1><<<grid, kDecThreads, lds, st>>>(a, n_ub); break;
    default: dec_gateup_kernel<MAXT, 2><<<grid, kDecThreads, lds, st>>>(a, n_ub); break;
  }
  return hipGetLastError();
}

hipError_t launch_dec_gateup(const ProjArgs& a_in, hipStream_t st) {
  ProjArgs a = a_in;
  const int cpl = dec_cpl(a.K, kDecGuLanes);
  if (cpl == 0) return hipErrorInvalidValue;
  a.sh_tile = a.maxt;
  a.n_sh_slots = a.n_shared * ((a.T + a.sh_tile - 1) / a.sh_tile);
  const int Umax = max(a.U, a.n_shared > 0 ? a.U_sh : 0);
  const int n_ub = (Umax + 2 * kDecWaves - 1) / (2 * kDecWaves);
  const long long blocks = (long long)(a.n_sh_slots + a.max_tiles) * n_ub;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = ((size_t)a.maxt * a.K * 2 + (size_t)a.maxt * (a.K / 32) * 4 + 15) / 16 * 16 +
                     (size_t)(a.E + a.n_shared) * sizeof(moe_qmat) +
                     (a.P <= kDecSortedLds ? (size_t)a.P * 4 : 0);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  switch (a.maxt) {
    case 1: return gu_cpl<1>(a, cpl, grid, lds, n_ub, st);
    case 2: return gu_cpl<2>(a, cpl, grid, lds, n_ub, st);
    case 4: return gu_cpl<4>(a, cpl, grid, lds, n_ub, st);
    case 8: return gu_cpl<8>(a, cpl, grid, lds, n_ub, st);
    default: return gu_cpl<16>(a, cpl, grid, lds, n_ub, st);
  }
}

bool dec_route_gateup_ok(int T, int H, int E, int k, int tile_m) {
  return T * k <= kFusedMaxP && E <= 512 && dec_gateup_ok(T, H, tile_m);
}

template <int MAXT, int CPL>
static hipError_t rgu_nv(const ProjArgs& a, const RouteOut& ro, dim3 grid, size_t lds, int n_ub,
                         const float* logits, int renorm, int tile_m, hipStream_t st) {
  const int nv = (a.E + 63) / 64;
  if (nv <= 1)
    dec_route_gateup_kernel<MAXT, CPL, 1><<<grid, kDecThreads, lds, st>>>(a, ro, n_ub, logits, renorm, tile_m);
  else if (nv <= 2)
    dec_route_gateup_kernel<MAXT, CPL, 2><<<grid, kDecThreads, lds, st>>>(a, ro, n_ub, logits, renorm, tile_m);
  else if (nv <= 4)
    dec_route_gateup_kernel<MAXT, CPL, 4><<<grid, kDecThreads, lds, st>>>(a, ro, n_ub, logits, renorm, tile_m);
  else
    dec_route_gateup_kernel<MAXT, CPL, 8><<<grid, kDecThreads, lds, st>>>(a, ro, n_ub, logits, renorm, tile_m);
  return hipGetLastError();
}

template <int MAXT>
static hipError_t rgu_cpl(const ProjArgs& a, const RouteOut& ro, int cpl, dim3 grid, size_t lds,
                          int n_ub, const float* logits, int renorm, int tile_m, hipStream_t st) {
  if (cpl == 1) return rgu_nv<MAXT, 1>(a, ro, grid, lds, n_ub, logits, renorm, tile_m, st);
  return rgu_nv<MAXT, 2>(a, ro, grid, lds, n_ub, logits, renorm, tile_m, st);
}

hipError_t launch_dec_route_gateup(const ProjArgs& a_in, const float* logits, int renorm,
                                   int tile_m, int32_t* ids, float* w, int32_t* counts,
                                   int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                   int32_t* tiles, int32_t* n_tiles, hipStream_t st) {
  ProjArgs a = a_in;
  const int cpl = dec_cpl(a.K, kDecGuLanes);
  if (cpl == 0 || a.P > kFusedMaxP || a.E > 512) return hipErrorInvalidValue;
  a.sh_tile = a.maxt;
  a.n_sh_slots = a.n_shared * ((a.T + a.sh_tile - 1) / a.sh_tile);
  const int Umax = max(a.U, a.n_shared > 0 ? a.U_sh : 0);
  const int n_ub = (Umax + 2 * kDecWaves - 1) / (2 * kDecWaves);
  const long long blocks = (long long)(a.n_sh_slots + a.max_tiles) * n_ub;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = ((size_t)a.maxt * a.K * 2 + (size_t)a.maxt * (a.K / 32) * 4 + 15) / 16 * 16 +
                     (size_t)(a.E + a.n_shared) * sizeof(moe_qmat) + (size_t)kFusedMaxP * 28 + 16;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  RouteOut ro{ids, w, counts, offsets, sorted_pair, pair_pos, tiles, n_tiles};
  const dim3 grid((unsigned)blocks);
  switch (a.maxt) {
    case 1: return rgu_cpl<1>(a, ro, cpl, grid, lds, n_ub, logits, renorm, tile_m, st);
    case 2: return rgu_cpl<2>(a, ro, cpl, grid, lds, n_ub, logits, renorm, tile_m, st);
    case 4: return rgu_cpl<4>(a, ro, cpl, grid, lds, n_ub, logits, renorm, tile_m, st);
    case 8: return rgu_cpl<8>(a, ro, cpl, grid, lds, n_ub, logits, renorm, tile_m, st);
    default: return rgu_cpl<16>(a, ro, cpl, grid, lds, n_ub, logits, renorm, tile_m, st);
  }
}

template <int MAXT>
static hipError_t dn_cpl(const ProjArgs& a, int cpl, dim3 grid, size_t lds, int R_rows,
                         uint16_t* out, hipStream_t st) {
  switch (cpl) {
    case 1: dec_down_combine_kernel<MAXT, 1><<<grid, kDecThreads, lds, st>>>(a, R_rows, out); break;
    default: dec_down_combine_kernel<MAXT, 2><<<grid, kDecThreads, lds, st>>>(a, R_rows, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_dec_down_combine(const ProjArgs& a_in, uint16_t* out, hipStream_t st) {
  ProjArgs a = a_in;
  const int Kmax = a.n_shared > 0 && a.K_sh > a.K ? a.K_sh : a.K;
  const int cpl = dec_cpl(Kmax, kDecDnLanes);
  if (cpl == 0 || a.U % kDecDnCols != 0) return hipErrorInvalidValue;
  a.sh_tile = a.maxt;
  a.n_sh_slots = a.n_shared * ((a.T + a.sh_tile - 1) / a.sh_tile);
  const int R_rows = a.P + a.n_shared * a.T;
  const size_t lds = dec_down_lds(a.T, a.k, a.E, a.n_shared, a.max_tiles, a.ld_in);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.U / kDecDnCols));
  switch (a.maxt) {
    case 1: return dn_cpl<1>(a, cpl, grid, lds, R_rows, out, st);
    case 2: return dn_cpl<2>(a, cpl, grid, lds, R_rows, out, st);
    case 4: return dn_cpl<4>(a, cpl, grid, lds, R_rows, out, st);
    case 8: return dn_cpl<8>(a, 2, grid, lds, R_rows, out, st);   // the 1-chunk form spills
    default: return dn_cpl<16>(a, 2, grid, lds, R_rows, out, st);
  }
}

}  // namespace moe
