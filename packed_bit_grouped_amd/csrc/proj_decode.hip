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
#include <mutex>

#include "gemv_common.h"
#include "route_common.h"

namespace moe {

// Phase clock stamps (a build with MOE_DEC_STAMPS only, for the timeline
// measurement; compiled out otherwise): thread 0 of workgroup b writes the
// 100 MHz realtime counter into slot i of stamps[b][8] at each phase end,
// with an ordinary vector store.
#ifdef MOE_DEC_STAMPS
__constant__ unsigned long long* g_dec_stamps = nullptr;
#define DEC_STAMP(i)                                                            \
  do {                                                                          \
    if (g_dec_stamps && threadIdx.x == 0)                                       \
      g_dec_stamps[(size_t)blockIdx.x * 8 + (i)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define DEC_STAMP(i) \
  do {               \
  } while (0)
#endif

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecGuLanes = 32;   // lanes per weight row, gate/up
constexpr int kDecDnLanes = 16;   // lanes per weight row, down
constexpr int kDecDnCols = 64 / kDecDnLanes;   // output columns per workgroup
constexpr int kDecDnRounds = 2;   // tiles per wave with loads in flight together
constexpr int kDecSortedLds = 2048;   // pairs whose sorted list is copied to LDS

// Kernel arguments live in memory and reach the scalar cache one 64-byte
// line at a time; the compiler reads a field where it is first used, so a
// line first touched in the middle of a kernel costs a memory round trip
// there.  These read one field of every line of the argument block at the
// start, where the first loads of the kernel wait anyway.
__device__ __forceinline__ void touch_args(const ProjArgs& a) {
  // lines at 0, 64, 128 and 192 bytes of the 224-byte block
  __asm__ volatile("" ::"s"(a.mode), "s"(a.K), "s"(a.n_tiles), "s"(a.topk_w));
}

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

// Copies of small global tables into LDS in two halves: fetch() issues
// this thread's loads (words tid, tid + blockDim, ... up to PER of them)
// and put() stores them, so the loads of every table a kernel needs, and
// of anything else issued in between, share one memory round trip.
// Entries past PER * blockDim are copied by a plain loop inside put().
template <class W, int PER>
struct TableCopy {
  W v[PER];
  __device__ __forceinline__ void fetch(const W* src, int n) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = threadIdx.x + r * kDecThreads;
      if (i < n) v[r] = ld_global(src + i);
    }
  }
  __device__ __forceinline__ void put(W* dst, const W* src, int n) const {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = threadIdx.x + r * kDecThreads;
      if (i < n) dst[i] = v[r];
    }
    for (int i = threadIdx.x + PER * kDecThreads; i < n; i += kDecThreads)
      dst[i] = ld_global(src + i);
  }
};

// Descriptor tables (routed then shared) in LDS: [E + n_shared] moe_qmat,
// two 16-byte words each.
template <int PER>
struct DescCopy {
  static constexpr int kW = sizeof(moe_qmat) / 16;
  TableCopy<u32x4_v, PER> routed, shared;
  __device__ __forceinline__ void fetch(const ProjArgs& a) {
    routed.fetch(reinterpret_cast<const u32x4_v*>(a.w), a.E * kW);
    if (a.n_shared > 0) shared.fetch(reinterpret_cast<const u32x4_v*>(a.w_sh), a.n_shared * kW);
  }
  __device__ __forceinline__ void put(moe_qmat* dst, const ProjArgs& a) const {
    routed.put(reinterpret_cast<u32x4_v*>(dst), reinterpret_cast<const u32x4_v*>(a.w), a.E * kW);
    if (a.n_shared > 0)
      shared.put(reinterpret_cast<u32x4_v*>(dst + a.E),
                 reinterpret_cast<const u32x4_v*>(a.w_sh), a.n_shared * kW);
  }
};

// Scale word of code chunk c (int2 with 32-wide groups: two scales).
__device__ __forceinline__ uint32_t dec_scale(const uint16_t* sp, const RowGeom& G, int c) {
  return (G.bits == 2 && G.group == 32) ? ld_global(reinterpret_cast<const uint32_t*>(sp + 2 * c))
                                        : (uint32_t)ld_global(sp + (c * G.CK) / G.group);
}
// The same without a branch (two 16-bit loads, then a select), for the
// gate/up weight issue: loads issued under conditions leave the compiler
// unsure how many are still in flight after them, and it then waits for
// all of them before the activation staging that follows.
__device__ __forceinline__ uint32_t dec_scale_flat(const uint16_t* sp, const RowGeom& G, int c) {
  const bool two = G.bits == 2 && G.group == 32;
  const int i0 = two ? 2 * c : (c * G.CK) / G.group;
  const uint32_t lo = ld_global(sp + i0), hi = ld_global(sp + (two ? i0 + 1 : i0));
  return two ? (lo | (hi << 16)) : lo;
}

// ---------------------------------------------------------------------
// gate/up + SiLU*mul.  Grid: (n_sh_slots + max_tiles) * n_ub workgroups;
// workgroup (slot, ub) owns units [16 ub, 16 ub + 16) of its tile's
// expert.  Wave w: units 16 ub + w and 16 ub + 8 + w, the loads of both
// issued together; lanes 0-31 hold a unit's gate row, lanes 32-63 its up
// row.  srow: the sorted pair list in LDS, or null (read from memory).
//
// Split in two: gu_issue starts every weight load of the wave (nothing
// waits), gu_compute applies the staged activation rows and writes h.
template <int CPL>
struct GuRows {
  int unit[2], wr[2];
  bool vrow[2];
  RowGeom G;
  uint4 wv[2][CPL];
  uint32_t sv[2][CPL];
};

template <int CPL>
__device__ __forceinline__ void gu_issue(GuRows<CPL>& g, const ProjArgs& a, bool is_sh,
                                         const moe_qmat& q, int ub) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int U = is_sh ? a.U_sh : a.U;
  g.G = row_geom(q, a.K, 0);
  const int lis = lane & (kDecGuLanes - 1);
  const bool up = lane >= kDecGuLanes;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    g.unit[r] = ub * 2 * kDecWaves + r * kDecWaves + wave;
    g.vrow[r] = g.unit[r] < U;
    g.wr[r] = g.vrow[r] ? g.unit[r] + (up ? U : 0) : 0;
  }
  // every load unconditional (an idle slot reads chunk 0 of its row, which
  // exists, and keeps zeros), so the compiler's wait counts stay exact
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint4* cp = reinterpret_cast<const uint4*>(q.codes + (size_t)g.wr[r] * g.G.row_bytes);
    const uint16_t* sp = q.scales + (size_t)g.wr[r] * g.G.ng;
#pragma unroll
    for (int b = 0; b < CPL; ++b) {
      const int c = lis + kDecGuLanes * b;
      const bool ok = g.vrow[r] && c < g.G.C_r;
      const int cc = ok ? c : 0;
      const u32x4_v t4 = ld_global_nt(reinterpret_cast<const u32x4_v*>(cp + cc));
      const uint32_t sv = dec_scale_flat(sp, g.G, cc);
      g.wv[r][b] = ok ? make_uint4(t4.x, t4.y, t4.z, t4.w) : make_uint4(0u, 0u, 0u, 0u);
      g.sv[r][b] = ok ? sv : 0u;
    }
  }
}

// COHERENT: h is stored at device scope (read back by other workgroups of
// the same launch).
template <int MAXT, int CPL, bool COHERENT = false>
__device__ __forceinline__ void gu_compute(const GuRows<CPL>& g, const ProjArgs& a, bool is_sh,
                                           int e, int r_begin, int nt, const uint32_t* xs,
                                           const float* xsum) {
  const int lane = threadIdx.x & 63;
  const int K = a.K;
  const int lis = lane & (kDecGuLanes - 1);
  const int xs_row = K / 2, xsum_row = K / 32;
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
      if (c < g.G.C_r)
        chunk_dot<MOE_A16, MAXT, false>(a, g.wv[r][b], g.sv[r][b], c, g.G, nt, xs, xs_row, xsum,
                                        xsum_row, acc, lis, g.vrow[r], g.wr[r], 0);
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t >= nt) break;
      // rows of 16 lanes, then row 0 into row 1 and row 2 into row 3:
      // lane 16 ends with the gate sum, lane 48 with the up sum
      float gs = group_sum(acc[t], 16);
      gs += dpp_f<kDppRowBcast15, 0xA>(0.0f, gs);
      const float u = __shfl_down(gs, 32);
      if (lane == 16 && g.vrow[r]) {
        uint16_t* hp = h + (size_t)(orow0 + t) * a.ld_out + g.unit[r];
        const uint16_t hv = (uint16_t)f32_to_bf16(silu_mul(gs, u));
        if (COHERENT)
          __hip_atomic_store(hp, hv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *hp = hv;
      }
    }
  }
}

template <int MAXT, int CPL>
__device__ __forceinline__ void gateup_tile(const ProjArgs& a, bool is_sh, int e, int r_begin,
                                            int r_end, const moe_qmat& q, int ub,
                                            const int* srow, uint32_t* xs, float* xsum) {
  const int tid = threadIdx.x;
  const int K = a.K;
  // ---- the tile's activation rows first, then every weight load of the
  // workgroup: the staging waits only for the activations, and each wave
  // starts its products as its own weights arrive
  const int xs_row = K / 2, xsum_row = K / 32, nb32 = K / 32;
  // one pass: the launcher guarantees a tile has at most MAXT rows (and K
  // at most 2048: 64 blocks per row)
  const int nt = min(MAXT, r_end - r_begin);
  constexpr int XI = (MAXT * 64 + kDecThreads - 1) / kDecThreads;
  uint32_t xv[XI][16];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int u = tid + i * kDecThreads;
    if (u < nt * nb32) {
      const int m = u / nb32, b = u - m * nb32;
      int row = r_begin + m;
      if (!is_sh) row = (srow ? srow[row] : ld_global(a.sorted_pair + row)) / a.k;
      load_a16_block(a.in_bf16 + (size_t)row * a.ld_in, b, xv[i]);
    }
  }
  GuRows<CPL> g;
  gu_issue<CPL>(g, a, is_sh, q, ub);
  DEC_STAMP(3);   // weight loads issued
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int u = tid + i * kDecThreads;
    if (u < nt * nb32) {
      const int m = u / nb32, b = u - m * nb32;
      store_a16_block(xv[i], b, K, g.G.bits, xs + m * xs_row, xsum + m * xsum_row);
    }
  }
  lds_barrier();
  DEC_STAMP(4);   // activations staged
  gu_compute<MAXT, CPL>(g, a, is_sh, e, r_begin, nt, xs, xsum);
  DEC_STAMP(5);   // products and h stores done
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
  touch_args(a);
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
  DescCopy<1> dc;
  TableCopy<int, 1> sc;
  dc.fetch(a);
  if (srow_lds) sc.fetch(a.sorted_pair, a.P);
  dc.put(descs, a);
  if (srow_lds) sc.put(srow, a.sorted_pair, a.P);
  lds_barrier();

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
// holds pair p; expert ids below 2^kPermIdBits).  One radix pass over the
// id bits with ballots gives each pair the set of pairs sorted before it
// (a smaller expert, or the same expert and a smaller pair index); its
// position is that set's size.  A pair starts a tile when its rank inside
// its expert is a multiple of tile_m, and the tile's index is the number
// of tile starts sorted before it.  Straight-line lane-mask arithmetic: a
// loop over the pairs with lane reads costs about a microsecond of
// dependent instructions in a single wave.  The same outputs as the
// block-wide sort of the routing kernels; the writer's per-expert counts
// and offsets come from wave_counts.
template <int NV>
__device__ void wave_permute(const int* ids, int P, int E, int tile_m, int* srt_l, int4* til_l,
                             int* ntl_l, int* ppos_l, const RouteOut* ro) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < P;
  const int ep = in ? ids[lane] : 0;
  // eq: valid pairs whose id agrees with mine on the bits seen so far;
  // lt: pairs already known to have a smaller id
  uint64_t eq = __ballot(in), lt = 0;
#pragma unroll
  for (int b = kPermIdBits - 1; b >= 0; --b) {
    const bool bit = (ep >> b) & 1;
    const uint64_t ones = __ballot(in && bit);
    lt = bit ? (lt | (eq & ~ones)) : lt;
    eq = bit ? (eq & ones) : (eq & ~ones);
  }
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));   // lanes < lane
  const uint64_t ahead = lt | (eq & below);                           // sorted before me
  const int n_lt = __popcll(lt), same = __popcll(eq), before = __popcll(eq & below);
  const int pos = n_lt + before;
  const bool start = in && before % tile_m == 0;
  const uint64_t starts = __ballot(start);
  const int tidx = __popcll(starts & ahead);
  const int n_tiles = __popcll(starts);
  const int4 tile = make_int4(ep, pos, min(pos + tile_m, n_lt + same), 0);
  if (in) srt_l[pos] = lane;
  if (in && ppos_l) ppos_l[lane] = pos;
  if (start) til_l[tidx] = tile;
  if (lane == 0) *ntl_l = n_tiles;
  if (ro) {
    if (in) {
      ro->sorted_pair[pos] = lane;
      ro->pair_pos[lane] = pos;
    }
    if (start) reinterpret_cast<int4*>(ro->tiles)[tidx] = tile;
    if (lane == 0) {
      *ro->n_tiles = n_tiles;
      ro->offsets[E] = P;
    }
  }
}

// Per-expert pair counts and offsets (pairs of a smaller expert) of the
// experts [64 j, 64 j + 64), by one wave reading the ids from LDS; run by
// the writer workgroup's otherwise idle waves while wave 0 sorts.
__device__ void wave_counts(const int* ids, int P, int E, int j, const RouteOut& ro) {
  const int ex = (threadIdx.x & 63) + 64 * j;
  int c = 0, o = 0;
  for (int q = 0; q < P; ++q) {
    const int eq = ids[q];
    c += eq == ex;
    o += eq < ex;
  }
  if (ex < E) {
    ro.counts[ex] = c;
    ro.offsets[ex] = o;
  }
}

// The sort and, in the writer workgroup, the counts: wave 0 sorts, waves
// 1.. count experts [64 (w - 1), 64 w); experts past the waves' reach are
// counted by wave 0 after its sort.
template <int NV>
__device__ __forceinline__ void block_permute(const int* ids, int P, int E, int tile_m, int* srt_l,
                                              int4* til_l, int* ntl_l, int* ppos_l, bool writer,
                                              const RouteOut& ro) {
  const int wave = threadIdx.x >> 6;
  if (wave == 0) {
    wave_permute<NV>(ids, P, E, tile_m, srt_l, til_l, ntl_l, ppos_l, writer ? &ro : nullptr);
    if (writer)
      for (int j = kDecWaves - 1; j < NV; ++j) wave_counts(ids, P, E, j, ro);
  } else if (writer && wave - 1 < NV) {
    wave_counts(ids, P, E, wave - 1, ro);
  }
}

template <int MAXT, int CPL, int NV>
__global__ __launch_bounds__(kDecThreads) void dec_route_gateup_kernel(ProjArgs a, RouteOut ro,
                                                                       int n_ub,
                                                                       const float* logits,
                                                                       int renorm, int tile_m) {
  extern __shared__ __align__(16) unsigned char smem[];
  // the argument block: ProjArgs, then the routing outputs and scalars
  touch_args(a);
  __asm__ volatile("" ::"s"(ro.sorted_pair), "s"(logits));
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

  // ---- round trip 1: descriptors and logits together; routing and sorting
  DEC_STAMP(0);   // entry
  DescCopy<1> dc;
  dc.fetch(a);
  const bool writer = blockIdx.x == 0;
  static_assert(kFusedMaxP <= 8 * kDecWaves, "every token routed in two passes");
  route_tokens<NV, 2>(logits, a.T, E, a.k, renorm, lane, wave, kDecWaves,
                      writer ? ro.ids : nullptr, writer ? ro.w : nullptr, rid, rw);
  dc.put(descs, a);
  lds_barrier();
  DEC_STAMP(1);   // logits and descriptors in, top-k done
  block_permute<NV>(rid, P, E, tile_m, srt, til, ntl, nullptr, writer, ro);
  lds_barrier();
  DEC_STAMP(2);   // sorted, tile list in LDS

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
//
// The pieces (dn_issue, dn_stage, dn_run, dn_combine) are shared with the
// one-launch layer kernel below.

// LDS carve-up of the down part: per-row bits, the staged h rows, their
// block sums and the per-row results.
struct DnLds {
  int* rbits;      // [R_rows]
  uint32_t* xs;    // [R_rows][ld/2]
  float* xsum;     // [R_rows][ld/32]
  float* yb;       // [R_rows][kDecDnCols]
};
__device__ __forceinline__ size_t dn_rows_bytes(int R_rows, int ld) {
  return (size_t)R_rows * ((size_t)ld * 2 + (size_t)(ld / 32) * 4 + kDecDnCols * 4);
}
// base: 16-byte aligned; rbits first, then the rows from the next 16 bytes.
__device__ __forceinline__ DnLds dn_lds(unsigned char* base, int R_rows, int ld) {
  DnLds d;
  d.rbits = reinterpret_cast<int*>(base);
  d.xs = reinterpret_cast<uint32_t*>(base + ((size_t)R_rows * 4 + 15) / 16 * 16);
  d.xsum = reinterpret_cast<float*>(d.xs + (size_t)R_rows * (ld / 2));
  d.yb = d.xsum + (size_t)R_rows * (ld / 32);
  return d;
}

template <int CPL>
struct DnSlots {
  bool ok[kDecDnRounds], shr[kDecDnRounds];
  int te[kDecDnRounds], tr0[kDecDnRounds], tr1[kDecDnRounds];
  RowGeom G[kDecDnRounds];
  uint4 wv[kDecDnRounds][CPL];
  uint32_t sv[kDecDnRounds][CPL];
};

// This wave's tiles of batch `batch` (kDecDnRounds of them): every weight
// load of the four columns n0..n0+3, nothing waits.
template <int CPL>
__device__ __forceinline__ void dn_issue(DnSlots<CPL>& d, const ProjArgs& a, int batch, int S,
                                         int n_tiles, const int4* tls, const moe_qmat* descs,
                                         int n) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lis = lane & (kDecDnLanes - 1);
  const int H = a.U;
#pragma unroll
  for (int i = 0; i < kDecDnRounds; ++i) {
    const int slot = wave + kDecWaves * (batch * kDecDnRounds + i);
    d.ok[i] = slot < S && dec_tile_lds(a, slot, n_tiles, tls, d.shr[i], d.te[i], d.tr0[i], d.tr1[i]);
    if (d.ok[i] && !d.shr[i] && (unsigned)d.te[i] >= (unsigned)a.E) {
      if (lane == 0) atomicOr(a.err, 2);
      d.ok[i] = false;
    }
    moe_qmat q;
    if (d.ok[i]) {
      q = descs[d.shr[i] ? a.E + d.te[i] : d.te[i]];
      const int K = d.shr[i] ? a.K_sh : a.K;
      if (!qmat_usable(q, H, K)) {
        if (lane == 0) atomicOr(a.err, 1);
        d.ok[i] = false;
      } else {
        d.G[i] = row_geom(q, K, 1);
      }
    }
#pragma unroll
    for (int b = 0; b < CPL; ++b) {
      const int c = lis + kDecDnLanes * b;
      if (d.ok[i] && c < d.G[i].C_r) {
        const uint4* cp = reinterpret_cast<const uint4*>(q.codes + (size_t)n * d.G[i].row_bytes);
        const u32x4_v t4 = ld_global_nt(reinterpret_cast<const u32x4_v*>(cp + c));
        d.wv[i][b] = make_uint4(t4.x, t4.y, t4.z, t4.w);
        d.sv[i][b] = dec_scale(q.scales + (size_t)n * d.G[i].ng, d.G[i], c);
      } else {
        d.wv[i][b] = make_uint4(0u, 0u, 0u, 0u);
        d.sv[i][b] = 0u;
      }
    }
  }
}

// Bits of every staged row (routed rows from their tiles, shared rows from
// their expert), then the h rows themselves (routed rows past the valid
// ones are never read).  Ends with the block in step.
template <bool COHERENT = false>
__device__ __forceinline__ void dn_stage(const ProjArgs& a, int S, int n_tiles, const int4* tls,
                                         const moe_qmat* descs, int R_rows, int total_valid,
                                         const DnLds& L) {
  const int tid = threadIdx.x;
  const int ld = a.ld_in;
  const int xs_row = ld / 2, xsum_row = ld / 32;
  for (int j = tid; j < S; j += kDecThreads) {
    bool is_sh;
    int e, r0, r1;
    if (!dec_tile_lds(a, j, n_tiles, tls, is_sh, e, r0, r1)) continue;
    if (!is_sh && (unsigned)e >= (unsigned)a.E) continue;
    const int bits = descs[is_sh ? a.E + e : e].bits;
    const int base = is_sh ? a.P + e * a.T : 0;
    for (int r = r0; r < r1; ++r) L.rbits[base + r] = bits;
  }
  lds_barrier();
  const int nbmax = ld / 32;
  for (int u = tid; u < R_rows * nbmax; u += kDecThreads) {
    const int row = u / nbmax, b = u - row * nbmax;
    const int K = row < a.P ? a.K : a.K_sh;
    if (b >= K / 32 || (row < a.P && row >= total_valid)) continue;
    uint32_t v[16];
    if (COHERENT)
      load_a16_block_coherent(a.in_bf16 + (size_t)row * ld, b, v);
    else
      load_a16_block(a.in_bf16 + (size_t)row * ld, b, v);
    store_a16_block(v, b, K, L.rbits[row], L.xs + (size_t)row * xs_row,
                    L.xsum + (size_t)row * xsum_row);
  }
  lds_barrier();
}

// Round i of the wave's batch: the 4 rows (columns n0..n0+3) of the tile
// against every token of it.  One pass: the launcher guarantees a tile has
// at most MAXT rows; a wave without a tile in this round computes nothing
// and stores nothing (no early exit, so the rounds stay one straight block).
template <int MAXT, int CPL>
__device__ __forceinline__ void dn_run(const DnSlots<CPL>& d, int i, const ProjArgs& a,
                                       const DnLds& L, int n) {
  const int lane = threadIdx.x & 63;
  const int lis = lane & (kDecDnLanes - 1), col = lane / kDecDnLanes;
  const int xs_row = a.ld_in / 2, xsum_row = a.ld_in / 32;
  const int nt = d.ok[i] ? min(MAXT, d.tr1[i] - d.tr0[i]) : 0;
  const int hrow0 = d.ok[i] ? (d.shr[i] ? a.P + d.te[i] * a.T : 0) + d.tr0[i] : 0;
  const int C_r = d.ok[i] ? d.G[i].C_r : 0;
  float acc[MAXT];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) acc[t] = 0.0f;
#pragma unroll
  for (int b = 0; b < CPL; ++b) {
    const int c = lis + kDecDnLanes * b;
    if (c < C_r)
      chunk_dot<MOE_A16, MAXT, false>(a, d.wv[i][b], d.sv[i][b], c, d.G[i], nt,
                                      L.xs + (size_t)hrow0 * xs_row, xs_row,
                                      L.xsum + (size_t)hrow0 * xsum_row, xsum_row, acc, lis,
                                      true, n, 0);
  }
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t >= nt) break;
    const float v = group_sum(acc[t], kDecDnLanes);
    if (lis == 0) L.yb[(size_t)(hrow0 + t) * kDecDnCols + col] = v;
  }
}

// out[t][n] = sum_j w[t][j] * y[pair_pos[t*k+j]][n] + sum_s y_s[t][n] for
// the columns n0..n0+3, in that order.
__device__ __forceinline__ void dn_combine(const ProjArgs& a, const int* ppos, const float* gw,
                                           const float* yb, void* __restrict__ out, int n0) {
  const int H = a.U;
  for (int idx = threadIdx.x; idx < a.T * kDecDnCols; idx += kDecThreads) {
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
    for (int s = 0; s < a.n_shared; ++s) {
      // weight 1 (fmaf(1, y, acc) is acc + y) or the token's sigmoid gate
      const float g = a.sh_gate ? shared_gate_weight(a.sh_gate[t * a.n_shared + s]) : 1.0f;
      acc = fmaf(g, yb[(size_t)(a.P + s * a.T + t) * kDecDnCols + cc], acc);
    }
    if (a.out_f32) static_cast<float*>(out)[(size_t)t * H + n0 + cc] = acc;
    else static_cast<uint16_t*>(out)[(size_t)t * H + n0 + cc] = (uint16_t)f32_to_bf16(acc);
  }
}

template <int MAXT, int CPL>
__global__ __launch_bounds__(kDecThreads) void dec_down_combine_kernel(ProjArgs a, int R_rows,
                                                                       void* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char smem[];
  touch_args(a);
  // LDS: tile list, descriptor tables, pair positions and gate weights
  // first (16-byte aligned), then the down part's rows
  int4* tls = reinterpret_cast<int4*>(smem);                             // [max_tiles]
  moe_qmat* descs = reinterpret_cast<moe_qmat*>(tls + a.max_tiles);      // [E + n_shared]
  int* ppos = reinterpret_cast<int*>(descs + a.E + a.n_shared);          // [P]
  float* gw = reinterpret_cast<float*>(ppos + a.P);                      // [P]
  const DnLds L = dn_lds(smem + ((size_t)a.max_tiles * 16 +
                                 (size_t)(a.E + a.n_shared) * sizeof(moe_qmat) +
                                 (size_t)a.P * 8 + 15) / 16 * 16,
                         R_rows, a.ld_in);
  const int n0 = blockIdx.x * kDecDnCols;
  const int n = n0 + (threadIdx.x & 63) / kDecDnLanes;

  // ---- round trip 1, all independent: counts and every table
  DEC_STAMP(0);   // entry
  const int n_tiles = min(ld_global(a.n_tiles), a.max_tiles);
  const int total_valid = ld_global(a.offsets + a.E);
  const u32x4_v* tsrc = reinterpret_cast<const u32x4_v*>(a.tiles);
  const int* wsrc = reinterpret_cast<const int*>(a.topk_w);
  TableCopy<u32x4_v, 1> tc;
  DescCopy<1> dc;
  TableCopy<int, 1> pc, wc;
  tc.fetch(tsrc, a.max_tiles);
  dc.fetch(a);
  pc.fetch(a.pair_pos, a.P);
  wc.fetch(wsrc, a.P);
  tc.put(reinterpret_cast<u32x4_v*>(tls), tsrc, a.max_tiles);
  dc.put(descs, a);
  pc.put(ppos, a.pair_pos, a.P);
  wc.put(reinterpret_cast<int*>(gw), wsrc, a.P);
  lds_barrier();
  DEC_STAMP(1);   // tables in
  const int S = a.n_sh_slots + n_tiles;

  // ---- this wave's tiles, kDecDnRounds at a time: every weight load of
  // the batch (round trip 2, together with the h rows below)
  DnSlots<CPL> d;
  dn_issue<CPL>(d, a, 0, S, n_tiles, tls, descs, n);
  DEC_STAMP(2);   // weight loads issued
  dn_stage(a, S, n_tiles, tls, descs, R_rows, total_valid, L);
  DEC_STAMP(3);   // h rows staged

  static_assert(kDecDnRounds == 2, "one dn_run() per round below");
  const int n_batches = (S + kDecWaves * kDecDnRounds - 1) / (kDecWaves * kDecDnRounds);
  for (int batch = 0; batch < n_batches; ++batch) {
    if (batch > 0) dn_issue<CPL>(d, a, batch, S, n_tiles, tls, descs, n);
    dn_run<MAXT, CPL>(d, 0, a, L, n);
    dn_run<MAXT, CPL>(d, 1, a, L, n);
  }
  lds_barrier();
  DEC_STAMP(4);   // products done
  dn_combine(a, ppos, gw, L.yb, out, n0);
  DEC_STAMP(5);   // outputs stored
}

// ---------------------------------------------------------------------
// The whole decode layer in one launch (bf16 activations, T * k <= 64).
// Workgroup b routes and sorts the batch itself (as above), loads the
// activation rows of gate/up work item b (tile, unit block), issues the
// weight loads of that item and of down column block b together, writes
// its h values and meets every other workgroup at a grid-wide barrier (h
// complete); then it stages every h row and finishes the down projection
// and the combine of its four output columns.  The W2 stream overlaps the
// gate/up work and no second launch waits on the first.
//
// The barrier needs every workgroup resident at once: the launcher checks
// the occupancy before it launches, and the wait is bounded by the
// constant clock (an expired wait sets bit 2 of the error word and the
// workgroup skips its down work), so every wave reaches the end.

constexpr long long kBarrierTicks = 2000000;   // 20 ms at the 100 MHz constant clock

struct LayerArgs {
  const float* logits;
  int renorm, tile_m;
  int n_ub;        // gate/up unit blocks per tile
  int n_gu;        // gate/up work items
  int n_dn;        // down column blocks
  int R_rows;      // h rows: P + n_shared * T
  void* out;       // bf16 or fp32 (ad.out_f32)
  uint32_t* flags; // kLayerFlags barrier flags, all equal between launches
};

// Grid-wide barrier over n <= kLayerFlags workgroups without atomics:
// workgroup b flips the flags b, b + n, b + 2n, ... (so every launch flips
// each flag exactly once and they are all equal again when it ends); a
// workgroup has passed once every flag holds the flipped value.  One wave
// polls, 16 flags per lane.  Flags and h are stored and loaded at device
// scope (they bypass the per-XCD L2 rather than being written back or
// invalidated there: whole-cache maintenance from hundreds of workgroups
// costs far more than the barrier itself); every wave waits for its own h
// stores to be acknowledged before the flags are stored, so a workgroup
// that sees every flag flipped reads complete h.  Returns false when the
// wait expired.
__device__ __forceinline__ bool grid_barrier(uint32_t* flags, int n, int32_t* err,
                                             int* ok_lds) {
  const int tid = threadIdx.x;
  // phase of this launch: every flag still holds the previous launch's value
  const uint32_t target =
      1u - __hip_atomic_load(flags + blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // Ordering (h before the flags, flags before the h reads) without L2
  // write-back or invalidation: every h store and h load of this launch is
  // an agent-scope access (it goes through to the memory side, which all
  // XCDs share), and so are the flag accesses.  (1) The compiler may not
  // move a memory access across the signal fences below.  (2) The wait
  // for every outstanding memory operation of the wave returns only once
  // its h stores are acknowledged at agent scope, so they are visible to
  // every workgroup before any flag store of the workgroup is issued
  // (the LDS barrier orders the waves of the workgroup).  (3) A poller
  // leaves the loop only after its flag loads have returned the target
  // (the exit depends on their values), and its h loads are issued after
  // that, at agent scope, so they read the stored h.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);   // this wave's h stores (and loads) complete
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  lds_barrier();
  for (int i = blockIdx.x + tid * n; i < kLayerFlags; i += kDecThreads * n)
    __hip_atomic_store(flags + i, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid < 64) {
    const long long t0 = wall_clock64();
    int ok = 1;
    while (true) {
      bool mine = true;
#pragma unroll
      for (int j = 0; j < kLayerFlags / 64; ++j)
        mine &= __hip_atomic_load(flags + tid + 64 * j, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT) == target;
      if (__all(mine)) break;
      if (wall_clock64() - t0 > kBarrierTicks) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (tid == 0) {
      if (!ok) atomicOr(err, 4);
      *ok_lds = ok;
    }
  }
  lds_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);   // no h load above the wait
  return *ok_lds != 0;
}

// Chunks per lane of the one-launch kernel: 2 for gate/up (H <= 2048) and
// down (I <= 1024); smaller K leaves slots idle.
constexpr int kLayerCpl = 2;

template <int MAXT, int NV>
__global__ __launch_bounds__(kDecThreads, 4) void dec_layer_kernel(ProjArgs ag, ProjArgs ad,
                                                                RouteOut ro, LayerArgs la) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int bar_ok;
  // the argument block: both ProjArgs, the routing outputs, LayerArgs
  touch_args(ag);
  touch_args(ad);
  __asm__ volatile("" ::"s"(ro.ids), "s"(ro.n_tiles), "s"(la.logits), "s"(la.flags));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = ag.K, E = ag.E, P = ag.P;
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem);                    // [MAXT][K/2]
  float* xsum = reinterpret_cast<float*>(xs + MAXT * (K / 2));         // [MAXT][K/32]
  moe_qmat* d13 = reinterpret_cast<moe_qmat*>(gateup_tables<MAXT>(smem, K));
  moe_qmat* d2 = d13 + E + ag.n_shared;
  int4* til = reinterpret_cast<int4*>(d2 + E + ad.n_shared);         // [64]
  int* rid = reinterpret_cast<int*>(til + kFusedMaxP);               // [64]
  float* rw = reinterpret_cast<float*>(rid + kFusedMaxP);            // [64]
  int* srt = reinterpret_cast<int*>(rw + kFusedMaxP);                // [64]
  int* ppos = srt + kFusedMaxP;                                      // [64]
  int* ntl = ppos + kFusedMaxP;                                      // [4]
  const DnLds L = dn_lds(reinterpret_cast<unsigned char*>(ntl + 4), la.R_rows, ad.ld_in);

  // ---- round trip 1: both descriptor tables and the logits together;
  // routing and sorting
  DescCopy<1> c13, c2;
  c13.fetch(ag);
  c2.fetch(ad);
  const bool writer = blockIdx.x == 0;
  static_assert(kFusedMaxP <= 8 * kDecWaves, "every token routed in two passes");
  route_tokens<NV, 2>(la.logits, ag.T, E, ag.k, la.renorm, lane, wave, kDecWaves,
                      writer ? ro.ids : nullptr, writer ? ro.w : nullptr, rid, rw);
  c13.put(d13, ag);
  c2.put(d2, ad);
  lds_barrier();
  block_permute<NV>(rid, P, E, la.tile_m, srt, til, ntl, ppos, writer, ro);
  lds_barrier();
  const int n_tiles = min(*ntl, ag.max_tiles);

  // ---- gate/up work item of this workgroup (uniform over the block)
  bool gu = (int)blockIdx.x < la.n_gu;
  bool is_sh = false;
  int e = 0, r_begin = 0, r_end = 0;
  const int slot = blockIdx.x / la.n_ub, ub = blockIdx.x - slot * la.n_ub;
  if (gu) gu = dec_tile_lds(ag, slot, n_tiles, til, is_sh, e, r_begin, r_end);
  if (gu) gu = ub * 2 * kDecWaves < (is_sh ? ag.U_sh : ag.U);
  moe_qmat q13;
  int gbits = 4;
  if (gu) {
    q13 = d13[is_sh ? E + e : e];
    if (!qmat_usable(q13, 2 * (is_sh ? ag.U_sh : ag.U), K)) {
      if (tid == 0) atomicOr(ag.err, 1);
      gu = false;
    } else {
      gbits = q13.bits;
    }
  }

  // ---- round trip 2: the tile's activation rows first (their wait does
  // not cover the weights), then every weight load of both items
  const int nb32 = K / 32;
  const int nt = gu ? min(MAXT, r_end - r_begin) : 0;
  constexpr int XI = (MAXT * 64 + kDecThreads - 1) / kDecThreads;   // K <= 2048
  uint32_t xv[XI][16];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int u = tid + i * kDecThreads;
    if (u < nt * nb32) {
      const int m = u / nb32, b = u - m * nb32;
      const int row = is_sh ? r_begin + m : srt[r_begin + m] / ag.k;
      load_a16_block(ag.in_bf16 + (size_t)row * ag.ld_in, b, xv[i]);
    }
  }
  GuRows<kLayerCpl> g;
  if (gu) gu_issue<kLayerCpl>(g, ag, is_sh, q13, ub);
  const bool dn = (int)blockIdx.x < la.n_dn;
  const int n0 = blockIdx.x * kDecDnCols;
  const int n = n0 + lane / kDecDnLanes;
  const int S = ad.n_sh_slots + n_tiles;
  DnSlots<kLayerCpl> d;
  if (dn) dn_issue<kLayerCpl>(d, ad, 0, S, n_tiles, til, d2, n);

  // ---- gate/up + SiLU*mul of the item, h to memory
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int u = tid + i * kDecThreads;
    if (u < nt * nb32) {
      const int m = u / nb32, b = u - m * nb32;
      store_a16_block(xv[i], b, K, gbits, xs + m * (K / 2), xsum + m * nb32);
    }
  }
  lds_barrier();
  if (gu) gu_compute<MAXT, kLayerCpl, true>(g, ag, is_sh, e, r_begin, nt, xs, xsum);

  // ---- every h value of the layer stored
  if (!grid_barrier(la.flags, gridDim.x, ag.err, &bar_ok) || !dn) return;

  // ---- down + combine of columns n0..n0+3
  dn_stage<true>(ad, S, n_tiles, til, d2, la.R_rows, P, L);
  static_assert(kDecDnRounds == 2, "one dn_run() per round below");
  const int n_batches = (S + kDecWaves * kDecDnRounds - 1) / (kDecWaves * kDecDnRounds);
  for (int batch = 0; batch < n_batches; ++batch) {
    if (batch > 0) dn_issue<kLayerCpl>(d, ad, batch, S, n_tiles, til, d2, n);
    dn_run<MAXT, kLayerCpl>(d, 0, ad, L, n);
    dn_run<MAXT, kLayerCpl>(d, 1, ad, L, n);
  }
  lds_barrier();
  dn_combine(ad, ppos, rw, L.yb, la.out, n0);
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
  const size_t meta = ((size_t)max_tiles * 16 + (size_t)(E + n_shared) * 32 + P * 8 + 15) / 16 * 16;
  return meta + (R_rows * 4 + 15) / 16 * 16 +
         R_rows * ((size_t)ld * 2 + (size_t)(ld / 32) * 4 + kDecDnCols * 4);
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
                         void* out, hipStream_t st) {
  switch (cpl) {
    case 1: dec_down_combine_kernel<MAXT, 1><<<grid, kDecThreads, lds, st>>>(a, R_rows, out); break;
    default: dec_down_combine_kernel<MAXT, 2><<<grid, kDecThreads, lds, st>>>(a, R_rows, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_dec_down_combine(const ProjArgs& a_in, void* out, hipStream_t st) {
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

// One-launch layer: eligibility, LDS and grid.
bool dec_layer_ok(int T, int H, int I, int I_shared, int E, int k, int n_shared, int tile_m,
                  int max_tiles, int ld_h) {
  const int Kd = n_shared > 0 && I_shared > I ? I_shared : I;
  return E <= 128 && dec_route_gateup_ok(T, H, E, k, tile_m) &&
         dec_cpl(H, kDecGuLanes) <= kLayerCpl &&
         dec_cpl(Kd, kDecDnLanes) != 0 && dec_cpl(Kd, kDecDnLanes) <= kLayerCpl &&
         dec_down_ok(T, k, E, n_shared, H, I, I_shared, ld_h, tile_m, max_tiles) &&
         max_tiles <= kFusedMaxP;
}

static size_t dec_layer_lds(int T, int k, int E, int n_shared, int K, int maxt, int ld_h) {
  const size_t P = (size_t)T * k, R = P + (size_t)n_shared * T;
  size_t lds = ((size_t)maxt * K * 2 + (size_t)maxt * (K / 32) * 4 + 15) / 16 * 16;
  lds += 2 * (size_t)(E + n_shared) * sizeof(moe_qmat);
  lds += (size_t)kFusedMaxP * 16 + 4 * (size_t)kFusedMaxP * 4 + 16;
  lds += (R * 4 + 15) / 16 * 16 + R * ((size_t)ld_h * 2 + (size_t)(ld_h / 32) * 4 + kDecDnCols * 4);
  return lds;
}

// Workgroups of kernel f (dynamic LDS lds) resident on one CU of the
// current device, and the device's CU count; both cached.
static bool resident_capacity(const void* f, size_t lds, long long& cap) {
  struct Entry {
    const void* f;
    size_t lds;
    int dev;
    long long cap;
  };
  static Entry cache[64];
  static int n_cache = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n_cache; ++i)
    if (cache[i].f == f && cache[i].lds == lds && cache[i].dev == dev) {
      cap = cache[i].cap;
      return true;
    }
  int nb = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, kDecThreads, lds) != hipSuccess)
    return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  cap = (long long)nb * cus;
  if (n_cache < 64) cache[n_cache++] = Entry{f, lds, dev, cap};
  return true;
}

// The kernel instance of a shape: rows per tile pass, and one or two
// logits per lane (E <= 128: wider routing does not fit the registers of
// four waves per SIMD).
template <int MAXT>
static const void* layer_fn_nv(int E) {
  return E <= 64 ? reinterpret_cast<const void*>(&dec_layer_kernel<MAXT, 1>)
                 : reinterpret_cast<const void*>(&dec_layer_kernel<MAXT, 2>);
}
static const void* layer_fn(int maxt, int E) {
  switch (maxt) {
    case 1: return layer_fn_nv<1>(E);
    case 2: return layer_fn_nv<2>(E);
    case 4: return layer_fn_nv<4>(E);
    case 8: return layer_fn_nv<8>(E);
    default: return layer_fn_nv<16>(E);
  }
}

// Grid, LDS and residency of the one-launch layer for a shape.
struct LayerPlan {
  int n_ub, n_gu, n_dn, grid;
  size_t lds;
  const void* fn;
  bool resident;
};
static LayerPlan layer_plan(int T, int H, int I, int I_shared, int E, int k, int n_shared,
                            int tile_m, int max_tiles, int ld_h) {
  LayerPlan p{};
  const int maxt = dec_maxt(T, tile_m);
  const int n_sh_slots = n_shared * ((T + maxt - 1) / maxt);
  const int Umax = max(I, n_shared > 0 ? I_shared : 0);
  p.n_ub = (Umax + 2 * kDecWaves - 1) / (2 * kDecWaves);
  p.n_gu = (n_sh_slots + max_tiles) * p.n_ub;
  p.n_dn = H / kDecDnCols;
  p.grid = max(p.n_gu, p.n_dn);
  p.lds = dec_layer_lds(T, k, E, n_shared, H, maxt, ld_h);
  p.fn = layer_fn(maxt, E);
  long long cap = 0;
  p.resident = p.grid > 0 && p.grid <= kLayerFlags && p.lds <= 160 * 1024 &&
               resident_capacity(p.fn, p.lds, cap) && cap >= p.grid;
  return p;
}

int dec_layer_one_launch(int T, int H, int I, int I_shared, int E, int k, int n_shared,
                         int tile_m, int max_tiles, int ld_h) {
  if (!dec_layer_ok(T, H, I, I_shared, E, k, n_shared, tile_m, max_tiles, ld_h)) return 0;
  return layer_plan(T, H, I, I_shared, E, k, n_shared, tile_m, max_tiles, ld_h).resident ? 1 : 0;
}

hipError_t launch_dec_layer(const ProjArgs& ag_in, const ProjArgs& ad_in, const float* logits,
                            int renorm, int tile_m, int32_t* ids, float* w, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                            int32_t* tiles, int32_t* n_tiles, void* out, uint32_t* flags,
                            bool& launched, hipStream_t st) {
  launched = false;
  ProjArgs ag = ag_in, ad = ad_in;
  if (ag.P > kFusedMaxP || ag.E > 128 || ag.max_tiles > kFusedMaxP || ad.U % kDecDnCols != 0 ||
      ag.maxt != dec_maxt(ag.T, tile_m))
    return hipErrorInvalidValue;
  const LayerPlan p = layer_plan(ag.T, ag.K, ad.K, ag.U_sh, ag.E, ag.k, ag.n_shared, tile_m,
                                 ag.max_tiles, ad.ld_in);
  if (!p.resident) return hipSuccess;
  for (ProjArgs* a : {&ag, &ad}) {
    a->sh_tile = a->maxt;
    a->n_sh_slots = a->n_shared * ((a->T + a->sh_tile - 1) / a->sh_tile);
  }
  LayerArgs la;
  la.logits = logits;
  la.renorm = renorm;
  la.tile_m = tile_m;
  la.n_ub = p.n_ub;
  la.n_gu = p.n_gu;
  la.n_dn = p.n_dn;
  la.R_rows = ag.P + ag.n_shared * ag.T;
  la.out = out;
  la.flags = flags;
  RouteOut ro{ids, w, counts, offsets, sorted_pair, pair_pos, tiles, n_tiles};
  void* args[] = {&ag, &ad, &ro, &la};
  const hipError_t e = hipLaunchKernel(p.fn, dim3((unsigned)p.grid), dim3(kDecThreads), args,
                                       p.lds, st);
  launched = e == hipSuccess;
  return e;
}

}  // namespace moe

// The phase-stamp buffer of the decode kernels (the MOE_DEC_STAMPS build;
// otherwise MOE_E_UNSUPPORTED and nothing is touched).
extern "C" moe_status moe_dbg_dec_stamps(unsigned long long* stamps) {
#ifdef MOE_DEC_STAMPS
  return hipMemcpyToSymbol(HIP_SYMBOL(moe::g_dec_stamps), &stamps, sizeof(stamps)) == hipSuccess
             ? MOE_OK
             : MOE_E_DEVICE;
#else
  (void)stamps;
  return MOE_E_UNSUPPORTED;
#endif
}
