// Router top-k with softmax gating, and the stable counting sort of
// (token, expert) pairs by expert, on the device.
//
// Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", sections
// "Keep low-bit weights packed, do the work on the NPU" (tokens are routed
// to experts on the device, grouped projections with routing and tile
// reuse) and "Remove sync and launch overhead from the token loop" (no
// device-to-host scalar reads; routing moved off the host; fused operators
// where a step is many small launches).
#include "route_common.h"

namespace moe {

// One row of x to int8 codes and its scale by one workgroup of THREADS
// threads: the row's absolute maximum (a block reduction: order-free), then
// the row quantizer's a8_scale / a8_code, so the codes equal that launch's.
// 16-byte loads of 8 values; the second pass reloads them (cache hits).
template <int THREADS>
__device__ void quant_x_row(const XPrep& xq, int t) {
  __shared__ float red[THREADS / 64];
  const int tid = threadIdx.x;
  const uint16_t* row = xq.x + (size_t)t * xq.H;
  float amax = 0.0f;
  for (int c = tid * 8; c < xq.H; c += THREADS * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(bf16_to_f32(u[j] & 0xFFFFu)));
      amax = fmaxf(amax, fabsf(bf16_to_f32(u[j] >> 16)));
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int i = 1; i < THREADS / 64; ++i) amax = fmaxf(amax, red[i]);
  const float sc = a8_scale(amax);
  int8_t* qrow = xq.q + (size_t)t * xq.H;
  for (int c = tid * 8; c < xq.H; c += THREADS * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      lo |= ((uint32_t)a8_code(bf16_to_f32(u[j] & 0xFFFFu), sc) & 0xFFu) << (16 * j);
      lo |= ((uint32_t)a8_code(bf16_to_f32(u[j] >> 16), sc) & 0xFFu) << (16 * j + 8);
      hi |= ((uint32_t)a8_code(bf16_to_f32(u[j + 2] & 0xFFFFu), sc) & 0xFFu) << (16 * j);
      hi |= ((uint32_t)a8_code(bf16_to_f32(u[j + 2] >> 16), sc) & 0xFFu) << (16 * j + 8);
    }
    *reinterpret_cast<uint2*>(qrow + c) = make_uint2(lo, hi);
  }
  if (tid == 0) xq.s[t] = sc;
}

// The fp16 copy of x in the unpack order (what the matrix-core gate/up
// stages), by workgroup b of nb workgroups of THREADS threads, the same
// conversion as that path's own.  A thread takes 8-value blocks u, u + S,
// ... (S = nb * THREADS) eight at a time: the eight loads are issued
// before the first store, so the copy streams instead of waiting one
// memory latency per block.
template <int THREADS>
__device__ void convert_x_rows(const XPrep& xp, int T, int b, int nb) {
  const long long units = (long long)T * (xp.H / 8);   // x rows are contiguous
  const long long S = (long long)nb * THREADS;
  const uint4* src = reinterpret_cast<const uint4*>(xp.x);
  uint4* dst = reinterpret_cast<uint4*>(xp.x16);
  for (long long u0 = (long long)b * THREADS + threadIdx.x; u0 < units; u0 += 8 * S) {
    // x is read once here (non-temporal loads); the fp16 copy, read by
    // every gate/up workgroup of a tile, is stored normally
    typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (u0 + i * S < units) {
        const u32x4_nt t =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(src + u0 + i * S));
        v[i] = make_uint4(t.x, t.y, t.z, t.w);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (u0 + i * S < units) dst[u0 + i * S] = convert8(v[i]);
  }
}

// The preparing workgroups of a routing launch: b of nb.
template <int THREADS>
__device__ void prep_x(const XPrep& xp, int T, int b, int nb) {
  if (xp.q) quant_x_row<THREADS>(xp, b);
  else convert_x_rows<THREADS>(xp, T, b, nb);
}

int xprep_convert_blocks(int T, int H) {
  const long long units = (long long)T * (H / 8);
  const long long nb = (units + 256 * 8 - 1) / (256 * 8);   // about 8 blocks per thread
  return (int)(nb < 1 ? 1 : nb > 1024 ? 1024 : nb);
}

// Workgroups [0, nrb) route, 16 tokens each: four per wave (one per row of
// 16 lanes, or one after another for E > 256); the workgroups after them
// prepare x (xp: int8 rows, one workgroup per row, or the fp16 copy).
template <int NV>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ w, int nrb, XPrep xp) {
  if ((int)blockIdx.x >= nrb) {
    prep_x<256>(xp, T, blockIdx.x - nrb, gridDim.x - nrb);
    return;
  }
  route_tokens<NV, 1>(logits, T, E, k, renorm, threadIdx.x & 63,
                      blockIdx.x * 4 + (threadIdx.x >> 6), nrb * 4, ids, w, nullptr,
                      nullptr);
}

// ---------------------------------------------------------------------
// Stable counting sort in one workgroup of 16 waves.
//  1. Wave w owns the contiguous pair range [w*seg, (w+1)*seg) and counts
//     its pairs per expert in LDS (integer atomics: exact).
//  2. Per expert: total, the base of each wave's range inside the expert
//     (prefix over waves), the exclusive scan over experts -> offsets, and
//     the tile list (ceil(count / tile_m) tiles per expert).
//  3. Each wave walks its range in order, 64 pairs at a time: lanes with
//     the same expert find each other with ballots over the expert id's
//     bits, rank = number of such lanes below, and the last of them
//     advances the wave's cursor for that expert.  Ranges are in pair
//     order and bases are prefix sums over waves, so within an expert the
//     pairs land in increasing p: the sort is stable.
constexpr int kPermWaves = 16;

struct PermSmem {
  int hist[kPermWaves * kPermMaxE];
  int tmp[2 * (kPermWaves + 1)];
  int total_valid;
};

// Exclusive scans of two values over the workgroup's 16 waves at once:
// shuffle scans inside each wave, then the 16 wave totals scanned by 16
// lanes of wave 0 (integer sums: exact in any order).  tmp: 2 * (kPermWaves
// + 1) ints; every thread of the workgroup calls it.
__device__ int2 block_exclusive_scan2(int a, int b, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int oa = __shfl_up(ia, off), ob = __shfl_up(ib, off);
    if (lane >= off) {
      ia += oa;
      ib += ob;
    }
  }
  if (lane == 63) {
    tmp[wave] = ia;
    tmp[kPermWaves + 1 + wave] = ib;
  }
  __syncthreads();
  if (wave == 0) {
    const int ta = lane < kPermWaves ? tmp[lane] : 0;
    const int tb = lane < kPermWaves ? tmp[kPermWaves + 1 + lane] : 0;
    int sa = ta, sb = tb;
#pragma unroll
    for (int off = 1; off < kPermWaves; off <<= 1) {
      const int oa = __shfl_up(sa, off), ob = __shfl_up(sb, off);
      if (lane >= off) {
        sa += oa;
        sb += ob;
      }
    }
    if (lane < kPermWaves) {
      tmp[lane] = sa - ta;
      tmp[kPermWaves + 1 + lane] = sb - tb;
    }
    if (lane == kPermWaves - 1) {
      tmp[kPermWaves] = sa;
      tmp[2 * kPermWaves + 1] = sb;
    }
  }
  __syncthreads();
  const int2 r = make_int2(tmp[wave] + ia - a, tmp[kPermWaves + 1 + wave] + ib - b);
  __syncthreads();
  return r;
}

// ids: global or LDS pointer to the P expert ids.
__device__ void permute_body(const int32_t* ids, int P, int E, int tile_m,
                             int32_t* __restrict__ counts,
                             int32_t* __restrict__ offsets,
                             int32_t* __restrict__ sorted_pair,
                             int32_t* __restrict__ pair_pos,
                             int32_t* __restrict__ tiles,
                             int32_t* __restrict__ n_tiles, PermSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kPermWaves * kPermMaxE; i += 1024) sm.hist[i] = 0;
  __syncthreads();
  const int seg = (P + kPermWaves - 1) / kPermWaves;
  const int p0 = min(P, wave * seg), p1 = min(P, p0 + seg);
  for (int p = p0 + lane; p < p1; p += 64) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&sm.hist[wave * kPermMaxE + e], 1);
  }
  __syncthreads();
  // per expert: the 16 wave counts read together (the waves' start
  // positions are written below, once the expert's offset is known)
  int cnt = 0;
  int wc[kPermWaves];
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) wc[w] = sm.hist[w * kPermMaxE + tid];
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) cnt += wc[w];
  }
  const int ntile = tid < E ? (cnt + tile_m - 1) / tile_m : 0;
  const int2 sc = block_exclusive_scan2(cnt, ntile, sm.tmp);
  const int excl = sc.x, texcl = sc.y;
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid] = excl;
    // wave w's first position: the offset plus the counts of waves 0..w-1
    int run = excl;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) {
      sm.hist[w * kPermMaxE + tid] = run;
      run += wc[w];
    }
    for (int i = 0; i < ntile; ++i) {
      const int r0 = excl + i * tile_m;
      int4 tl;
      tl.x = tid;
      tl.y = r0;
      tl.z = min(r0 + tile_m, excl + cnt);
      tl.w = 0;
      reinterpret_cast<int4*>(tiles)[texcl + i] = tl;
    }
    if (tid == E - 1) {
      offsets[E] = excl + cnt;
      *n_tiles = texcl + ntile;
      sm.total_valid = excl + cnt;
    }
  }
  __syncthreads();
  const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
  for (int base = p0; base < p1; base += 64) {
    const int p = base + lane;
    const bool in = p < p1;
    const int e = in ? ids[p] : -1;
    const bool valid = in && (unsigned)e < (unsigned)E;
    unsigned long long m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < kPermIdBits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const unsigned long long bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    if (valid) {
      const int pos = sm.hist[wave * kPermMaxE + e] + __popcll(m & below);
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
      if ((m >> lane) == 1ull) sm.hist[wave * kPermMaxE + e] = pos + 1;
    } else if (in) {
      pair_pos[p] = -1;
    }
  }
  __syncthreads();
  for (int i = sm.total_valid + tid; i < P; i += 1024) sorted_pair[i] = -1;
}

// ---------------------------------------------------------------------
// The same sort over many workgroups, for large batches (the layer call,
// with its workspace): workgroup b takes pairs [b * kPermChunk, +kPermChunk).
// Two launches: (1) each workgroup counts its chunk per expert ->
// hist[b][e]; (2) each workgroup forms the offsets from all the counts
// (workgroup 0 also writes counts, offsets and the tile list), its first
// sorted position of every expert: offsets[e] plus the counts of
// workgroups 0..b-1, and places its chunk from there with the per-wave
// counts and ballot ranks of permute_body.  Pairs of an expert stay in
// increasing p, so the result is the single workgroup's, bit for bit.
constexpr int kPermChunk = 2048;   // pairs per workgroup (128 per wave)

__global__ __launch_bounds__(1024) void perm_hist_kernel(const int32_t* __restrict__ ids, int P,
                                                         int E, int32_t* __restrict__ hist) {
  __shared__ int h[kPermMaxE];
  for (int i = threadIdx.x; i < E; i += 1024) h[i] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kPermChunk, p1 = min(P, p0 + kPermChunk);
  for (int p = p0 + threadIdx.x; p < p1; p += 1024) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += 1024) hist[(size_t)blockIdx.x * E + i] = h[i];
}

// (2) + (3) in one launch: every workgroup sums the chunks' counts into the
// expert totals (all of hist: nb * E ints from the cache), scans them into
// the offsets, adds the counts of chunks 0..b-1 for its own first positions
// and places its chunk; workgroup 0 also writes counts, offsets, the tile
// list, n_tiles and the -1 tail of sorted_pair.
__global__ __launch_bounds__(1024) void perm_place_kernel(const int32_t* __restrict__ ids, int P,
                                                          int E, int nb, int tile_m,
                                                          const int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pair,
                                                          int32_t* __restrict__ pair_pos,
                                                          int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ n_tiles) {
  __shared__ int wh[kPermWaves * kPermMaxE];
  __shared__ int tmp[2 * (kPermWaves + 1)];
  __shared__ int total;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  // the chunk's counts per wave and expert (exact integer atomics)
  for (int i = tid; i < kPermWaves * kPermMaxE; i += 1024) wh[i] = 0;
  __syncthreads();
  constexpr int seg = kPermChunk / kPermWaves;
  const int p0 = min(P, b * kPermChunk + wave * seg), p1 = min(P, p0 + seg);
  for (int p = p0 + lane; p < p1; p += 64) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&wh[wave * kPermMaxE + e], 1);
  }
  // expert totals and the counts of the chunks before this one, eight
  // chunks' loads in flight at a time
  int cnt = 0, before = 0;
  if (tid < E) {
    for (int c0 = 0; c0 < nb; c0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = c0 + u < nb ? hist[(size_t)(c0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        cnt += v[u];
        before += c0 + u < b ? v[u] : 0;
      }
    }
  }
  const int ntile = tid < E ? (cnt + tile_m - 1) / tile_m : 0;
  const int2 sc = block_exclusive_scan2(cnt, ntile, tmp);
  const int excl = sc.x;
  if (b == 0) {
    const int texcl = sc.y;
    if (tid < E) {
      counts[tid] = cnt;
      offsets[tid] = excl;
      for (int i = 0; i < ntile; ++i) {
        const int r0 = excl + i * tile_m;
        int4 tl;
        tl.x = tid;
        tl.y = r0;
        tl.z = min(r0 + tile_m, excl + cnt);
        tl.w = 0;
        reinterpret_cast<int4*>(tiles)[texcl + i] = tl;
      }
      if (tid == E - 1) {
        offsets[E] = excl + cnt;
        *n_tiles = texcl + ntile;
      }
    }
  }
  if (tid == E - 1) total = excl + cnt;
  __syncthreads();   // the wave counts are complete
  if (tid < E) {
    // wave w of this chunk starts expert tid after waves 0..w-1
    int run = excl + before;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = wh[w * kPermMaxE + tid];
      wh[w * kPermMaxE + tid] = run;
      run += c;
    }
  }
  __syncthreads();
  const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
  for (int base = p0; base < p1; base += 64) {
    const int p = base + lane;
    const bool in = p < p1;
    const int e = in ? ids[p] : -1;
    const bool valid = in && (unsigned)e < (unsigned)E;
    unsigned long long m = __ballot(valid);
#pragma unroll
    for (int bb = 0; bb < kPermIdBits; ++bb) {
      const bool bit = valid && ((e >> bb) & 1);
      const unsigned long long bm = __ballot(bit);
      m &= bit ? bm : ~bm;
    }
    if (valid) {
      const int pos = wh[wave * kPermMaxE + e] + __popcll(m & below);
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
      if ((m >> lane) == 1ull) wh[wave * kPermMaxE + e] = pos + 1;
    } else if (in) {
      pair_pos[p] = -1;
    }
  }
  if (b == 0)
    for (int i = total + tid; i < P; i += 1024) sorted_pair[i] = -1;
}

__global__ __launch_bounds__(1024) void permute_kernel(
    const int32_t* __restrict__ ids, int P, int E, int tile_m,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ PermSmem sm;
  permute_body(ids, P, E, tile_m, counts, offsets, sorted_pair, pair_pos, tiles,
               n_tiles, sm);
}

// Stable counting sort of P <= 128 pairs by one wave (valid ids below
// 2^kPermIdBits; lane l holds pairs l and l + 64): one radix pass over the
// id bits with ballots gives, for each of a lane's pairs and each of the
// two pair slots, the lanes whose id is smaller (lt) and equal (eq); a
// pair's position is the number of pairs sorted before it (smaller id, or
// equal id and smaller index), its rank in its expert the equal-id pairs
// before it, a tile starts where that rank is a multiple of tile_m, and
// the tile's index is the number of starts sorted before it.  Straight-line
// mask arithmetic, the same outputs as permute_body (counts and offsets
// per expert come from count_experts).
template <int NV>
__device__ void wave_sort128(const int32_t* ids, int P, int E, int tile_m,
                             int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
                             int32_t* __restrict__ pair_pos, int32_t* __restrict__ tiles,
                             int32_t* __restrict__ n_tiles) {
  const int lane = threadIdx.x & 63;
  const bool in0 = lane < P, in1 = lane + 64 < P;
  const int e0 = in0 ? ids[lane] : 0, e1 = in1 ? ids[lane + 64] : 0;
  const uint64_t v0 = __ballot(in0), v1 = __ballot(in1);
  // [my pair][slot]
  uint64_t eq00 = v0, eq01 = v1, eq10 = v0, eq11 = v1;
  uint64_t lt00 = 0, lt01 = 0, lt10 = 0, lt11 = 0;
  // ids below E <= 64 NV: the bits of 64 NV - 1
  constexpr int kBits = NV <= 1 ? 6 : NV <= 2 ? 7 : NV <= 4 ? 8 : kPermIdBits;
  static_assert(kBits <= kPermIdBits, "ids below 2^kPermIdBits");
#pragma unroll
  for (int b = kBits - 1; b >= 0; --b) {
    const bool b0 = (e0 >> b) & 1, b1 = (e1 >> b) & 1;
    const uint64_t o0 = __ballot(in0 && b0), o1 = __ballot(in1 && b1);
    lt00 = b0 ? (lt00 | (eq00 & ~o0)) : lt00;
    lt01 = b0 ? (lt01 | (eq01 & ~o1)) : lt01;
    eq00 = b0 ? (eq00 & o0) : (eq00 & ~o0);
    eq01 = b0 ? (eq01 & o1) : (eq01 & ~o1);
    lt10 = b1 ? (lt10 | (eq10 & ~o0)) : lt10;
    lt11 = b1 ? (lt11 | (eq11 & ~o1)) : lt11;
    eq10 = b1 ? (eq10 & o0) : (eq10 & ~o0);
    eq11 = b1 ? (eq11 & o1) : (eq11 & ~o1);
  }
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;   // lanes < lane
  // pair lane: same-id pairs before it are slot-0 lanes below; pair lane +
  // 64: every same-id slot-0 pair and the slot-1 lanes below
  const uint64_t ahead00 = lt00 | (eq00 & below), ahead01 = lt01;
  const uint64_t ahead10 = lt10 | eq10, ahead11 = lt11 | (eq11 & below);
  const int nlt0 = __popcll(lt00) + __popcll(lt01);
  const int nlt1 = __popcll(lt10) + __popcll(lt11);
  const int bef0 = __popcll(eq00 & below);
  const int bef1 = __popcll(eq10) + __popcll(eq11 & below);
  const int end0 = nlt0 + __popcll(eq00) + __popcll(eq01);
  const int end1 = nlt1 + __popcll(eq10) + __popcll(eq11);
  const int pos0 = nlt0 + bef0, pos1 = nlt1 + bef1;
  const bool st0 = in0 && bef0 % tile_m == 0, st1 = in1 && bef1 % tile_m == 0;
  const uint64_t s0 = __ballot(st0), s1 = __ballot(st1);
  const int tix0 = __popcll(s0 & ahead00) + __popcll(s1 & ahead01);
  const int tix1 = __popcll(s0 & ahead10) + __popcll(s1 & ahead11);
  if (in0) {
    sorted_pair[pos0] = lane;
    pair_pos[lane] = pos0;
  }
  if (in1) {
    sorted_pair[pos1] = lane + 64;
    pair_pos[lane + 64] = pos1;
  }
  if (st0) reinterpret_cast<int4*>(tiles)[tix0] = make_int4(e0, pos0, min(pos0 + tile_m, end0), 0);
  if (st1) reinterpret_cast<int4*>(tiles)[tix1] = make_int4(e1, pos1, min(pos1 + tile_m, end1), 0);
  if (lane == 0) {
    *n_tiles = __popcll(s0) + __popcll(s1);
    offsets[E] = P;
  }
}

// Per-expert pair counts and offsets (pairs of a smaller expert) of the
// experts e = first, first + stride, ... by one thread each, reading the
// P ids from LDS (every thread reads the same ids at a time: broadcasts),
// eight 16-byte reads in flight per turn.  ids: 16-byte aligned, padded
// with an id no expert has up to a multiple of 32.
__device__ void count_experts(const int32_t* ids, int P, int E, int first, int stride,
                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  const int4* v = reinterpret_cast<const int4*>(ids);
  for (int ex = first; ex < E; ex += stride) {
    int c = 0, o = 0;
    for (int q = 0; q < P; q += 32) {
      int4 r[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) r[u] = v[q / 4 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        c += (r[u].x == ex) + (r[u].y == ex) + (r[u].z == ex) + (r[u].w == ex);
        o += (r[u].x < ex) + (r[u].y < ex) + (r[u].z < ex) + (r[u].w < ex);
      }
    }
    counts[ex] = c;
    offsets[ex] = o;
  }
}

// Route and permute in one launch for small batches: the 16 waves route
// the tokens (ids kept in LDS as well), then the same workgroup sorts: up
// to 128 pairs wave 0 alone (the other waves count the experts), more with
// the block-wide sort.
template <int NV>
__global__ __launch_bounds__(1024) void route_permute_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int tile_m, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles, XPrep xp) {
  if (blockIdx.x > 0) {   // the workgroups after the first prepare x
    prep_x<1024>(xp, T, blockIdx.x - 1, gridDim.x - 1);
    return;
  }
  __shared__ PermSmem sm;
  __shared__ __align__(16) int32_t lds_ids[kFusedRouteMaxP];
  static_assert(kFusedRouteMaxT == 4 * kPermWaves, "one token per row of 16 lanes");
  route_tokens<NV, 1>(logits, T, E, k, renorm, threadIdx.x & 63, threadIdx.x >> 6, kPermWaves,
                      ids, w, lds_ids, nullptr);
  __syncthreads();
  const int P = T * k;
  if (P <= 128) {
    // ids past P read by the counting threads: an id no expert has
    if (threadIdx.x >= P && threadIdx.x < 128) lds_ids[threadIdx.x] = 0x7fffffff;
    __syncthreads();
    if (threadIdx.x < 64)
      wave_sort128<NV>(lds_ids, P, E, tile_m, offsets, sorted_pair, pair_pos, tiles, n_tiles);
    else
      count_experts(lds_ids, P, E, threadIdx.x - 64, 1024 - 64, counts, offsets);
    return;
  }
  permute_body(lds_ids, P, E, tile_m, counts, offsets, sorted_pair, pair_pos,
               tiles, n_tiles, sm);
}

#define MOE_NV_DISPATCH(NVV, ...)               \
  do {                                          \
    const int nv_ = (E + 63) / 64;              \
    if (nv_ <= 1) { constexpr int NVV = 1; __VA_ARGS__; }       \
    else if (nv_ <= 2) { constexpr int NVV = 2; __VA_ARGS__; }  \
    else if (nv_ <= 4) { constexpr int NVV = 4; __VA_ARGS__; }  \
    else if (nv_ <= 8) { constexpr int NVV = 8; __VA_ARGS__; }  \
    else { constexpr int NVV = 16; __VA_ARGS__; }               \
  } while (0)

// ---------------------------------------------------------------------
// Router logits on the device: logits[t][e] = sum_h x[t][h] * W[h][e]
// (+ prior[e]), fp32, summed in a fixed order: within a chunk of H in
// increasing h, then the chunks in increasing order.  Workgroup (chunk,
// token tile, expert tile) = 64 tokens x 64 experts; each thread owns a
// 4 x 4 block of outputs.  H advances 32 rows per step through LDS ([h]
// [token] and [h][expert] fp32, double-buffered): the next step's loads
// are in flight while the current step's 32 x 16 fused multiply-adds run.
// Small batches split H into chunks (partial sums to the workspace, then
// router_reduce_kernel) so that the launch has about 256 workgroups.
constexpr int kRtT = 64, kRtE = 64, kRtK = 32, kRtThreads = 256;
constexpr int kRtLd = (kRtK * kRtT) / kRtThreads;   // loads per thread per step and operand

__global__ __launch_bounds__(kRtThreads) void router_logits_kernel(
    const uint16_t* __restrict__ x, int T, int H, const float* __restrict__ W, int E,
    const float* __restrict__ prior, int hc, int n_chunks, float* __restrict__ out) {
  __shared__ __align__(16) float xs[2][kRtK * kRtT];   // [h][token]
  __shared__ __align__(16) float ws[2][kRtK * kRtE];   // [h][expert]
  const int tid = threadIdx.x;
  const int t0 = blockIdx.y * kRtT, e0 = blockIdx.z * kRtE;
  const int h_begin = blockIdx.x * hc, h_end = min(H, h_begin + hc);
  const int n_steps = (h_end - h_begin + kRtK - 1) / kRtK;
  // staging: x element i -> (token i / 32, h i % 32); W element i ->
  // (h i / 64, expert i % 64); consecutive threads read consecutive memory
  float xr[kRtLd], wr[kRtLd];
  auto load = [&](int st) {
    const int h0 = h_begin + st * kRtK;
#pragma unroll
    for (int j = 0; j < kRtLd; ++j) {
      const int i = tid + j * kRtThreads;
      const int xt = i / kRtK, xh = i % kRtK;
      const int wh = i / kRtE, we = i % kRtE;
      xr[j] = (t0 + xt < T && h0 + xh < h_end)
                  ? bf16_to_f32(x[(size_t)(t0 + xt) * H + h0 + xh]) : 0.0f;
      wr[j] = (h0 + wh < h_end && e0 + we < E) ? W[(size_t)(h0 + wh) * E + e0 + we] : 0.0f;
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int j = 0; j < kRtLd; ++j) {
      const int i = tid + j * kRtThreads;
      xs[b][(i % kRtK) * kRtT + i / kRtK] = xr[j];
      ws[b][i] = wr[j];
    }
  };
  const int tg = tid / (kRtE / 4), eg = tid % (kRtE / 4);   // 4 tokens x 4 experts
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
  if (n_steps > 0) {
    load(0);
    store(0);
    __syncthreads();
  }
  for (int st = 0; st < n_steps; ++st) {
    const int b = st & 1;
    if (st + 1 < n_steps) load(st + 1);
#pragma unroll 8
    for (int h = 0; h < kRtK; ++h) {
      const float4 xv = *reinterpret_cast<const float4*>(&xs[b][h * kRtT + 4 * tg]);
      const float4 wv = *reinterpret_cast<const float4*>(&ws[b][h * kRtE + 4 * eg]);
      const float xa[4] = {xv.x, xv.y, xv.z, xv.w}, wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(xa[a], wa[c], acc[a][c]);
    }
    if (st + 1 < n_steps) store(b ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int t = t0 + 4 * tg + a;
    if (t >= T) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = e0 + 4 * eg + c;
      if (e >= E) continue;
      if (n_chunks == 1)
        out[(size_t)t * E + e] = prior ? acc[a][c] + prior[e] : acc[a][c];
      else
        out[((size_t)blockIdx.x * T + t) * E + e] = acc[a][c];
    }
  }
}

// Chunk partials [n_chunks][T][E] -> logits [T][E], chunks in order, then
// the prior.
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ part,
                                                            int T, int E, int n_chunks,
                                                            const float* __restrict__ prior,
                                                            float* __restrict__ logits) {
  const size_t n = (size_t)T * E;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    // 16 loads in flight at a time, summed in chunk order
    float v = 0.0f;
    for (int c0 = 0; c0 < n_chunks; c0 += 16) {
      float p[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = c0 + j < n_chunks ? part[(size_t)(c0 + j) * n + i] : 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (c0 + j < n_chunks) v += p[j];
    }
    logits[i] = prior ? v + prior[i % E] : v;
  }
}

// Chunks of H for a batch (the launch should hold about 256 workgroups),
// and their length (a multiple of 32).
void router_chunks(int T, int H, int E, int& n_chunks, int& hc) {
  const long long groups = (long long)((T + kRtT - 1) / kRtT) * ((E + kRtE - 1) / kRtE);
  long long n = (256 + groups - 1) / groups;
  const long long n_max = (H + kRtK - 1) / kRtK;
  n = n < 1 ? 1 : n > n_max ? n_max : n;
  hc = (int)(((H + n - 1) / n + kRtK - 1) / kRtK * kRtK);
  n_chunks = (H + hc - 1) / hc;
}

size_t router_workspace_bytes(int T, int H, int E) {
  int n, hc;
  router_chunks(T, H, E, n, hc);
  return n > 1 ? (size_t)n * T * E * sizeof(float) : 0;
}

hipError_t launch_router_logits(const uint16_t* x, int T, int H, const float* W, int E,
                                const float* prior, float* logits, float* part,
                                hipStream_t st) {
  if (T == 0) return hipSuccess;
  int n_chunks, hc;
  router_chunks(T, H, E, n_chunks, hc);
  const dim3 grid(n_chunks, (T + kRtT - 1) / kRtT, (E + kRtE - 1) / kRtE);
  router_logits_kernel<<<grid, kRtThreads, 0, st>>>(x, T, H, W, E, prior, hc, n_chunks,
                                                    n_chunks == 1 ? logits : part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_chunks == 1) return e;
  const size_t n = (size_t)T * E;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  router_reduce_kernel<<<blocks, 256, 0, st>>>(part, T, E, n_chunks, prior, logits);
  return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k,
                             int renorm, int32_t* ids, float* w,
                             hipStream_t st, const XPrep* xp) {
  if (T == 0) return hipSuccess;
  const int nrb = (T + 15) / 16;
  const XPrep p = xp ? *xp : XPrep{nullptr, 0, nullptr, nullptr, nullptr};
  const int np = !xp ? 0 : p.q ? T : xprep_convert_blocks(T, p.H);
  MOE_NV_DISPATCH(NV, route_topk_kernel<NV><<<nrb + np, 256, 0, st>>>(
                          logits, T, E, k, renorm, ids, w, nrb, p));
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int P, int E, int tile_m,
                          int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos,
                          int32_t* tiles, int32_t* n_tiles, hipStream_t st) {
  permute_kernel<<<1, 1024, 0, st>>>(ids, P, E, tile_m, counts, offsets,
                                     sorted_pair, pair_pos, tiles, n_tiles);
  return hipGetLastError();
}

int permute_multi_blocks(int P) {
  return P >= kPermMultiMinP ? (P + kPermChunk - 1) / kPermChunk : 0;
}

hipError_t launch_permute_multi(const int32_t* ids, int P, int E, int tile_m, int32_t* counts,
                                int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                int32_t* tiles, int32_t* n_tiles, int32_t* scratch,
                                hipStream_t st) {
  const int nb = (P + kPermChunk - 1) / kPermChunk;
  if (nb == 0) return launch_permute(ids, P, E, tile_m, counts, offsets, sorted_pair, pair_pos,
                                     tiles, n_tiles, st);
  perm_hist_kernel<<<nb, 1024, 0, st>>>(ids, P, E, scratch);
  perm_place_kernel<<<nb, 1024, 0, st>>>(ids, P, E, nb, tile_m, scratch, counts, offsets,
                                         sorted_pair, pair_pos, tiles, n_tiles);
  return hipGetLastError();
}

hipError_t launch_route_permute(const float* logits, int T, int E, int k,
                                int renorm, int tile_m, int32_t* ids, float* w,
                                int32_t* counts, int32_t* offsets,
                                int32_t* sorted_pair, int32_t* pair_pos,
                                int32_t* tiles, int32_t* n_tiles,
                                hipStream_t st, const XPrep* xq) {
  // from 16 tokens on the routing is worth more than one compute unit: the
  // multi-workgroup router, then the sort (same functions, same results)
  if (T >= kRouteMultiMinT) {
    const hipError_t e = launch_route_topk(logits, T, E, k, renorm, ids, w, st, xq);
    if (e != hipSuccess) return e;
    return launch_permute(ids, T * k, E, tile_m, counts, offsets, sorted_pair, pair_pos, tiles,
                          n_tiles, st);
  }
  const XPrep q = xq ? *xq : XPrep{nullptr, 0, nullptr, nullptr, nullptr};
  // preparing workgroups of 1024 threads: one per row (int8), or the
  // fp16 copy at about 8 blocks per thread
  const int nq = !xq ? 0 : q.q ? T : (xprep_convert_blocks(T, q.H) + 3) / 4;
  MOE_NV_DISPATCH(NV, route_permute_kernel<NV><<<1 + nq, 1024, 0, st>>>(
                          logits, T, E, k, renorm, tile_m, ids, w, counts,
                          offsets, sorted_pair, pair_pos, tiles, n_tiles, q));
  return hipGetLastError();
}

}  // namespace moe
