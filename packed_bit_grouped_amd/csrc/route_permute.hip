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

template <int NV>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ w) {
  // 16 tokens per workgroup: four per wave (one per row of 16 lanes, or
  // one after another for E > 256)
  route_tokens<NV, 1>(logits, T, E, k, renorm, threadIdx.x & 63,
                      blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4, ids, w, nullptr,
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
  int tmp[kPermWaves + 1];
  int total_valid;
};

__device__ int block_exclusive_scan(int v, int* tmp /* kPermWaves + 1 */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < kPermWaves; ++i) {
      const int c = tmp[i];
      tmp[i] = run;
      run += c;
    }
    tmp[kPermWaves] = run;
  }
  __syncthreads();
  const int r = tmp[wave] + incl - v;
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
  int cnt = 0;
  if (tid < E) {
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = sm.hist[w * kPermMaxE + tid];
      sm.hist[w * kPermMaxE + tid] = cnt;
      cnt += c;
    }
  }
  const int excl = block_exclusive_scan(cnt, sm.tmp);
  const int ntile = tid < E ? (cnt + tile_m - 1) / tile_m : 0;
  const int texcl = block_exclusive_scan(ntile, sm.tmp);
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid] = excl;
    for (int w = 0; w < kPermWaves; ++w) sm.hist[w * kPermMaxE + tid] += excl;
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

__global__ __launch_bounds__(1024) void permute_kernel(
    const int32_t* __restrict__ ids, int P, int E, int tile_m,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ PermSmem sm;
  permute_body(ids, P, E, tile_m, counts, offsets, sorted_pair, pair_pos, tiles,
               n_tiles, sm);
}

// Route and permute in one launch for small batches: the 16 waves route
// the tokens (ids kept in LDS as well), then the same workgroup sorts.
template <int NV>
__global__ __launch_bounds__(1024) void route_permute_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int tile_m, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ PermSmem sm;
  __shared__ int32_t lds_ids[kFusedRouteMaxP];
  static_assert(kFusedRouteMaxT == 4 * kPermWaves, "one token per row of 16 lanes");
  route_tokens<NV, 1>(logits, T, E, k, renorm, threadIdx.x & 63, threadIdx.x >> 6, kPermWaves,
                      ids, w, lds_ids, nullptr);
  __syncthreads();
  permute_body(lds_ids, T * k, E, tile_m, counts, offsets, sorted_pair, pair_pos,
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
// token group, expert group): 16 tokens x 256 experts (one per thread) x
// one H chunk; the chunk's activations are staged in LDS 128 h at a time
// as [h][token] fp32, so each step is one coalesced 1 KB row of W and 16
// FMAs against four broadcast LDS reads.  Small batches split H over up
// to ceil(H / 128) chunks (partial sums to the workspace, then
// router_reduce_kernel) so that the launch fills the chip; large ones use
// one chunk and write the logits directly.
constexpr int kRtTok = 16, kRtExp = 256, kRtStep = 128;

__global__ __launch_bounds__(kRtExp) void router_logits_kernel(
    const uint16_t* __restrict__ x, int T, int H, const float* __restrict__ W, int E,
    const float* __restrict__ prior, int hc, int n_chunks, float* __restrict__ out) {
  __shared__ __align__(16) float xs[kRtStep * kRtTok];   // [h][token]
  const int tid = threadIdx.x;
  const int e = blockIdx.z * kRtExp + tid;
  const int t0 = blockIdx.y * kRtTok, nt = min(kRtTok, T - t0);
  const int h_begin = blockIdx.x * hc, h_end = min(H, h_begin + hc);
  float acc[kRtTok];
#pragma unroll
  for (int t = 0; t < kRtTok; ++t) acc[t] = 0.0f;
  for (int h0 = h_begin; h0 < h_end; h0 += kRtStep) {
    const int hn = min(kRtStep, h_end - h0);
    for (int i = tid; i < kRtStep * kRtTok; i += kRtExp) {
      const int t = i / kRtStep, hh = i - t * kRtStep;
      xs[hh * kRtTok + t] =
          (t < nt && hh < hn) ? bf16_to_f32(x[(size_t)(t0 + t) * H + h0 + hh]) : 0.0f;
    }
    __syncthreads();
    if (e < E) {
      const float* wp = W + (size_t)h0 * E + e;
#pragma unroll 8
      for (int hh = 0; hh < hn; ++hh) {
        const float wv = wp[(size_t)hh * E];
        const float4* xr = reinterpret_cast<const float4*>(xs + hh * kRtTok);
#pragma unroll
        for (int q = 0; q < kRtTok / 4; ++q) {
          const float4 xv = xr[q];
          acc[4 * q + 0] = fmaf(xv.x, wv, acc[4 * q + 0]);
          acc[4 * q + 1] = fmaf(xv.y, wv, acc[4 * q + 1]);
          acc[4 * q + 2] = fmaf(xv.z, wv, acc[4 * q + 2]);
          acc[4 * q + 3] = fmaf(xv.w, wv, acc[4 * q + 3]);
        }
      }
    }
    __syncthreads();
  }
  if (e >= E) return;
  const float pe = (n_chunks == 1 && prior) ? prior[e] : 0.0f;
#pragma unroll
  for (int t = 0; t < kRtTok; ++t) {
    if (t >= nt) break;
    const size_t o = n_chunks == 1 ? (size_t)(t0 + t) * E + e
                                   : ((size_t)blockIdx.x * T + t0 + t) * E + e;
    out[o] = acc[t] + pe;
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
    float v = 0.0f;
    for (int c = 0; c < n_chunks; ++c) v += part[(size_t)c * n + i];
    logits[i] = prior ? v + prior[i % E] : v;
  }
}

// Chunks of H for a batch (the launch should hold about 256 workgroups),
// and their length (a multiple of 32).
void router_chunks(int T, int H, int E, int& n_chunks, int& hc) {
  const long long groups = (long long)((T + kRtTok - 1) / kRtTok) * ((E + kRtExp - 1) / kRtExp);
  long long n = (256 + groups - 1) / groups;
  const long long n_max = (H + kRtStep - 1) / kRtStep;
  n = n < 1 ? 1 : n > n_max ? n_max : n;
  hc = (int)(((H + n - 1) / n + 31) / 32 * 32);
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
  const dim3 grid(n_chunks, (T + kRtTok - 1) / kRtTok, (E + kRtExp - 1) / kRtExp);
  router_logits_kernel<<<grid, kRtExp, 0, st>>>(x, T, H, W, E, prior, hc, n_chunks,
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
                             hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 15) / 16), block(256);
  MOE_NV_DISPATCH(NV, route_topk_kernel<NV><<<grid, block, 0, st>>>(
                          logits, T, E, k, renorm, ids, w));
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

hipError_t launch_route_permute(const float* logits, int T, int E, int k,
                                int renorm, int tile_m, int32_t* ids, float* w,
                                int32_t* counts, int32_t* offsets,
                                int32_t* sorted_pair, int32_t* pair_pos,
                                int32_t* tiles, int32_t* n_tiles,
                                hipStream_t st) {
  // from 16 tokens on the routing is worth more than one compute unit: the
  // multi-workgroup router, then the sort (same functions, same results)
  if (T >= kRouteRowMinT) {
    const hipError_t e = launch_route_topk(logits, T, E, k, renorm, ids, w, st);
    if (e != hipSuccess) return e;
    return launch_permute(ids, T * k, E, tile_m, counts, offsets, sorted_pair, pair_pos, tiles,
                          n_tiles, st);
  }
  MOE_NV_DISPATCH(NV, route_permute_kernel<NV><<<1, 1024, 0, st>>>(
                          logits, T, E, k, renorm, tile_m, ids, w, counts,
                          offsets, sorted_pair, pair_pos, tiles, n_tiles));
  return hipGetLastError();
}

}  // namespace moe
