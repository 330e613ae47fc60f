// Grouped expert projections for decode shapes: a split-K wavefront GEMV
// over packed int4/int2 weights.
//
// Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", section "Keep
// low-bit weights packed, do the work on the NPU": grouped expert
// projections straight from packed weights, fused gate/up handling,
// blocked reduction, routing and tile reuse, a dedicated W4A8 mode, and
// no transiently expanded expert bank.  On gfx950 at 1-16 tokens per
// expert this work is bound by HBM, not by the matrix cores, so it runs on
// the vector ALUs:
//
//  * a fixed grid of about one workgroup per CU covers every tile (tile =
//    up to tile_m sorted rows of one expert, or a shared-expert token
//    block): the device-side tile count decides how many workgroups split
//    a tile's output units (gate/up row pairs or down rows), so no
//    workgroup waits on an empty tile and none straddles two tiles;
//  * a workgroup stages a tile's activations once in LDS, in the pair
//    order of the code unpack, and applies every weight row it reads to
//    all of the tile's tokens (tile reuse); each weight byte is read once;
//  * a weight row is cut into 16-byte chunks; `seg` lanes share a row
//    (split-K) and add their partial sums with DPP exchanges inside the
//    segment (blocked reduction); the rows of the next iteration are
//    loaded into a second register set while the current ones are
//    reduced (software pipelining), so HBM latency overlaps the VALU work;
//  * gate row i and up row I+i of W13 are in the same iteration and meet
//    in LDS for the fused SiLU(g) * u epilogue;
//  * A16: codes expand to bf16 (exact, biased) and v_dot2_f32_bf16 forms
//    the products; A8: codes expand to int8 and v_dot4_i32_i8 forms exact
//    int32 per-group partial sums, scaled in fp32.
#include "gemv_common.h"

namespace moe {

// Stage the activation rows [pass, pass + nt) of a tile into LDS.
template <int ACT>
__device__ void stage_rows(const ProjArgs& a, bool is_sh, int e, int pass, int nt,
                           int K, int bits, uint32_t* xs, int xs_row, float* xsum,
                           float* xsc, int xsum_row) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb32 = K / 32;
  if (ACT == MOE_A16) {
    for (int u = tid; u < nt * nb32; u += kGemvThreads) {
      const int m = u / nb32, b = u - m * nb32;
      int row;
      if (a.mode == 0) row = is_sh ? pass + m : a.sorted_pair[pass + m] / a.k;
      else row = is_sh ? a.P + e * a.T + pass + m : pass + m;
      stage_a16_block(a.in_bf16 + (size_t)row * a.ld_in, b, K, bits, xs + m * xs_row,
                      xsum + m * xsum_row);
    }
  } else if (a.mode == 0) {  // A8 gate/up: pre-quantized x
    for (int u = tid; u < nt * nb32; u += kGemvThreads) {
      const int m = u / nb32, b = u - m * nb32;
      const int t = is_sh ? pass + m : a.sorted_pair[pass + m] / a.k;
      const uint4* src = reinterpret_cast<const uint4*>(a.in_q + (size_t)t * a.ld_in + b * 32);
      const uint4 lo = src[0], hi = src[1];
      const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      uint32_t pr[8];
      auto xb = [&](int j) -> uint32_t { return (d[j >> 2] >> (8 * (j & 3))) & 0xFFu; };
      if (bits == 4) {       // 8-blocks: even quad, odd quad
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          pr[2 * blk] = xb(8 * blk) | xb(8 * blk + 2) << 8 | xb(8 * blk + 4) << 16 | xb(8 * blk + 6) << 24;
          pr[2 * blk + 1] = xb(8 * blk + 1) | xb(8 * blk + 3) << 8 | xb(8 * blk + 5) << 16 | xb(8 * blk + 7) << 24;
        }
      } else {               // 16-blocks: quads (i, i+4, i+8, i+12)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pr[4 * blk + i] = xb(16 * blk + i) | xb(16 * blk + i + 4) << 8 |
                              xb(16 * blk + i + 8) << 16 | xb(16 * blk + i + 12) << 24;
      }
      store_a8_planes(xs + m * xs_row, pr, b, K, bits);
      if (b == 0) xsc[m] = a.in_s[t];
    }
  } else {                   // A8 down: quantize fp32 h rows here
    for (int m = wave; m < nt; m += kGemvWaves) {
      const int row = is_sh ? a.P + e * a.T + pass + m : pass + m;
      const float* src = a.in_f32 + (size_t)row * a.ld_in;
      float amax = 0.0f;
      for (int c = lane; c < K; c += 64) amax = fmaxf(amax, fabsf(src[c]));
      amax = wave_max(amax);
      const float sc = a8_scale(amax);
      for (int b = lane; b < nb32; b += 64) {
        int cq[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) cq[j] = a8_code(src[b * 32 + j], sc) & 0xFF;
        uint32_t pr[8];
        if (bits == 4) {
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            pr[2 * blk] = cq[8 * blk] | cq[8 * blk + 2] << 8 | cq[8 * blk + 4] << 16 | cq[8 * blk + 6] << 24;
            pr[2 * blk + 1] = cq[8 * blk + 1] | cq[8 * blk + 3] << 8 | cq[8 * blk + 5] << 16 | cq[8 * blk + 7] << 24;
          }
        } else {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pr[4 * blk + i] = cq[16 * blk + i] | cq[16 * blk + i + 4] << 8 |
                                cq[16 * blk + i + 8] << 16 | (uint32_t)cq[16 * blk + i + 12] << 24;
        }
        store_a8_planes(xs + m * xs_row, pr, b, K, bits);
      }
      if (lane == 0) xsc[m] = sc;
    }
  }
}

template <int ACT, int MAXT, bool DUMP>
__global__ __launch_bounds__(kGemvThreads) void proj_gemv_kernel(ProjArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Kl = max(a.K, a.K_sh);

  // ---- LDS carve-up
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem);
  const int xs_row = ACT == MOE_A16 ? Kl / 2 : Kl / 4;   // dwords per staged row
  const int xsum_row = Kl / 32;
  float* xsum = reinterpret_cast<float*>(xs + MAXT * xs_row);  // A16: [MAXT][Kl/32]
  float* xsc = xsum;                                           // A8: [MAXT]
  float* res = ACT == MOE_A16 ? xsum + MAXT * xsum_row : xsc + MAXT;  // [2][res_rows][MAXT]

  // ---- this workgroup's work: S = shared + routed tiles (device count).
  // With S <= grid, each tile gets floor(grid / S) workgroups splitting its
  // units evenly; otherwise workgroups take whole tiles in a strided loop.
  // No workgroup straddles two tiles.
  const int S = a.n_sh_slots + *a.n_tiles;
  const int n_wg = gridDim.x;
  const int bps = S > 0 && S <= n_wg ? n_wg / S : 1;
  int slot = S <= n_wg ? blockIdx.x / bps : blockIdx.x;
  const int part = S <= n_wg ? blockIdx.x - slot * bps : 0;
  const int slot_step = S <= n_wg ? S : n_wg;

  for (; slot < S; slot += slot_step) {
    // ---- the tile and this workgroup's unit range inside it
    bool is_sh;
    int e, r_begin, r_end, U, K;
    if (slot < a.n_sh_slots) {
      const int per_sh = (a.T + a.sh_tile - 1) / a.sh_tile;
      const int s = slot / per_sh, ti = slot - s * per_sh;
      is_sh = true;
      e = s;
      r_begin = ti * a.sh_tile;
      r_end = min(a.T, r_begin + a.sh_tile);
      U = a.U_sh;
      K = a.K_sh;
    } else {
      const int4 tl = reinterpret_cast<const int4*>(a.tiles)[slot - a.n_sh_slots];
      is_sh = false;
      e = tl.x;
      r_begin = tl.y;
      r_end = tl.z;
      U = a.U;
      K = a.K;
    }
    const int unit0 = (int)((long long)U * part / bps);
    const int unit1 = (int)((long long)U * (part + 1) / bps);
    const int nunits = unit1 - unit0;
    if (nunits <= 0) continue;
    if (!is_sh && (unsigned)e >= (unsigned)a.E) {
      if (tid == 0) atomicOr(a.err, 2);
      continue;
    }
    const moe_qmat q = is_sh ? a.w_sh[e] : a.w[e];
    if (!qmat_usable(q, a.mode == 0 ? 2 * U : U, K)) {
      if (tid == 0) atomicOr(a.err, 1);
      continue;
    }
    const RowGeom G = row_geom(q, K, a.mode);
    const int lis = lane & (G.seg - 1);
    const int sid = lane >> G.lseg;
    const int qrow = wave * G.segs_w + sid;     // row slot inside an iteration
    const int n_it = (nunits + G.UPI - 1) / G.UPI;

    // weight row of iteration `it` for this lane's row slot
    auto wrow = [&](int it, bool& vrow) -> int {
      const int ub = it * G.UPI;
      int unit, wr;
      if (a.mode == 0) {
        const bool up = qrow >= G.UPI;
        unit = ub + (up ? qrow - G.UPI : qrow);
        wr = unit0 + unit + (up ? U : 0);
      } else {
        unit = ub + qrow;
        wr = unit0 + unit;
      }
      vrow = unit < nunits;
      return vrow ? wr : 0;
    };
    auto load = [&](int it, int c0, uint4 (&wv)[kCplMax], uint32_t (&sv)[kCplMax]) {
      bool vrow;
      const int wr = wrow(it, vrow);
      const uint4* cp = reinterpret_cast<const uint4*>(q.codes + (size_t)wr * G.row_bytes);
      const uint16_t* sp = q.scales + (size_t)wr * G.ng;
#pragma unroll
      for (int b = 0; b < kCplMax; ++b) {
        const int c = lis + G.seg * (c0 + b);
        if (c0 + b < G.cpl && vrow) {
          const u32x4_v t4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_v*>(cp + c));
          wv[b] = make_uint4(t4.x, t4.y, t4.z, t4.w);
          sv[b] = (G.bits == 2 && G.group == 32) ? *reinterpret_cast<const uint32_t*>(sp + 2 * c)
                                                 : (uint32_t)sp[(c * G.CK) / G.group];
        } else {
          wv[b] = make_uint4(0u, 0u, 0u, 0u);
          sv[b] = 0u;
        }
      }
    };

    for (int pass = r_begin; pass < r_end; pass += MAXT) {
      const int nt = min(MAXT, r_end - pass);
      const int orow_base = is_sh ? a.P + e * a.T + pass : pass;

      // one iteration: dot products of the iteration's rows, reduction,
      // then the epilogue of its units
      auto iterate = [&](int it, uint4 (&wv)[kCplMax], uint32_t (&sv)[kCplMax], int rbuf) {
        bool vrow;
        const int wr = wrow(it, vrow);
        float acc[MAXT];
#pragma unroll
        for (int t = 0; t < MAXT; ++t) acc[t] = 0.0f;
        for (int c0 = 0; c0 < G.cpl; c0 += kCplMax) {
          if (c0 > 0) load(it, c0, wv, sv);
#pragma unroll
          for (int b = 0; b < kCplMax; ++b) {
            if (c0 + b >= G.cpl) break;
            chunk_dot<ACT, MAXT, DUMP>(a, wv[b], sv[b], lis + G.seg * (c0 + b), G, nt, xs,
                                       xs_row, xsum, xsum_row, acc, lis, vrow, wr, orow_base);
          }
        }
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
          if (t >= nt) break;
          acc[t] = group_sum(acc[t], G.seg);
        }
        float* rs = res + rbuf * a.res_rows * MAXT;
        if (lis == 0 && vrow) {
#pragma unroll
          for (int t = 0; t < MAXT; ++t) {
            if (t >= nt) break;
            rs[qrow * MAXT + t] = acc[t];
          }
        }
        __syncthreads();
        const int ub = it * G.UPI;
        const int nu = min(G.UPI, nunits - ub);
        if (a.mode == 0) {
          for (int idx = tid; idx < nu * nt; idx += kGemvThreads) {
            const int m = idx / nu, i = idx - m * nu;
            float gv = rs[i * MAXT + m], uv = rs[(G.UPI + i) * MAXT + m];
            if (ACT == MOE_A8) {
              gv *= xsc[m];
              uv *= xsc[m];
            }
            const float hv = silu_mul(gv, uv);
            const size_t o = (size_t)(orow_base + m) * a.ld_out + unit0 + ub + i;
            if (ACT == MOE_A16) static_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16(hv);
            else static_cast<float*>(a.out)[o] = hv;
          }
        } else {
          for (int idx = tid; idx < nu * nt; idx += kGemvThreads) {
            const int m = idx / nu, i = idx - m * nu;
            float y = rs[i * MAXT + m];
            if (ACT == MOE_A8) y *= xsc[m];
            static_cast<float*>(a.out)[(size_t)(orow_base + m) * a.ld_out + unit0 + ub + i] = y;
          }
        }
      };

      uint4 wvA[kCplMax], wvB[kCplMax];
      uint32_t svA[kCplMax], svB[kCplMax];
      load(0, 0, wvA, svA);              // in flight while the activations are staged
      __syncthreads();                   // previous users of xs / res are done
      stage_rows<ACT>(a, is_sh, e, pass, nt, K, G.bits, xs, xs_row, xsum, xsc, xsum_row);
      __syncthreads();
      for (int it = 0; it < n_it; it += 2) {
        if (it + 1 < n_it) load(it + 1, 0, wvB, svB);
        iterate(it, wvA, svA, 0);
        if (it + 1 >= n_it) break;
        if (it + 2 < n_it) load(it + 2, 0, wvA, svA);
        iterate(it + 1, wvB, svB, 1);
      }
    }
  }
}

template <int ACT, int MAXT, bool DUMP>
static hipError_t launch_t(const ProjArgs& a, int grid, hipStream_t st) {
  const int Kl = max(a.K, a.K_sh);
  size_t lds;
  if (ACT == MOE_A16)
    lds = (size_t)MAXT * Kl * 2 + (size_t)MAXT * (Kl / 32) * 4;
  else
    lds = (size_t)MAXT * Kl + (size_t)MAXT * 4;
  lds += (size_t)2 * a.res_rows * MAXT * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  proj_gemv_kernel<ACT, MAXT, DUMP><<<grid, kGemvThreads, lds, st>>>(a);
  return hipGetLastError();
}

template <int ACT, bool DUMP>
static hipError_t launch_act(const ProjArgs& a, int grid, hipStream_t st) {
  switch (a.maxt) {
    case 1: return launch_t<ACT, 1, DUMP>(a, grid, st);
    case 2: return launch_t<ACT, 2, DUMP>(a, grid, st);
    case 4: return launch_t<ACT, 4, DUMP>(a, grid, st);
    default: return launch_t<ACT, 8, DUMP>(a, grid, st);
  }
}

// Tokens staged per pass: the largest row count a tile can hold, rounded
// up to 1, 2, 4 or 8 (tiles with more rows take several passes).
int gemv_maxt(int T, int tile_m) {
  const int b = min(T, tile_m);
  return b <= 1 ? 1 : b <= 2 ? 2 : b <= 4 ? 4 : 8;
}

// Rows per iteration of the widest geometry any expert of the call can
// have (the fewest lanes per row: K and bits decide it).
int gemv_res_rows(int K, int K_sh) {
  int rows = 0;
  for (int kk : {K, K_sh}) {
    for (int bits : {4, 2}) {
      const int C_r = kk * bits / 128;
      if (C_r <= 0) continue;
      int seg = C_r & (-C_r);
      if (seg > 16) seg = 16;
      rows = max(rows, kGemvWaves * (64 / seg));
    }
  }
  return rows;
}

hipError_t launch_proj_gemv(const ProjArgs& a_in, int act, int grid, hipStream_t st) {
  ProjArgs a = a_in;
  a.res_rows = gemv_res_rows(a.K, a.K_sh);
  if (grid <= 0) return hipSuccess;
  const bool dump = a.partials != nullptr;
  if (act == MOE_A16) return launch_act<MOE_A16, false>(a, grid, st);
  if (dump) return launch_act<MOE_A8, true>(a, grid, st);
  return launch_act<MOE_A8, false>(a, grid, st);
}

}  // namespace moe
