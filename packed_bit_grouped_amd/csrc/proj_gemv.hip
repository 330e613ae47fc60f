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
//  * work item = (tile of up to tile_m sorted rows of one expert, block of
//    output units); the tile's activations are staged once in LDS in the
//    pair order of the code unpack, and every weight row of the block is
//    read once from HBM and applied to all of the tile's tokens (tile
//    reuse);
//  * a weight row is split into 16-byte chunks; `seg` lanes share a row
//    (split-K) and combine their partial sums with a butterfly over the
//    segment (blocked reduction); a wave covers 64/seg rows at a time;
//  * gate row i and up row I+i of W13 are in the same work item and meet
//    in LDS for the fused SiLU(g) * u epilogue;
//  * A16: codes expand to bf16 (exact, biased) and v_dot2_f32_bf16 forms
//    the products; A8: codes expand to int8 and v_dot4_i32_i8 forms exact
//    int32 per-group partial sums, scaled in fp32.
#include "moe_internal.h"

namespace moe {

constexpr int kGemvThreads = 256;

typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));

// Input row pointers of pass row m.
__device__ __forceinline__ int token_of(const ProjArgs& a, bool is_sh, int r) {
  return is_sh ? r : a.sorted_pair[r] / a.k;
}

template <int ACT, int MAXT, bool DUMP>
__global__ __launch_bounds__(kGemvThreads) void proj_gemv_kernel(ProjArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = blockIdx.x / a.n_rb;
  const int rbi = blockIdx.x - slot * a.n_rb;

  // ---- which expert and which rows
  bool is_sh;
  int e, r_begin, r_end;  // routed: sorted rows; shared: token indices
  if (slot < a.n_sh_slots) {
    const int per = (a.T + a.sh_tile - 1) / a.sh_tile;
    const int s = slot / per, ti = slot - s * per;
    is_sh = true;
    e = s;
    r_begin = ti * a.sh_tile;
    r_end = min(a.T, r_begin + a.sh_tile);
  } else {
    const int j = slot - a.n_sh_slots;
    if (j >= *a.n_tiles) return;
    const int4 tl = reinterpret_cast<const int4*>(a.tiles)[j];
    if ((unsigned)tl.x >= (unsigned)a.E) {
      if (tid == 0) atomicOr(a.err, 2);
      return;
    }
    is_sh = false;
    e = tl.x;
    r_begin = tl.y;
    r_end = tl.z;
  }
  const int K = is_sh ? a.K_sh : a.K;
  const int U = is_sh ? a.U_sh : a.U;
  const int unit0 = rbi * a.rb;
  if (unit0 >= U || r_end <= r_begin) return;
  const int nunits = min(a.rb, U - unit0);
  const moe_qmat q = is_sh ? a.w_sh[e] : a.w[e];
  if (!qmat_usable(q, a.mode == 0 ? 2 * U : U, K)) {
    if (tid == 0) atomicOr(a.err, 1);
    return;
  }
  const int bits = q.bits, group = q.group;
  const int CK = 128 / bits;          // K positions per 16-byte chunk
  const int C_r = K / CK;             // chunks per row
  int seg = C_r & (-C_r);
  if (seg > 16) seg = 16;
  const int lseg = __builtin_ctz(seg);
  const int cpl = C_r >> lseg;        // chunks per lane per row
  const int segs_w = 64 >> lseg;
  const int lis = lane & (seg - 1);
  const int sid = lane >> lseg;
  const int rows_item = a.mode == 0 ? 2 * nunits : nunits;
  const int row_stride = 4 * segs_w;
  const int iters = (rows_item + row_stride - 1) / row_stride;
  const size_t row_bytes = (size_t)K * bits / 8;
  const int ng = K / group;
  const int Kl = max(a.K, a.K_sh);
  const int rows_max = a.mode == 0 ? 2 * a.rb : a.rb;

  // ---- LDS carve-up
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem);
  float* xsum = nullptr;     // A16: [MAXT][Kl/32]
  float* xsc = nullptr;      // A8: [MAXT]
  float* res;
  if (ACT == MOE_A16) {
    xsum = reinterpret_cast<float*>(xs + MAXT * (Kl / 2));
    res = xsum + MAXT * (Kl / 32);
  } else {
    xsc = reinterpret_cast<float*>(xs + MAXT * (Kl / 4));
    res = xsc + MAXT;
  }
  const int xs_row = ACT == MOE_A16 ? Kl / 2 : Kl / 4;  // dwords per staged row
  const int nb32 = K / 32;

  for (int pass = r_begin; pass < r_end; pass += MAXT) {
    const int nt = min(MAXT, r_end - pass);
    __syncthreads();
    // ---- stage the pass's activation rows
    if (ACT == MOE_A16) {
      for (int u = tid; u < nt * nb32; u += kGemvThreads) {
        const int m = u / nb32, b = u - m * nb32;
        int row;
        if (a.mode == 0) row = token_of(a, is_sh, pass + m);
        else row = is_sh ? a.P + e * a.T + pass + m : pass + m;
        const uint4* src =
            reinterpret_cast<const uint4*>(a.in_bf16 + (size_t)row * a.ld_in + b * 32);
        uint32_t v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 t4 = src[i];
          v[4 * i] = t4.x; v[4 * i + 1] = t4.y; v[4 * i + 2] = t4.z; v[4 * i + 3] = t4.w;
        }
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sum += bf16_to_f32(v[i] & 0xFFFFu);
          sum += bf16_to_f32(v[i] >> 16);
        }
        uint32_t* dst = xs + m * xs_row + b * 16;
        auto xv = [&](int j) -> uint32_t {
          return (v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        };
        if (bits == 4) {       // four 8-blocks, pairs (i, i+4)
#pragma unroll
          for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              dst[blk * 4 + i] = xv(8 * blk + i) | (xv(8 * blk + i + 4) << 16);
        } else {               // two 16-blocks, pairs (i, i+8)
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 8; ++i)
              dst[blk * 8 + i] = xv(16 * blk + i) | (xv(16 * blk + i + 8) << 16);
        }
        xsum[m * (Kl / 32) + b] = sum;
      }
    } else if (a.mode == 0) {  // A8 gate/up: pre-quantized x
      for (int u = tid; u < nt * nb32; u += kGemvThreads) {
        const int m = u / nb32, b = u - m * nb32;
        const int t = token_of(a, is_sh, pass + m);
        const uint4* src = reinterpret_cast<const uint4*>(a.in_q + (size_t)t * a.ld_in + b * 32);
        const uint4 lo = src[0], hi = src[1];
        const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        uint32_t* dst = xs + m * xs_row + b * 8;
        auto xb = [&](int j) -> uint32_t { return (d[j >> 2] >> (8 * (j & 3))) & 0xFFu; };
        if (bits == 4) {       // 8-blocks: even quad, odd quad
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            dst[2 * blk] = xb(8 * blk) | xb(8 * blk + 2) << 8 | xb(8 * blk + 4) << 16 | xb(8 * blk + 6) << 24;
            dst[2 * blk + 1] = xb(8 * blk + 1) | xb(8 * blk + 3) << 8 | xb(8 * blk + 5) << 16 | xb(8 * blk + 7) << 24;
          }
        } else {               // 16-blocks: quads (i, i+4, i+8, i+12)
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              dst[4 * blk + i] = xb(16 * blk + i) | xb(16 * blk + i + 4) << 8 |
                                 xb(16 * blk + i + 8) << 16 | xb(16 * blk + i + 12) << 24;
        }
        if (b == 0) xsc[m] = a.in_s[t];
      }
    } else {                   // A8 down: quantize fp32 h rows here
      for (int m = wave; m < nt; m += 4) {
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
          uint32_t* dst = xs + m * xs_row + b * 8;
          if (bits == 4) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
              dst[2 * blk] = cq[8 * blk] | cq[8 * blk + 2] << 8 | cq[8 * blk + 4] << 16 | cq[8 * blk + 6] << 24;
              dst[2 * blk + 1] = cq[8 * blk + 1] | cq[8 * blk + 3] << 8 | cq[8 * blk + 5] << 16 | cq[8 * blk + 7] << 24;
            }
          } else {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                dst[4 * blk + i] = cq[16 * blk + i] | cq[16 * blk + i + 4] << 8 |
                                   cq[16 * blk + i + 8] << 16 | (uint32_t)cq[16 * blk + i + 12] << 24;
          }
        }
        if (lane == 0) xsc[m] = sc;
      }
    }
    __syncthreads();

    // ---- weight rows of the work item
    for (int it = 0; it < iters; ++it) {
      const int qrow = it * row_stride + wave * segs_w + sid;
      const bool vrow = qrow < rows_item;
      int wr;
      if (a.mode == 0) wr = qrow < nunits ? unit0 + qrow : U + unit0 + (qrow - nunits);
      else wr = unit0 + qrow;
      if (!vrow) wr = 0;
      const uint4* cp = reinterpret_cast<const uint4*>(q.codes + (size_t)wr * row_bytes);
      const uint16_t* sp = q.scales + (size_t)wr * ng;
      float acc[MAXT];
#pragma unroll
      for (int t = 0; t < MAXT; ++t) acc[t] = 0.0f;

      for (int c0 = 0; c0 < cpl; c0 += 8) {
        uint4 wv[8];
        uint32_t sv[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int c = lis + seg * (c0 + b);
          if (c0 + b < cpl && vrow) {
            const u32x4_v t4 =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4_v*>(cp + c));
            wv[b] = make_uint4(t4.x, t4.y, t4.z, t4.w);
            if (bits == 2 && group == 32)
              sv[b] = *reinterpret_cast<const uint32_t*>(sp + 2 * c);
            else
              sv[b] = sp[(c * CK) / group];
          } else {
            wv[b] = make_uint4(0u, 0u, 0u, 0u);
            sv[b] = 0u;
          }
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          if (c0 + b >= cpl) break;
          const int c = lis + seg * (c0 + b);
          const uint32_t W[4] = {wv[b].x, wv[b].y, wv[b].z, wv[b].w};
          if (ACT == MOE_A16) {
            if (bits == 4) {
              uint32_t wb[16];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t w = W[j] ^ 0x88888888u;
                wb[4 * j + 0] = (w & 0x000F000Fu) | 0x43004300u;
                wb[4 * j + 1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
                wb[4 * j + 2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
                wb[4 * j + 3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
              }
              const float s = fp16_to_f32(sv[b] & 0xFFFFu);
#pragma unroll
              for (int t = 0; t < MAXT; ++t) {
                if (t >= nt) break;
                const uint4* xp = reinterpret_cast<const uint4*>(xs + t * xs_row + c * 16);
                float D = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const uint4 xv4 = xp[i];
                  D = dot2_bf16(wb[4 * i + 0], xv4.x, D);
                  D = dot2_bf16(wb[4 * i + 1], xv4.y, D);
                  D = dot2_bf16(wb[4 * i + 2], xv4.z, D);
                  D = dot2_bf16(wb[4 * i + 3], xv4.w, D);
                }
                acc[t] = fmaf(s, D - 136.0f * xsum[t * (Kl / 32) + c], acc[t]);
              }
            } else {  // int2: 4 words x 8 pairs
              uint32_t wb[32];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t w = W[j] ^ 0xAAAAAAAAu;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                  wb[8 * j + i] = ((w >> (2 * i)) & 0x00030003u) | 0x43004300u;
              }
              float s0, s1;
              if (group == 32) {
                s0 = fp16_to_f32(sv[b] & 0xFFFFu);
                s1 = fp16_to_f32(sv[b] >> 16);
              } else {
                s0 = s1 = fp16_to_f32(sv[b] & 0xFFFFu);
              }
#pragma unroll
              for (int t = 0; t < MAXT; ++t) {
                if (t >= nt) break;
                const uint4* xp = reinterpret_cast<const uint4*>(xs + t * xs_row + c * 32);
                float D0 = 0.0f, D1 = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const uint4 xv4 = xp[i];
                  D0 = dot2_bf16(wb[4 * i + 0], xv4.x, D0);
                  D0 = dot2_bf16(wb[4 * i + 1], xv4.y, D0);
                  D0 = dot2_bf16(wb[4 * i + 2], xv4.z, D0);
                  D0 = dot2_bf16(wb[4 * i + 3], xv4.w, D0);
                }
#pragma unroll
                for (int i = 4; i < 8; ++i) {
                  const uint4 xv4 = xp[i];
                  D1 = dot2_bf16(wb[4 * i + 0], xv4.x, D1);
                  D1 = dot2_bf16(wb[4 * i + 1], xv4.y, D1);
                  D1 = dot2_bf16(wb[4 * i + 2], xv4.z, D1);
                  D1 = dot2_bf16(wb[4 * i + 3], xv4.w, D1);
                }
                const float X0 = xsum[t * (Kl / 32) + 2 * c];
                const float X1 = xsum[t * (Kl / 32) + 2 * c + 1];
                acc[t] = fmaf(s0, D0 - 130.0f * X0, acc[t]);
                acc[t] = fmaf(s1, D1 - 130.0f * X1, acc[t]);
              }
            }
          } else {  // A8
            const int orow_base = is_sh ? a.P + e * a.T + pass : pass;
            if (bits == 4) {
              uint32_t wq[8];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                wq[2 * j] = (W[j] << 4) & 0xF0F0F0F0u;
                wq[2 * j + 1] = W[j] & 0xF0F0F0F0u;
              }
              const float s = fp16_to_f32(sv[b] & 0xFFFFu);
              const int cpg = group / 32;     // chunks per group (<= seg)
              const int g = (c * 32) / group;
#pragma unroll
              for (int t = 0; t < MAXT; ++t) {
                if (t >= nt) break;
                const uint4* xp = reinterpret_cast<const uint4*>(xs + t * xs_row + c * 8);
                const uint4 x0 = xp[0], x1 = xp[1];
                int d = 0;
                d = sdot4((int)wq[0], (int)x0.x, d);
                d = sdot4((int)wq[1], (int)x0.y, d);
                d = sdot4((int)wq[2], (int)x0.z, d);
                d = sdot4((int)wq[3], (int)x0.w, d);
                d = sdot4((int)wq[4], (int)x1.x, d);
                d = sdot4((int)wq[5], (int)x1.y, d);
                d = sdot4((int)wq[6], (int)x1.z, d);
                d = sdot4((int)wq[7], (int)x1.w, d);
                int P = group_sum_i(d >> 4, cpg);
                if ((lis & (cpg - 1)) == 0) {
                  acc[t] = fmaf(s, (float)P, acc[t]);
                  if (DUMP && vrow)
                    a.partials[((size_t)(orow_base + t) * a.part_rows + wr) * a.ng_ld + g] = P;
                }
              }
            } else {  // int2
              uint32_t wq[16];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                wq[4 * j + 0] = (W[j] << 6) & 0xC0C0C0C0u;
                wq[4 * j + 1] = (W[j] << 4) & 0xC0C0C0C0u;
                wq[4 * j + 2] = (W[j] << 2) & 0xC0C0C0C0u;
                wq[4 * j + 3] = W[j] & 0xC0C0C0C0u;
              }
#pragma unroll
              for (int t = 0; t < MAXT; ++t) {
                if (t >= nt) break;
                const uint4* xp = reinterpret_cast<const uint4*>(xs + t * xs_row + c * 16);
                int d0 = 0, d1 = 0;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                  const uint4 xv4 = xp[i];
                  d0 = sdot4((int)wq[4 * i + 0], (int)xv4.x, d0);
                  d0 = sdot4((int)wq[4 * i + 1], (int)xv4.y, d0);
                  d0 = sdot4((int)wq[4 * i + 2], (int)xv4.z, d0);
                  d0 = sdot4((int)wq[4 * i + 3], (int)xv4.w, d0);
                }
#pragma unroll
                for (int i = 2; i < 4; ++i) {
                  const uint4 xv4 = xp[i];
                  d1 = sdot4((int)wq[4 * i + 0], (int)xv4.x, d1);
                  d1 = sdot4((int)wq[4 * i + 1], (int)xv4.y, d1);
                  d1 = sdot4((int)wq[4 * i + 2], (int)xv4.z, d1);
                  d1 = sdot4((int)wq[4 * i + 3], (int)xv4.w, d1);
                }
                if (group == 32) {
                  const int P0 = d0 >> 6, P1 = d1 >> 6;
                  acc[t] = fmaf(fp16_to_f32(sv[b] & 0xFFFFu), (float)P0, acc[t]);
                  acc[t] = fmaf(fp16_to_f32(sv[b] >> 16), (float)P1, acc[t]);
                  if (DUMP && vrow) {
                    int32_t* pp = a.partials + ((size_t)(orow_base + t) * a.part_rows + wr) * a.ng_ld;
                    pp[2 * c] = P0;
                    pp[2 * c + 1] = P1;
                  }
                } else {
                  const int cpg = group / 64;
                  const int P = group_sum_i((d0 + d1) >> 6, cpg);
                  if ((lis & (cpg - 1)) == 0) {
                    acc[t] = fmaf(fp16_to_f32(sv[b] & 0xFFFFu), (float)P, acc[t]);
                    if (DUMP && vrow)
                      a.partials[((size_t)(orow_base + t) * a.part_rows + wr) * a.ng_ld +
                                 (c * 64) / group] = P;
                  }
                }
              }
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t >= nt) break;
        acc[t] = group_sum(acc[t], seg);
      }
      if (lis == 0 && vrow) {
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
          if (t >= nt) break;
          res[qrow * MAXT + t] = acc[t];
        }
      }
    }
    __syncthreads();

    // ---- epilogue
    const int orow0 = is_sh ? a.P + e * a.T + pass : pass;
    if (a.mode == 0) {
      for (int idx = tid; idx < nunits * nt; idx += kGemvThreads) {
        const int m = idx / nunits, i = idx - m * nunits;
        float g = res[i * MAXT + m], u = res[(nunits + i) * MAXT + m];
        if (ACT == MOE_A8) {
          g *= xsc[m];
          u *= xsc[m];
        }
        const float hv = silu_mul(g, u);
        const size_t o = (size_t)(orow0 + m) * a.ld_out + unit0 + i;
        if (ACT == MOE_A16) static_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16(hv);
        else static_cast<float*>(a.out)[o] = hv;
      }
    } else {
      for (int idx = tid; idx < nunits * nt; idx += kGemvThreads) {
        const int m = idx / nunits, i = idx - m * nunits;
        float y = res[i * MAXT + m];
        if (ACT == MOE_A8) y *= xsc[m];
        static_cast<float*>(a.out)[(size_t)(orow0 + m) * a.ld_out + unit0 + i] = y;
      }
    }
  }
  (void)rows_max;
}

template <int ACT, int MAXT, bool DUMP>
static hipError_t launch_t(const ProjArgs& a, hipStream_t st) {
  const int Kl = max(a.K, a.K_sh);
  const int rows_max = a.mode == 0 ? 2 * a.rb : a.rb;
  size_t lds;
  if (ACT == MOE_A16)
    lds = (size_t)MAXT * Kl * 2 + (size_t)MAXT * (Kl / 32) * 4 + (size_t)rows_max * MAXT * 4;
  else
    lds = (size_t)MAXT * Kl + (size_t)MAXT * 4 + (size_t)rows_max * MAXT * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const long long blocks = (long long)(a.n_sh_slots + a.max_tiles) * a.n_rb;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  proj_gemv_kernel<ACT, MAXT, DUMP><<<(unsigned)blocks, kGemvThreads, lds, st>>>(a);
  return hipGetLastError();
}

template <int ACT, bool DUMP>
static hipError_t launch_act(const ProjArgs& a, int maxt, hipStream_t st) {
  switch (maxt) {
    case 1: return launch_t<ACT, 1, DUMP>(a, st);
    case 2: return launch_t<ACT, 2, DUMP>(a, st);
    case 4: return launch_t<ACT, 4, DUMP>(a, st);
    default: return launch_t<ACT, 8, DUMP>(a, st);
  }
}

// Tokens staged per pass: the largest row count a tile can hold, rounded
// up to 1, 2, 4 or 8 (tiles with more rows take several passes).
int gemv_maxt(int T, int tile_m) {
  const int b = min(T, tile_m);
  return b <= 1 ? 1 : b <= 2 ? 2 : b <= 4 ? 4 : 8;
}

hipError_t launch_proj_gemv(const ProjArgs& a, int act, hipStream_t st) {
  const int maxt = a.maxt;
  const bool dump = a.partials != nullptr;
  if (act == MOE_A16) return launch_act<MOE_A16, false>(a, maxt, st);
  if (dump) return launch_act<MOE_A8, true>(a, maxt, st);
  return launch_act<MOE_A8, false>(a, maxt, st);
}

}  // namespace moe
