// Device helpers shared by the split-K GEMV kernels (decode shapes): row
// geometry of a packed weight matrix, the LDS planes that activation rows
// are staged into, and the dot product of one 16-byte code chunk with
// every staged token.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kGemvWaves = 8;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kCplMax = 4;   // 16-byte chunks per lane held per register set

typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));

// Loads through the global address space.  Pointers read out of
// descriptors or argument structs are generic to the compiler, which then
// emits flat loads; those count against the LDS counter as well, so every
// LDS wait would also wait for them.  All buffers here live in global
// memory.
template <class T>
__device__ __forceinline__ T ld_global(const T* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ T ld_global_nt(const T* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) T*)p);
}

// Geometry of the rows of one expert matrix.
struct RowGeom {
  int bits, group, CK, C_r, seg, lseg, cpl, segs_w, RPI, UPI, ng;
  size_t row_bytes;
};

__device__ __forceinline__ RowGeom row_geom(const moe_qmat& q, int K, int mode) {
  RowGeom g;
  g.bits = q.bits;
  g.group = q.group;
  g.CK = 128 / g.bits;                 // K positions per 16-byte chunk
  g.C_r = K / g.CK;                    // chunks per row
  int seg = g.C_r & (-g.C_r);
  g.seg = seg > 16 ? 16 : seg;
  g.lseg = __builtin_ctz(g.seg);
  g.cpl = g.C_r >> g.lseg;             // chunks per lane per row
  g.segs_w = 64 >> g.lseg;             // rows per wave
  g.RPI = kGemvWaves * g.segs_w;       // rows per iteration
  g.UPI = mode == 0 ? g.RPI / 2 : g.RPI;
  g.ng = K / g.group;
  g.row_bytes = (size_t)K * g.bits / 8;
  return g;
}

// LDS layout of a staged activation row.  The activations that meet one
// 16-byte code chunk c (in unpack order) span NJ 16-byte words (A16: 4 for
// int4, 8 for int2; A8: 2 for int4, 4 for int2).  Word j of chunk c is
// stored at 16-byte index j * C_r + c (C_r = chunks per row), so the lanes
// of a segment, which hold consecutive chunks, read consecutive 16-byte
// words: no LDS bank conflicts on the ds_read_b128.
//
// A8: the 8 dwords of a 32-K staging block b go to words (int4: chunk b,
// words 0-1; int2: chunk b/2, words 2*(b%2) + 0-1).
__device__ __forceinline__ void store_a8_planes(uint32_t* row, const uint32_t (&pr)[8], int b,
                                                int K, int bits) {
  const int C_r = K * bits / 128;
  const int c = bits == 4 ? b : b >> 1;
  const int p0 = bits == 4 ? 0 : (b & 1) * 2;
  uint4* dst = reinterpret_cast<uint4*>(row);
  dst[p0 * C_r + c] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
  dst[(p0 + 1) * C_r + c] = make_uint4(pr[4], pr[5], pr[6], pr[7]);
}

// Stage one 32-K block b of a bf16 activation row into its LDS planes
// (layout above) and record the block's sum of activations (it removes
// the code bias of the exact bf16 unpack).
// Split in two so a caller can issue the loads early and store later.
__device__ __forceinline__ void load_a16_block(const uint16_t* row, int b, uint32_t (&v)[16]) {
  const u32x4_v* src = reinterpret_cast<const u32x4_v*>(row + b * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_v t4 = ld_global(src + i);
    v[4 * i] = t4.x; v[4 * i + 1] = t4.y; v[4 * i + 2] = t4.z; v[4 * i + 3] = t4.w;
  }
}

// The same loads at device scope (coherent across XCDs without a cache
// write-back or invalidate): rows written by other workgroups of the same
// launch.
__device__ __forceinline__ void load_a16_block_coherent(const uint16_t* row, int b,
                                                        uint32_t (&v)[16]) {
  const uint64_t* src = reinterpret_cast<const uint64_t*>(row + b * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint64_t t = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v[2 * i] = (uint32_t)t;
    v[2 * i + 1] = (uint32_t)(t >> 32);
  }
}

__device__ __forceinline__ void store_a16_block(const uint32_t (&v)[16], int b, int K, int bits,
                                                uint32_t* xs_row, float* xsum_row) {
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sum += bf16_to_f32(v[i] & 0xFFFFu);
    sum += bf16_to_f32(v[i] >> 16);
  }
  // 16 dwords of pairs -> planes (see the layout note above)
  uint32_t pr[16];
  auto xv = [&](int j) -> uint32_t { return (v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu; };
  if (bits == 4) {       // four 8-blocks, pairs (i, i+4)
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pr[blk * 4 + i] = xv(8 * blk + i) | (xv(8 * blk + i + 4) << 16);
  } else {               // two 16-blocks, pairs (i, i+8)
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pr[blk * 8 + i] = xv(16 * blk + i) | (xv(16 * blk + i + 8) << 16);
  }
  const int C_r = K * bits / 128;
  const int c = bits == 4 ? b : b >> 1;
  const int p0 = bits == 4 ? 0 : (b & 1) * 4;
  uint4* dst = reinterpret_cast<uint4*>(xs_row);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dst[(p0 + i) * C_r + c] = make_uint4(pr[4 * i], pr[4 * i + 1], pr[4 * i + 2], pr[4 * i + 3]);
  xsum_row[b] = sum;
}

__device__ __forceinline__ void stage_a16_block(const uint16_t* row, int b, int K, int bits,
                                                uint32_t* xs_row, float* xsum_row) {
  uint32_t v[16];
  load_a16_block(row, b, v);
  store_a16_block(v, b, K, bits, xs_row, xsum_row);
}

// One 16-byte chunk c of a weight row against every staged token.
template <int ACT, int MAXT, bool DUMP>
__device__ __forceinline__ void chunk_dot(const ProjArgs& a, const uint4 wv, const uint32_t sv,
                                          int c, const RowGeom& G, int nt, const uint32_t* xs,
                                          int xs_row, const float* xsum, int xsum_row,
                                          float (&acc)[MAXT], int lis, bool vrow, int wr,
                                          int orow_base) {
  const uint32_t W[4] = {wv.x, wv.y, wv.z, wv.w};
  if (ACT == MOE_A16) {
    if (G.bits == 4) {
      uint32_t wb[16];
      // code c -> bf16 136 + c: field (c ^ 8) OR-ed into 128 = 0x4300, written
      // as one AND and one XOR (the offset 8 folded into the constant)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = W[j];
        wb[4 * j + 0] = (w & 0x000F000Fu) ^ 0x43084308u;
        wb[4 * j + 1] = ((w >> 4) & 0x000F000Fu) ^ 0x43084308u;
        wb[4 * j + 2] = ((w >> 8) & 0x000F000Fu) ^ 0x43084308u;
        wb[4 * j + 3] = ((w >> 12) & 0x000F000Fu) ^ 0x43084308u;
      }
      const float s = fp16_to_f32(sv & 0xFFFFu);
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t >= nt) break;
        const uint4* xp = reinterpret_cast<const uint4*>(xs + t * xs_row) + c;
        float D = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 x4 = xp[i * G.C_r];
          D = dot2_bf16(wb[4 * i + 0], x4.x, D);
          D = dot2_bf16(wb[4 * i + 1], x4.y, D);
          D = dot2_bf16(wb[4 * i + 2], x4.z, D);
          D = dot2_bf16(wb[4 * i + 3], x4.w, D);
        }
        acc[t] = fmaf(s, D - 136.0f * xsum[t * xsum_row + c], acc[t]);
      }
    } else {  // int2: 4 words x 8 pairs
      uint32_t wb[32];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = W[j];
#pragma unroll
        for (int i = 0; i < 8; ++i) wb[8 * j + i] = ((w >> (2 * i)) & 0x00030003u) ^ 0x43024302u;
      }
      const float s0 = fp16_to_f32(sv & 0xFFFFu);
      const float s1 = G.group == 32 ? fp16_to_f32(sv >> 16) : s0;
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t >= nt) break;
        const uint4* xp = reinterpret_cast<const uint4*>(xs + t * xs_row) + c;
        float D0 = 0.0f, D1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 x4 = xp[i * G.C_r];
          D0 = dot2_bf16(wb[4 * i + 0], x4.x, D0);
          D0 = dot2_bf16(wb[4 * i + 1], x4.y, D0);
          D0 = dot2_bf16(wb[4 * i + 2], x4.z, D0);
          D0 = dot2_bf16(wb[4 * i + 3], x4.w, D0);
        }
#pragma unroll
        for (int i = 4; i < 8; ++i) {
          const uint4 x4 = xp[i * G.C_r];
          D1 = dot2_bf16(wb[4 * i + 0], x4.x, D1);
          D1 = dot2_bf16(wb[4 * i + 1], x4.y, D1);
          D1 = dot2_bf16(wb[4 * i + 2], x4.z, D1);
          D1 = dot2_bf16(wb[4 * i + 3], x4.w, D1);
        }
        acc[t] = fmaf(s0, D0 - 130.0f * xsum[t * xsum_row + 2 * c], acc[t]);
        acc[t] = fmaf(s1, D1 - 130.0f * xsum[t * xsum_row + 2 * c + 1], acc[t]);
      }
    }
  } else {  // A8
    if (G.bits == 4) {
      uint32_t wq[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wq[2 * j] = (W[j] << 4) & 0xF0F0F0F0u;
        wq[2 * j + 1] = W[j] & 0xF0F0F0F0u;
      }
      const float s = fp16_to_f32(sv & 0xFFFFu);
      const int cpg = G.group / 32;   // chunks per group (<= seg)
      const int g = (c * 32) / G.group;
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t >= nt) break;
        const uint4* xp = reinterpret_cast<const uint4*>(xs + t * xs_row) + c;
        const uint4 x0 = xp[0], x1 = xp[G.C_r];
        int d = 0;
        d = sdot4((int)wq[0], (int)x0.x, d);
        d = sdot4((int)wq[1], (int)x0.y, d);
        d = sdot4((int)wq[2], (int)x0.z, d);
        d = sdot4((int)wq[3], (int)x0.w, d);
        d = sdot4((int)wq[4], (int)x1.x, d);
        d = sdot4((int)wq[5], (int)x1.y, d);
        d = sdot4((int)wq[6], (int)x1.z, d);
        d = sdot4((int)wq[7], (int)x1.w, d);
        const int P = group_sum_i(d >> 4, cpg);
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
        const uint4* xp = reinterpret_cast<const uint4*>(xs + t * xs_row) + c;
        int d0 = 0, d1 = 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 x4 = xp[i * G.C_r];
          d0 = sdot4((int)wq[4 * i + 0], (int)x4.x, d0);
          d0 = sdot4((int)wq[4 * i + 1], (int)x4.y, d0);
          d0 = sdot4((int)wq[4 * i + 2], (int)x4.z, d0);
          d0 = sdot4((int)wq[4 * i + 3], (int)x4.w, d0);
        }
#pragma unroll
        for (int i = 2; i < 4; ++i) {
          const uint4 x4 = xp[i * G.C_r];
          d1 = sdot4((int)wq[4 * i + 0], (int)x4.x, d1);
          d1 = sdot4((int)wq[4 * i + 1], (int)x4.y, d1);
          d1 = sdot4((int)wq[4 * i + 2], (int)x4.z, d1);
          d1 = sdot4((int)wq[4 * i + 3], (int)x4.w, d1);
        }
        if (G.group == 32) {
          const int P0 = d0 >> 6, P1 = d1 >> 6;
          acc[t] = fmaf(fp16_to_f32(sv & 0xFFFFu), (float)P0, acc[t]);
          acc[t] = fmaf(fp16_to_f32(sv >> 16), (float)P1, acc[t]);
          if (DUMP && vrow) {
            int32_t* pp = a.partials + ((size_t)(orow_base + t) * a.part_rows + wr) * a.ng_ld;
            pp[2 * c] = P0;
            pp[2 * c + 1] = P1;
          }
        } else {
          const int cpg = G.group / 64;
          const int P = group_sum_i((d0 + d1) >> 6, cpg);
          if ((lis & (cpg - 1)) == 0) {
            acc[t] = fmaf(fp16_to_f32(sv & 0xFFFFu), (float)P, acc[t]);
            if (DUMP && vrow)
              a.partials[((size_t)(orow_base + t) * a.part_rows + wr) * a.ng_ld +
                         (c * 64) / G.group] = P;
          }
        }
      }
    }
  }
}

}  // namespace moe
