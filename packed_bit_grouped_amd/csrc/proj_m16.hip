// Grouped expert projections for tiles of at most 16 rows on the matrix
// cores (v_mfma_f32_16x16x32_bf16 for bf16 activations,
// v_mfma_i32_16x16x32_i8 for the W4A8 mode).
//
// Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", section "Keep
// low-bit weights packed, do the work on the NPU": grouped expert
// projections straight from the packed weights, fused gate/up handling and
// tile reuse.  With several rows per expert tile (batched or speculative
// decode) the layer still streams every touched expert once, but a split-K
// GEMV spends one dot instruction per two (bf16) or four (int8) products
// and reads the activations from LDS again for every weight row; at a few
// rows per tile it runs out of VALU issue and LDS bandwidth before HBM runs
// out of bytes.  Here the tile's rows are the M side of a 16x16 MFMA:
//
//  * lane l feeds token row l%16 of A and weight row l%16 of B, each with
//    the 8-wide K slice l/16 of a 32-K step.  Codes come with buffer loads
//    (the step offset is a scalar) into a ring of loads: for int4 with scale
//    groups of 128 or more, 16 bytes of the lane's row per 4 steps (MFMA m
//    of the 4 takes dword m, so the four lane slices of one MFMA span 128 K
//    of one group) with the workgroup's row scales copied to LDS once;
//    otherwise one 32-bit (int4) or 16-bit (int2) word and the row's scale
//    per step.  Every load is issued unconditionally (steps past the end
//    re-read the last one), so the compiler's wait counts stay graded.
//  * Codes expand in registers to exact integers: bf16 136 + v (int4) or
//    130 + v (int2), the bias removed per scale group with the staged sum
//    of the tile's activations over that group; or int8 16 v / 64 v, whose
//    int32 MFMA sums are exact.
//  * Scale groups are at least 32 K, so every MFMA lies inside one group:
//    the group's result is scaled in fp32 by the row's scale when the
//    group ends and added to the fp32 accumulator.
//  * The activations are staged once per workgroup in LDS, each 8-K slice
//    stored in the item order of the code expansion (the two operands of
//    an MFMA must list K in the same order; the order inside a slice is
//    free).
//  * A wave owns the gate tile and the up tile of the same 16 units, so
//    SiLU(g) * u is formed in registers; down waves own four 16-row tiles.
#include <type_traits>

#include "gemv_common.h"

namespace moe {

constexpr int kM16Waves = 4;
constexpr int kM16Threads = 64 * kM16Waves;
constexpr int kM16MaxRows = 16;     // MFMA M: tokens of a tile
constexpr int kM16StageIt = 4;      // staging items per thread and batch

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef int i32x4_v __attribute__((ext_vector_type(4)));

template <int MODE>
struct M16Shape;
template <>
struct M16Shape<0> {                // gate tile + up tile of 16 units
  static constexpr int NT = 2, R = 16, UPW = 16;
};
template <>
struct M16Shape<1> {                // four 16-row tiles of the down matrix
  static constexpr int NT = 4, R = 8, UPW = 64;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t m16_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// B operand of one step from the lane's code word: 8 codes at K 0..7 of
// the lane's slice, items ordered (0,4)(1,5)(2,6)(3,7) as bf16 pairs.
template <int BITS>
__device__ __forceinline__ bf16x8_v m16_b_a16(uint32_t w) {
  u32x4_v b;
  if (BITS == 4) {
    const uint32_t u = w ^ 0x88888888u;              // offset binary c + 8
    b.x = (u & 0x000F000Fu) | 0x43004300u;
    b.y = ((u >> 4) & 0x000F000Fu) | 0x43004300u;
    b.z = ((u >> 8) & 0x000F000Fu) | 0x43004300u;
    b.w = ((u >> 12) & 0x000F000Fu) | 0x43004300u;
  } else {
    // codes 0..3 to bits 0..7, codes 4..7 to bits 16..23; offset binary c + 2
    const uint32_t u = ((w & 0xFFu) | ((w & 0xFF00u) << 8)) ^ 0x00AA00AAu;
    b.x = (u & 0x00030003u) | 0x43004300u;
    b.y = ((u >> 2) & 0x00030003u) | 0x43004300u;
    b.z = ((u >> 4) & 0x00030003u) | 0x43004300u;
    b.w = ((u >> 6) & 0x00030003u) | 0x43004300u;
  }
  return __builtin_bit_cast(bf16x8_v, b);
}

// B operand for int8 activations: items (0,2,4,6,1,3,5,7) as 16 v (int4),
// (0,1,4,5,2,3,6,7) as 64 v (int2).
template <int BITS>
__device__ __forceinline__ long m16_b_a8(uint32_t w) {
  uint32_t lo, hi;
  if (BITS == 4) {
    lo = (w << 4) & 0xF0F0F0F0u;
    hi = w & 0xF0F0F0F0u;
  } else {
    const uint32_t u = (w & 0xFFu) | ((w & 0xFF00u) << 8);
    lo = ((u << 6) & 0x00C000C0u) | ((u << 12) & 0xC000C000u);
    hi = ((u << 2) & 0x00C000C0u) | ((u << 8) & 0xC000C000u);
  }
  return (long)(((uint64_t)hi << 32) | lo);
}

// The same item orders applied to 8 activations x0..x7 (natural order).
// bf16: d[0..3] hold (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> (x0,x4)(x1,x5)(x2,x6)(x3,x7).
__device__ __forceinline__ u32x4_v m16_order_a16(u32x4_v d) {
  u32x4_v o;
  o.x = (d.x & 0xFFFFu) | (d.z << 16);
  o.y = (d.x >> 16) | (d.z & 0xFFFF0000u);
  o.z = (d.y & 0xFFFFu) | (d.w << 16);
  o.w = (d.y >> 16) | (d.w & 0xFFFF0000u);
  return o;
}
// int8: lo = x0..x3, hi = x4..x7 (one byte each).
template <int BITS>
__device__ __forceinline__ uint64_t m16_order_a8(uint32_t lo, uint32_t hi) {
  uint32_t a, b;
  if (BITS == 4) {   // (x0,x2,x4,x6) (x1,x3,x5,x7)
    a = (lo & 0xFFu) | ((lo >> 8) & 0xFF00u) | ((hi & 0xFFu) << 16) | ((hi & 0xFF0000u) << 8);
    b = ((lo >> 8) & 0xFFu) | ((lo >> 16) & 0xFF00u) | ((hi & 0xFF00u) << 8) | (hi & 0xFF000000u);
  } else {           // (x0,x1,x4,x5) (x2,x3,x6,x7)
    a = (lo & 0xFFFFu) | (hi << 16);
    b = (lo >> 16) | (hi & 0xFFFF0000u);
  }
  return ((uint64_t)b << 32) | a;
}

// Row of the staged activations for tile row t.
template <int MODE>
__device__ __forceinline__ int m16_src_row(const ProjArgs& a, bool is_sh, int e, int r_begin,
                                           int t) {
  if (MODE == 0) return is_sh ? r_begin + t : a.sorted_pair[r_begin + t] / a.k;
  return is_sh ? a.P + e * a.T + r_begin + t : r_begin + t;
}

// Activation staging (layout in the file comment).  Work item = (tile row
// t, 32-K block b), it = t * S + b; a thread takes items tid + i * threads.
// The rows of the first batch are resolved before the weight descriptor
// is read (m16_first_rows), their loads are issued before the weight ring
// (m16_x_load), and the LDS stores follow the ring issue (m16_x_store).
template <int ACT>
struct M16XRegs {
  u32x4_v v[kM16StageIt][ACT == MOE_A16 ? 4 : 2];
};

template <int MODE>
__device__ __forceinline__ void m16_row_loads(const ProjArgs& a, int r_begin, int nt, int S,
                                              int (&srow)[kM16StageIt],
                                              int (&trow)[kM16StageIt]) {
  // every index clamped into the tile (r_begin + t < P also for shared
  // slots, whose rows are tokens), so the loads are issued together
#pragma unroll
  for (int i = 0; i < kM16StageIt; ++i) {
    trow[i] = min((i * kM16Threads + (int)threadIdx.x) / S, nt - 1);
    if (MODE == 0) srow[i] = ld_global(a.sorted_pair + r_begin + trow[i]);
  }
}
template <int MODE>
__device__ __forceinline__ void m16_row_finish(const ProjArgs& a, bool is_sh, int e, int r_begin,
                                               int (&srow)[kM16StageIt],
                                               const int (&trow)[kM16StageIt]) {
#pragma unroll
  for (int i = 0; i < kM16StageIt; ++i) {
    if (MODE == 0) srow[i] = is_sh ? r_begin + trow[i] : srow[i] / a.k;
    else srow[i] = m16_src_row<MODE>(a, is_sh, e, r_begin, trow[i]);
  }
}

template <int ACT>
__device__ __forceinline__ void m16_x_load(const ProjArgs& a, int base, int items, int S,
                                           const int (&srow)[kM16StageIt], M16XRegs<ACT>& x) {
#pragma unroll
  for (int i = 0; i < kM16StageIt; ++i) {
    const int it = base + i * kM16Threads + threadIdx.x;
    if (it < items) {
      const int b = it - (it / S) * S;
      if (ACT == MOE_A16) {
        const u32x4_v* src =
            reinterpret_cast<const u32x4_v*>(a.in_bf16 + (size_t)srow[i] * a.ld_in + 32 * b);
#pragma unroll
        for (int c = 0; c < 4; ++c) x.v[i][c] = ld_global(src + c);
      } else {
        const u32x4_v* src =
            reinterpret_cast<const u32x4_v*>(a.in_q + (size_t)srow[i] * a.ld_in + 32 * b);
        x.v[i][0] = ld_global(src);
        x.v[i][1] = ld_global(src + 1);
      }
    }
  }
}

template <int ACT, int BITS>
__device__ __forceinline__ void m16_x_store(int base, int items, int S, const M16XRegs<ACT>& x,
                                            unsigned char* xs, int xstride, float* bsum, int Sl) {
#pragma unroll
  for (int i = 0; i < kM16StageIt; ++i) {
    const int it = base + i * kM16Threads + threadIdx.x;
    if (it < items) {
      const int t = it / S, b = it - t * S;
      if (ACT == MOE_A16) {
        u32x4_v* dst = reinterpret_cast<u32x4_v*>(xs + t * xstride + 64 * b);
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4_v d = x.v[i][c];
          dst[c] = m16_order_a16(d);
          sum += bf16_to_f32(d.x & 0xFFFFu) + bf16_to_f32(d.x >> 16);
          sum += bf16_to_f32(d.y & 0xFFFFu) + bf16_to_f32(d.y >> 16);
          sum += bf16_to_f32(d.z & 0xFFFFu) + bf16_to_f32(d.z >> 16);
          sum += bf16_to_f32(d.w & 0xFFFFu) + bf16_to_f32(d.w >> 16);
        }
        bsum[t * Sl + b] = sum;
      } else {
        uint64_t* dst = reinterpret_cast<uint64_t*>(xs + t * xstride + 32 * b);
        dst[0] = m16_order_a8<BITS>(x.v[i][0].x, x.v[i][0].y);
        dst[1] = m16_order_a8<BITS>(x.v[i][0].z, x.v[i][0].w);
        dst[2] = m16_order_a8<BITS>(x.v[i][1].x, x.v[i][1].y);
        dst[3] = m16_order_a8<BITS>(x.v[i][1].z, x.v[i][1].w);
      }
    }
  }
}

// W4A8 with the int8 rows made here (the row quantizer's rule, a8_scale /
// a8_code, over each staged row): items of the first batch only (the host
// checks that every item fits it).  Gate/up reads bf16 x, down fp32 h.
template <int MODE>
struct M16QRegs {
  static constexpr int kIt = MODE == 0 ? kM16StageIt : kM16StageIt / 2;   // items per thread
  static constexpr int kVec = MODE == 0 ? 4 : 8;                          // 16-byte words per item
  u32x4_v v[kIt][kVec];
};

template <int MODE>
__device__ __forceinline__ void m16_q_load(const ProjArgs& a, int items, int S,
                                           const int (&srow)[kM16StageIt], M16QRegs<MODE>& x) {
#pragma unroll
  for (int i = 0; i < M16QRegs<MODE>::kIt; ++i) {
    const int it = i * kM16Threads + threadIdx.x;
    if (it < items) {
      const int b = it - (it / S) * S;
      const u32x4_v* src =
          MODE == 0 ? reinterpret_cast<const u32x4_v*>(a.in_bf16 + (size_t)srow[i] * a.ld_in + 32 * b)
                    : reinterpret_cast<const u32x4_v*>(a.in_f32 + (size_t)srow[i] * a.ld_in + 32 * b);
#pragma unroll
      for (int c = 0; c < M16QRegs<MODE>::kVec; ++c) x.v[i][c] = ld_global(src + c);
    }
  }
}

// value j (0..31) of an item
template <int MODE>
__device__ __forceinline__ float m16_q_val(const u32x4_v (&v)[M16QRegs<MODE>::kVec], int j) {
  if (MODE == 0) {
    const uint32_t w = v[j >> 3][(j >> 1) & 3];
    return bf16_to_f32((j & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
  return __uint_as_float(v[j >> 2][j & 3]);
}

// row maxima of |v| into rmax (unsigned bits of non-negative floats)
template <int MODE>
__device__ __forceinline__ void m16_q_amax(int items, int S, const M16QRegs<MODE>& x,
                                           uint32_t* rmax) {
#pragma unroll
  for (int i = 0; i < M16QRegs<MODE>::kIt; ++i) {
    const int it = i * kM16Threads + threadIdx.x;
    if (it < items) {
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) m = fmaxf(m, fabsf(m16_q_val<MODE>(x.v[i], j)));
      atomicMax(rmax + it / S, __float_as_uint(m));
    }
  }
}

// a8_code(v, s) without a division per element: for a normal reciprocal,
// y = v * (1/s) lies within a few ulps of the IEEE quotient, so the two round to the same integer
// unless the quotient is within 2^-13 of a half-integer (|y| <= 127.5 and
// an ulp there is 2^-17); those rare elements take the exact path.
__device__ __forceinline__ int m16_a8_code(float v, float s, float rs) {
  if (s == 0.0f) return 0;
  // a scale below 2^-128 has no finite reciprocal (v * inf would give inf
  // or NaN): those rows take the exact division
  if (!(rs <= 0x1.fffffep127f)) return a8_code(v, s);
  const float y = v * rs;
  const float f = y - floorf(y);
  if (fabsf(f - 0.5f) < 0x1p-13f) return a8_code(v, s);
  const float q = fminf(fmaxf(rintf(y), -127.0f), 127.0f);
  return (int)q;
}

template <int MODE, int BITS>
__device__ __forceinline__ void m16_q_store(int items, int S, const M16QRegs<MODE>& x,
                                            const uint32_t* rmax, unsigned char* xs, int xstride) {
#pragma unroll
  for (int i = 0; i < M16QRegs<MODE>::kIt; ++i) {
    const int it = i * kM16Threads + threadIdx.x;
    if (it < items) {
      const int t = it / S, b = it - t * S;
      const float sc = a8_scale(__uint_as_float(rmax[t]));
      const float rs = sc != 0.0f ? 1.0f / sc : 0.0f;
      uint64_t* dst = reinterpret_cast<uint64_t*>(xs + t * xstride + 32 * b);
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {     // 8-K slices
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo |= ((uint32_t)m16_a8_code(m16_q_val<MODE>(x.v[i], 8 * sl + j), sc, rs) & 0xFFu)
                << (8 * j);
          hi |= ((uint32_t)m16_a8_code(m16_q_val<MODE>(x.v[i], 8 * sl + 4 + j), sc, rs) & 0xFFu)
                << (8 * j);
        }
        dst[sl] = m16_order_a8<BITS>(lo, hi);
      }
    }
  }
}

// Rows of the down matrix or gate/up rows a workgroup covers.
template <int MODE>
struct M16Rows {
  static constexpr int kBlock = M16Shape<MODE>::UPW * kM16Waves;   // rows per block
  static constexpr int kBlocks = MODE == 0 ? 2 : 1;                 // gate + up blocks
};

// The scale of LDS row `lrow` (workgroup row) and group g.
__device__ __forceinline__ float m16_scale(const uint16_t* ssc, int lrow, int ng, int g) {
  return fp16_to_f32(ssc[lrow * ng + g]);
}

template <int MODE, int ACT, int BITS, bool WIDE, bool QX, bool PART>
__device__ __forceinline__ void m16_tile(const ProjArgs& a, const moe_qmat& q, bool is_sh, int e,
                                         int r_begin, int nt, int U, int K, int u0, int mt,
                                         const int (&srow)[kM16StageIt], unsigned char* smem) {
  using Sh = M16Shape<MODE>;
  constexpr int NT = Sh::NT;
  // ring depth in loads per N-tile: WIDE loads cover 4 steps (64 bytes of a
  // row), the others one step.  Shallow on purpose: with every resident
  // wave streaming, deeper rings measured slower (more scattered requests
  // outstanding per CU, not more bandwidth).
  constexpr int R = WIDE ? (MODE == 0 ? 4 : 2) : Sh::R;
  constexpr int SPL = WIDE ? 4 : 1;                      // steps per load
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, qd = lane >> 4;
  const int S = K >> 5;                                  // 32-K steps
  const int L = S / SPL;                                 // loads per N-tile
  const int row_bytes = K * BITS / 8;
  const int group = __builtin_amdgcn_readfirstlane(q.group);
  const int ng = K / group;
  const int lbpg = __builtin_ctz(group >> 5);            // log2(steps per group)
  const int Kl = max(a.K, a.K_sh);
  const int Sl = Kl >> 5;
  const int xstride = ACT == MOE_A16 ? 2 * Kl + 16 : Kl + 8;
  unsigned char* xs = smem;
  float* aux = reinterpret_cast<float*>(smem + mt * xstride);
  float* bsum = aux;                   // A16: [16][Sl]
  float* xsum = aux + 16 * Sl;         // A16: [Sl][16]
  float* xsc = aux;                    // A8: [16]
  uint32_t* rmax = reinterpret_cast<uint32_t*>(aux + kM16MaxRows);   // A8, QX: [16]
  uint16_t* ssc = reinterpret_cast<uint16_t*>(
      aux + (ACT == MOE_A16 ? 32 * Sl : 2 * kM16MaxRows));   // [blocks * block rows][ng]

  // ---- first batch of the activations, then the scales, then the ring
  const int items = nt * S;
  M16XRegs<ACT> xr;
  M16QRegs<MODE> xq;
  if constexpr (QX) {
    if (tid < kM16MaxRows) rmax[tid] = 0u;
    m16_q_load<MODE>(a, items, S, srow, xq);
  } else {
    m16_x_load<ACT>(a, 0, items, S, srow, xr);
  }

  // the rows' scales: one contiguous block per row block (gate, up / down)
  constexpr int kBR = M16Rows<MODE>::kBlock;
  const int nr = min(kBR, U - u0);                        // rows of each block
  const int ndw = nr * ng / 2;                            // dwords per block (nr is even)
  constexpr int kSclIt = 8;
  const uint32_t* s0 = reinterpret_cast<const uint32_t*>(q.scales + (size_t)u0 * ng);
  const uint32_t* s1 = reinterpret_cast<const uint32_t*>(q.scales + (size_t)(U + u0) * ng);
  uint32_t* d32 = reinterpret_cast<uint32_t*>(ssc);
  const int blk_dw = kBR * ng / 2;
  const int tot = ndw * M16Rows<MODE>::kBlocks;
  uint32_t sv[kSclIt];
#pragma unroll
  for (int i = 0; i < kSclIt; ++i) {
    const int idx = i * kM16Threads + tid;
    if (idx < tot) sv[i] = ld_global(idx < ndw ? s0 + idx : s1 + (idx - ndw));
  }

  // this wave's weight rows and the ring of code loads
  const int nrows = MODE == 0 ? 2 * U : U;
  const __amdgpu_buffer_rsrc_t crs = m16_rsrc(q.codes, (uint32_t)((size_t)nrows * row_bytes));
  int coff[NT], lrow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int row = MODE == 0 ? (j == 0 ? 0 : U) + u0 + wave * 16 + n
                              : u0 + wave * 64 + 16 * j + n;
    lrow[j] = MODE == 0 ? j * M16Rows<0>::kBlock + wave * 16 + n : wave * 64 + 16 * j + n;
    coff[j] = row * row_bytes + (WIDE ? 16 : (BITS == 4 ? 4 : 2)) * qd;
  }
  using RingT = typename std::conditional<WIDE, u32x4_v, uint32_t>::type;
  RingT rc[R][NT];
  auto load = [&](int l, int r) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (WIDE) {
        rc[r][j] = __builtin_bit_cast(RingT, __builtin_amdgcn_raw_buffer_load_b128(
                                                 crs, coff[j], l * 64, 0));
      } else if constexpr (BITS == 4) {
        rc[r][j] = __builtin_amdgcn_raw_buffer_load_b32(crs, coff[j], l * 16, 0);
      } else {
        rc[r][j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(crs, coff[j], l * 8, 0);
      }
    }
  };
#pragma unroll
  for (int r = 0; r < R; ++r) load(min(r, L - 1), r);

  // ---- LDS stores (the ring stays in flight), further batches if any
  if constexpr (QX) {
    __syncthreads();                     // row maxima cleared
    m16_q_amax<MODE>(items, S, xq, rmax);
    __syncthreads();
    m16_q_store<MODE, BITS>(items, S, xq, rmax, xs, xstride);
    if (tid < kM16MaxRows) xsc[tid] = a8_scale(__uint_as_float(rmax[tid]));
  } else {
    m16_x_store<ACT, BITS>(0, items, S, xr, xs, xstride, bsum, Sl);
  }
#pragma unroll
  for (int i = 0; i < kSclIt; ++i) {
    const int idx = i * kM16Threads + tid;
    if (idx < tot) d32[idx < ndw ? idx : blk_dw + (idx - ndw)] = sv[i];
  }
  for (int idx = kSclIt * kM16Threads + tid; idx < tot; idx += kM16Threads)
    d32[idx < ndw ? idx : blk_dw + (idx - ndw)] = ld_global(idx < ndw ? s0 + idx : s1 + (idx - ndw));
  for (int base = kM16Threads * kM16StageIt; !QX && base < items;
       base += kM16Threads * kM16StageIt) {
    int rows[kM16StageIt];
#pragma unroll
    for (int i = 0; i < kM16StageIt; ++i) {
      const int it = base + i * kM16Threads + tid;
      rows[i] = it < items ? m16_src_row<MODE>(a, is_sh, e, r_begin, it / S) : 0;
    }
    m16_x_load<ACT>(a, base, items, S, rows, xr);
    m16_x_store<ACT, BITS>(base, items, S, xr, xs, xstride, bsum, Sl);
  }
  if (ACT == MOE_A8 && !QX && tid < kM16MaxRows)
    xsc[tid] = tid < nt ? ld_global(a.in_s + m16_src_row<MODE>(a, is_sh, e, r_begin, tid)) : 0.0f;
  __syncthreads();
  if (ACT == MOE_A16) {   // per-group sums of the staged rows
    const int bpg = 1 << lbpg;
    for (int it = tid; it < ng * kM16MaxRows; it += kM16Threads) {
      const int g = it >> 4, t = it & 15;
      float sm = 0.0f;
      if (t < nt)
        for (int b = g * bpg; b < (g + 1) * bpg; ++b) sm += bsum[t * Sl + b];
      xsum[it] = sm;
    }
    __syncthreads();
  }

  // ---- K loop
  constexpr int AS = ACT == MOE_A16 ? 16 : 8;            // bytes of one 8-K A slice
  // slice of this lane: non-WIDE step s -> 4 s + qd; WIDE load l, MFMA m ->
  // 16 l + 4 qd + m
  const unsigned char* ap = xs + min(n, nt - 1) * xstride + (WIDE ? 4 : 1) * AS * qd;
  const float bias = BITS == 4 ? 136.0f : 130.0f;
  const float a8_unit = BITS == 4 ? 0.0625f : 0.015625f;   // 1/16, 1/64
  f32x4_v acc[NT];
  f32x4_v D[NT];
  i32x4_v Di[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    acc[j] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
    D[j] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
    Di[j] = i32x4_v{0, 0, 0, 0};
  }
  // one MFMA per N-tile on step s: code word w of each tile; the A slice of
  // the step for this lane starts at byte offset `ao` of the staged row
  auto mma = [&](int ao, const uint32_t (&w)[NT]) {
    if (ACT == MOE_A16) {
      const bf16x8_v A = *reinterpret_cast<const bf16x8_v*>(ap + ao);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        D[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, m16_b_a16<BITS>(w[j]), D[j], 0, 0, 0);
    } else {
      const long A = *reinterpret_cast<const long*>(ap + ao);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        Di[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, m16_b_a8<BITS>(w[j]), Di[j], 0, 0, 0);
    }
  };
  auto group_end = [&](int g) {
    if (ACT == MOE_A16) {
      const f32x4_v xg = *reinterpret_cast<const f32x4_v*>(xsum + g * 16 + 4 * qd);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float sc = m16_scale(ssc, lrow[j], ng, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(sc, fmaf(-bias, xg[i], D[j][i]), acc[j][i]);
        D[j] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
      }
    } else {
      if constexpr (PART) {
        // the exact int32 sums of the group (the MFMA sums hold 16 v or
        // 64 v per code, so an arithmetic shift divides exactly)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int wr = MODE == 0 ? (j == 0 ? 0 : U) + u0 + wave * 16 + n
                                   : u0 + wave * 64 + 16 * j + n;
          if (wr - (MODE == 0 && j == 1 ? U : 0) < U) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t = 4 * qd + i;
              if (t < nt) {
                const int orow = (is_sh ? a.P + e * a.T : 0) + r_begin + t;
                a.partials[((size_t)orow * a.part_rows + wr) * a.ng_ld + g] =
                    Di[j][i] >> (BITS == 4 ? 4 : 6);
              }
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float sc = m16_scale(ssc, lrow[j], ng, g) * a8_unit;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(sc, (float)Di[j][i], acc[j][i]);
        Di[j] = i32x4_v{0, 0, 0, 0};
      }
    }
  };
  const int lgpl = lbpg - (WIDE ? 2 : 0);                // log2(loads per group), WIDE: >= 0
  const int gmask = (1 << lgpl) - 1;
  for (int l0 = 0; l0 < L; l0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int l = l0 + r;
      if (l < L) {
        if constexpr (WIDE) {
          // load l = steps 4l..4l+3; lane slice qd of step 4l+m is dword m of
          // the lane's 16 bytes, i.e. K = 128 l + 32 qd + 8 m
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            uint32_t w[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) w[j] = rc[r][j][m];
            mma(AS * (16 * l + m), w);
          }
        } else {
          uint32_t w[NT];
#pragma unroll
          for (int j = 0; j < NT; ++j) w[j] = rc[r][j];
          mma(AS * 4 * l, w);
        }
        if (((l + 1) & gmask) == 0) group_end(l >> lgpl);
      }
      load(min(l + R, L - 1), r);
    }
  }

  // ---- epilogue: lane holds tokens 4*qd + i of weight row n of each tile
  const int orow0 = is_sh ? a.P + e * a.T + r_begin : r_begin;
  if (MODE == 0) {
    const int unit = u0 + wave * 16 + n;
    if (unit < U) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * qd + i;
        if (t < nt) {
          float gv = acc[0][i], uv = acc[1][i];
          if (ACT == MOE_A8) {
            gv *= xsc[t];
            uv *= xsc[t];
          }
          const float hv = silu_mul(gv, uv);
          const size_t o = (size_t)(orow0 + t) * a.ld_out + unit;
          if (ACT == MOE_A16) static_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16(hv);
          else static_cast<float*>(a.out)[o] = hv;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int col = u0 + wave * 64 + 16 * j + n;
      if (col < U) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * qd + i;
          if (t < nt) {
            float y = acc[j][i];
            if (ACT == MOE_A8) y *= xsc[t];
            static_cast<float*>(a.out)[(size_t)(orow0 + t) * a.ld_out + col] = y;
          }
        }
      }
    }
  }
}

// Grid: (shared slots + host bound of tiles) x blocks of units; blocks past
// the device-side tile count or past an expert's units exit at once.
template <int MODE, int ACT, bool QX, bool PART>
__global__ __launch_bounds__(kM16Threads) void proj_m16_kernel(ProjArgs a, int mt, int nblk) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int slot = blockIdx.x / nblk;
  const int blk = blockIdx.x - slot * nblk;
  // the tile entry is read together with the tile count (slot - shared
  // slots < max_tiles for every block of the grid)
  int4 tl = reinterpret_cast<const int4*>(a.tiles)[max(slot - a.n_sh_slots, 0)];
  int n_tiles = *a.n_tiles;
  __asm__ volatile("" : "+s"(tl.x), "+s"(tl.y), "+s"(tl.z), "+s"(n_tiles));
  if (slot >= a.n_sh_slots + n_tiles) return;
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
    is_sh = false;
    e = tl.x;
    r_begin = tl.y;
    r_end = tl.z;
    U = a.U;
    K = a.K;
  }
  const int u0 = blk * M16Shape<MODE>::UPW * kM16Waves;
  if (u0 >= U) return;
  const int nt = r_end - r_begin;
  if (nt <= 0 || nt > mt || (!is_sh && (unsigned)e >= (unsigned)a.E)) {
    if (threadIdx.x == 0) atomicOr(a.err, 2);
    return;
  }
  // the 32-byte descriptor (two 16-byte loads) and the pair numbers of the
  // first staged rows are in flight together
  const u32x4_v* dp = reinterpret_cast<const u32x4_v*>(is_sh ? a.w_sh + e : a.w + e);
  u32x4_v d0 = ld_global(dp), d1 = ld_global(dp + 1);
  int srow[kM16StageIt], trow[kM16StageIt];   // activation rows of the first staging batch
  m16_row_loads<MODE>(a, r_begin, nt, K >> 5, srow, trow);
  __asm__ volatile("" : "+v"(d0), "+v"(d1));
  m16_row_finish<MODE>(a, is_sh, e, r_begin, srow, trow);
  // the descriptor is the same for the whole workgroup: scalar registers,
  // so the buffer resources built from it need no per-lane loop
  u32x4_v lo, hi;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)d0[i]);
    hi[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)d1[i]);
  }
  struct {
    u32x4_v lo, hi;
  } raw = {lo, hi};
  const moe_qmat q = __builtin_bit_cast(moe_qmat, raw);
  if (!qmat_usable(q, MODE == 0 ? 2 * U : U, K)) {
    if (threadIdx.x == 0) atomicOr(a.err, 1);
    return;
  }
  if (q.bits == 4 && q.group >= 128)
    m16_tile<MODE, ACT, 4, true, QX, PART>(a, q, is_sh, e, r_begin, nt, U, K, u0, mt, srow, smem);
  else if (q.bits == 4)
    m16_tile<MODE, ACT, 4, false, QX, PART>(a, q, is_sh, e, r_begin, nt, U, K, u0, mt, srow, smem);
  else
    m16_tile<MODE, ACT, 2, false, QX, PART>(a, q, is_sh, e, r_begin, nt, U, K, u0, mt, srow, smem);
}

int m16_rows(int T) { return T < kM16MaxRows ? T : kM16MaxRows; }

size_t m16_lds(int act, int mode, int T, int K, int K_sh) {
  const int Kl = K > K_sh ? K : K_sh;
  const size_t x = (size_t)m16_rows(T) * (act == MOE_A16 ? 2 * Kl + 16 : Kl + 8);
  const size_t aux = act == MOE_A16 ? (size_t)2 * kM16MaxRows * (Kl / 32) * 4
                                    : (size_t)2 * kM16MaxRows * 4;
  const size_t rows = mode == 0 ? 2 * M16Rows<0>::kBlock : M16Rows<1>::kBlock;
  return x + aux + rows * (Kl / 32) * 2;
}

bool m16_quant_ok(int mode, int T, int K, int K_sh) {
  // down: every workgroup of a tile would quantize the same fp32 h rows
  // (a division per element); the row quantizer launch measured faster
  if (mode != 0) return false;
  const int Kl = K > K_sh ? K : K_sh;
  const int it = mode == 0 ? M16QRegs<0>::kIt : M16QRegs<1>::kIt;
  return (long long)m16_rows(T) * (Kl / 32) <= (long long)kM16Threads * it;
}

bool m16_ok(int act, int mode, int T, int K, int K_sh, int tile_m) {
  return T > 0 && tile_m <= kM16MaxRows && m16_lds(act, mode, T, K, K_sh) <= 160 * 1024;
}

hipError_t launch_proj_m16(const ProjArgs& a_in, int act, hipStream_t st) {
  ProjArgs a = a_in;
  a.sh_tile = kM16MaxRows;
  a.n_sh_slots = a.n_shared * ((a.T + kM16MaxRows - 1) / kM16MaxRows);
  const int upwg = (a.mode == 0 ? M16Shape<0>::UPW : M16Shape<1>::UPW) * kM16Waves;
  const int umax = a.n_shared > 0 && a.U_sh > a.U ? a.U_sh : a.U;
  const int nblk = (umax + upwg - 1) / upwg;
  const long long grid = (long long)(a.n_sh_slots + a.max_tiles) * nblk;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int mt = m16_rows(a.T);
  const size_t lds = m16_lds(act, a.mode, a.T, a.K, a.K_sh);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  // A8 with int8 rows made in the kernel when a.in_q is null
  const bool qx = act == MOE_A8 && a.in_q == nullptr;
  if (qx && !m16_quant_ok(a.mode, a.T, a.K, a.K_sh)) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(kM16Threads);
  // A8 test hook: the same kernels, also storing the exact group sums
  const bool part = act == MOE_A8 && a.partials != nullptr;
  if (a.mode == 0) {
    if (act == MOE_A16) proj_m16_kernel<0, MOE_A16, false, false><<<g, b, lds, st>>>(a, mt, nblk);
    else if (qx && part) proj_m16_kernel<0, MOE_A8, true, true><<<g, b, lds, st>>>(a, mt, nblk);
    else if (qx) proj_m16_kernel<0, MOE_A8, true, false><<<g, b, lds, st>>>(a, mt, nblk);
    else if (part) proj_m16_kernel<0, MOE_A8, false, true><<<g, b, lds, st>>>(a, mt, nblk);
    else proj_m16_kernel<0, MOE_A8, false, false><<<g, b, lds, st>>>(a, mt, nblk);
  } else {
    if (act == MOE_A16) proj_m16_kernel<1, MOE_A16, false, false><<<g, b, lds, st>>>(a, mt, nblk);
    else if (qx && part) proj_m16_kernel<1, MOE_A8, true, true><<<g, b, lds, st>>>(a, mt, nblk);
    else if (qx) proj_m16_kernel<1, MOE_A8, true, false><<<g, b, lds, st>>>(a, mt, nblk);
    else if (part) proj_m16_kernel<1, MOE_A8, false, true><<<g, b, lds, st>>>(a, mt, nblk);
    else proj_m16_kernel<1, MOE_A8, false, false><<<g, b, lds, st>>>(a, mt, nblk);
  }
  return hipGetLastError();
}

}  // namespace moe
