// Grouped expert GEMMs for prefill shapes on the CDNA4 matrix cores, two
// waves per SIMD.
//
// Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", sections "Keep
// low-bit weights packed, do the work on the NPU" (grouped expert
// projections on the matrix unit, fused gate/up, routing and tile reuse, a
// weight layout made for the matrix unit, no expanded expert bank) and
// "GLM is my next, harder model" (a blocked-dequant matrix kernel over a
// mixed int2/int4 expert bank).  With ~128 tokens per expert the work is a
// dense contraction on v_mfma_f32_32x32x16_f16:
//
//  * workgroup = one tile chunk (up to 160 sorted rows of one expert) x 128
//    gate/up units (256 weight rows) or 256 down rows; 8 waves, two per
//    SIMD, so one wave's waits (LDS, memory, the step barrier) are covered
//    by the other's matrix work.  Wave w owns 32 weight rows: for gate/up
//    the gate rows of 16 units and the up rows of the same units (SiLU*mul
//    pairs them through LDS in the epilogue), for down 32 output
//    rows; every wave owns all of the chunk's activation rows (up to 5 x 1
//    accumulator tiles of 32x32: 80 accumulation registers);
//  * the K loop walks 64 K per step, four 16-K MFMA sub-steps.  A
//    (activations, fp16, in the K order of the unpack) is staged through a
//    double-buffered LDS tile [row][8 x 16-byte chunks], chunk c of row m at
//    slot c ^ ((m >> 1) & 7): a 128-bit LDS access is served 16 lanes at a
//    time, and 16 consecutive rows' chunk c then cover the 64 banks once;
//  * weights go from HBM straight into registers (16 bytes (int4) or 8
//    bytes (int2) per lane and step, four steps ahead) and are dequantized
//    there: a code field OR-ed into the mantissa of an fp16 power of two
//    reads as that power plus the field, a packed subtract gives the exact
//    code, a packed multiply the fp16 scale (one rounding).  An int2 word's
//    bytes are reordered (0, 2, 1, 3) first, so int2 codes unpack in the
//    same K order as int4 and one fp16 copy of x serves both;
//  * canonical layout: lane (row c, half h) of a 32-row block reads bytes
//    [32 s + 16 h, +16) (int4; int2 [16 s + 8 h, +8)) of its row at step s;
//    prepacked layout (moe_w4_prepack): those 16 (8) bytes of the 64 lanes
//    stored contiguously per block and step, so a wave's step is one 1 KB
//    (512 B) coalesced load, with the int2 byte order applied once;
//  * workgroups of one tile land on one XCD (blockIdx mod 8 picks the
//    XCD), so the tile's activation rows are shared in that XCD's L2.
#include "moe_internal.h"

namespace moe {

namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_v;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_v;
typedef __attribute__((ext_vector_type(16))) float f32x16_v;
typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_v __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;       // 8 waves, two per SIMD
constexpr int kUnits = 128;         // gate/up units per workgroup (shared-expert tile rows too)
constexpr int kRowsMax = 160;       // activation rows per tile chunk (5 row blocks of 32)
constexpr int kRing = 4;            // steps in flight
constexpr int kKS = 64;             // K per step
constexpr int kChunks = kKS / 8;    // 16-byte fp16 chunks per row and step
constexpr int kXcd = 8;

__device__ __forceinline__ f16x2_v as_h2(uint32_t v) { return __builtin_bit_cast(f16x2_v, v); }

// Exact unpack of one pair of codes (one per 16-bit half of w, BITS wide at
// bit offset OFS < 10), times the fp16 scale pair s2: the field OR-ed into
// fp16 2^(10 - OFS) with its top bit flipped reads 2^(10 - OFS) + code + 8
// (int2: + 2); one packed subtract leaves the code, one packed multiply
// scales it.
template <int OFS, int BITS>
__device__ __forceinline__ f16x2_v unpack_pair(uint32_t w, f16x2_v s2) {
  constexpr uint32_t field = (BITS == 4 ? 0xFu : 0x3u) << OFS;
  constexpr uint32_t flip = (BITS == 4 ? 0x8u : 0x2u) << OFS;
  constexpr uint32_t pow2 = (uint32_t)(25 - OFS) << 10;
  constexpr uint32_t mask = field * 0x10001u;
  constexpr uint32_t c = (flip | pow2) * 0x10001u;
  constexpr float bias_f = (float)(1 << (10 - OFS)) + (BITS == 4 ? 8.0f : 2.0f);
  const f16x2_v bias = {(_Float16)bias_f, (_Float16)bias_f};
  return (as_h2((w & mask) ^ c) - bias) * s2;
}

__device__ __forceinline__ void put_pair(f16x8_v& r, int i, f16x2_v p) {
  r[2 * i] = p.x;
  r[2 * i + 1] = p.y;
}

// 8 int4 codes (K order k0..k7 at bits 4k) -> fragment in the order
// k0,k4,k1,k5,k2,k6,k3,k7.
__device__ __forceinline__ f16x8_v deq_int4(uint32_t w, f16x2_v s2) {
  f16x8_v r;
  const uint32_t w8 = w >> 8;
  put_pair(r, 0, unpack_pair<0, 4>(w, s2));
  put_pair(r, 1, unpack_pair<4, 4>(w, s2));
  put_pair(r, 2, unpack_pair<0, 4>(w8, s2));
  put_pair(r, 3, unpack_pair<4, 4>(w8, s2));
  return r;
}

// int2 word with bytes reordered (0, 2, 1, 3): HALF 0 -> codes k0..k7, HALF
// 1 -> k8..k15, each in the order of deq_int4.
template <int HALF>
__device__ __forceinline__ f16x8_v deq_int2(uint32_t w, f16x2_v s2) {
  f16x8_v r;
  const uint32_t v = HALF ? w >> 8 : w;
  put_pair(r, 0, unpack_pair<0, 2>(v, s2));
  put_pair(r, 1, unpack_pair<2, 2>(v, s2));
  put_pair(r, 2, unpack_pair<4, 2>(v, s2));
  put_pair(r, 3, unpack_pair<6, 2>(v, s2));
  return r;
}

__device__ __forceinline__ uint32_t int2_order(uint32_t w) {
  return __builtin_amdgcn_perm(w, w, 0x03010200u);   // bytes 0, 2, 1, 3
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

struct Tile {
  const uint16_t* asrc;   // fp16 activations in the unpack's K order
  uint32_t a_bytes;       // bytes of asrc the tile may address
  const uint8_t* codes;
  const uint16_t* scales;
  int K, U, group, u0, e, r_begin, r_end;
  bool is_sh;
};

// This lane's weight row, its code buffer descriptor and its scales in LDS.
struct Lane {
  __amdgpu_buffer_rsrc_t crs;
  int coff;                // byte offset of step 0 (+ step * stride)
  int cstride;             // bytes per step
  const uint16_t* sc;      // LDS: this lane's row of group scales
  int wrow;                // weight row (gate/up: unit of the lane's column)
  bool wval;
  int n_st, gsh;
};

template <int BITS>
struct BReg {
  uint32_t c[BITS];        // 16 (int4) or 8 (int2) bytes
};

template <int MB>
struct AReg {
  u32x4_v a[(MB * 32 * kChunks + kThreads - 1) / kThreads];
};

// K loop and epilogue of one chunk of up to 32 * MB rows (tok[] holds
// their activation rows).  Straight-line loop body, every load
// unconditional (steps past the end re-read the last step with a zero
// scale), so the wait counts stay graded.
template <int MODE, int BITS, int MB, bool PP>
__device__ __forceinline__ void chunk(const ProjArgs& a, const Tile& t, const Lane& ln_,
                                      u32x4_v* As, const int* tok, int mc, int nrows) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int lc = lane & 31, kh = lane >> 5;
  const int n_st = ln_.n_st;
  constexpr int kAN = (MB * 32 * kChunks + kThreads - 1) / kThreads;   // A chunks per thread
  constexpr int kAChunks = MB * 32 * kChunks;

  auto load_b = [&](int st, BReg<BITS>& b) {
    st = min(st, n_st - 1);
    if constexpr (BITS == 4) {
      const u32x4_v v =
          __builtin_amdgcn_raw_buffer_load_b128(ln_.crs, ln_.coff, st * ln_.cstride, 0);
      b.c[0] = v.x; b.c[1] = v.y; b.c[2] = v.z; b.c[3] = v.w;
    } else {
      const u32x2_v v =
          __builtin_amdgcn_raw_buffer_load_b64(ln_.crs, ln_.coff, st * ln_.cstride, 0);
      b.c[0] = PP ? v.x : int2_order(v.x);
      b.c[1] = PP ? v.y : int2_order(v.y);
    }
  };
  // A staging: chunk q = tid + kThreads * i (row q >> 3, chunk q & 7); a
  // thread past the chunk count re-reads a valid chunk and stores nothing
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(t.asrc, t.a_bytes);
  int aoff[kAN], adst[kAN];
#pragma unroll
  for (int i = 0; i < kAN; ++i) {
    const int q = tid + kThreads * i;
    const int qq = q < kAChunks ? q : tid;
    const int m = qq >> 3, ci = qq & 7;
    aoff[i] = tok[m] * a.ld_in * 2 + ci * 16;
    adst[i] = q < kAChunks ? m * kChunks + (ci ^ ((m >> 1) & 7)) : -1;
  }
  auto load_a = [&](int st, AReg<MB>& ar) {
    const int o = min(st, n_st - 1) * (kKS * 2);
#pragma unroll
    for (int i = 0; i < kAN; ++i) ar.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ars, aoff[i], o, 0);
  };
  auto store_a = [&](int buf, const AReg<MB>& ar) {
    u32x4_v* d = As + buf * kChunks * kRowsMax;
#pragma unroll
    for (int i = 0; i < kAN; ++i)
      if (adst[i] >= 0) d[adst[i]] = ar.a[i];
  };

  f32x16_v acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[mb][j] = 0.0f;

  // fragment read offsets (16-byte units) of this lane's rows 32 mb + lc
  const int rsw = (lc >> 1) & 7;
  auto compute = [&](int buf, const BReg<BITS>& b, int stg) {
    const bool live = stg < n_st;
    const int gi = (min(stg, n_st - 1) * kKS + kh * 32) >> ln_.gsh;
    const uint32_t m16 = live ? 0x10001u : 0u;
    const f16x2_v s2 = as_h2((uint32_t)ln_.sc[gi] * m16);
    const u32x4_v* Ab = As + buf * kChunks * kRowsMax + lc * kChunks;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      f16x8_v bf;
      if constexpr (BITS == 4) {
        bf = deq_int4(b.c[ks], s2);
      } else {
        if ((ks & 1) == 0) bf = deq_int2<0>(b.c[ks >> 1], s2);
        else bf = deq_int2<1>(b.c[ks >> 1], s2);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const f16x8_v av =
            __builtin_bit_cast(f16x8_v, Ab[32 * kChunks * mb + ((kh * 4 + ks) ^ rsw)]);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bf, acc[mb], 0, 0, 0);
      }
    }
  };

  // weights kRing steps ahead in a register ring; activations two steps
  // ahead in two register slots (A of step k lives in slot k & 1): step s
  // computes from LDS buffer s & 1, writes A(s + 1) into the other buffer,
  // refills that slot with A(s + 3) and the weight slot with step s + 4
  AReg<MB> ar0, ar1;
  BReg<BITS> b0, b1, b2, b3;
  load_a(0, ar0); load_b(0, b0);
  load_a(1, ar1); load_b(1, b1);
  load_b(2, b2);
  load_b(3, b3);
  store_a(0, ar0);
  load_a(2, ar0);
  __syncthreads();
#define MOE8_STEP(J, AS, BC)                        \
  compute(J & 1, BC, base + J);                     \
  store_a((J + 1) & 1, AS);                         \
  load_a(base + J + 3, AS);                         \
  load_b(base + J + kRing, BC);                     \
  __syncthreads();
  for (int base = 0; base < n_st; base += kRing) {
    MOE8_STEP(0, ar1, b0)
    MOE8_STEP(1, ar0, b1)
    MOE8_STEP(2, ar1, b2)
    MOE8_STEP(3, ar0, b3)
  }
#undef MOE8_STEP

  // ---- epilogue: lane holds column lc (rows 32 mb + 8 (j >> 2) + 4 kh + (j & 3))
  const int orow0 = t.is_sh ? a.P + t.e * a.T + mc : mc;
  // gate/up: the gate of a unit sits in column c < 16, its up in column
  // c + 16 (lane + 16); the pairs meet through this wave's own 4 KB of the
  // A tile, free once every wave has passed the K loop's last barrier.
  // Lane L reads what lane L ^ 16 wrote, which the compiler cannot see as
  // a dependence: barriers order the writes, the reads and the next writes.
  float* xch = reinterpret_cast<float*>(As) + (threadIdx.x >> 6) * (16 * 64);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (MODE == 0) {
      if (mb > 0) __syncthreads();   // the previous row block's reads are done
#pragma unroll
      for (int j = 0; j < 16; ++j) xch[j * 64 + lane] = acc[mb][j];
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int m = 32 * mb + (j >> 2) * 8 + kh * 4 + (j & 3);
      if (MODE == 0) {
        const float up = xch[j * 64 + (lane ^ 16)];
        if (lc < 16 && m < nrows && ln_.wval) {
          const float hv = silu_mul(acc[mb][j], up);
          const uint32_t hb = f32_to_bf16(hv);
          const size_t o = (size_t)(orow0 + m) * a.ld_out;
          static_cast<uint16_t*>(a.out)[o + ln_.wrow] = (uint16_t)hb;
          if (a.out16) {
            // the down projection's fp16 input: the bf16 value (exact in
            // fp16's normal range) at its place in the unpack order of its
            // 8-block, (0,4)(1,5)(2,6)(3,7)
            const int u = ln_.wrow;
            const int pos = (u & ~7) | ((u & 3) << 1) | ((u >> 2) & 1);
            const uint32_t f16 = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(hb << 16), 0.0f));
            a.out16[o + pos] = (uint16_t)(f16 & 0xFFFFu);
          }
        }
      } else {
        if (m < nrows && ln_.wval)
          static_cast<float*>(a.out)[(size_t)(orow0 + m) * a.ld_out + ln_.wrow] = acc[mb][j];
      }
    }
  }
}

template <int MODE, int BITS, bool PP>
__device__ __forceinline__ void tile(const ProjArgs& a, const Tile& t, u32x4_v* As, int* tok,
                                     uint16_t* ssc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 31, kh = lane >> 5;
  const int K = t.K, U = t.U;
  const int ng = K / t.group;
  const int row_bytes = K * BITS / 8;
  const int n_wrows = MODE == 0 ? 2 * U : U;

  Lane L;
  L.n_st = K / kKS;
  int brow, lrow;   // this lane's weight row and its row in the staged scales
  if (MODE == 0) {
    const int unit = t.u0 + 16 * wave + (lc & 15);
    L.wval = unit < U;
    L.wrow = unit;
    brow = lc < 16 ? unit : U + unit;
    lrow = (lc < 16 ? 0 : kUnits) + 16 * wave + (lc & 15);
  } else {
    const int r = t.u0 + 32 * wave + lc;
    L.wval = r < U;
    L.wrow = r;
    brow = r;
    lrow = 32 * wave + lc;
  }
  L.crs = make_rsrc(t.codes, (uint32_t)((size_t)n_wrows * row_bytes));
  constexpr int kLaneBytes = kKS * BITS / 16;   // per lane half and step
  if (PP) {
    // block of 32 weight rows: gate/up block (u0 + 16 wave) / 16 pairs 16
    // gate and 16 up rows, down block (u0 + 32 wave) / 32
    const int blk = MODE == 0 ? t.u0 / 16 + wave : t.u0 / 32 + wave;
    L.cstride = 64 * kLaneBytes;
    L.coff = L.wval ? blk * L.n_st * L.cstride + lane * kLaneBytes : 0;
  } else {
    L.cstride = kKS * BITS / 8;
    L.coff = (L.wval ? brow : 0) * row_bytes + kh * kLaneBytes;
  }
  L.gsh = 31 - __builtin_clz(t.group);

  // ---- the group scales of the workgroup's weight rows into LDS, [local
  // row][group]: gate rows u0.. then up rows U+u0.. (gate/up), or down
  // rows u0..; contiguous runs of the scale matrix copied in 16-byte words
  // (runs start at multiples of 128 rows, so they are 16-byte aligned).
  {
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(t.scales, (uint32_t)(n_wrows * ng * 2));
    const int run_rows = MODE == 0 ? kUnits : min(2 * kUnits, U - t.u0);
    const int run_words = run_rows * ng * 2 / 16;
    const int n_runs = MODE == 0 ? 2 : 1;
    for (int q = tid; q < n_runs * run_words; q += kThreads) {
      const int run = q >= run_words, qq = q - run * run_words;
      const int row0 = run ? U + t.u0 : t.u0;
      const u32x4_v v =
          __builtin_amdgcn_raw_buffer_load_b128(srs, row0 * ng * 2 + qq * 16, 0, 0);
      reinterpret_cast<u32x4_v*>(ssc + (size_t)run * kUnits * ng)[qq] = v;
    }
  }
  L.sc = ssc + lrow * ng;

  for (int mc = t.r_begin; mc < t.r_end; mc += kRowsMax) {
    const int nrows = min(kRowsMax, t.r_end - mc);
    __syncthreads();   // previous chunk's readers of tok / As are done
    if (tid < kRowsMax) {
      const int mm = tid < nrows ? tid : 0;   // padding rows re-read row 0 (discarded)
      int r;
      if (MODE == 0) r = t.is_sh ? mc + mm : a.sorted_pair[mc + mm] / a.k;
      else r = t.is_sh ? a.P + t.e * a.T + mc + mm : mc + mm;
      tok[tid] = r;
    }
    __syncthreads();
    if (nrows > 128) chunk<MODE, BITS, 5, PP>(a, t, L, As, tok, mc, nrows);
    else if (nrows > 64) chunk<MODE, BITS, 4, PP>(a, t, L, As, tok, mc, nrows);
    else if (nrows > 32) chunk<MODE, BITS, 2, PP>(a, t, L, As, tok, mc, nrows);
    else chunk<MODE, BITS, 1, PP>(a, t, L, As, tok, mc, nrows);
  }
}

template <int MODE, bool PP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void proj_mfma8_kernel(ProjArgs a, const uint16_t* x16) {
  extern __shared__ __align__(16) unsigned char smem[];
  u32x4_v* As = reinterpret_cast<u32x4_v*>(smem);                        // [2][kRowsMax][kChunks]
  int* tok = reinterpret_cast<int*>(smem + 2 * kChunks * kRowsMax * 16);  // [kRowsMax]
  uint16_t* ssc = reinterpret_cast<uint16_t*>(tok + kRowsMax);             // [256][K / group]
  const int tid = threadIdx.x;

  // block -> (tile slot, unit block): XCD b mod 8 takes a contiguous range
  // of the device-side slots, so the blocks of one tile (they share its
  // activation rows) and the tiles of one expert (its weights) meet in one L2
  const int b = blockIdx.x;
  const int xcd = b % kXcd, li = b / kXcd;
  const int nb = li % a.n_rb;
  const int n_slots = a.n_sh_slots + min(*a.n_tiles, a.max_tiles);
  const int per_xcd = (n_slots + kXcd - 1) / kXcd;
  const int local = li / a.n_rb;
  if (local >= per_xcd) return;
  const int slot = xcd * per_xcd + local;
  if (slot >= n_slots) return;
  Tile t;
  if (slot < a.n_sh_slots) {
    const int per = (a.T + a.sh_tile - 1) / a.sh_tile;
    const int s = slot / per, ti = slot - s * per;
    t.is_sh = true;
    t.e = s;
    t.r_begin = ti * a.sh_tile;
    t.r_end = min(a.T, t.r_begin + a.sh_tile);
  } else {
    const int j = slot - a.n_sh_slots;
    if (j >= a.max_tiles) return;
    const int4 tl = reinterpret_cast<const int4*>(a.tiles)[j];
    if (j >= *a.n_tiles) return;
    if ((unsigned)tl.x >= (unsigned)a.E) {
      if (tid == 0) atomicOr(a.err, 2);
      return;
    }
    t.is_sh = false;
    t.e = tl.x;
    t.r_begin = tl.y;
    t.r_end = tl.z;
  }
  t.K = t.is_sh ? a.K_sh : a.K;
  t.U = t.is_sh ? a.U_sh : a.U;
  t.u0 = nb * (MODE == 0 ? kUnits : 2 * kUnits);
  if (t.u0 >= t.U) return;
  const moe_qmat q = t.is_sh ? a.w_sh[t.e] : a.w[t.e];
  if (!qmat_usable(q, MODE == 0 ? 2 * t.U : t.U, t.K) || t.K % (2 * kKS) != 0) {
    if (tid == 0) atomicOr(a.err, 1);
    return;
  }
  t.codes = q.codes;
  t.scales = q.scales;
  t.group = q.group;
  // rows the activation source holds: T token rows, or every h row
  t.a_bytes = (uint32_t)((size_t)(MODE == 0 ? a.T : a.P + a.n_shared * a.T) * a.ld_in * 2);
  t.asrc = MODE == 0 ? x16 : a.in_bf16;
  if (q.bits == 4) tile<MODE, 4, PP>(a, t, As, tok, ssc);
  else tile<MODE, 2, PP>(a, t, As, tok, ssc);
}

// fp16 copy of bf16 rows, every 8-block in the order (0,4)(1,5)(2,6)(3,7)
// (the unpack order of int4, and of int2 after its byte reorder).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t lo_bf16, uint32_t hi_bf16) {
  const float x0 = __uint_as_float(lo_bf16 << 16);
  const float x1 = __uint_as_float(hi_bf16 << 16);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0, x1));
}
__device__ __forceinline__ uint4 convert8(uint4 v) {
  const uint32_t e[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                         v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
  return make_uint4(bf16x2_to_f16x2(e[0], e[4]), bf16x2_to_f16x2(e[1], e[5]),
                    bf16x2_to_f16x2(e[2], e[6]), bf16x2_to_f16x2(e[3], e[7]));
}

// rows [R][ld] bf16 -> fp16 in the unpack order: the first K columns of
// every row (K % 8 == 0), one 8-block per thread.
__global__ __launch_bounds__(256) void convert8_kernel(const uint16_t* __restrict__ src,
                                                       long long R, int K, int ld,
                                                       uint16_t* __restrict__ dst) {
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  const int upr = K / 8;
  if (u >= R * upr) return;
  const long long r = u / upr;
  const int c = (int)(u - r * upr);
  const size_t o = (size_t)r * ld + (size_t)c * 8;
  reinterpret_cast<uint4*>(dst + o)[0] = convert8(reinterpret_cast<const uint4*>(src + o)[0]);
}

}  // namespace

bool mfma_available() { return true; }

hipError_t launch_proj_mfma8(const ProjArgs& a_in, uint16_t* a16, bool prepacked,
                             hipStream_t st) {
  ProjArgs a = a_in;
  a.sh_tile = kUnits;
  a.n_sh_slots = a.n_shared * ((a.T + kUnits - 1) / kUnits);
  const int Umax = a.U > a.U_sh ? a.U : a.U_sh;
  a.n_rb = a.mode == 0 ? (Umax + kUnits - 1) / kUnits : (a.U + 2 * kUnits - 1) / (2 * kUnits);
  const long long slots = (long long)a.n_sh_slots + a.max_tiles;
  const long long groups = (slots + kXcd - 1) / kXcd;
  const long long blocks = groups * kXcd * a.n_rb;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  // one fp16 copy of the activations in the unpack's K order
  if (a.mode == 0) {
    const long long units = (long long)a.T * (a.K / 8);
    convert8_kernel<<<(unsigned)((units + 255) / 256), 256, 0, st>>>(a.in_bf16, a.T, a.K,
                                                                     a.K, a16);
  } else if (!a.in16_ready) {
    const long long R = (long long)a.P + (long long)a.n_shared * a.T;
    const int Kc = a.K_sh > a.K ? a.K_sh : a.K;
    const long long units = R * (Kc / 8);
    convert8_kernel<<<(unsigned)((units + 255) / 256), 256, 0, st>>>(a.in_bf16, R, Kc,
                                                                     a.ld_in, a16);
    a.in_bf16 = a16;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int Kmax = a.K_sh > a.K ? a.K_sh : a.K;
  const size_t lds = (size_t)2 * kChunks * kRowsMax * 16 + kRowsMax * sizeof(int) +
                     (size_t)2 * kUnits * (Kmax / 32) * 2;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const dim3 g((unsigned)blocks), blk(kThreads);
  if (a.mode == 0) {
    if (prepacked) proj_mfma8_kernel<0, true><<<g, blk, lds, st>>>(a, a16);
    else proj_mfma8_kernel<0, false><<<g, blk, lds, st>>>(a, a16);
  } else {
    if (prepacked) proj_mfma8_kernel<1, true><<<g, blk, lds, st>>>(a, nullptr);
    else proj_mfma8_kernel<1, false><<<g, blk, lds, st>>>(a, nullptr);
  }
  return hipGetLastError();
}

}  // namespace moe

namespace moe {
namespace {

// One 16-byte (int4) or 8-byte (int2) unit of the prepacked layout per
// thread: unit u = (block, step, lane); lane = half * 32 + column; the
// column's row is 16 gate rows then the same 16 up rows (gate_up) or 32
// consecutive rows; the unit holds bytes [step * 32 + half * 16, +16) of
// that row (int2: [step * 16 + half * 8, +8), each 4-byte word's bytes
// reordered (0, 2, 1, 3)).
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t* __restrict__ src, int bits,
                                                      int N, int K, int gate_up,
                                                      uint8_t* __restrict__ dst) {
  const int n_st = K / kKS;
  const long long units = (long long)(N / 32) * n_st * 64;
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int lane = (int)(u & 63);
  const long long bs = u >> 6;
  const int st = (int)(bs % n_st);
  const int blk = (int)(bs / n_st);
  const int c = lane & 31, half = lane >> 5;
  const int row = gate_up ? (c < 16 ? 16 * blk + c : N / 2 + 16 * blk + c - 16) : 32 * blk + c;
  const size_t row_bytes = (size_t)K * bits / 8;
  if (bits == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + row * row_bytes + st * 32 + half * 16);
    reinterpret_cast<uint4*>(dst)[u] = v;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(src + row * row_bytes + st * 16 + half * 8);
    reinterpret_cast<uint2*>(dst)[u] = make_uint2(int2_order(v.x), int2_order(v.y));
  }
}

}  // namespace

hipError_t launch_prepack(const uint8_t* src, int bits, int N, int K, int gate_up, uint8_t* dst,
                          hipStream_t st) {
  const long long units = (long long)(N / 32) * (K / kKS) * 64;
  if (units <= 0) return hipSuccess;
  prepack_kernel<<<(unsigned)((units + 255) / 256), 256, 0, st>>>(src, bits, N, K, gate_up, dst);
  return hipGetLastError();
}

}  // namespace moe
