// Grouped expert GEMMs for prefill shapes on the CDNA4 matrix cores.
//
// Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", sections "Keep
// low-bit weights packed, do the work on the NPU" (grouped expert
// projections on the matrix unit, fused gate/up, routing and tile reuse,
// no expanded expert bank) and "GLM is my next, harder model" (a
// blocked-dequant matrix kernel over a mixed int2/int4 expert bank).  With
// ~128 tokens per expert the work is a dense contraction, so it runs on
// v_mfma_f32_32x32x16_f16:
//
//  * workgroup = one tile chunk (up to 128 sorted rows of one expert) x
//    one block of output units: 128 gate/up row pairs (fused SiLU*mul
//    epilogue: gate and up accumulators of a unit sit in the same lane) or
//    256 down rows; 4 waves, one per SIMD, each owning all 128 activation
//    rows x 64 weight rows (4 x 2 accumulator tiles of 32x32), so every
//    dequantized weight fragment feeds four MFMAs;
//  * the K loop walks 64 K per step.  A (activations) comes from an fp16
//    copy made once per call in the K order of the weight unpack, so a
//    step's A tile is a plain copy: each thread holds its share of the
//    next steps in a four-slot register ring (8 lanes fetch one whole
//    128-byte row slice) and writes one step into a double-buffered LDS
//    tile laid out [row][16-byte K chunk] with an XOR swizzle of the chunk
//    slot by the row, so LDS writes and MFMA fragment reads are both free
//    of bank conflicts;
//  * packed weights go from HBM straight into registers (16 bytes (int4)
//    or 8 bytes (int2) per lane, row and step, four steps ahead) and are
//    dequantized there, never in LDS or HBM: a code field OR-ed into the
//    mantissa of a suitable fp16 power of two reads as that power plus
//    the field, a packed fp16 subtract gives the exact code, a packed fp16
//    multiply applies the fp16 group scale (one rounding to fp16, relative
//    error <= 2^-11);
//  * the K order inside each MFMA step is permuted the same way on both
//    operands (a contraction does not depend on the order of K);
//  * int4 and int2 experts mix freely: a tile takes its expert's format;
//  * workgroups of one tile land on one XCD (blockIdx mod 8 picks the
//    XCD), so the tile's activation rows are shared in that XCD's L2.
#include "moe_internal.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_v;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_v;
typedef __attribute__((ext_vector_type(16))) float f32x16_v;
typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_v __attribute__((ext_vector_type(2)));

constexpr int kMThreads = 256;    // 4 waves, one per SIMD
constexpr int kBM = 128;            // weight units per workgroup (gate/up), shared-expert tile rows
constexpr int kRowsMax = 160;       // activation rows per tile chunk (5 row blocks of 32)
constexpr int kRing = 4;            // steps in flight (register ring slots)
constexpr int kKS = 64;             // K per pipeline step
constexpr int kChunks = kKS / 8;    // 16-byte fp16 chunks per row and step
constexpr int kXcd = 8;

bool mfma_available() { return true; }

__device__ __forceinline__ f16x2_v as_h2(uint32_t v) { return __builtin_bit_cast(f16x2_v, v); }

// fp16 pair from two bf16 values (exact in fp16's normal range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t lo_bf16, uint32_t hi_bf16) {
  const float a = __uint_as_float(lo_bf16 << 16);
  const float b = __uint_as_float(hi_bf16 << 16);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// Shift-free exact unpack of one pair of codes (one per 16-bit half of
// w, BITS wide at bit offset OFS < 10).  OR-ed into the fp16 power of two
// 2^(10 - OFS), the field lands in the mantissa where its unit is worth
// exactly 1, so the half reads 2^(10 - OFS) + field.  With the field's top
// bit flipped (offset binary: code + 8 for int4, + 2 for int2) a packed
// fp16 subtract of 2^(10 - OFS) + 8 (or + 2) leaves the signed code
// exactly, and a packed fp16 multiply applies the group scale with one
// rounding.  Mask, flip and OR fold into one three-input bit operation.
template <int OFS, int BITS>
__device__ __forceinline__ f16x2_v unpack_pair(uint32_t w, f16x2_v s2) {
  constexpr uint32_t field = (BITS == 4 ? 0xFu : 0x3u) << OFS;
  constexpr uint32_t flip = (BITS == 4 ? 0x8u : 0x2u) << OFS;
  constexpr uint32_t pow2 = (uint32_t)(25 - OFS) << 10;   // fp16 bits of 2^(10 - OFS)
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

// One int4 code word (8 codes, K order k0..k7 at bits 4k) -> MFMA
// fragment of 8 fp16 in the order k0,k4,k1,k5,k2,k6,k3,k7, each = code *
// scale.
__device__ __forceinline__ f16x8_v deq_int4(uint32_t w, f16x2_v s2) {
  f16x8_v r;
  const uint32_t w8 = w >> 8;
  put_pair(r, 0, unpack_pair<0, 4>(w, s2));
  put_pair(r, 1, unpack_pair<4, 4>(w, s2));
  put_pair(r, 2, unpack_pair<0, 4>(w8, s2));
  put_pair(r, 3, unpack_pair<4, 4>(w8, s2));
  return r;
}
// One int2 code word (16 codes k0..k15 at bits 2k) -> fragment HALF (0:
// pairs (k0,k8)..(k3,k11); 1: pairs (k4,k12)..(k7,k15)).
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

// ---------------------------------------------------------------------
// fp16 copy of bf16 rows in the K order of the weight unpack:
// perm 4: every 8-block as (0,4)(1,5)(2,6)(3,7); perm 2: every 16-block
// as (0,8)(1,9)..(7,15).  One 16-element unit per thread.
__device__ __forceinline__ void convert_unit(const uint16_t* src, uint16_t* dst, int perm) {
  const uint4 lo = reinterpret_cast<const uint4*>(src)[0];
  const uint4 hi = reinterpret_cast<const uint4*>(src)[1];
  const uint32_t v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  auto bf = [&](int j) -> uint32_t { return (v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu; };
  uint32_t o[8];
  if (perm == 4) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int p = 0; p < 4; ++p) o[4 * blk + p] = bf16x2_to_f16x2(bf(8 * blk + p), bf(8 * blk + p + 4));
  } else {
#pragma unroll
    for (int p = 0; p < 8; ++p) o[p] = bf16x2_to_f16x2(bf(p), bf(p + 8));
  }
  reinterpret_cast<uint4*>(dst)[0] = make_uint4(o[0], o[1], o[2], o[3]);
  reinterpret_cast<uint4*>(dst)[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// x [T][H] -> x16_4 and x16_2 [T][H].
__global__ __launch_bounds__(256) void convert_x_kernel(const uint16_t* __restrict__ x, int T,
                                                         int H, uint16_t* __restrict__ x4,
                                                         uint16_t* __restrict__ x2) {
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long upr = H / 16;
  if (u >= (long long)T * upr) return;
  const long long t = u / upr, c = u - t * upr;
  const size_t o = (size_t)t * H + c * 16;
  convert_unit(x + o, x4 + o, 4);
  convert_unit(x + o, x2 + o, 2);
}

// h rows -> h16 rows permuted for the bit width of the row's down matrix.
// One wave per row; rows of a routed tile belong to its expert, rows past
// T*k to the shared experts.
__global__ __launch_bounds__(256) void convert_h_kernel(ProjArgs a, uint16_t* __restrict__ h16) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int R = a.P + a.n_shared * a.T;
  if (row >= R) return;
  int bits = 4, K = a.K;
  if (row < a.P) {
    // expert of sorted row `row`: the last e with offsets[e] <= row
    int lo = 0, hi = a.E;   // offsets has E+1 entries
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.offsets[mid] <= row) lo = mid; else hi = mid;
    }
    bits = a.w[lo].bits;
  } else {
    const int s = (row - a.P) / a.T;
    bits = a.w_sh[s].bits;
    K = a.K_sh;
  }
  const int perm = bits == 2 ? 2 : 4;
  const uint16_t* src = a.in_bf16 + (size_t)row * a.ld_in;
  uint16_t* dst = h16 + (size_t)row * a.ld_in;
  for (int c = lane; c < K / 16; c += 64) convert_unit(src + c * 16, dst + c * 16, perm);
}

// 32-bit buffer descriptor over [p, p + bytes) (bytes < 2^31): loads
// take a per-lane 32-bit offset plus a wave-uniform one, and out-of-range
// offsets read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

template <int MB>
struct AStep {
  u32x4_v a[MB];   // this thread's 16-byte A chunks of one step
};

template <int BITS>
struct BStep {
  uint32_t c[2][BITS];   // code words of the two weight rows (16 or 8 bytes each)
};

// Where one workgroup works: a tile chunk of sorted rows of one matrix.
struct TileCtx {
  const uint16_t* asrc;   // fp16 activations in the unpack's K order
  uint32_t a_bytes;       // bytes of asrc the tile may address
  const uint8_t* codes;
  const uint16_t* scales;
  int K, U, group, u0, e, r_begin, r_end;
  bool is_sh;
};

// This lane's weight rows, their code buffer descriptor and their group
// scales, staged in LDS once per tile.
struct WeightCtx {
  __amdgpu_buffer_rsrc_t crs;
  int coff[2];
  const uint16_t* sc[2];   // LDS: this lane's two rows of group scales
  int wrow[2];
  bool wval[2];
  int n_st, gsh;           // steps, log2(group)
};

// K loop and epilogue of one chunk of up to 32 * MB rows (tok[] holds
// their activation rows).  The loop body is straight-line code (format
// and row blocks fixed, no data-dependent branches, every load
// unconditional) so that the compiler's counters let the loads of the
// next kRing steps stay in flight while the matrix cores work on the
// current one.
template <int MODE, int BITS, int MB>
__device__ __forceinline__ void mfma_chunk(const ProjArgs& a, const TileCtx& c,
                                           const WeightCtx& w, u32x4_v* As, const int* tok,
                                           int mc, int nrows) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int ln = lane & 31, kh = lane >> 5;
  const int n_st = w.n_st;
  constexpr int kStepBytes = kKS * BITS / 8;   // 32 (int4) or 16 (int2)

  auto load_b = [&](int st, BStep<BITS>& b) {
    st = min(st, n_st - 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (BITS == 4) {
        const u32x4_v t =
            __builtin_amdgcn_raw_buffer_load_b128(w.crs, w.coff[s], st * kStepBytes, 0);
        b.c[s][0] = t.x; b.c[s][1] = t.y; b.c[s][2] = t.z; b.c[s][3] = t.w;
      } else {
        const u32x2_v t =
            __builtin_amdgcn_raw_buffer_load_b64(w.crs, w.coff[s], st * kStepBytes, 0);
        b.c[s][0] = t.x; b.c[s][1] = t.y;
      }
    }
  };
  // A staging: 32 * MB rows x 128 bytes per step, LDS laid out [row m][8
  // 16-byte K chunks] with chunk ci of row m stored at slot ci ^ ((m >> 1)
  // & 7).  A 128-bit LDS access is served 16 lanes (256 bytes, the 64
  // banks) at a time: the fragment read of 16 consecutive rows' chunk ci
  // then covers every bank once (even rows take the lower 128 bytes of the
  // bank space, odd rows the upper, and within a parity the 8 rows have 8
  // distinct slots); with ci ^ (m & 7), rows m and m + 8 collided.  Thread tid
  // moves chunk tid & 7 of rows (tid >> 3) + 32 i (i < MB): 8 lanes read
  // one whole 128-byte line from memory.
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(c.asrc, c.a_bytes);
  const int ci_own = tid & 7, m_own = tid >> 3;
  int aoff[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) aoff[i] = tok[m_own + 32 * i] * a.ld_in * 2 + ci_own * 16;
  auto load_a = [&](int st, AStep<MB>& ar) {
    const int o = min(st, n_st - 1) * (kKS * 2);
#pragma unroll
    for (int i = 0; i < MB; ++i) ar.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ars, aoff[i], o, 0);
  };
  auto store_a = [&](int buf, const AStep<MB>& ar) {
    u32x4_v* d = As + buf * kChunks * kRowsMax + m_own * kChunks + (ci_own ^ ((m_own >> 1) & 7));
#pragma unroll
    for (int i = 0; i < MB; ++i) d[32 * kChunks * i] = ar.a[i];
  };

  f32x16_v acc[2][MB];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[s][mb][j] = 0.0f;

  // steps past the last one (the loop runs whole trips of kRing steps)
  // re-read the last step with a zero scale: they add exact zeros
  auto compute = [&](int buf, const BStep<BITS>& b, int stg) {
    const bool live = stg < n_st;
    // group scales of this step (64 stg + 32 kh lies in group (..) >> gsh)
    const int gi = (min(stg, n_st - 1) * kKS + kh * 32) >> w.gsh;
    const uint32_t sc0 = w.sc[0][gi], sc1 = w.sc[1][gi];
    const u32x4_v* Ab = As + buf * kChunks * kRowsMax + ln * kChunks;
    // the whole step's A fragments first: one LDS round trip per step
    u32x4_v af[4][MB];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[st][mb] = Ab[32 * kChunks * mb + ((kh * 4 + st) ^ ((ln >> 1) & 7))];
    const uint32_t m16 = live ? 0x10001u : 0u;
    const f16x2_v s0 = as_h2(sc0 * m16);
    const f16x2_v s1 = as_h2(sc1 * m16);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      f16x8_v b0, b1;
      if constexpr (BITS == 4) {
        b0 = deq_int4(b.c[0][st], s0);
        b1 = deq_int4(b.c[1][st], s1);
      } else {
        if ((st & 1) == 0) {
          b0 = deq_int2<0>(b.c[0][st >> 1], s0);
          b1 = deq_int2<0>(b.c[1][st >> 1], s1);
        } else {
          b0 = deq_int2<1>(b.c[0][st >> 1], s0);
          b1 = deq_int2<1>(b.c[1][st >> 1], s1);
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const f16x8_v av = __builtin_bit_cast(f16x8_v, af[st][mb]);
        acc[0][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, b0, acc[0][mb], 0, 0, 0);
        acc[1][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, b1, acc[1][mb], 0, 0, 0);
      }
    }
    // Issue order for the step: the A fragments of the first two
    // sub-steps, the unpack of sub-step 0, then each MFMA followed by a
    // share of the next sub-step's unpack (one wave per SIMD, so the
    // VALU work has to run in the shadow of its own MFMAs) and the LDS
    // reads of the sub-step after next.
    constexpr int kMfmaPerSub = 2 * MB;
    constexpr int kValuPerSub = 26;
    constexpr int kValuPerMfma = (kValuPerSub + kMfmaPerSub - 1) / kMfmaPerSub;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * MB, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValuPerSub, 0);
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
#pragma unroll
      for (int i = 0; i < kMfmaPerSub; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
        if (sub < 2 && i < MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };

  // ---- K loop over a ring of kRing register slots: step s computes
  // from LDS buffer s & 1 and weight slot s % kRing, writes the
  // activations of step s + 1 (loaded three steps earlier) into the
  // other LDS buffer, then refills slot s % kRing with step s + kRing.
  AStep<MB> ar0, ar1, ar2, ar3;
  BStep<BITS> b0, b1, b2, b3;
  load_a(0, ar0); load_b(0, b0);
  load_a(1, ar1); load_b(1, b1);
  load_a(2, ar2); load_b(2, b2);
  load_a(3, ar3); load_b(3, b3);
  store_a(0, ar0);
  __syncthreads();
#define MOE_STEP(J, AC, BC, AN)                     \
  compute(J & 1, BC, base + J);                     \
  store_a((J + 1) & 1, AN);                         \
  load_a(base + J + kRing, AC);                     \
  load_b(base + J + kRing, BC);                     \
  __syncthreads();
  for (int base = 0; base < n_st; base += kRing) {
    MOE_STEP(0, ar0, b0, ar1)
    MOE_STEP(1, ar1, b1, ar2)
    MOE_STEP(2, ar2, b2, ar3)
    MOE_STEP(3, ar3, b3, ar0)
  }
#undef MOE_STEP

  // ---- epilogue
  const int orow0 = c.is_sh ? a.P + c.e * a.T + mc : mc;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int m = 32 * mb + (j >> 2) * 8 + kh * 4 + (j & 3);
      if (m >= nrows) continue;
      if (MODE == 0) {
        if (!w.wval[0]) continue;
        const float hv = silu_mul(acc[0][mb][j], acc[1][mb][j]);
        static_cast<uint16_t*>(a.out)[(size_t)(orow0 + m) * a.ld_out + w.wrow[0]] =
            (uint16_t)f32_to_bf16(hv);
      } else {
        float* y = static_cast<float*>(a.out) + (size_t)(orow0 + m) * a.ld_out;
        if (w.wval[0]) y[w.wrow[0]] = acc[0][mb][j];
        if (w.wval[1]) y[w.wrow[1]] = acc[1][mb][j];
      }
    }
  }
}

// Every chunk of one tile for one weight format: chunks of up to 32, 64
// or 128 rows take matching row-block counts, so a tile's ragged tail
// costs what its rows need.
template <int MODE, int BITS>
__device__ __forceinline__ void mfma_tile(const ProjArgs& a, const TileCtx& c, u32x4_v* As,
                                          int* tok, uint16_t* ssc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, kh = lane >> 5;
  const int K = c.K, U = c.U;
  const int ng = K / c.group;
  constexpr int kLaneBytes = kKS * BITS / 16;   // per lane half and step
  const int row_bytes = K * BITS / 8;

  WeightCtx w;
  w.n_st = K / kKS;
  // this lane's two weight rows: gate/up of one unit, or two down rows
  if (MODE == 0) {
    const int unit = c.u0 + 32 * wave + ln;
    w.wval[0] = w.wval[1] = unit < U;
    w.wrow[0] = unit;
    w.wrow[1] = U + unit;
  } else {
    const int r0 = c.u0 + 64 * wave + ln;
    w.wval[0] = r0 < U;
    w.wval[1] = r0 + 32 < U;
    w.wrow[0] = r0;
    w.wrow[1] = r0 + 32;
  }
  const int n_wrows = MODE == 0 ? 2 * U : U;
  w.crs = make_rsrc(c.codes, (uint32_t)(n_wrows * row_bytes));
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int r = w.wval[s] ? w.wrow[s] : 0;
    w.coff[s] = r * row_bytes + kh * kLaneBytes;
  }
  w.gsh = 31 - __builtin_clz(c.group);

  // ---- the group scales of the workgroup's 256 weight rows into LDS,
  // [local row][group]: gate rows u0.. then up rows U+u0.. (gate/up), or
  // down rows u0..; two contiguous runs of the scale matrix, copied in
  // 16-byte words (row runs start at multiples of 128 rows, so they are
  // 16-byte aligned).  The first barrier of the chunk loop publishes them.
  {
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(c.scales, (uint32_t)(n_wrows * ng * 2));
    const int run_rows = MODE == 0 ? kBM : min(2 * kBM, U - c.u0);
    const int run_words = run_rows * ng * 2 / 16;
    const int n_runs = MODE == 0 ? 2 : 1;
    for (int q = tid; q < n_runs * run_words; q += kMThreads) {
      const int run = q >= run_words, qq = q - run * run_words;
      const int row0 = run ? U + c.u0 : c.u0;
      const u32x4_v v =
          __builtin_amdgcn_raw_buffer_load_b128(srs, row0 * ng * 2 + qq * 16, 0, 0);
      reinterpret_cast<u32x4_v*>(ssc + (size_t)run * kBM * ng)[qq] = v;
    }
  }
  if (MODE == 0) {
    w.sc[0] = ssc + (32 * wave + ln) * ng;
    w.sc[1] = ssc + (kBM + 32 * wave + ln) * ng;
  } else {
    w.sc[0] = ssc + (64 * wave + ln) * ng;
    w.sc[1] = ssc + (64 * wave + ln + 32) * ng;
  }

  for (int mc = c.r_begin; mc < c.r_end; mc += kRowsMax) {
    const int nrows = min(kRowsMax, c.r_end - mc);
    __syncthreads();   // previous chunk's readers of tok / As are done
    if (tid < kRowsMax) {
      const int mm = tid < nrows ? tid : 0;   // padding rows re-read row 0 (discarded)
      int r;
      if (MODE == 0) r = c.is_sh ? mc + mm : a.sorted_pair[mc + mm] / a.k;
      else r = c.is_sh ? a.P + c.e * a.T + mc + mm : mc + mm;
      tok[tid] = r;
    }
    __syncthreads();
    if (nrows > 128) mfma_chunk<MODE, BITS, 5>(a, c, w, As, tok, mc, nrows);
    else if (nrows > 64) mfma_chunk<MODE, BITS, 4>(a, c, w, As, tok, mc, nrows);
    else if (nrows > 32) mfma_chunk<MODE, BITS, 2>(a, c, w, As, tok, mc, nrows);
    else mfma_chunk<MODE, BITS, 1>(a, c, w, As, tok, mc, nrows);
  }
}

template <int MODE>
__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void proj_mfma_kernel(ProjArgs a, const uint16_t* x16_4,
                                                              const uint16_t* x16_2) {
  extern __shared__ __align__(16) unsigned char smem[];
  u32x4_v* As = reinterpret_cast<u32x4_v*>(smem);                        // [2][kRowsMax][kChunks]
  int* tok = reinterpret_cast<int*>(smem + 2 * kChunks * kRowsMax * 16);  // [kRowsMax]
  uint16_t* ssc = reinterpret_cast<uint16_t*>(tok + kRowsMax);             // [256][K / group]
  const int tid = threadIdx.x;

  // ---- block -> (tile slot, unit block).  Block b runs on XCD b mod 8; each
  // XCD takes a contiguous range of the device-side slots, in order, so
  // the blocks of one tile (they share its activation rows) and the tiles
  // of one expert (they share its weights) run on one XCD at about the
  // same time and meet in its L2.
  const int b = blockIdx.x;
  const int xcd = b % kXcd, li = b / kXcd;
  const int nb = li % a.n_rb;
  const int n_slots = a.n_sh_slots + min(*a.n_tiles, a.max_tiles);
  const int per_xcd = (n_slots + kXcd - 1) / kXcd;
  const int local = li / a.n_rb;
  if (local >= per_xcd) return;
  const int slot = xcd * per_xcd + local;
  if (slot >= n_slots) return;
  TileCtx c;
  if (slot < a.n_sh_slots) {
    const int per = (a.T + a.sh_tile - 1) / a.sh_tile;
    const int s = slot / per, ti = slot - s * per;
    c.is_sh = true;
    c.e = s;
    c.r_begin = ti * a.sh_tile;
    c.r_end = min(a.T, c.r_begin + a.sh_tile);
  } else {
    const int j = slot - a.n_sh_slots;
    if (j >= a.max_tiles) return;
    const int4 tl = reinterpret_cast<const int4*>(a.tiles)[j];
    if (j >= *a.n_tiles) return;
    if ((unsigned)tl.x >= (unsigned)a.E) {
      if (tid == 0) atomicOr(a.err, 2);
      return;
    }
    c.is_sh = false;
    c.e = tl.x;
    c.r_begin = tl.y;
    c.r_end = tl.z;
  }
  c.K = c.is_sh ? a.K_sh : a.K;
  c.U = c.is_sh ? a.U_sh : a.U;
  c.u0 = nb * (MODE == 0 ? 128 : 256);
  if (c.u0 >= c.U) return;
  const moe_qmat q = c.is_sh ? a.w_sh[c.e] : a.w[c.e];
  if (!qmat_usable(q, MODE == 0 ? 2 * c.U : c.U, c.K) || c.K % (2 * kKS) != 0) {
    if (tid == 0) atomicOr(a.err, 1);
    return;
  }
  c.codes = q.codes;
  c.scales = q.scales;
  c.group = q.group;
  // rows the activation source holds: T token rows, or every h row
  c.a_bytes = (uint32_t)((size_t)(MODE == 0 ? a.T : a.P + a.n_shared * a.T) * a.ld_in * 2);
  if (q.bits == 4) {
    c.asrc = MODE == 0 ? x16_4 : a.in_bf16;
    mfma_tile<MODE, 4>(a, c, As, tok, ssc);
  } else {
    c.asrc = MODE == 0 ? x16_2 : a.in_bf16;
    mfma_tile<MODE, 2>(a, c, As, tok, ssc);
  }
}

hipError_t launch_proj_mfma(const ProjArgs& a_in, uint16_t* a16_4, uint16_t* a16_2,
                            hipStream_t st) {
  ProjArgs a = a_in;
  a.sh_tile = kBM;
  a.n_sh_slots = a.n_shared * ((a.T + kBM - 1) / kBM);
  const int Umax = a.U > a.U_sh ? a.U : a.U_sh;
  a.n_rb = a.mode == 0 ? (Umax + 127) / 128 : (a.U + 255) / 256;
  const long long slots = (long long)a.n_sh_slots + a.max_tiles;
  const long long groups = (slots + kXcd - 1) / kXcd;
  const long long blocks = groups * kXcd * a.n_rb;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  // one fp16 copy of the activations in the unpack's K order
  if (a.mode == 0) {
    const long long units = (long long)a.T * (a.K / 16);
    convert_x_kernel<<<(unsigned)((units + 255) / 256), 256, 0, st>>>(a.in_bf16, a.T, a.K,
                                                                       a16_4, a16_2);
  } else {
    const int R = a.P + a.n_shared * a.T;
    convert_h_kernel<<<(unsigned)((R + 3) / 4), 256, 0, st>>>(a, a16_4);
    a.in_bf16 = a16_4;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // A tile, row table, and the scales of 256 weight rows at the smallest
  // group (32)
  const int Kmax = a.K_sh > a.K ? a.K_sh : a.K;
  const size_t lds = (size_t)2 * kChunks * kRowsMax * 16 + kRowsMax * sizeof(int) +
                     (size_t)2 * kBM * (Kmax / 32) * 2;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  if (a.mode == 0)
    proj_mfma_kernel<0><<<(unsigned)blocks, kMThreads, lds, st>>>(a, a16_4, a16_2);
  else
    proj_mfma_kernel<1><<<(unsigned)blocks, kMThreads, lds, st>>>(a, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace moe
