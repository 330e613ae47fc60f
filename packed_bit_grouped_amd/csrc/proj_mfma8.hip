// Grouped expert GEMMs for prefill shapes on the CDNA4 matrix cores, one
// wave per SIMD.
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
//    gate/up units or 256 down rows; 4 waves, one per SIMD (512 registers:
//    the accumulators in AGPRs).  Wave w owns 64 weight rows - the gate
//    rows and the up rows of 32 units (SiLU*mul then pairs registers of the
//    same lane), or 64 down rows - against all of the chunk's rows: up to
//    2 x 5 accumulator tiles of 32x32, so every activation fragment read
//    from LDS feeds two MFMAs;
//  * the K loop walks 64 K per step, four 16-K MFMA sub-steps; each
//    sub-step reads the next sub-step's activation fragments and
//    dequantizes its weights while its own MFMAs run;
//  * a chunk whose last block would hold 1..16 rows runs those rows as a
//    16-row half block on v_mfma_f32_16x16x32_f16 (two sub-steps at once,
//    the weight fragments rearranged by permlane16 swaps), so padding
//    stays under 16 rows per chunk;
//  * activations (fp16, in the K order of the unpack) go from memory
//    straight into a ring of six LDS buffers [row][8 x 16-byte chunks] with
//    buffer loads that write LDS, five steps ahead, a step's loads spread
//    over three sub-steps; chunk c of row m sits in
//    slot c ^ ((m >> 1) & 7) (a 128-bit LDS access is served 16 lanes at a
//    time, and 16 consecutive rows' chunk c then cover the 64 banks once);
//    a load writes its 64 lanes' 16 bytes contiguously, so each lane loads
//    the global chunk that belongs in its slot;
//  * weights and their fp16 group scales go from memory into a register
//    ring eight steps ahead (16 bytes (int4) or 8 bytes (int2) of codes and
//    one scale per part, lane and step) and are dequantized in registers: a
//    code field OR-ed into the mantissa of an fp16 power of two reads as
//    that power plus the field, a packed subtract gives the exact code, a
//    packed multiply the fp16 scale (one rounding).  An int2 word's bytes
//    are reordered (0, 2, 1, 3) first, so int2 codes unpack in the same K
//    order as int4 and one fp16 copy of x serves both;
//  * one barrier per step, with the wait for the activation loads counted
//    by hand (every step issues the same loads in the same order) and the
//    LDS wait leaving the next step's first fragment reads in flight;
//  * canonical layout: lane (row c, half h) of a 32-row block reads bytes
//    [32 s + 16 h, +16) (int4; int2 [16 s + 8 h, +8)) of its row at step s;
//    prepacked layout (moe_w4_prepack): those 16 (8) bytes of the 64 lanes
//    stored contiguously per block and step (gate/up: the gate block of 32
//    units, then the up block of the same units), so each of a wave's loads
//    is one 1 KB (512 B) coalesced piece, with the int2 byte order applied
//    once;
//  * the results leave through the wave's part of the idle activation ring
//    as 16-byte stores;
//  * workgroups of one tile land on one XCD (blockIdx mod 8 picks the
//    XCD), so the tile's activation rows are shared in that XCD's L2.
#include "moe_internal.h"

namespace moe {

namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_v;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_v;
typedef __attribute__((ext_vector_type(16))) float f32x16_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;
typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_v __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;       // 4 waves, one per SIMD
constexpr int kUnits = 128;         // gate/up units per workgroup (shared-expert tile rows too)
constexpr int kRowsMax = 160;       // activation rows per tile chunk (5 row blocks of 32)
constexpr int kSclGroupsMax = 64;   // prepacked scales: groups per row staged in LDS
constexpr int kRing = 8;            // weight steps in flight (registers)
constexpr int kKS = 64;             // K per step
constexpr int kChunks = kKS / 8;    // 16-byte fp16 chunks per row and step
constexpr int kXcd = 8;
constexpr int kAD = 5;              // activation steps in flight (LDS)
constexpr int kABufs = 6;           // LDS activation buffers (> kAD)
constexpr int kABuf = kChunks * kRowsMax;   // 16-byte slots per buffer

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

// This lane's two weight rows (parts p = 0, 1: the gate and up rows of one
// unit, or two down rows 32 apart), their code and scale offsets.
struct Lane {
  __amdgpu_buffer_rsrc_t crs, srs;
  int coff[2];             // code byte offset of step 0 (+ step * cstride)
  int cstride;             // code bytes per step
  int soff[2];             // scale byte offset of the row's group 0 (prepacked:
                           // soff[0], both parts' scales in one word)
  int wrow[2];             // output column (gate/up: the unit; down: the row)
  const uint32_t* ss;      // prepacked: this wave's staged scale words + lane column
  bool wval[2];
  int n_st, gsh;
};

// SiLU(g) * u with the hardware exp2 and reciprocal (relative error a few
// fp32 units; the result is rounded to bf16)
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Eight bf16 values (units 8q..8q+7) as fp16 in the unpack order of an
// 8-block, (0,4)(1,5)(2,6)(3,7) (exact in fp16's normal range)
__device__ __forceinline__ u32x4_v bf16x8_to_f16_unpack(u32x4_v v) {
  const uint32_t e[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                         v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
  u32x4_v r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(e[0] << 16),
                                                               __uint_as_float(e[4] << 16)));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(e[1] << 16),
                                                               __uint_as_float(e[5] << 16)));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(e[2] << 16),
                                                               __uint_as_float(e[6] << 16)));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(e[3] << 16),
                                                               __uint_as_float(e[7] << 16)));
  return r;
}

// One step of this lane's weights: codes of both parts and their scales.
template <int BITS>
struct BReg {
  uint32_t c[2][BITS];     // per part 16 (int4) or 8 (int2) bytes
  uint32_t s[2];           // fp16 scale bits (prepacked: s[0] holds part 0 in
                           // its low half and part 1 in its high half)
};

// Wait until at most N vector-memory operations of this wave are in flight
// and every LDS access but the last LG has completed (LDS accesses complete
// in order; an outstanding scalar load only makes the count stricter), then
// the workgroup barrier.  The scheduling fences keep the compiler from
// moving any instruction across it, so the count of loads issued after a
// given one is the program's.
template <int N, int LG = 0>
__device__ __forceinline__ void vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  static_assert(LG >= 0 && LG < 16, "lgkmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (LG << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// K loop and epilogue of one chunk of up to 32 * MBT + 16 * HT rows (tok[]
// holds their activation rows): the wave's 64 weight rows against all of
// them.  Per step every wave issues the same loads in the same order
// (MBT + HT activation loads into LDS, two code loads, two scale loads),
// every load unconditional (steps past the end re-read the last step with a
// zero scale), so the number of loads issued after any given one is fixed.
//
// HT = 1 adds a half block of 16 rows on v_mfma_f32_16x16x32_f16 (a chunk
// of 32 MBT + 1 .. 32 MBT + 16 rows then pays for 16 padding rows at most,
// not 31).  Its MFMA contracts two consecutive 16-K sub-steps at once: the
// weight fragments of both (32x32 layout: lane (c, h) holds row c, chunk
// 4 h + ks) pass through one permlane16 swap per register, which leaves
// rows 0..15 of the 32-row tile in one register and rows 16..31 in the
// other, lane (c, g) = (lane & 15, lane >> 4) holding chunk 4 (g >> 1) + ks
// - 1 + (g & 1) of its row (ks odd); the half block's activation fragment
// takes the same chunks of its rows, so both operands agree on K.
template <int MODE, int BITS, int MBT, int HT, bool PP>
__device__ __forceinline__ void chunk(const ProjArgs& a, const Tile& t, const Lane& ln_,
                                      u32x4_v* As, int* tok, int mc, int nrows) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lc = lane & 31, kh = lane >> 5;
  const int n_st = ln_.n_st;

  // the weight stream is read once: non-temporal loads (cache policy nt),
  // so it does not push the tile's activation rows out of L2
  constexpr int kWeightCpol = 2;
  auto load_c = [&](int st, BReg<BITS>& b) {
    st = min(st, n_st - 1);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if constexpr (BITS == 4) {
        const u32x4_v v =
            __builtin_amdgcn_raw_buffer_load_b128(ln_.crs, ln_.coff[p], st * ln_.cstride,
                                                  kWeightCpol);
        b.c[p][0] = v.x; b.c[p][1] = v.y; b.c[p][2] = v.z; b.c[p][3] = v.w;
      } else {
        const u32x2_v v =
            __builtin_amdgcn_raw_buffer_load_b64(ln_.crs, ln_.coff[p], st * ln_.cstride,
                                                 kWeightCpol);
        b.c[p][0] = PP ? v.x : int2_order(v.x);
        b.c[p][1] = PP ? v.y : int2_order(v.y);
      }
    }
  };
  auto load_s = [&](int st, BReg<BITS>& b) {
    st = min(st, n_st - 1);
    const int gi = (st * kKS + kh * 32) >> ln_.gsh;
    if constexpr (PP) {
      // both parts' scales of the lane's row pair, from the wave's copy of
      // its block's scale words in LDS (32 words per group)
      b.s[0] = ln_.ss[gi * 32];
      b.s[1] = 0u;
    } else {
#pragma unroll
      for (int p = 0; p < 2; ++p)
        b.s[p] = __builtin_amdgcn_raw_buffer_load_b16(ln_.srs, ln_.soff[p] + gi * 2, 0, 0);
    }
  };
  auto load_b = [&](int st, BReg<BITS>& b) {
    load_c(st, b);
    load_s(st, b);
  };
  // the weight ring is issued first (it needs only the descriptor), then
  // the chunk's activation rows are read and published in LDS
  constexpr int kBLoads = PP ? 2 : 4;   // code and scale loads per step
  constexpr int MBA = MBT + HT;         // 32-row pieces staged in LDS per step
  constexpr int kStepLoads = MBA + kBLoads;
  // Loads issued after A(s + 2) by the end of step s: from step 3 on, the
  // weight and scale loads of its own step and three whole steps (at least
  // (kAD - 2) whole steps, counted without the former); in steps 0 and 1,
  // whose A(s + 2) the prologue issued (after the weight ring), the
  // prologue's later activation loads and the steps so far:
  // (kAD - 2) * MBA + kBLoads (s + 1).  The prologue's barrier waits for A(1):
  // A(2) .. A(kAD - 1) come after it.
  constexpr int kWaitSteady = (kAD - 2) * kStepLoads;
  constexpr int kWaitFirst = (kAD - 2) * MBA;
  static_assert(kAD == 5, "the early-step counts below assume five steps ahead");
  // the chunk's activation rows (a load that needs only the tile), then
  // the weight ring (it needs the descriptor), then the rows are published
  int r = 0;
  if (tid < kRowsMax) {
    const int mm = tid < nrows ? tid : 0;   // padding rows re-read row 0 (discarded)
    if (MODE == 0) r = t.is_sh ? mc + mm : a.sorted_pair[mc + mm];
    else r = t.is_sh ? a.P + t.e * a.T + mc + mm : mc + mm;
  }
  BReg<BITS> b0, b1, b2, b3, b4, b5, b6, b7;
  if (PP) {
    // codes only: the scale words of these steps are read from LDS after
    // the prologue barrier, once their copy (issued before) has landed
    load_c(0, b0); load_c(1, b1); load_c(2, b2); load_c(3, b3);
    load_c(4, b4); load_c(5, b5); load_c(6, b6); load_c(7, b7);
  } else {
    load_b(0, b0); load_b(1, b1); load_b(2, b2); load_b(3, b3);
    load_b(4, b4); load_b(5, b5); load_b(6, b6); load_b(7, b7);
  }
  __syncthreads();   // previous chunk's readers of tok are done
  if (tid < kRowsMax) tok[tid] = (MODE == 0 && !t.is_sh) ? r / a.k : r;
  __syncthreads();
  // activations: piece q = (wave * MBA + i) * 64 + lane of a step (row q >>
  // 3, LDS slot q & 7) holds global chunk (q & 7) ^ ((row >> 1) & 7) of the
  // row; a load writes its 64 lanes' 16 bytes contiguously from its LDS base
  // (a half block stages a whole 32-row piece: rows past the chunk re-read
  // row 0, and every wave keeps one load count)
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(t.asrc, t.a_bytes);
  int aoff[MBA];
#pragma unroll
  for (int i = 0; i < MBA; ++i) {
    const int q = (wave * MBA + i) * 64 + lane;
    const int m = q >> 3;
    aoff[i] = tok[m] * a.ld_in * 2 + (((q & 7) ^ ((m >> 1) & 7)) * 16);
  }
  // pieces i with i % 3 == part of step st (part < 0: all of them)
  auto dma_a = [&](int st, int buf, int part) {
    const int o = min(st, n_st - 1) * (kKS * 2);
#pragma unroll
    for (int i = 0; i < MBA; ++i)
      if (part < 0 || i % 3 == part)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ars,
            (__attribute__((address_space(3))) void*)(As + buf * kABuf + (wave * MBA + i) * 64),
            16, aoff[i], o, 0, 0);
  };

  f32x16_v acc[2][MBT];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int mb = 0; mb < MBT; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[p][mb][j] = 0.0f;
  // half block: [part][rows 0..15 / 16..31 of the part's 32-row tile]
  f32x4_v acch[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 2; ++q) acch[p][q] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};

  // fragment of row tile mb, 16-K sub-step ks, from LDS buffer buf: lane
  // (lc, kh) reads row 32 mb + lc, chunk kh * 4 + ks
  const int rsw = (lc >> 1) & 7;
  auto read_frags = [&](int buf, int ks, f16x8_v* f) {
    const u32x4_v* Ab = As + buf * kABuf + lc * kChunks + ((kh * 4 + ks) ^ rsw);
#pragma unroll
    for (int mb = 0; mb < MBT; ++mb) f[mb] = __builtin_bit_cast(f16x8_v, Ab[32 * kChunks * mb]);
  };
  // half-block fragment for sub-steps ks, ks + 1 (ks even): lane (c, g)
  // reads row 32 MBT + c, chunk 4 (g >> 1) + ks + (g & 1)
  const int hc = lane & 15, hg = lane >> 4;
  const int hoff = (32 * MBT + hc) * kChunks;
  const int hsw = (hc >> 1) & 7;
  auto read_half = [&](int buf, int ks) {
    return __builtin_bit_cast(
        f16x8_v, As[buf * kABuf + hoff + ((4 * (hg >> 1) + ks + (hg & 1)) ^ hsw)]);
  };
  // 16x16x32 weight operands of one part from its 32x32 fragments of
  // sub-steps ks - 1 (x) and ks (y): rows 0..15 (t0) and 16..31 (t1)
  auto swap16 = [&](const f16x8_v& x, const f16x8_v& y, f16x8_v& t0, f16x8_v& t1) {
    const u32x4_v xv = __builtin_bit_cast(u32x4_v, x), yv = __builtin_bit_cast(u32x4_v, y);
    u32x4_v a0, a1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto r = __builtin_amdgcn_permlane16_swap(xv[i], yv[i], false, false);
      a0[i] = r[0];
      a1[i] = r[1];
    }
    t0 = __builtin_bit_cast(f16x8_v, a0);
    t1 = __builtin_bit_cast(f16x8_v, a1);
  };
  // steps past the last one (the loop runs whole rings) get a zero scale
  auto deq = [&](const BReg<BITS>& b, int ks, int stg, f16x8_v* bq) {
    const uint32_t m16 = stg < n_st ? 0x10001u : 0u;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t sv = PP ? (p ? b.s[0] >> 16 : b.s[0] & 0xFFFFu) : b.s[p];
      const f16x2_v s2 = as_h2(sv * m16);
      if constexpr (BITS == 4) bq[p] = deq_int4(b.c[p][ks], s2);
      else if ((ks & 1) == 0) bq[p] = deq_int2<0>(b.c[p][ks >> 1], s2);
      else bq[p] = deq_int2<1>(b.c[p][ks >> 1], s2);
    }
  };
  f16x8_v fr[2][MBT];
  f16x8_v bq[2][2];
  // one 64-K step from LDS buffer buf with the weights of b; sub-step ks
  // reads the fragments of ks + 1 and dequantizes its weights while its own
  // MFMAs run; the last sub-step does so for the first sub-step of the next
  // step (buffer nbuf, weights bn)
  // Sub-steps 0..2 also issue the activation loads of step dst into LDS
  // buffer dbuf (piece i in sub-step i mod 3, so the four waves' 1 KB loads
  // do not queue up at the CU's address unit at once), sub-step 3 the
  // weight and scale loads of step stg + kRing into b (its codes are last
  // read by sub-step 2); the loads are spread between the MFMAs.  Sub-steps
  // end with scheduling fences, so the order of the loads (activations,
  // then weights and scales) is the same in every step.
  auto step = [&](int buf, int nbuf, BReg<BITS>& b, const BReg<BITS>& bn, int stg, int dst,
                  int dbuf) {
    // prepacked: the scale word of step stg + kRing is read from LDS in
    // sub-step 0 (b's own scale is still in use until sub-step 2) and moved
    // into b with its codes in sub-step 3, so the read has landed long
    // before the step's barrier waits for the LDS
    BReg<BITS> sn;
    f16x8_v fh, bprev[2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (PP && ks == 0) load_s(stg + kRing, sn);
      if (HT && cur == 0) {
        fh = read_half(buf, ks);
        bprev[0] = bq[cur][0];
        bprev[1] = bq[cur][1];
      }
      f16x8_v th[2][2];
      if (HT && cur == 1) {
        swap16(bprev[0], bq[cur][0], th[0][0], th[0][1]);
        swap16(bprev[1], bq[cur][1], th[1][0], th[1][1]);
      }
      if (ks < 3) {
        read_frags(buf, ks + 1, fr[nxt]);
        deq(b, ks + 1, stg, bq[nxt]);
      } else {
        read_frags(nbuf, 0, fr[nxt]);
        deq(bn, 0, stg + 1, bq[nxt]);
      }
      if (ks < 3) dma_a(dst, dbuf, ks);
      if (ks == 3) {
        if (PP) {
          load_c(stg + kRing, b);
          b.s[0] = sn.s[0];
        } else {
          load_b(stg + kRing, b);
        }
      }
#pragma unroll
      for (int mb = 0; mb < MBT; ++mb) {
        acc[0][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[cur][mb], bq[cur][0], acc[0][mb], 0, 0, 0);
        acc[1][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[cur][mb], bq[cur][1], acc[1][mb], 0, 0, 0);
      }
      if (HT && cur == 1) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int q = 0; q < 2; ++q)
            acch[p][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fh, th[p][q], acch[p][q], 0, 0, 0);
      }
      // issue order: the LDS reads, then the MFMAs with the loads (one per
      // MFMA) and the dequantization between them
      const int kLd = ks < 3 ? (MBA - ks + 2) / 3 : kBLoads;
      const bool ds_s = PP && ks == 0, ds_h = HT && cur == 0;
      if (ds_s && ds_h) __builtin_amdgcn_sched_group_barrier(0x100, MBT + 2, 0);
      else if (ds_s || ds_h) __builtin_amdgcn_sched_group_barrier(0x100, MBT + 1, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, MBT, 0);
#pragma unroll
      for (int i = 0; i < 2 * MBT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < kLd) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
      if (HT && cur == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (2 * MBT + i < kLd) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Activations kAD steps ahead in a ring of kABufs LDS buffers (step s in
  // buffer s % kABufs); weights and scales kRing steps ahead in registers.
  // Step s computes, loads A(s + kAD) into the buffer step s - 1 read, and
  // B(s + kRing) into the register slot it consumed; the barrier that ends
  // it waits for A(s + 2), whose first fragments step s + 1 reads early
  // (the counts above).
#pragma unroll
  for (int j = 0; j < kAD; ++j) {
    __builtin_amdgcn_sched_barrier(0);
    dma_a(j, j, -1);
  }
  vm_barrier<kWaitFirst>();
  if (PP) {
    load_s(0, b0); load_s(1, b1); load_s(2, b2); load_s(3, b3);
    load_s(4, b4); load_s(5, b5); load_s(6, b6); load_s(7, b7);
  }
  read_frags(0, 0, fr[0]);
  deq(b0, 0, 0, bq[0]);
  int buf = 0;
#define MOE8_STEP(J, BC, BN)                                  \
  {                                                           \
    const int nb = buf == kABufs - 1 ? 0 : buf + 1;           \
    const int db = buf + kAD >= kABufs ? buf + kAD - kABufs : buf + kAD; \
    step(buf, nb, BC, BN, base + J, base + J + kAD, db);      \
    if (J < 2 && base == 0)                                   \
      vm_barrier<(kAD - 2) * MBA + kBLoads * (J + 1), MBT>(); \
    else                                                      \
      vm_barrier<kWaitSteady, MBT>();                         \
    buf = nb;                                                 \
  }
  for (int base = 0; base < n_st; base += kRing) {
    MOE8_STEP(0, b0, b1)
    MOE8_STEP(1, b1, b2)
    MOE8_STEP(2, b2, b3)
    MOE8_STEP(3, b3, b4)
    MOE8_STEP(4, b4, b5)
    MOE8_STEP(5, b5, b6)
    MOE8_STEP(6, b6, b7)
    MOE8_STEP(7, b7, b0)
  }
#undef MOE8_STEP
  // the loads still in flight (past the last step) land before the LDS is
  // reused
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue: lane holds column lc of both parts (rows 32 mb + 8 (j >>
  // 2) + 4 kh + (j & 3)); gate/up: part 0 is the gate, part 1 the up of the
  // same unit, so SiLU(g) * u needs no exchange.  The wave's results pass
  // through its own part of the (now idle) activation ring, so the global
  // stores are 16 bytes per lane.
  const int orow0 = t.is_sh ? a.P + t.e * a.T + mc : mc;
  __syncthreads();   // every wave is past its last read of the ring
  if (MODE == 0) {
    // h tile [rows][32 units] bf16, row stride 80 bytes (rows 4 apart land
    // on different banks)
    constexpr int kRowB = 80;
    unsigned char* stg = reinterpret_cast<unsigned char*>(As) + wave * (kRowsMax * kRowB);
    // two rows of one column at a time: one packed round-to-nearest-even
    // conversion, then the two halves
    auto put2 = [&](int m, int c, float g0, float u0, float g1, float u1) {
      const bf16x2_v v = {(__bf16)silu_mul_fast(g0, u0), (__bf16)silu_mul_fast(g1, u1)};
      const uint32_t w = __builtin_bit_cast(uint32_t, v);
      *reinterpret_cast<uint16_t*>(stg + m * kRowB + c * 2) = (uint16_t)w;
      *reinterpret_cast<uint16_t*>(stg + (m + 1) * kRowB + c * 2) = (uint16_t)(w >> 16);
    };
#pragma unroll
    for (int mb = 0; mb < MBT; ++mb)
#pragma unroll
      for (int j = 0; j < 16; j += 2)
        put2(32 * mb + (j >> 2) * 8 + kh * 4 + (j & 3), lc, acc[0][mb][j], acc[1][mb][j],
             acc[0][mb][j + 1], acc[1][mb][j + 1]);
    // half block: lane holds column 16 q + (lane & 15) of both parts, rows
    // 32 MBT + 4 (lane >> 4) + j
    if (HT) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int j = 0; j < 4; j += 2)
          put2(32 * MBT + 4 * hg + j, 16 * q + hc, acch[0][q][j], acch[1][q][j],
               acch[0][q][j + 1], acch[1][q][j + 1]);
    }
    __syncthreads();   // lanes read what other lanes wrote
    const int q = lane & 3;
    const int u = ln_.wrow[0] - lc + 8 * q;   // first unit of the lane's 16 bytes
#pragma unroll
    for (int i = 0; i < (MBT * 32 + HT * 16 + 15) / 16; ++i) {
      const int m = 16 * i + (lane >> 2);
      const u32x4_v v = *reinterpret_cast<const u32x4_v*>(stg + m * kRowB + q * 16);
      if (m < nrows && ln_.wval[0]) {
        const size_t o = (size_t)(orow0 + m) * a.ld_out + u;
        *reinterpret_cast<u32x4_v*>(static_cast<uint16_t*>(a.out) + o) = v;
        if (a.out16) *reinterpret_cast<u32x4_v*>(a.out16 + o) = bf16x8_to_f16_unpack(v);
      }
    }
  } else {
    // y tile of one part [rows][32] fp32, row stride 160 bytes
    constexpr int kRowB = 160;
    unsigned char* stg = reinterpret_cast<unsigned char*>(As) + wave * (kRowsMax * kRowB);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (p > 0) __syncthreads();   // the previous part's reads are done
#pragma unroll
      for (int mb = 0; mb < MBT; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int m = 32 * mb + (j >> 2) * 8 + kh * 4 + (j & 3);
          *reinterpret_cast<float*>(stg + m * kRowB + lc * 4) = acc[p][mb][j];
        }
      if (HT) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float*>(stg + (32 * MBT + 4 * hg + j) * kRowB + (16 * q + hc) * 4) =
                acch[p][q][j];
      }
      __syncthreads();   // lanes read what other lanes wrote
      const int q = lane & 7;
      const int col = ln_.wrow[p] - lc + 4 * q;
#pragma unroll
      for (int i = 0; i < (MBT * 32 + HT * 16 + 7) / 8; ++i) {
        const int m = 8 * i + (lane >> 3);
        const u32x4_v v = *reinterpret_cast<const u32x4_v*>(stg + m * kRowB + q * 16);
        // y is read once, by the combine after the whole launch: streamed
        // out with non-temporal stores, which keep the caches for the
        // tiles' h rows and weights
        if (m < nrows && ln_.wval[p])
          __builtin_nontemporal_store(
              v, reinterpret_cast<u32x4_v*>(static_cast<float*>(a.out) +
                                            (size_t)(orow0 + m) * a.ld_out + col));
      }
    }
  }
}

template <int MODE, int BITS, bool PP>
__device__ __forceinline__ void tile(const ProjArgs& a, const Tile& t, u32x4_v* As, int* tok) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = __builtin_amdgcn_readfirstlane(tid >> 6);   // weight block of the wave
  const int lc = lane & 31, kh = lane >> 5;
  const int K = t.K, U = t.U;
  const int ng = K / t.group;
  const int row_bytes = K * BITS / 8;
  const int n_wrows = MODE == 0 ? 2 * U : U;

  Lane L;
  L.n_st = K / kKS;
  int brow[2];   // this lane's weight rows
  if (MODE == 0) {
    const int unit = t.u0 + 32 * n + lc;
    L.wval[0] = L.wval[1] = unit < U;
    L.wrow[0] = L.wrow[1] = unit;
    brow[0] = unit;
    brow[1] = U + unit;
  } else {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = t.u0 + 64 * n + 32 * p + lc;
      L.wval[p] = r < U;
      L.wrow[p] = r;
      brow[p] = r;
    }
  }
  L.crs = make_rsrc(t.codes, (uint32_t)((size_t)n_wrows * row_bytes));
  L.srs = make_rsrc(t.scales, (uint32_t)((size_t)n_wrows * ng * 2));
#pragma unroll
  for (int p = 0; p < 2; ++p) L.soff[p] = (L.wval[p] ? brow[p] : 0) * ng * 2;
  // prepacked scales: [block][group][32 rows][2 parts] fp16, a block being
  // a gate/up unit block of 32 (gate, up) or a down pair of 32-row blocks;
  // staged in LDS below (soff unused)
  constexpr int kLaneBytes = kKS * BITS / 16;   // per lane half and step
  if (PP) {
    // gate/up: [unit block of 32][step][gate, up][64 lane slots]; down:
    // [row block of 32][step][64 lane slots]
    if (MODE == 0) {
      const int blk = t.u0 / 32 + n;
      L.cstride = 2 * 64 * kLaneBytes;
#pragma unroll
      for (int p = 0; p < 2; ++p)
        L.coff[p] = L.wval[p] ? blk * L.n_st * L.cstride + p * 64 * kLaneBytes + lane * kLaneBytes
                              : 0;
    } else {
      L.cstride = 64 * kLaneBytes;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int blk = (t.u0 + 64 * n) / 32 + p;
        L.coff[p] = L.wval[p] ? blk * L.n_st * L.cstride + lane * kLaneBytes : 0;
      }
    }
  } else {
    L.cstride = kKS * BITS / 8;
#pragma unroll
    for (int p = 0; p < 2; ++p) L.coff[p] = (L.wval[p] ? brow[p] : 0) * row_bytes + kh * kLaneBytes;
  }
  L.gsh = 31 - __builtin_clz(t.group);
  if (PP) {
    // the wave's block of prepacked scale words ([group][32 rows][2 parts],
    // ng * 128 bytes) into its LDS region once per tile, 1 KB per load;
    // issued before every load of the chunks, so the first chunk's prologue
    // barrier (it waits for an activation load issued later) covers them
    uint32_t* sw = reinterpret_cast<uint32_t*>(As + kABufs * kABuf) + kRowsMax +
                   n * (kSclGroupsMax * 32);
    const int sblk = MODE == 0 ? t.u0 / 32 + n : (t.u0 + 64 * n) / 64;
    const int nld = (ng * 128 + 1023) / 1024;
    for (int i = 0; i < nld; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          L.srs, (__attribute__((address_space(3))) void*)(sw + 256 * i), 16,
          lane * 16, sblk * ng * 128 + i * 1024, 0, 0);
    L.ss = sw + lc;
  }

  for (int mc = t.r_begin; mc < t.r_end; mc += kRowsMax) {
    const int nrows = min(kRowsMax, t.r_end - mc);
    // whole 32-row blocks, plus a 16-row half block when the last 1..16
    // rows would otherwise fill a block of their own
    const int full = nrows >> 5, rem = nrows & 31;
    const bool half = full > 0 && rem > 0 && rem <= 16;
    const int mbt = half ? full : (nrows + 31) >> 5;
    if (mbt == 5) chunk<MODE, BITS, 5, 0, PP>(a, t, L, As, tok, mc, nrows);
    else if (mbt == 4) {
      if (half) chunk<MODE, BITS, 4, 1, PP>(a, t, L, As, tok, mc, nrows);
      else chunk<MODE, BITS, 4, 0, PP>(a, t, L, As, tok, mc, nrows);
    } else if (mbt == 3) {
      if (half) chunk<MODE, BITS, 3, 1, PP>(a, t, L, As, tok, mc, nrows);
      else chunk<MODE, BITS, 3, 0, PP>(a, t, L, As, tok, mc, nrows);
    } else if (mbt == 2) {
      if (half) chunk<MODE, BITS, 2, 1, PP>(a, t, L, As, tok, mc, nrows);
      else chunk<MODE, BITS, 2, 0, PP>(a, t, L, As, tok, mc, nrows);
    } else {
      if (half) chunk<MODE, BITS, 1, 1, PP>(a, t, L, As, tok, mc, nrows);
      else chunk<MODE, BITS, 1, 0, PP>(a, t, L, As, tok, mc, nrows);
    }
  }
}

template <int MODE, bool PP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void proj_mfma8_kernel(ProjArgs a, const uint16_t* x16) {
  extern __shared__ __align__(16) unsigned char smem[];
  u32x4_v* As = reinterpret_cast<u32x4_v*>(smem);                         // [kABufs][kRowsMax][kChunks]
  int* tok = reinterpret_cast<int*>(smem + kABufs * kABuf * 16);           // [kRowsMax]
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
  if (!qmat_usable(q, MODE == 0 ? 2 * t.U : t.U, t.K) || t.K % (2 * kKS) != 0 ||
      (PP && (t.K / q.group > kSclGroupsMax ||
              (reinterpret_cast<uintptr_t>(q.scales) & 15) != 0))) {
    if (tid == 0) atomicOr(a.err, 1);
    return;
  }
  t.codes = q.codes;
  t.scales = q.scales;
  t.group = q.group;
  // rows the activation source holds: T token rows, or every h row
  t.a_bytes = (uint32_t)((size_t)(MODE == 0 ? a.T : a.P + a.n_shared * a.T) * a.ld_in * 2);
  t.asrc = MODE == 0 ? x16 : a.in_bf16;
  if (q.bits == 4) tile<MODE, 4, PP>(a, t, As, tok);
  else tile<MODE, 2, PP>(a, t, As, tok);
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
  // one fp16 copy of the activations in the unpack's K order (gate/up:
  // unless the routing launch made it, a.in16_ready)
  if (a.mode == 0 && !a.in16_ready) {
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
  // prepacked banks: the four waves' scale words after the row numbers
  const size_t lds = (size_t)kABufs * kABuf * 16 + kRowsMax * sizeof(int) +
                     (prepacked ? (size_t)4 * kSclGroupsMax * 32 * 4 : 0);
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
// thread.  gate_up: u = ((block * n_st + step) * 2 + part) * 64 + lane, the
// row of lane (half * 32 + column) being gate row 32 block + column (part
// 0) or up row N / 2 + 32 block + column (part 1); down: u = (block * n_st
// + step) * 64 + lane, row 32 block + column.  The unit holds bytes
// [step * 32 + half * 16, +16) of that row (int2: [step * 16 + half * 8,
// +8), each 4-byte word's bytes reordered (0, 2, 1, 3)).
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t* __restrict__ src, int bits,
                                                      int N, int K, int gate_up,
                                                      uint8_t* __restrict__ dst) {
  const int n_st = K / kKS;
  const long long units = (long long)(N / 32) * n_st * 64;
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int lane = (int)(u & 63);
  long long bs = u >> 6;
  const int part = gate_up ? (int)(bs & 1) : 0;
  if (gate_up) bs >>= 1;
  const int st = (int)(bs % n_st);
  const int blk = (int)(bs / n_st);
  const int c = lane & 31, half = lane >> 5;
  const int row = (part ? N / 2 : 0) + 32 * blk + c;
  const size_t row_bytes = (size_t)K * bits / 8;
  if (bits == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + row * row_bytes + st * 32 + half * 16);
    reinterpret_cast<uint4*>(dst)[u] = v;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(src + row * row_bytes + st * 16 + half * 8);
    reinterpret_cast<uint2*>(dst)[u] = make_uint2(int2_order(v.x), int2_order(v.y));
  }
}

// One 4-byte word of the prepacked scales per thread: word u = (b * ng + g)
// * 32 + c holds group g of rows r0 (low half) and r1 (high half), gate/up
// r0 = 32b + c, r1 = N/2 + 32b + c; down r0 = 64b + c, r1 = 64b + 32 + c.
__global__ __launch_bounds__(256) void prepack_scales_kernel(const uint16_t* __restrict__ src,
                                                             int N, int ng, int gate_up,
                                                             uint32_t* __restrict__ dst) {
  const long long words = (long long)(N / 2) * ng;
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  if (u >= words) return;
  const int c = (int)(u & 31);
  const long long bg = u >> 5;
  const int g = (int)(bg % ng);
  const int b = (int)(bg / ng);
  const int r0 = gate_up ? 32 * b + c : 64 * b + c;
  const int r1 = gate_up ? N / 2 + 32 * b + c : 64 * b + 32 + c;
  dst[u] = (uint32_t)src[(size_t)r0 * ng + g] | ((uint32_t)src[(size_t)r1 * ng + g] << 16);
}

}  // namespace

hipError_t launch_prepack_scales(const uint16_t* src, int N, int ng, int gate_up, uint16_t* dst,
                                 hipStream_t st) {
  const long long words = (long long)(N / 2) * ng;
  if (words <= 0) return hipSuccess;
  prepack_scales_kernel<<<(unsigned)((words + 255) / 256), 256, 0, st>>>(
      src, N, ng, gate_up, reinterpret_cast<uint32_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_prepack(const uint8_t* src, int bits, int N, int K, int gate_up, uint8_t* dst,
                          hipStream_t st) {
  const long long units = (long long)(N / 32) * (K / kKS) * 64;
  if (units <= 0) return hipSuccess;
  prepack_kernel<<<(unsigned)((units + 255) / 256), 256, 0, st>>>(src, bits, N, K, gate_up, dst);
  return hipGetLastError();
}

}  // namespace moe
