// Device helpers shared by the MoE W4 kernels (gfx950, wave64).
//
// Packed-code unpacking.  Expert weights stay packed in device memory and
// are expanded only in registers (build log "Two 96 GB Ascend cards run
// Qwen3.8 Flash-Next", section "Keep low-bit weights packed, do the work
// on the NPU").  Three exact expansions are used:
//
//  * bf16 for the VALU dot2 path: a 4-bit code c (two's complement) is
//    turned into the offset value u = c ^ 8 = v + 8 in [0, 15] and OR-ed
//    into the mantissa of bf16 128.0 (0x4300): the bf16 value is exactly
//    128 + u = 136 + v.  The dot product against x therefore carries a
//    bias 136 * sum(x), removed with a precomputed per-chunk sum of x.
//    2-bit codes use u = c ^ 2 = v + 2 and bias 130.  Two codes of one
//    32-bit word are expanded per OR: lanes (c_i, c_{i+4}) for int4,
//    (c_i, c_{i+8}) for int2, so the activations are stored in that
//    pair order.
//  * int8 for the A8 sdot4 path: a 4-bit code placed in the top nibble of
//    a byte reads as the signed byte 16 * v, a 2-bit code in the top two
//    bits as 64 * v; one AND/shift expands four codes, and the int32 dot
//    is divided by 16 or 64 exactly (an arithmetic shift).
//  * fp16 for the MFMA path: u OR-ed into fp16 1024.0 (0x6400) is exactly
//    1024 + u; one packed fp16 subtract yields v.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_w4.h"

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float -> bf16 bit pattern, round to nearest even (finite input).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fp16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a),
                                         __builtin_bit_cast(bf16x2_v, b), c,
                                         false);
}

__device__ __forceinline__ int sdot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

// ---------------------------------------------------------------------
// Cross-lane exchange with DPP (data-parallel primitives: the operand of a
// VALU instruction is read from another lane of the same row of 16 lanes,
// or broadcast between rows), a few cycles each instead of the LDS round
// trip of ds_bpermute.
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;    // lane i <- 15 - i within a row
constexpr int kDppRowHalfMirror = 0x141;// lane i <- 7 - i within 8 lanes
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of row r -> row r+1
constexpr int kDppRowBcast31 = 0x143;   // lane 31 -> rows 2 and 3

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Workgroup barrier for data exchanged through LDS only.  Unlike
// __syncthreads() it does not wait for this wave's outstanding global
// loads and stores (gfx9 counts both on one counter), so weight streams
// stay in flight across it; each use still waits for its own loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over aligned groups of `width` lanes, width in {1, 2, 4, 8, 16}; every
// lane of a group ends with the group's sum, formed in a fixed order.
// width 16: mirror, half mirror, xor 2, xor 1; width 8: the last three.
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width >= 16) v += dpp_f<kDppRowMirror>(v, v);
  if (width >= 8) v += dpp_f<kDppRowHalfMirror>(v, v);
  if (width >= 4) v += dpp_f<kDppXor2>(v, v);
  if (width >= 2) v += dpp_f<kDppXor1>(v, v);
  return v;
}
__device__ __forceinline__ int group_sum_i(int v, int width) {
  if (width >= 16) v += dpp_i<kDppRowMirror>(v, v);
  if (width >= 8) v += dpp_i<kDppRowHalfMirror>(v, v);
  if (width >= 4) v += dpp_i<kDppXor2>(v, v);
  if (width >= 2) v += dpp_i<kDppXor1>(v, v);
  return v;
}

// (value, index) order of the router: larger value first, ties to the
// lower index.
__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = dpp_f<CTRL, ROW_MASK>(v, v);
  const int oi = dpp_i<CTRL, ROW_MASK>(i, i);
  if (beats(ov, oi, v, i)) { v = ov; i = oi; }
}
// Wave-wide arg-max; the result is returned uniform (read from lane 63).
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<kDppXor1>(v, i);
  argmax_step<kDppXor2>(v, i);
  argmax_step<kDppRowHalfMirror>(v, i);
  argmax_step<kDppRowMirror>(v, i);
  argmax_step<kDppRowBcast15, 0xA>(v, i);
  argmax_step<kDppRowBcast31, 0xC>(v, i);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}
__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ---------------------------------------------------------------------
// int8 row quantizer of the A8 mode: s = fp32(amax) / 127 (IEEE division),
// q = clamp(rint(v / s), -127, 127); amax == 0 gives s = 0 and q = 0.
// The projections and the standalone call use these same two functions.
// Weight of a shared expert for one token from its gate logit l:
// sigmoid(l) = 1 / (1 + exp(-l)) in fp32 (every combine uses this one).
__device__ __forceinline__ float shared_gate_weight(float l) {
  return 1.0f / (1.0f + expf(-l));
}

__device__ __forceinline__ float a8_scale(float amax) {
  return amax / 127.0f;
}
__device__ __forceinline__ int a8_code(float v, float s) {
  if (s == 0.0f) return 0;
  float q = rintf(v / s);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return (int)q;
}

// ---------------------------------------------------------------------
// Activation pair order matching the unpack order of one 32-bit code word.
// A16 (bf16 pairs): int4 word = K positions 0..7 -> pairs (0,4)(1,5)(2,6)(3,7);
// int2 word = K 0..15 -> pairs (0,8)(1,9)...(7,15).  Given the position j
// inside the word's block, return where it is stored.
__device__ __forceinline__ int a16_slot(int j, int bits) {
  if (bits == 4) {               // block of 8
    int i = j & 3, hi = j >> 2;  // pair i, half hi
    return 2 * i + hi;
  } else {                       // block of 16
    int i = j & 7, hi = j >> 3;
    return 2 * i + hi;
  }
}
// A8 (int8 quads): int4 word = K 0..7 -> quads (0,2,4,6)(1,3,5,7);
// int2 word = K 0..15 -> quads (0,4,8,12)(1,5,9,13)(2,6,10,14)(3,7,11,15).
__device__ __forceinline__ int a8_slot(int j, int bits) {
  if (bits == 4) {               // block of 8: even positions first
    return (j & 1) * 4 + (j >> 1);
  } else {                       // block of 16
    return (j & 3) * 4 + (j >> 2);
  }
}

// Bias of the bf16 expansion (see the file comment).
__device__ __forceinline__ float a16_bias(int bits) {
  return bits == 4 ? 136.0f : 130.0f;
}

// Dot product of one 32-bit code word with activations already in pair
// order (bf16 pairs), bias included.  int4: 4 pairs; int2: 8 pairs.
__device__ __forceinline__ float dot_word_a16_int4(uint32_t w, const uint32_t* xp,
                                                   float acc) {
  w ^= 0x88888888u;
  acc = dot2_bf16((w & 0x000F000Fu) | 0x43004300u, xp[0], acc);
  acc = dot2_bf16(((w >> 4) & 0x000F000Fu) | 0x43004300u, xp[1], acc);
  acc = dot2_bf16(((w >> 8) & 0x000F000Fu) | 0x43004300u, xp[2], acc);
  acc = dot2_bf16(((w >> 12) & 0x000F000Fu) | 0x43004300u, xp[3], acc);
  return acc;
}
__device__ __forceinline__ float dot_word_a16_int2(uint32_t w, const uint32_t* xp,
                                                   float acc) {
  w ^= 0xAAAAAAAAu;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    acc = dot2_bf16(((w >> (2 * i)) & 0x00030003u) | 0x43004300u, xp[i], acc);
  return acc;
}

// int8 x packed-code dot of one word; the result is 16x (int4) or 64x
// (int2) the true integer dot product.
__device__ __forceinline__ int dot_word_a8_int4(uint32_t w, const uint32_t* xq,
                                                int acc) {
  acc = sdot4((int)((w << 4) & 0xF0F0F0F0u), (int)xq[0], acc);
  acc = sdot4((int)(w & 0xF0F0F0F0u), (int)xq[1], acc);
  return acc;
}
__device__ __forceinline__ int dot_word_a8_int2(uint32_t w, const uint32_t* xq,
                                                int acc) {
  acc = sdot4((int)((w << 6) & 0xC0C0C0C0u), (int)xq[0], acc);
  acc = sdot4((int)((w << 4) & 0xC0C0C0C0u), (int)xq[1], acc);
  acc = sdot4((int)((w << 2) & 0xC0C0C0C0u), (int)xq[2], acc);
  acc = sdot4((int)(w & 0xC0C0C0C0u), (int)xq[3], acc);
  return acc;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

__device__ __forceinline__ bool qmat_usable(const moe_qmat& q, int N, int K) {
  if (q.codes == nullptr || q.scales == nullptr) return false;
  if (q.bits != 4 && q.bits != 2) return false;
  if (q.group != 32 && q.group != 64 && q.group != 128 && q.group != 256)
    return false;
  if (q.N != N || q.K != K) return false;
  if (K % q.group) return false;
  if ((K * q.bits / 8) % 16) return false;
  return true;
}

// fp16 copy of 8 bf16 values in the order (0,4)(1,5)(2,6)(3,7): the order
// in which the matrix-core path unpacks 8 int4 codes (and int2 codes after
// their byte reorder), so one copy of x serves both formats.  Exact for
// values within fp16 range (bf16 has fewer mantissa bits).
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

}  // namespace moe
