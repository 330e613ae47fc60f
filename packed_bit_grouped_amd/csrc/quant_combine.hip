// Dynamic int8 row quantizer (the W4A8 mode of the build log "Two 96 GB
// Ascend cards run Qwen3.8 Flash-Next", section "Keep low-bit weights
// packed, do the work on the NPU") and the weighted combine of expert
// outputs into token outputs.
#include "moe_internal.h"

namespace moe {

// One workgroup (256 threads) per row: amax by block reduction, then the
// shared a8_scale / a8_code rule.
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const void* __restrict__ src, int is_f32, int C, int ld,
    int8_t* __restrict__ q, int ldq, float* __restrict__ s) {
  __shared__ float red[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  const uint16_t* rb = static_cast<const uint16_t*>(src) + (size_t)r * ld;
  const float* rf = static_cast<const float*>(src) + (size_t)r * ld;
  float amax = 0.0f;
  for (int c = tid; c < C; c += 256) {
    const float v = is_f32 ? rf[c] : bf16_to_f32(rb[c]);
    amax = fmaxf(amax, fabsf(v));
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = a8_scale(amax);
  for (int c = tid; c < C; c += 256) {
    const float v = is_f32 ? rf[c] : bf16_to_f32(rb[c]);
    q[(size_t)r * ldq + c] = (int8_t)a8_code(v, sc);
  }
  if (tid == 0) s[r] = sc;
}

hipError_t launch_quant_a8(const void* src, int is_f32, int R, int C, int ld,
                           int8_t* q, int ldq, float* s, hipStream_t st) {
  if (R == 0) return hipSuccess;
  quant_rows_kernel<<<R, 256, 0, st>>>(src, is_f32, C, ld, q, ldq, s);
  return hipGetLastError();
}

// out[t][n] = bf16( sum_j w[t][j] * y[pair_pos[t*k+j]][n] + sum_s y[P+s*T+t][n] ),
// accumulated in fp32 in that fixed order (deterministic).  Four outputs
// per thread with 16-byte loads; the y rows of eight pairs are loaded
// before the first of their multiply-adds, so they are in flight together.
// Every y value is read once: non-temporal loads.
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ y, int ld_y, const float* __restrict__ topk_w,
    const int32_t* __restrict__ pair_pos, int T, int k, int H, int P,
    int n_shared, const float* __restrict__ sh_gate, void* __restrict__ out, int out_f32) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += 8) {
    int pp[8];
    float wj[8];
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool in = j0 + u < k;
      pp[u] = in ? pair_pos[t * k + j0 + u] : -1;
      wj[u] = in ? topk_w[t * k + j0 + u] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (pp[u] >= 0) {
        const f32x4_nt t = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_nt*>(y + (size_t)pp[u] * ld_y + n));
        v[u] = make_float4(t.x, t.y, t.z, t.w);
      } else {
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (pp[u] < 0) continue;
      acc.x = fmaf(wj[u], v[u].x, acc.x);
      acc.y = fmaf(wj[u], v[u].y, acc.y);
      acc.z = fmaf(wj[u], v[u].z, acc.z);
      acc.w = fmaf(wj[u], v[u].w, acc.w);
    }
  }
  for (int s = 0; s < n_shared; ++s) {
    const float4 v =
        *reinterpret_cast<const float4*>(y + (size_t)(P + s * T + t) * ld_y + n);
    // weight 1 (fmaf(1, v, acc) is acc + v) or the token's sigmoid gate
    const float g = sh_gate ? shared_gate_weight(sh_gate[t * n_shared + s]) : 1.0f;
    acc.x = fmaf(g, v.x, acc.x);
    acc.y = fmaf(g, v.y, acc.y);
    acc.z = fmaf(g, v.z, acc.z);
    acc.w = fmaf(g, v.w, acc.w);
  }
  if (out_f32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)t * H + n) = acc;
  } else {
    uint2 o;
    o.x = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
    o.y = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)t * H + n) = o;
  }
}

hipError_t launch_combine(const float* y, int ld_y, const float* topk_w,
                          const int32_t* pair_pos, int T, int k, int H, int P,
                          int n_shared, const float* sh_gate, void* out, int out_f32,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid((H / 4 + 255) / 256, T);
  combine_kernel<<<grid, 256, 0, st>>>(y, ld_y, topk_w, pair_pos, T, k, H, P,
                                       n_shared, sh_gate, out, out_f32);
  return hipGetLastError();
}

}  // namespace moe
