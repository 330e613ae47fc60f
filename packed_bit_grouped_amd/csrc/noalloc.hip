// moe_w4_layer_noalloc: the whole layer with no workspace argument, for
// callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).  The
// workspace the kernels use (error word, barrier flags, int8 rows, fp32
// per-pair outputs, fp16 activation copies) is the file-scope device
// array `scratch` below: one copy per GPU the library runs on, resident
// until the process ends.  Nothing here allocates.
#include <hip/hip_runtime.h>

#include <atomic>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch is used as a 256-byte aligned workspace");

// Zero-initialised when the code object is loaded on a device; every call
// leaves the barrier flags (bytes 256..4351) equal, as the layer requires.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of this device's copy of `scratch` (the array's name in
// host code is only a stand-in for the symbol, never an address).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

__global__ void err_clear_kernel(int32_t* w) { *w = 0; }

__global__ void err_report_kernel(const int32_t* w, int32_t* out) { *out = *w; }

}  // namespace

extern "C" moe_status moe_w4_layer_noalloc(
    int act, const float* logits, const uint16_t* x, int T, int H, int I, int E, int k,
    int renormalize, const moe_qmat* w13, const moe_qmat* w2, const moe_qmat* w13_shared,
    const moe_qmat* w2_shared, int n_shared, int I_shared, const float* shared_gate,
    int tile_m, int32_t* topk_ids,
    float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
    int32_t* tiles, int32_t* n_tiles, void* h, void* out, int32_t* err_out, int flags,
    void* stream) {
  if (act != MOE_A16 && act != MOE_A8) return MOE_E_INVAL;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || n_shared < 0) return MOE_E_INVAL;
  if (n_shared > 0 && I_shared <= 0) return MOE_E_INVAL;
  // the shape's workspace must fit the static array
  if (ws_layout(act, T, H, I, E, k, n_shared, I_shared).total > kScratchBytes)
    return MOE_E_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return MOE_E_DEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* err = static_cast<int32_t*>(ws);   // the workspace's error word
  if (err_out) {
    err_clear_kernel<<<1, 1, 0, s>>>(err);
    if (hipGetLastError() != hipSuccess) return MOE_E_DEVICE;
  }
  const moe_status st = moe_w4_layer(
      act, logits, x, T, H, I, E, k, renormalize, w13, w2, w13_shared, w2_shared, n_shared,
      I_shared, shared_gate, tile_m, topk_ids, topk_w, counts, offsets, sorted_pair, pair_pos, tiles,
      n_tiles, h, out, ws, kScratchBytes, flags, stream);
  if (st != MOE_OK || !err_out) return st;
  err_report_kernel<<<1, 1, 0, s>>>(err, err_out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_DEVICE;
}
