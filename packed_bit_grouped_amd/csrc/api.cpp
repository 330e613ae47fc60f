// C ABI of the MoE W4 FFN layer: host-side argument checks, workspace
// layout, path choice and kernel dispatch.  Nothing here allocates,
// synchronizes with the device or reads device memory (build log "Two 96 GB
// Ascend cards run Qwen3.8 Flash-Next", section "Remove sync and launch
// overhead from the token loop").
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

moe_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_E_DEVICE;
  if (dev < kMaxDevices) {
    const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return MOE_OK;
    if (c == 2) return MOE_E_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_E_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MOE_OK : MOE_E_DEVICE;
}

int g_cu_count[kMaxDevices];

// Compute units of the current device (queried once per device).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices && g_cu_count[dev] > 0) return g_cu_count[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < kMaxDevices) g_cu_count[dev] = n;
  return n;
}

// GEMV grid: one workgroup per CU, fewer when there is little work.
int gemv_grid(const ProjArgs& a) {
  const long long units = (long long)a.n_sh_slots * a.U_sh + (long long)a.max_tiles * a.U;
  long long g = (units + 15) / 16;
  const long long cap = cu_count();   // one 8-wave workgroup per CU (about 230 VGPRs)
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_DEVICE; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

// Shapes shared by both projections.
moe_status check_layer(int act, int T, int H, int I, int E, int k, int n_shared,
                       int I_shared, int tile_m, int flags) {
  if (act != MOE_A16 && act != MOE_A8) return MOE_E_INVAL;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || n_shared < 0) return MOE_E_INVAL;
  if (k > E) return MOE_E_INVAL;
  if (n_shared > 0 && I_shared <= 0) return MOE_E_INVAL;
  if (tile_m <= 0 || tile_m > 4096) return MOE_E_INVAL;
  if (flags & ~(MOE_PATH_MASK | MOE_QUANT_SEPARATE | MOE_OUT_F32 | MOE_W_PREPACKED |
                MOE_X_PREPARED))
    return MOE_E_INVAL;
  if (H % 32 || I % 32 || (n_shared > 0 && I_shared % 32)) return MOE_E_UNSUPPORTED;
  if (E > kPermMaxE) return MOE_E_UNSUPPORTED;
  if ((long long)T * k >= (1LL << 24)) return MOE_E_UNSUPPORTED;
  if ((long long)T * (k + n_shared) * H >= (1LL << 31)) return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

int ld_h_of(int I, int n_shared, int I_shared) {
  return n_shared > 0 && I_shared > I ? I_shared : I;
}

// The MFMA path covers bf16 activations, K dimensions that are whole
// pairs of 64-wide steps for int4 and int2 alike (H, I, I_shared % 128 ==
// 0), and fp16 activation copies the kernel addresses with 32-bit byte
// offsets (x: T*H, h: T*(k + n_shared) rows of max(I, I_shared)).
bool mfma_shape_ok(int act, int T, int H, int I, int k, int n_shared, int I_shared) {
  if (act != MOE_A16 || H % 128 != 0 || I % 128 != 0) return false;
  if (n_shared > 0 && I_shared % 128 != 0) return false;
  const long long ld_h = n_shared > 0 && I_shared > I ? I_shared : I;
  const long long rows = (long long)T * (k + n_shared);
  return (long long)T * H * 2 < (1LL << 31) && rows * ld_h * 2 < (1LL << 31);
}

// Decode batches up to this many pairs take the vector-ALU decode kernels
// (about one row per expert tile); larger ones the 16-row MFMA tiles.
constexpr long long kDecPairs = 64;

bool use_mfma(int act, int T, int H, int I, int E, int k, int n_shared,
              int I_shared, int flags) {
  const int path = flags & MOE_PATH_MASK;
  if (path == MOE_PATH_GEMV || path == MOE_PATH_MFMA16) return false;
  if (path == MOE_PATH_MFMA) return true;
  return mfma_available() && mfma_shape_ok(act, T, H, I, k, n_shared, I_shared) &&
         (long long)T * k >= 32LL * E;
}

}  // namespace

namespace moe {
WsLayout ws_layout(int act, int T, int H, int I, int E, int k, int n_shared,
                   int I_shared) {
  (void)I; (void)E; (void)I_shared;
  WsLayout L;
  size_t off = 0;
  L.err = off;
  off += 256;
  L.flags = off;
  off += kLayerFlags * 4;
  L.qx = off;
  if (act == MOE_A8) off += up256((size_t)T * H);
  L.sx = off;
  if (act == MOE_A8) off += up256((size_t)T * 4);
  L.qh = off;
  L.sh = off;
  if (act == MOE_A8) {
    const size_t R = (size_t)T * (k + n_shared);
    off += up256(R * (size_t)ld_h_of(I, n_shared, I_shared));
    L.sh = off;
    off += up256(R * 4);
  }
  L.y = off;
  off += up256((size_t)T * (k + n_shared) * H * 4);
  L.perm = off;
  off += up256((size_t)permute_multi_blocks((int)((long long)T * k)) * E * 4);
  L.a16 = off;
  L.h16 = off;
  if (act == MOE_A16 && mfma_shape_ok(act, T, H, I, k, n_shared, I_shared)) {
    const size_t ld_h = (size_t)(n_shared > 0 && I_shared > I ? I_shared : I);
    const size_t xs = (size_t)T * H * 2;
    const size_t hs = (size_t)T * (k + n_shared) * ld_h * 2;
    off += up256(xs > hs ? xs : hs);
    L.h16 = off;
    off += up256(hs);
  }
  L.total = off;
  return L;
}
}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_W4_ABI_VERSION; }

const char* moe_status_str(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_INVAL: return "invalid argument";
    case MOE_E_UNSUPPORTED: return "unsupported shape or format";
    case MOE_E_DEVICE: return "HIP error or device is not gfx950";
    case MOE_E_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int moe_permute_max_tiles(int T, int k, int E, int tile_m) {
  if (T <= 0 || k <= 0 || E <= 0 || tile_m <= 0) return 0;
  const long long P = (long long)T * k;
  const long long b = P / tile_m + (E < P ? E : P);
  return (int)(b < P ? b : P);
}

int moe_preferred_tile_m(int act, int T, int E, int k) {
  if (act == MOE_A16 && (long long)T * k >= 32LL * E) return 160;
  return 16;
}

size_t moe_workspace_bytes(int act, int T, int H, int I, int E, int k,
                           int n_shared, int I_shared) {
  if (T < 0 || H <= 0 || k <= 0 || n_shared < 0) return 0;
  return ws_layout(act, T, H, I, E, k, n_shared, I_shared).total;
}

static moe_status route_topk_impl(const float* logits, int T, int E, int k,
                                  int renormalize, int32_t* topk_ids, float* topk_w,
                                  void* stream, const XPrep* xp) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return MOE_E_INVAL;
  if (renormalize != 0 && renormalize != 1) return MOE_E_INVAL;
  if (E > kRouteMaxE) return MOE_E_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_E_INVAL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(launch_route_topk(logits, T, E, k, renormalize, topk_ids,
                                    topk_w, static_cast<hipStream_t>(stream), xp));
}

moe_status moe_route_topk(const float* logits, int T, int E, int k,
                          int renormalize, int32_t* topk_ids, float* topk_w,
                          void* stream) {
  return route_topk_impl(logits, T, E, k, renormalize, topk_ids, topk_w, stream, nullptr);
}

size_t moe_router_workspace_bytes(int T, int H, int E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  return router_workspace_bytes(T, H, E);
}

moe_status moe_router_topk(const uint16_t* x, int T, int H, const float* router_w,
                           const float* prior, int E, int k, int renormalize, float* logits,
                           int32_t* topk_ids, float* topk_w, void* workspace, size_t ws_bytes,
                           void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > E) return MOE_E_INVAL;
  if (renormalize != 0 && renormalize != 1) return MOE_E_INVAL;
  if (E > kRouteMaxE) return MOE_E_UNSUPPORTED;
  if ((long long)T * H >= (1LL << 31) || (long long)H * E >= (1LL << 31) ||
      (long long)T * E >= (1LL << 31))
    return MOE_E_UNSUPPORTED;
  if ((T + 63) / 64 > 65535) return MOE_E_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !router_w || !logits || !topk_ids || !topk_w) return MOE_E_INVAL;
  const size_t need = router_workspace_bytes(T, H, E);
  if (need > 0 && (!workspace || !aligned(workspace, 16) || ws_bytes < need))
    return MOE_E_WORKSPACE;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = launch_router_logits(x, T, H, router_w, E, prior, logits,
                                            static_cast<float*>(workspace), s);
  if (e != hipSuccess) return MOE_E_DEVICE;
  return from_hip(launch_route_topk(logits, T, E, k, renormalize, topk_ids, topk_w, s));
}

moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E,
                       int tile_m, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_pair, int32_t* pair_pos,
                       int32_t* tiles, int32_t* n_tiles, void* stream) {
  if (T < 0 || k <= 0 || E <= 0 || tile_m <= 0 || tile_m > 4096) return MOE_E_INVAL;
  if (E > kPermMaxE) return MOE_E_UNSUPPORTED;
  if ((long long)T * k >= (1LL << 24)) return MOE_E_UNSUPPORTED;
  if (!counts || !offsets || !n_tiles) return MOE_E_INVAL;
  if (T > 0 && (!topk_ids || !sorted_pair || !pair_pos || !tiles)) return MOE_E_INVAL;
  if (tiles && !aligned(tiles, 16)) return MOE_E_INVAL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(launch_permute(topk_ids, T * k, E, tile_m, counts, offsets,
                                 sorted_pair, pair_pos, tiles, n_tiles,
                                 static_cast<hipStream_t>(stream)));
}

static moe_status route_permute_impl(const float* logits, int T, int E, int k,
                                     int renormalize, int tile_m, int32_t* topk_ids,
                                     float* topk_w, int32_t* counts, int32_t* offsets,
                                     int32_t* sorted_pair, int32_t* pair_pos,
                                     int32_t* tiles, int32_t* n_tiles, void* stream,
                                     const XPrep* xq) {
  if (T < 0 || E <= 0 || k <= 0 || k > E || tile_m <= 0 || tile_m > 4096) return MOE_E_INVAL;
  if (renormalize != 0 && renormalize != 1) return MOE_E_INVAL;
  if (E > kPermMaxE || T > kFusedRouteMaxT || T * k > kFusedRouteMaxP) return MOE_E_UNSUPPORTED;
  if (!counts || !offsets || !n_tiles) return MOE_E_INVAL;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_pair || !pair_pos || !tiles))
    return MOE_E_INVAL;
  if (tiles && !aligned(tiles, 16)) return MOE_E_INVAL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(launch_route_permute(logits, T, E, k, renormalize, tile_m,
                                       topk_ids, topk_w, counts, offsets,
                                       sorted_pair, pair_pos, tiles, n_tiles,
                                       static_cast<hipStream_t>(stream), xq));
}

moe_status moe_route_permute(const float* logits, int T, int E, int k,
                             int renormalize, int tile_m, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_pair, int32_t* pair_pos,
                             int32_t* tiles, int32_t* n_tiles, void* stream) {
  return route_permute_impl(logits, T, E, k, renormalize, tile_m, topk_ids, topk_w, counts,
                            offsets, sorted_pair, pair_pos, tiles, n_tiles, stream, nullptr);
}

moe_status moe_quant_a8_rows(const void* src, int src_is_f32, int R, int C,
                             int ld, int8_t* q, float* s, void* stream) {
  if (R < 0 || C <= 0 || ld < C) return MOE_E_INVAL;
  if (src_is_f32 != 0 && src_is_f32 != 1) return MOE_E_INVAL;
  if (R == 0) return MOE_OK;
  if (!src || !q || !s) return MOE_E_INVAL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(launch_quant_a8(src, src_is_f32, R, C, ld, q, C, s,
                                  static_cast<hipStream_t>(stream)));
}

static moe_status gateup_impl(int act, const uint16_t* x, int T, int H, int I,
                              int E, int k, const moe_qmat* w13,
                              const moe_qmat* w13_shared, int n_shared,
                              int I_shared, const int32_t* offsets,
                              const int32_t* sorted_pair, const int32_t* tiles,
                              const int32_t* n_tiles, int tile_m, void* h,
                              void* workspace, size_t ws_bytes, int flags,
                              int32_t* partials, int ng_ld, void* stream,
                              bool stage_h16 = false) {
  moe_status st = check_layer(act, T, H, I, E, k, n_shared, I_shared, tile_m, flags);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !w13 || !offsets || !sorted_pair || !tiles || !n_tiles || !h) return MOE_E_INVAL;
  if (n_shared > 0 && !w13_shared) return MOE_E_INVAL;
  if (!aligned(x, 16) || !aligned(h, 16) || !aligned(tiles, 16)) return MOE_E_INVAL;
  const WsLayout L = ws_layout(act, T, H, I, E, k, n_shared, I_shared);
  if (!workspace || !aligned(workspace, 256) || ws_bytes < L.total) return MOE_E_WORKSPACE;
  if (partials && ng_ld <= 0) return MOE_E_INVAL;
  const int path = flags & MOE_PATH_MASK;
  const bool m16 = m16_ok(act, 0, T, H, H, tile_m);
  if (path == MOE_PATH_MFMA16 && !m16) return MOE_E_UNSUPPORTED;
  if (path == MOE_PATH_MFMA && !mfma_shape_ok(act, T, H, I, k, n_shared, I_shared))
    return MOE_E_UNSUPPORTED;
  st = check_device();
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int ld_h = ld_h_of(I, n_shared, I_shared);

  ProjArgs a;
  std::memset(&a, 0, sizeof(a));
  a.mode = 0;
  a.ld_in = H;
  a.w = w13;
  a.w_sh = w13_shared;
  a.K = H;
  a.K_sh = H;
  a.U = I;
  a.U_sh = n_shared > 0 ? I_shared : 0;
  a.T = T;
  a.k = k;
  a.P = T * k;
  a.E = E;
  a.n_shared = n_shared;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.tiles = tiles;
  a.n_tiles = n_tiles;
  a.max_tiles = moe_permute_max_tiles(T, k, E, tile_m);
  a.out = h;
  a.ld_out = ld_h;
  a.err = reinterpret_cast<int32_t*>(ws + L.err);
  a.partials = partials;
  a.ng_ld = ng_ld;
  a.part_rows = 2 * ld_h;

  const bool pp = (flags & MOE_W_PREPACKED) != 0;
  if (use_mfma(act, T, H, I, E, k, n_shared, I_shared, flags)) {
    if (!mfma_shape_ok(act, T, H, I, k, n_shared, I_shared)) return MOE_E_UNSUPPORTED;
    a.in_bf16 = x;
    uint16_t* x16 = reinterpret_cast<uint16_t*>(ws + L.a16);
    // the routing launch of moe_w4_layer made the fp16 copy of x already
    if (flags & MOE_X_PREPARED) a.in16_ready = 1;
    if (stage_h16) a.out16 = reinterpret_cast<uint16_t*>(ws + L.h16);
    return from_hip(launch_proj_mfma8(a, x16, pp, s));
  }
  if (pp) return MOE_E_UNSUPPORTED;   // the prepacked layout is read by the matrix-core path only
  const bool dec = act == MOE_A16 && !partials && dec_gateup_ok(T, H, tile_m);
  const bool on_m16 = path == MOE_PATH_MFMA16 ||
                      (path == MOE_PATH_AUTO && m16 && !(dec && (long long)T * k <= kDecPairs));
  a.in_bf16 = x;
  if (act == MOE_A8 && (flags & MOE_X_PREPARED)) {
    // the int8 rows the routing launch of moe_w4_route_gateup_silu made
    a.in_q = reinterpret_cast<const int8_t*>(ws + L.qx);
    a.in_s = reinterpret_cast<const float*>(ws + L.sx);
  } else if (act == MOE_A8 &&
             !(on_m16 && !(flags & MOE_QUANT_SEPARATE) && m16_quant_ok(0, T, H, H))) {
    // int8 x rows for the kernels that read them (the 16-row matrix tiles
    // quantize their staged rows themselves when a tile's rows fit)
    int8_t* qx = reinterpret_cast<int8_t*>(ws + L.qx);
    float* sx = reinterpret_cast<float*>(ws + L.sx);
    hipError_t e = launch_quant_a8(x, 0, T, H, H, qx, H, sx, s);
    if (e != hipSuccess) return MOE_E_DEVICE;
    a.in_q = qx;
    a.in_s = sx;
  }
  if (on_m16) return from_hip(launch_proj_m16(a, act, s));
  a.maxt = gemv_maxt(T, tile_m);
  a.sh_tile = a.maxt;
  a.n_sh_slots = n_shared * ((T + a.sh_tile - 1) / a.sh_tile);
  if (dec) {
    a.maxt = dec_maxt(T, tile_m);
    return from_hip(launch_dec_gateup(a, s));
  }
  return from_hip(launch_proj_gemv(a, act, gemv_grid(a), s));
}

static moe_status down_impl(int act, const void* h, int T, int H, int I, int E,
                            int k, const moe_qmat* w2, const moe_qmat* w2_shared,
                            int n_shared, int I_shared, const float* shared_gate,
                            const float* topk_w,
                            const int32_t* offsets, const int32_t* sorted_pair,
                            const int32_t* pair_pos, const int32_t* tiles,
                            const int32_t* n_tiles, int tile_m, void* out,
                            void* workspace, size_t ws_bytes, int flags,
                            int32_t* partials, int ng_ld, void* stream,
                            bool h16_staged = false) {
  moe_status st = check_layer(act, T, H, I, E, k, n_shared, I_shared, tile_m, flags);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!h || !w2 || !topk_w || !offsets || !sorted_pair || !pair_pos || !tiles ||
      !n_tiles || !out)
    return MOE_E_INVAL;
  if (n_shared > 0 && !w2_shared) return MOE_E_INVAL;
  const int out_f32 = (flags & MOE_OUT_F32) ? 1 : 0;
  if (!aligned(h, 16) || !aligned(out, out_f32 ? 16 : 8) || !aligned(tiles, 16))
    return MOE_E_INVAL;
  const WsLayout L = ws_layout(act, T, H, I, E, k, n_shared, I_shared);
  if (!workspace || !aligned(workspace, 256) || ws_bytes < L.total) return MOE_E_WORKSPACE;
  if (partials && ng_ld <= 0) return MOE_E_INVAL;
  const int path = flags & MOE_PATH_MASK;
  const bool m16 = m16_ok(act, 1, T, I, n_shared > 0 ? I_shared : I, tile_m);
  if (path == MOE_PATH_MFMA16 && !m16) return MOE_E_UNSUPPORTED;
  if (path == MOE_PATH_MFMA && !mfma_shape_ok(act, T, H, I, k, n_shared, I_shared))
    return MOE_E_UNSUPPORTED;
  st = check_device();
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int ld_h = ld_h_of(I, n_shared, I_shared);
  float* y = reinterpret_cast<float*>(ws + L.y);

  ProjArgs a;
  std::memset(&a, 0, sizeof(a));
  a.mode = 1;
  a.ld_in = ld_h;
  a.w = w2;
  a.w_sh = w2_shared;
  a.K = I;
  a.K_sh = n_shared > 0 ? I_shared : I;
  a.U = H;
  a.U_sh = H;
  a.T = T;
  a.k = k;
  a.P = T * k;
  a.E = E;
  a.n_shared = n_shared;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.tiles = tiles;
  a.n_tiles = n_tiles;
  a.max_tiles = moe_permute_max_tiles(T, k, E, tile_m);
  a.out = y;
  a.ld_out = H;
  a.err = reinterpret_cast<int32_t*>(ws + L.err);
  a.partials = partials;
  a.ng_ld = ng_ld;
  a.part_rows = H;

  hipError_t e;
  const bool pp = (flags & MOE_W_PREPACKED) != 0;
  if (use_mfma(act, T, H, I, E, k, n_shared, I_shared, flags)) {
    if (!mfma_shape_ok(act, T, H, I, k, n_shared, I_shared)) return MOE_E_UNSUPPORTED;
    a.in_bf16 = static_cast<const uint16_t*>(h);
    if (h16_staged) {
      a.in_bf16 = reinterpret_cast<const uint16_t*>(ws + L.h16);
      a.in16_ready = 1;
    }
    e = launch_proj_mfma8(a, reinterpret_cast<uint16_t*>(ws + L.a16), pp, s);
    if (e != hipSuccess) return MOE_E_DEVICE;
    return from_hip(launch_combine(y, H, topk_w, pair_pos, T, k, H, T * k,
                                   n_shared, shared_gate, out, out_f32, s));
  }
  if (pp) return MOE_E_UNSUPPORTED;   // the prepacked layout is read by the matrix-core path only
  if (act == MOE_A8) a.in_f32 = static_cast<const float*>(h);
  else a.in_bf16 = static_cast<const uint16_t*>(h);
  const bool dec = act == MOE_A16 && !partials &&
                   dec_down_ok(T, k, E, n_shared, H, I, I_shared, ld_h, tile_m, a.max_tiles);
  if (path == MOE_PATH_MFMA16 ||
      (path == MOE_PATH_AUTO && m16 && !(dec && (long long)T * k <= kDecPairs))) {
    if (act == MOE_A8 && !m16_quant_ok(1, T, I, n_shared > 0 ? I_shared : I)) {
      // int8 h rows for the int8 MFMA (made in the kernel when a tile's rows fit)
      int8_t* qh = reinterpret_cast<int8_t*>(ws + L.qh);
      float* sh = reinterpret_cast<float*>(ws + L.sh);
      const int P = T * k;
      e = launch_quant_a8(h, 1, P, I, ld_h, qh, ld_h, sh, s);
      if (e == hipSuccess && n_shared > 0)
        e = launch_quant_a8(static_cast<const float*>(h) + (size_t)P * ld_h, 1, n_shared * T,
                            I_shared, ld_h, qh + (size_t)P * ld_h, ld_h, sh + P, s);
      if (e != hipSuccess) return MOE_E_DEVICE;
      a.in_q = qh;
      a.in_s = sh;
    }
    e = launch_proj_m16(a, act, s);
    if (e != hipSuccess) return MOE_E_DEVICE;
    return from_hip(launch_combine(y, H, topk_w, pair_pos, T, k, H, T * k,
                                   n_shared, shared_gate, out, out_f32, s));
  }
  a.maxt = gemv_maxt(T, tile_m);
  a.sh_tile = a.maxt;
  a.n_sh_slots = n_shared * ((T + a.sh_tile - 1) / a.sh_tile);
  if (dec) {
    a.maxt = dec_maxt(T, tile_m);
    a.topk_w = topk_w;
    a.pair_pos = pair_pos;
    a.out_f32 = out_f32;
    a.sh_gate = n_shared > 0 ? shared_gate : nullptr;
    return from_hip(launch_dec_down_combine(a, out, s));
  }
  e = launch_proj_gemv(a, act, gemv_grid(a), s);
  if (e != hipSuccess) return MOE_E_DEVICE;
  return from_hip(launch_combine(y, H, topk_w, pair_pos, T, k, H, T * k,
                                 n_shared, shared_gate, out, out_f32, s));
}

moe_status moe_w4_gateup_silu(int act, const uint16_t* x, int T, int H, int I,
                              int E, int k, const moe_qmat* w13,
                              const moe_qmat* w13_shared, int n_shared,
                              int I_shared, const int32_t* offsets,
                              const int32_t* sorted_pair,
                              const int32_t* tiles, const int32_t* n_tiles,
                              int tile_m, void* h, void* workspace,
                              size_t ws_bytes, int flags, void* stream) {
  return gateup_impl(act, x, T, H, I, E, k, w13, w13_shared, n_shared, I_shared,
                     offsets, sorted_pair, tiles, n_tiles, tile_m, h, workspace,
                     ws_bytes, flags, nullptr, 0, stream);
}

moe_status moe_w4_route_gateup_silu(int act, const float* logits, const uint16_t* x, int T,
                                    int H, int I, int E, int k, int renormalize,
                                    const moe_qmat* w13, const moe_qmat* w13_shared,
                                    int n_shared, int I_shared, int tile_m, int32_t* topk_ids,
                                    float* topk_w, int32_t* counts, int32_t* offsets,
                                    int32_t* sorted_pair, int32_t* pair_pos, int32_t* tiles,
                                    int32_t* n_tiles, void* h, void* workspace,
                                    size_t ws_bytes, int flags, void* stream) {
  moe_status st = check_layer(act, T, H, I, E, k, n_shared, I_shared, tile_m, flags);
  if (st != MOE_OK) return st;
  if (renormalize != 0 && renormalize != 1) return MOE_E_INVAL;
  flags &= ~MOE_X_PREPARED;   // x is routed here: its int8 rows are made here too
  const bool fused = act == MOE_A16 && T > 0 && (flags & MOE_PATH_MASK) != MOE_PATH_MFMA16 &&
                     !(flags & MOE_W_PREPACKED) &&
                     !use_mfma(act, T, H, I, E, k, n_shared, I_shared, flags) &&
                     dec_route_gateup_ok(T, H, E, k, tile_m);
  if (!fused) {
    // the two calls, each with its own checks
    if (T <= kFusedRouteMaxT && (long long)T * k <= kFusedRouteMaxP && E <= kPermMaxE) {
      // W4A8: the routing launch also makes x's int8 rows (one extra
      // workgroup per token) and the gate/up call reads them
      const bool xq_ok = act == MOE_A8 && T > 0 && !(flags & MOE_QUANT_SEPARATE) &&
                         x && aligned(x, 16) && H % 8 == 0 &&
                         workspace && aligned(workspace, 256) &&
                         ws_bytes >= ws_layout(act, T, H, I, E, k, n_shared, I_shared).total;
      XPrep xq = {nullptr, 0, nullptr, nullptr, nullptr};
      if (xq_ok) {
        const WsLayout L = ws_layout(act, T, H, I, E, k, n_shared, I_shared);
        char* ws = static_cast<char*>(workspace);
        xq = XPrep{x, H, reinterpret_cast<int8_t*>(ws + L.qx),
                   reinterpret_cast<float*>(ws + L.sx), nullptr};
        flags |= MOE_X_PREPARED;
      }
      st = route_permute_impl(logits, T, E, k, renormalize, tile_m, topk_ids, topk_w, counts,
                              offsets, sorted_pair, pair_pos, tiles, n_tiles, stream,
                              xq_ok ? &xq : nullptr);
    } else {
      st = moe_route_topk(logits, T, E, k, renormalize, topk_ids, topk_w, stream);
      if (st == MOE_OK)
        st = moe_permute(topk_ids, T, k, E, tile_m, counts, offsets, sorted_pair, pair_pos,
                         tiles, n_tiles, stream);
    }
    if (st != MOE_OK) return st;
    return moe_w4_gateup_silu(act, x, T, H, I, E, k, w13, w13_shared, n_shared, I_shared,
                              offsets, sorted_pair, tiles, n_tiles, tile_m, h, workspace,
                              ws_bytes, flags, stream);
  }
  if (!logits || !x || !w13 || !topk_ids || !topk_w || !counts || !offsets || !sorted_pair ||
      !pair_pos || !tiles || !n_tiles || !h)
    return MOE_E_INVAL;
  if (n_shared > 0 && !w13_shared) return MOE_E_INVAL;
  if (!aligned(x, 16) || !aligned(h, 16) || !aligned(tiles, 16)) return MOE_E_INVAL;
  const WsLayout L = ws_layout(act, T, H, I, E, k, n_shared, I_shared);
  if (!workspace || !aligned(workspace, 256) || ws_bytes < L.total) return MOE_E_WORKSPACE;
  st = check_device();
  if (st != MOE_OK) return st;
  char* ws = static_cast<char*>(workspace);
  ProjArgs a;
  std::memset(&a, 0, sizeof(a));
  a.mode = 0;
  a.in_bf16 = x;
  a.ld_in = H;
  a.w = w13;
  a.w_sh = w13_shared;
  a.K = H;
  a.K_sh = H;
  a.U = I;
  a.U_sh = n_shared > 0 ? I_shared : 0;
  a.T = T;
  a.k = k;
  a.P = T * k;
  a.E = E;
  a.n_shared = n_shared;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.tiles = tiles;
  a.n_tiles = n_tiles;
  a.max_tiles = moe_permute_max_tiles(T, k, E, tile_m);
  a.maxt = dec_maxt(T, tile_m);
  a.out = h;
  a.ld_out = ld_h_of(I, n_shared, I_shared);
  a.err = reinterpret_cast<int32_t*>(ws + L.err);
  return from_hip(launch_dec_route_gateup(a, logits, renormalize, tile_m, topk_ids, topk_w,
                                          counts, offsets, sorted_pair, pair_pos, tiles,
                                          n_tiles, static_cast<hipStream_t>(stream)));
}

moe_status moe_w4_down_combine(int act, const void* h, int T, int H, int I,
                               int E, int k, const moe_qmat* w2,
                               const moe_qmat* w2_shared, int n_shared,
                               int I_shared, const float* shared_gate,
                               const float* topk_w,
                               const int32_t* offsets,
                               const int32_t* sorted_pair,
                               const int32_t* pair_pos, const int32_t* tiles,
                               const int32_t* n_tiles, int tile_m,
                               void* out, void* workspace,
                               size_t ws_bytes, int flags, void* stream) {
  return down_impl(act, h, T, H, I, E, k, w2, w2_shared, n_shared, I_shared,
                   shared_gate, topk_w, offsets, sorted_pair, pair_pos, tiles, n_tiles,
                   tile_m, out, workspace, ws_bytes, flags, nullptr, 0, stream);
}

moe_status moe_dbg_w4a8_gateup_partials(
    const uint16_t* x, int T, int H, int I, int E, int k,
    const moe_qmat* w13, const moe_qmat* w13_shared, int n_shared,
    int I_shared, const int32_t* offsets, const int32_t* sorted_pair,
    const int32_t* tiles, const int32_t* n_tiles, int tile_m, void* h,
    void* workspace, size_t ws_bytes, int flags, int32_t* partials, int ng_ld,
    void* stream) {
  if (!partials) return MOE_E_INVAL;
  if ((flags & MOE_PATH_MASK) == MOE_PATH_MFMA) return MOE_E_UNSUPPORTED;   // A16 only
  return gateup_impl(MOE_A8, x, T, H, I, E, k, w13, w13_shared, n_shared,
                     I_shared, offsets, sorted_pair, tiles, n_tiles, tile_m, h,
                     workspace, ws_bytes, flags, partials, ng_ld, stream);
}

moe_status moe_dbg_w4a8_down_partials(
    const void* h, int T, int H, int I, int E, int k, const moe_qmat* w2,
    const moe_qmat* w2_shared, int n_shared, int I_shared,
    const float* shared_gate, const float* topk_w, const int32_t* offsets, const int32_t* sorted_pair,
    const int32_t* pair_pos, const int32_t* tiles, const int32_t* n_tiles,
    int tile_m, void* out, void* workspace, size_t ws_bytes, int flags,
    int32_t* partials, int ng_ld, void* stream) {
  if (!partials) return MOE_E_INVAL;
  if ((flags & MOE_PATH_MASK) == MOE_PATH_MFMA) return MOE_E_UNSUPPORTED;   // A16 only
  return down_impl(MOE_A8, h, T, H, I, E, k, w2, w2_shared, n_shared, I_shared,
                   shared_gate, topk_w, offsets, sorted_pair, pair_pos, tiles, n_tiles,
                   tile_m, out, workspace, ws_bytes, flags, partials,
                   ng_ld, stream);
}

}  // extern "C"

extern "C" moe_status moe_w4_prepack(const uint8_t* codes, int bits, int N, int K, int gate_up,
                                     uint8_t* dst, void* stream) {
  if (bits != 2 && bits != 4) return MOE_E_UNSUPPORTED;
  if (N <= 0 || K <= 0 || (gate_up != 0 && gate_up != 1)) return MOE_E_INVAL;
  if (N % (gate_up ? 64 : 32) != 0 || K % 128 != 0) return MOE_E_UNSUPPORTED;
  if ((long long)N * K * bits / 8 >= (1LL << 31)) return MOE_E_UNSUPPORTED;
  if (!codes || !dst || codes == dst) return MOE_E_INVAL;
  if (!aligned(codes, 16) || !aligned(dst, 16)) return MOE_E_INVAL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(launch_prepack(codes, bits, N, K, gate_up, dst,
                                 static_cast<hipStream_t>(stream)));
}

extern "C" moe_status moe_w4_prepack_scales(const uint16_t* scales, int N, int K, int group,
                                            int gate_up, uint16_t* dst, void* stream) {
  if (N <= 0 || K <= 0 || (gate_up != 0 && gate_up != 1)) return MOE_E_INVAL;
  if (group != 32 && group != 64 && group != 128 && group != 256) return MOE_E_UNSUPPORTED;
  if (K % group != 0 || N % 64 != 0 || K / group > 64) return MOE_E_UNSUPPORTED;
  if ((long long)N * (K / group) * 2 >= (1LL << 31)) return MOE_E_UNSUPPORTED;
  if (!scales || !dst || scales == dst) return MOE_E_INVAL;
  if (!aligned(scales, 4) || !aligned(dst, 16)) return MOE_E_INVAL;
  const moe_status d = check_device();
  if (d != MOE_OK) return d;
  return from_hip(launch_prepack_scales(scales, N, K / group, gate_up, dst,
                                        static_cast<hipStream_t>(stream)));
}

// Shapes and flags for which moe_w4_layer issues one launch (before the
// device's residency check).
static bool layer_one_shape(int act, int T, int H, int I, int E, int k, int n_shared,
                            int I_shared, int tile_m, int flags) {
  const int path = flags & MOE_PATH_MASK;
  return act == MOE_A16 && T > 0 && (path == MOE_PATH_AUTO || path == MOE_PATH_GEMV) &&
         !(flags & MOE_W_PREPACKED) &&
         !use_mfma(act, T, H, I, E, k, n_shared, I_shared, flags) &&
         dec_layer_ok(T, H, I, I_shared, E, k, n_shared, tile_m,
                      moe_permute_max_tiles(T, k, E, tile_m), ld_h_of(I, n_shared, I_shared));
}

int moe_w4_layer_one_launch(int act, int T, int H, int I, int E, int k, int n_shared,
                            int I_shared, int tile_m, int flags) {
  const bool one = (flags & MOE_LAYER_ONE_LAUNCH) != 0;
  flags &= ~MOE_LAYER_ONE_LAUNCH;
  moe_status st = check_layer(act, T, H, I, E, k, n_shared, I_shared, tile_m, flags);
  if (st != MOE_OK) return st;
  if (!one) return 0;
  if (!layer_one_shape(act, T, H, I, E, k, n_shared, I_shared, tile_m, flags)) return 0;
  st = check_device();
  if (st != MOE_OK) return st;
  return dec_layer_one_launch(T, H, I, I_shared, E, k, n_shared, tile_m,
                              moe_permute_max_tiles(T, k, E, tile_m),
                              ld_h_of(I, n_shared, I_shared));
}

moe_status moe_w4_layer(int act, const float* logits, const uint16_t* x, int T, int H, int I,
                        int E, int k, int renormalize, const moe_qmat* w13, const moe_qmat* w2,
                        const moe_qmat* w13_shared, const moe_qmat* w2_shared, int n_shared,
                        int I_shared, const float* shared_gate, int tile_m, int32_t* topk_ids, float* topk_w,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                        int32_t* pair_pos, int32_t* tiles, int32_t* n_tiles, void* h,
                        void* out, void* workspace, size_t ws_bytes, int flags,
                        void* stream) {
  const bool one = (flags & MOE_LAYER_ONE_LAUNCH) != 0;
  flags &= ~MOE_LAYER_ONE_LAUNCH;   // the component calls do not take it
  moe_status st = check_layer(act, T, H, I, E, k, n_shared, I_shared, tile_m, flags);
  if (st != MOE_OK) return st;
  if (renormalize != 0 && renormalize != 1) return MOE_E_INVAL;
  const int ld_h = ld_h_of(I, n_shared, I_shared);
  const int max_tiles = moe_permute_max_tiles(T, k, E, tile_m);
  // every argument of both calls, before either form issues anything
  if (T > 0) {
    if (!logits || !x || !w13 || !w2 || !topk_ids || !topk_w || !counts || !offsets ||
        !sorted_pair || !pair_pos || !tiles || !n_tiles || !h || !out)
      return MOE_E_INVAL;
    if (n_shared > 0 && (!w13_shared || !w2_shared)) return MOE_E_INVAL;
    if (!aligned(x, 16) || !aligned(h, 16) || !aligned(tiles, 16) ||
        !aligned(out, (flags & MOE_OUT_F32) ? 16 : 8))
      return MOE_E_INVAL;
  }
  const WsLayout L = ws_layout(act, T, H, I, E, k, n_shared, I_shared);
  if (!workspace || !aligned(workspace, 256) || ws_bytes < L.total) return MOE_E_WORKSPACE;
  if (one && layer_one_shape(act, T, H, I, E, k, n_shared, I_shared, tile_m, flags)) {
    st = check_device();
    if (st != MOE_OK) return st;
    char* ws = static_cast<char*>(workspace);
    ProjArgs ag, ad;
    std::memset(&ag, 0, sizeof(ag));
    std::memset(&ad, 0, sizeof(ad));
    ag.mode = 0;
    ag.in_bf16 = x;
    ag.ld_in = H;
    ag.w = w13;
    ag.w_sh = w13_shared;
    ag.K = H;
    ag.K_sh = H;
    ag.U = I;
    ag.U_sh = n_shared > 0 ? I_shared : 0;
    ad.mode = 1;
    ad.in_bf16 = static_cast<const uint16_t*>(h);
    ad.ld_in = ld_h;
    ad.w = w2;
    ad.w_sh = w2_shared;
    ad.K = I;
    ad.K_sh = n_shared > 0 ? I_shared : I;
    ad.U = H;
    ad.U_sh = H;
    for (ProjArgs* a : {&ag, &ad}) {
      a->T = T;
      a->k = k;
      a->P = T * k;
      a->E = E;
      a->n_shared = n_shared;
      a->offsets = offsets;
      a->sorted_pair = sorted_pair;
      a->tiles = tiles;
      a->n_tiles = n_tiles;
      a->max_tiles = max_tiles;
      a->maxt = dec_maxt(T, tile_m);
      a->err = reinterpret_cast<int32_t*>(ws + L.err);
    }
    ag.out = h;
    ag.ld_out = ld_h;
    ad.topk_w = topk_w;
    ad.pair_pos = pair_pos;
    ad.out_f32 = (flags & MOE_OUT_F32) ? 1 : 0;
    ad.sh_gate = n_shared > 0 ? shared_gate : nullptr;
    bool launched = false;
    const hipError_t e = launch_dec_layer(
        ag, ad, logits, renormalize, tile_m, topk_ids, topk_w, counts, offsets, sorted_pair,
        pair_pos, tiles, n_tiles, out, reinterpret_cast<uint32_t*>(ws + L.flags), launched,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return MOE_E_DEVICE;
    if (launched) return MOE_OK;
  }
  if (T > 0 && use_mfma(act, T, H, I, E, k, n_shared, I_shared, flags) &&
      mfma_shape_ok(act, T, H, I, k, n_shared, I_shared)) {
    // matrix-core form: the routing launch also makes the fp16 copy of x the
    // gate/up stages (extra workgroups), and the gate/up epilogue writes the
    // fp16 copy of h the down projection reads, so no conversion pass runs
    const XPrep xp = {x, H, nullptr, nullptr,
                      reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + L.a16)};
    if (T <= kFusedRouteMaxT && (long long)T * k <= kFusedRouteMaxP && E <= kPermMaxE) {
      st = route_permute_impl(logits, T, E, k, renormalize, tile_m, topk_ids, topk_w, counts,
                              offsets, sorted_pair, pair_pos, tiles, n_tiles, stream, &xp);
    } else {
      st = route_topk_impl(logits, T, E, k, renormalize, topk_ids, topk_w, stream, &xp);
      if (st == MOE_OK && permute_multi_blocks(T * k) > 0) {
        // the sort over many workgroups, with its counts in the workspace
        st = from_hip(launch_permute_multi(
            topk_ids, T * k, E, tile_m, counts, offsets, sorted_pair, pair_pos, tiles, n_tiles,
            reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + L.perm),
            static_cast<hipStream_t>(stream)));
      } else if (st == MOE_OK) {
        st = moe_permute(topk_ids, T, k, E, tile_m, counts, offsets, sorted_pair, pair_pos,
                         tiles, n_tiles, stream);
      }
    }
    if (st != MOE_OK) return st;
    st = gateup_impl(act, x, T, H, I, E, k, w13, w13_shared, n_shared, I_shared, offsets,
                     sorted_pair, tiles, n_tiles, tile_m, h, workspace, ws_bytes,
                     flags | MOE_X_PREPARED, nullptr, 0, stream, true);
    if (st != MOE_OK) return st;
    return down_impl(act, h, T, H, I, E, k, w2, w2_shared, n_shared, I_shared, shared_gate,
                     topk_w, offsets, sorted_pair, pair_pos, tiles, n_tiles, tile_m, out,
                     workspace, ws_bytes, flags, nullptr, 0, stream, true);
  }
  st = moe_w4_route_gateup_silu(act, logits, x, T, H, I, E, k, renormalize, w13, w13_shared,
                                n_shared, I_shared, tile_m, topk_ids, topk_w, counts, offsets,
                                sorted_pair, pair_pos, tiles, n_tiles, h, workspace, ws_bytes,
                                flags, stream);
  if (st != MOE_OK) return st;
  return moe_w4_down_combine(act, h, T, H, I, E, k, w2, w2_shared, n_shared, I_shared,
                             shared_gate, topk_w, offsets, sorted_pair, pair_pos, tiles,
                             n_tiles, tile_m, out, workspace, ws_bytes, flags, stream);
}
