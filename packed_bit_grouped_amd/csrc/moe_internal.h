// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include "moe_common.h"

namespace moe {

constexpr int kPermMaxE = 512;      // permute: experts per launch
constexpr int kPermIdBits = 9;      // bits of an expert id below kPermMaxE
constexpr int kRouteMaxE = 1024;    // route: 16 logits per lane
constexpr int kFusedRouteMaxT = 64; // fused route+permute: tokens per launch
constexpr int kFusedRouteMaxP = 4096;  // fused route+permute: pairs per launch
constexpr int kLayerFlags = 1024;   // one-launch layer: barrier flags (and max grid)

// Workspace layout (byte offsets from the workspace base).
struct WsLayout {
  size_t err;        // int32 error word
  size_t flags;      // kLayerFlags uint32 barrier flags of the one-launch layer
  size_t qx;         // A8: int8 [T][H]
  size_t sx;         // A8: fp32 [T]
  size_t qh;         // A8: int8 h rows [R][ld_h] (matrix-core decode path)
  size_t sh;         // A8: fp32 [R]
  size_t y;          // fp32 [R][H]
  size_t a16;        // A16 MFMA path: fp16 copy of x (gate/up) or of h (down)
  size_t perm;       // moe_w4_layer: per-workgroup counts of the multi-workgroup sort
  size_t h16;        // A16 MFMA path: fp16 copy of h written by the gate/up epilogue
                     // (moe_w4_layer: the down call reads it instead of converting h)
  size_t total;
};
WsLayout ws_layout(int act, int T, int H, int I, int E, int k, int n_shared,
                   int I_shared);

// Arguments of the grouped projections (both kernels families).
struct ProjArgs {
  int mode;                    // 0: gate/up (+SiLU*mul), 1: down
  // inputs
  const uint16_t* in_bf16;     // A16: x [T][H] (gate/up) or h [R][ld_in] (down)
  const float* in_f32;         // A8 down: h fp32 [R][ld_in]
  const int8_t* in_q;          // A8 gate/up: qx [T][H]
  const float* in_s;           // A8 gate/up: sx [T]
  int ld_in;
  // weights
  const moe_qmat* w;           // routed experts
  const moe_qmat* w_sh;        // shared experts
  int K, K_sh;                 // reduction length (routed / shared)
  int U, U_sh;                 // output units per expert: I pairs (gate/up), H rows (down)
  // routing
  int T, k, P, E, n_shared;
  const int32_t* offsets;
  const int32_t* sorted_pair;
  const int32_t* tiles;
  const int32_t* n_tiles;
  int max_tiles;               // host upper bound of *n_tiles
  int maxt;                    // activation rows staged per pass (1, 2, 4, 8)
  int sh_tile;                 // tokens per shared-expert tile
  int n_sh_slots;              // n_shared * ceil(T / sh_tile)
  int rb;                      // units per work item (MFMA path)
  int n_rb;                    // work items per tile (MFMA path)
  int res_rows;                // rows of one result buffer in LDS (GEMV path)
  // outputs
  void* out;                   // gate/up: h (bf16 or fp32); down: y fp32
  int ld_out;
  int32_t* err;
  // down with the combine fused (decode kernels): gate weights and the
  // sorted row of every pair
  const float* topk_w;
  const int32_t* pair_pos;
  uint16_t* out16;             // MFMA gate/up: also write h as fp16 in the unpack order, or null
  int in16_ready;              // MFMA down: in_bf16 already holds that fp16 copy;
                               // MFMA gate/up: the fp16 copy of x is made
  int out_f32;                 // the combined output is fp32 (else bf16)
  const float* sh_gate;        // shared-expert gate logits [T][n_shared], or null (weight 1)
  int32_t* partials;           // A8 test hook (null otherwise)
  int ng_ld;
  int part_rows;               // row stride (in weight rows) of partials
};


// Router logits = x . W (+ prior), fp32 in a fixed order; part: the
// workspace of router_workspace_bytes (null when that is 0).
size_t router_workspace_bytes(int T, int H, int E);
hipError_t launch_router_logits(const uint16_t* x, int T, int H, const float* W, int E,
                                const float* prior, float* logits, float* part,
                                hipStream_t st);
hipError_t launch_permute(const int32_t* ids, int P, int E, int tile_m,
                          int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos,
                          int32_t* tiles, int32_t* n_tiles, hipStream_t st);
// The same sort over many workgroups for large batches: scratch holds
// permute_multi_blocks(P) * E ints (zero blocks: P below the threshold,
// the single-workgroup sort runs).
constexpr int kPermMultiMinP = 8192;
int permute_multi_blocks(int P);
hipError_t launch_permute_multi(const int32_t* ids, int P, int E, int tile_m, int32_t* counts,
                                int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                int32_t* tiles, int32_t* n_tiles, int32_t* scratch,
                                hipStream_t st);
// Copies of x made by extra workgroups of the routing launch, so that the
// gate/up projection needs no preparing launch of its own: W4A8 int8 rows
// and scales (q, s: one workgroup per row, the row quantizer's rule), or
// the matrix-core path's fp16 copy in the unpack order (x16).  x bf16
// [T][H], 16-byte aligned, H a multiple of 8.
struct XPrep {
  const uint16_t* x;
  int H;
  int8_t* q;        // [T][H], or null
  float* s;         // [T]
  uint16_t* x16;    // [T][H] fp16, or null
};
// workgroups of 256 threads that make the fp16 copy of T rows of H
int xprep_convert_blocks(int T, int H);
hipError_t launch_route_permute(const float* logits, int T, int E, int k,
                                int renorm, int tile_m, int32_t* ids, float* w,
                                int32_t* counts, int32_t* offsets,
                                int32_t* sorted_pair, int32_t* pair_pos,
                                int32_t* tiles, int32_t* n_tiles, hipStream_t st,
                                const XPrep* xq = nullptr);
hipError_t launch_route_topk(const float* logits, int T, int E, int k,
                             int renorm, int32_t* ids, float* w, hipStream_t st,
                             const XPrep* xp = nullptr);
// Rows [R][C] (row stride ld) to int8 rows of stride ldq and fp32 scales.
hipError_t launch_quant_a8(const void* src, int is_f32, int R, int C, int ld,
                           int8_t* q, int ldq, float* s, hipStream_t st);
hipError_t launch_proj_gemv(const ProjArgs& a, int act, int grid, hipStream_t st);
int gemv_maxt(int T, int tile_m);
// Matrix-core grouped GEMM (two waves per SIMD); a16: workspace for one
// fp16 copy of the activations; prepacked: the weight tables hold codes in
// the layout of launch_prepack.
hipError_t launch_proj_mfma8(const ProjArgs& a, uint16_t* a16, bool prepacked, hipStream_t st);
// Re-tile one packed matrix [N][K] into the matrix-core fragment layout
// (N % 32 == 0, K % 64 == 0); gate_up pairs gate rows with up rows.
hipError_t launch_prepack(const uint8_t* src, int bits, int N, int K, int gate_up, uint8_t* dst,
                          hipStream_t st);
// Scales in the prepacked layout (moe_w4_prepack_scales), ng groups per row.
hipError_t launch_prepack_scales(const uint16_t* src, int N, int ng, int gate_up, uint16_t* dst,
                                 hipStream_t st);
bool mfma_available();
// Decode-shape A16 projections (proj_decode.hip): tiles of at most 16
// rows, H <= 2048 (gate/up) and I <= 1024 (down), down with the combine
// fused when every h row of the layer fits in LDS.  a.maxt must be
// dec_maxt(T, tile_m).
int dec_maxt(int T, int tile_m);
bool dec_gateup_ok(int T, int H, int tile_m);
bool dec_down_ok(int T, int k, int E, int n_shared, int H, int I, int I_shared, int ld,
                 int tile_m, int max_tiles);
hipError_t launch_dec_gateup(const ProjArgs& a, hipStream_t st);
hipError_t launch_dec_down_combine(const ProjArgs& a, void* out, hipStream_t st);
// Route + permute + gate/up in one launch (T * k <= 64, E <= 512).
bool dec_route_gateup_ok(int T, int H, int E, int k, int tile_m);
hipError_t launch_dec_route_gateup(const ProjArgs& a, const float* logits, int renorm,
                                   int tile_m, int32_t* ids, float* w, int32_t* counts,
                                   int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                   int32_t* tiles, int32_t* n_tiles, hipStream_t st);
// The whole layer (route, permute, gate/up, down, combine) in one launch
// for bf16 decode batches: every workgroup resident at once, a grid-wide
// barrier on h.  `launched` is false (and nothing was issued) when the
// grid would not be resident or the LDS would not fit; the caller then
// issues the two-call form.  flags: kLayerFlags words, all equal (zeroed
// once; every launch leaves them equal again).
bool dec_layer_ok(int T, int H, int I, int I_shared, int E, int k, int n_shared, int tile_m,
                  int max_tiles, int ld_h);
// 1 when launch_dec_layer would launch for this shape on the current device.
int dec_layer_one_launch(int T, int H, int I, int I_shared, int E, int k, int n_shared,
                         int tile_m, int max_tiles, int ld_h);
hipError_t launch_dec_layer(const ProjArgs& ag, const ProjArgs& ad, const float* logits,
                            int renorm, int tile_m, int32_t* ids, float* w, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                            int32_t* tiles, int32_t* n_tiles, void* out, uint32_t* flags,
                            bool& launched, hipStream_t st);
// Tiles of at most 16 rows on 16x16 MFMAs (proj_m16.hip).  A8 inputs are
// int8 rows (a.in_q, stride a.ld_in) with fp32 row scales (a.in_s): x for
// gate/up, the quantized h rows for down.
bool m16_ok(int act, int mode, int T, int K, int K_sh, int tile_m);
// A8: the kernel makes the int8 rows of a tile itself (from bf16 x or fp32
// h, a.in_q null) when they fit one staging batch.
bool m16_quant_ok(int mode, int T, int K, int K_sh);
hipError_t launch_proj_m16(const ProjArgs& a, int act, hipStream_t st);
// out: bf16 [T][H], or fp32 [T][H] when out_f32
hipError_t launch_combine(const float* y, int ld_y, const float* topk_w,
                          const int32_t* pair_pos, int T, int k, int H, int P,
                          int n_shared, const float* sh_gate, void* out, int out_f32,
                          hipStream_t st);

}  // namespace moe
