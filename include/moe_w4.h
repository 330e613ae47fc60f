/*
 * moe_w4.h -- C ABI of a low-bit mixture-of-experts FFN layer for AMD
 * MI355X (gfx950).
 *
 * The layer follows the build log "Two 96 GB Ascend cards run Qwen3.8
 * Flash-Next" (ai-pulse-lab), section "Keep low-bit weights packed, do the
 * work on the NPU": expert weights stay packed in device memory, tokens
 * are routed to experts on the device, and the expert projections run as
 * grouped operations with fused gate/up handling, blocked reduction, tile
 * reuse and a dedicated W4A8 mode -- never by expanding the packed bank
 * into a dequantized copy.  Section "Remove sync and launch overhead from
 * the token loop" of the same log asks for a hot path with no
 * device-to-host reads and reused per-step buffers; section "Make the
 * hybrid model correct before making it fast" treats the kernel package
 * and its host code as one versioned ABI.  Hence:
 *
 *   - every call is asynchronous on the caller's HIP stream and never
 *     synchronizes with the host; sizes of device-side data (number of
 *     tiles, tokens per expert) stay on the device and grids are sized
 *     from host-known upper bounds;
 *   - the library allocates nothing and keeps no state: the caller owns
 *     every buffer (weights, descriptor tables, activations, outputs,
 *     workspace) and keeps it alive and unmodified until the stream has
 *     passed the call;
 *   - calls return a moe_status and never throw; arguments are checked
 *     on the host before anything is launched;
 *   - one generic contract (T, H, I, E, k, group size, bit width), with
 *     no per-model special cases.
 *
 * Layer definition (what the calls compute together):
 *   ids, w   = top-k of the router logits per token (descending logit,
 *              ties to the lower expert index); w = softmax over the
 *              chosen k logits (renormalize=1) or the plain softmax
 *              values (renormalize=0)
 *   pairs    = (t, j) with flat index p = t*k + j, grouped by expert
 *              (stable: increasing p within an expert)
 *   gate/up  = g = x_t . W13_e[i], u = x_t . W13_e[I+i], h = SiLU(g)*u
 *   down     = y = h . W2_e[n]
 *   combine  = out[t] = sum_j w[t][j] * y(t, ids[t][j]) + sum_s g_s(t) y_s(t)
 *   with W = code * scale (code int4 in [-8,7] or int2 in [-2,1], one
 *   fp16 scale per row per K-group).  Shared experts are always on and
 *   join with weight g = 1.0, or with a sigmoid gate g = sigmoid(l) of a
 *   per-token gate logit l when the caller passes shared-gate logits.
 *
 * Precision: A16 (bf16 activations): fp32 accumulation; h is rounded to
 * bf16 between the projections.  A8: activations are quantized per row to
 * int8 with scale = max|row| / 127 (fp32, round half to even); per-group
 * int8 x int code partial sums are exact int32; they are scaled in fp32.
 * out is bf16 (round to nearest even).
 *
 * All pointers are DEVICE pointers unless stated otherwise.
 */
#ifndef MOE_W4_H
#define MOE_W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_W4_ABI_VERSION 4

/* Version of the compiled library.  The Python binding refuses to load a
 * library whose version differs from the header it was written for. */
int moe_abi_version(void);

typedef enum {
  MOE_OK = 0,
  MOE_E_INVAL = -1,        /* bad argument (null pointer, size, shape)      */
  MOE_E_UNSUPPORTED = -2,  /* valid but unsupported (bits, group, E, ...)   */
  MOE_E_DEVICE = -3,       /* HIP error, or the current device is not gfx950 */
  MOE_E_WORKSPACE = -4     /* workspace missing or smaller than required    */
} moe_status;

/* Static string for a status code (host pointer, never null). */
const char* moe_status_str(int status);

typedef enum {
  MOE_A16 = 0,             /* bf16 activations                               */
  MOE_A8 = 1               /* dynamic per-row int8 activations               */
} moe_act;

/* One quantized matrix W [N][K], K contiguous.  Tables of these descriptors
 * live in DEVICE memory (one per expert); `codes` and `scales` point to
 * device memory.
 *   codes : N * K * bits / 8 bytes, row-major.  bits = 4: two codes per byte,
 *           even K index in the low nibble.  bits = 2: four codes per byte,
 *           lowest K index in the lowest two bits.  Two's complement.
 *   scales: N * (K / group) fp16 bit patterns, row-major.
 * Supported: bits in {2, 4}; group in {32, 64, 128, 256}; K % group == 0;
 * a row of codes is a whole number of 16-byte chunks (K % 32 == 0 for
 * int4, K % 64 == 0 for int2); codes 16-byte aligned, scales 4-byte
 * aligned.  A descriptor the kernels cannot use (other bits or group,
 * N/K different from the shape the call expects, null pointer) makes the
 * kernels skip that expert and set bit 0 of the workspace error word. */
typedef struct moe_qmat {
  const uint8_t* codes;
  const uint16_t* scales;
  int32_t bits;
  int32_t group;
  int32_t N;
  int32_t K;
} moe_qmat;                 /* 32 bytes */

/* ---------------------------------------------------------------------
 * moe_router_topk -- the router on the device: logits from the token
 * activations and the router weights, then moe_route_topk on them.
 * Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", section "Keep
 * low-bit weights packed, do the work on the NPU" (tokens are scored and
 * routed on the device).
 *   x         bf16 [T][H]
 *   router_w  fp32 [H][E] (row h holds every expert's weight for input h)
 *   prior     fp32 [E] added to every token's logits, or null
 *   logits    fp32 [T][E] (out): sum over h of x[t][h] * router_w[h][e] in
 *             fp32, in a fixed order (increasing h inside each chunk of H,
 *             then the chunks in order; the chunking depends only on T, H
 *             and E), then + prior[e]
 *   topk_ids, topk_w (out): as moe_route_topk on those logits
 *   workspace moe_router_workspace_bytes(T, H, E) bytes of device memory,
 *             16-byte aligned (may be null when that is 0)
 * Limits: those of moe_route_topk, T * H, H * E and T * E below 2^31.
 * Errors: MOE_E_INVAL (arguments), MOE_E_UNSUPPORTED (limits),
 * MOE_E_WORKSPACE, MOE_E_DEVICE.  The fp32 logits can differ from exact
 * ones by the rounding of the sum, so near-ties may select differently
 * from an exact router; the routing of the returned logits is exact.
 * ------------------------------------------------------------------- */
size_t moe_router_workspace_bytes(int T, int H, int E);
moe_status moe_router_topk(const uint16_t* x, int T, int H,
                           const float* router_w, const float* prior, int E,
                           int k, int renormalize, float* logits,
                           int32_t* topk_ids, float* topk_w, void* workspace,
                           size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * moe_route_topk -- router top-k and softmax gating on the device
 * (pages: tokens are routed to experts on the device; routing moved out of
 * the host loop).
 *   logits   fp32 [T][E]
 *   topk_ids int32 [T][k]  (out) experts in descending logit order, ties
 *                          to the lower index
 *   topk_w   fp32 [T][k]   (out) gate weights
 * Limits: 1 <= E <= 1024, 1 <= k <= E, T >= 0 (T = 0 launches nothing).
 * Logits must be finite.
 * ------------------------------------------------------------------- */
moe_status moe_route_topk(const float* logits, int T, int E, int k,
                          int renormalize, int32_t* topk_ids, float* topk_w,
                          void* stream);

/* ---------------------------------------------------------------------
 * moe_permute -- stable counting sort of the T*k (token, expert) pairs by
 * expert, plus the tile list the grouped projections walk (pages: grouped
 * expert projections with routing and tile reuse).
 *   topk_ids    int32 [T*k]   pair p = t*k + j goes to expert topk_ids[p]
 *   counts      int32 [E]     (out) pairs per expert
 *   offsets     int32 [E+1]   (out) exclusive prefix sum of counts
 *   sorted_pair int32 [T*k]   (out) pairs grouped by expert, increasing p
 *                             within an expert
 *   pair_pos    int32 [T*k]   (out) inverse: pair_pos[sorted_pair[r]] = r
 *   tiles       int32 [max_tiles][4] (out) (expert, first row, end row, 0):
 *                             per expert, consecutive runs of at most tile_m
 *                             sorted rows; experts in increasing order
 *   n_tiles     int32 [1]     (out) number of tiles written
 * max_tiles = moe_permute_max_tiles(T, k, E, tile_m).
 * An id outside [0, E) is skipped: its pair_pos is -1, it is not counted
 * (offsets[E] < T*k reveals it) and the tail of sorted_pair is -1.
 * Limits: 1 <= E <= 512, 1 <= tile_m <= 4096, T*k < 2^24.
 * ------------------------------------------------------------------- */
moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E,
                       int tile_m, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_pair, int32_t* pair_pos,
                       int32_t* tiles, int32_t* n_tiles, void* stream);

/* ---------------------------------------------------------------------
 * moe_route_permute -- moe_route_topk followed by moe_permute, in one launch
 * (one workgroup) for T < 16, where the two steps are each a handful of
 * microseconds of launch and latency (pages: fused operators where a decode
 * step is many small launches); from 16 tokens on the routing alone keeps a
 * compute unit busy for longer than a launch costs, so it issues the two
 * kernels.  Same outputs, bit for bit, as the two calls.  Limits: T <= 64,
 * T*k <= 4096, 1 <= E <= 512.
 * ------------------------------------------------------------------- */
moe_status moe_route_permute(const float* logits, int T, int E, int k,
                             int renormalize, int tile_m, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_pair, int32_t* pair_pos,
                             int32_t* tiles, int32_t* n_tiles, void* stream);

/* Host-side upper bound of n_tiles: min(T*k, floor(T*k / tile_m) + min(E, T*k)). */
int moe_permute_max_tiles(int T, int k, int E, int tile_m);

/* ---------------------------------------------------------------------
 * moe_quant_a8_rows -- the dynamic int8 row quantizer of the A8 mode, as a
 * standalone call (the projections run the same device code internally).
 * Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", section "Keep
 * low-bit weights packed, do the work on the NPU" (a dedicated W4A8
 * execution: int8 activations against the packed int4 weights).
 *   src   [R][ld] bf16 (src_is_f32 = 0) or fp32 (src_is_f32 = 1); the
 *         first C entries of each row are quantized
 *   q     int8 [R][C] (out), s fp32 [R] (out)
 *   s = fp32(max|row|) / 127 (IEEE division), q = clamp(rint(v / s), -127,
 *   127) with round half to even; a zero row gives s = 0, q = 0.
 * ------------------------------------------------------------------- */
moe_status moe_quant_a8_rows(const void* src, int src_is_f32, int R, int C,
                             int ld, int8_t* q, float* s, void* stream);

/* ---------------------------------------------------------------------
 * Workspace of the two projection calls.  One buffer of this size (device
 * memory, 256-byte aligned) may be passed to both calls of a layer.  Its
 * first 4 bytes are an error word the kernels OR bits into (bit 0: an
 * expert descriptor was unusable; bit 1: a tile named an expert outside
 * [0, E); bit 2: a grid-wide wait of moe_w4_layer expired, the output of
 * that call is incomplete).  Bytes 256-4351 hold the flags of
 * moe_w4_layer's grid-wide barrier, which are all equal again whenever a
 * call has ended.  The caller zeroes the first 4352 bytes once and reads
 * the error word when it wants to.
 * Rows of h / y: R = T*k + n_shared*T.
 * ------------------------------------------------------------------- */
size_t moe_workspace_bytes(int act, int T, int H, int I, int E, int k,
                           int n_shared, int I_shared);

/* Flags of the projection calls. */
#define MOE_PATH_AUTO 0       /* choose from the average pairs per expert   */
#define MOE_PATH_GEMV 1       /* split-K wavefront GEMV (decode shapes)      */
#define MOE_PATH_MFMA 2       /* MFMA grouped GEMM (prefill shapes); A16 only, */
                              /* H, I, I_shared multiples of 128, and fp16    */
                              /* copies of x (T*H) and h (T*(k+n_shared)      */
                              /* rows of max(I, I_shared)) under 2 GiB, else  */
                              /* MOE_E_UNSUPPORTED                            */
#define MOE_PATH_MFMA16 3     /* 16x16 MFMA tiles of at most 16 rows (decode */
                              /* batches; both modes): tile_m <= 16 and the   */
                              /* tile's activations within 160 KB of LDS,     */
                              /* else MOE_E_UNSUPPORTED                       */
#define MOE_PATH_MASK 3
#define MOE_QUANT_SEPARATE 4  /* W4A8: quantize x with the row quantizer    */
                              /* launch even where the gate/up kernel would */
                              /* make the int8 rows itself (same codes; a   */
                              /* check and a fallback)                      */
#define MOE_X_PREPARED 64     /* moe_w4_gateup_silu: read the prepared copy */
                              /* of x from the workspace instead of making  */
                              /* it: W4A8 int8 rows and scales, or the fp16 */
                              /* copy the matrix-core path stages (bf16,    */
                              /* prefill shapes).  The routing launch of    */
                              /* moe_w4_route_gateup_silu (W4A8, T <= 64,   */
                              /* H a multiple of 8) and of moe_w4_layer     */
                              /* (also the matrix-core path) leaves it for  */
                              /* that x and T; the caller guarantees it is  */
                              /* there.  Ignored where no copy is read      */
#define MOE_LAYER_ONE_LAUNCH 8 /* moe_w4_layer: one launch for the whole    */
                              /* layer where the shape allows it (same      */
                              /* results as the two calls)                  */
#define MOE_W_PREPACKED 32    /* the weight tables' codes are in the layout */
                              /* of moe_w4_prepack and their scales in that */
                              /* of moe_w4_prepack_scales; read by the      */
                              /* matrix-core path only: any other path      */
                              /* returns MOE_E_UNSUPPORTED                  */
#define MOE_OUT_F32 16        /* moe_w4_down_combine / moe_w4_layer: out is */
                              /* fp32 [T][H] (16-byte aligned) holding the  */
                              /* combined sum before any rounding to bf16;  */
                              /* without it out is bf16, the round-to-      */
                              /* nearest-even of exactly that value         */

/* Tile height to pass as moe_permute's tile_m: 160 (the MFMA path's row
 * chunk: an expert with up to 160 pairs streams its weights once) when
 * T*k >= 32*E with A16, else 16.  Both paths accept any tile_m; the MFMA
 * path walks longer tiles in 160-row chunks. */
int moe_preferred_tile_m(int act, int T, int E, int k);

/* ---------------------------------------------------------------------
 * moe_w4_prepack -- optional re-tiling of one packed code matrix into the
 * order the matrix-core path (MOE_PATH_MFMA, prefill shapes) loads it in,
 * the analogue of the operand layout the build log "Two 96 GB Ascend cards
 * run Qwen3.8 Flash-Next" adds for its matrix unit (section "Keep low-bit
 * weights packed, do the work on the NPU").  The canonical layout keeps
 * working everywhere; a prepacked bank is read only with MOE_W_PREPACKED.
 *   codes   canonical codes of a [N][K] matrix (moe_qmat layout), device
 *   bits    4 or 2
 *   gate_up 1 for a gate/up matrix [2I][H] (rows i and I + i are paired),
 *           0 for a down matrix [H][I]
 *   dst     device, N*K*bits/8 bytes (the same size), not overlapping codes
 * Layout of dst: pieces of 64 lane slots; slot h*32 + c of a piece holds
 * bytes [32 s + 16 h, +16) of one row for int4, [16 s + 8 h, +8) for int2
 * with every 4-byte word's bytes in the order (0, 2, 1, 3).  Down: piece
 * (b, s) = rows 32b + c at step s, in order b, s.  Gate/up: pieces (b, s,
 * p) in order b, s, p, p = 0 the gate rows 32b + c and p = 1 the up rows
 * I + 32b + c.  The scales are re-tiled by moe_w4_prepack_scales.
 * Limits: N % 32 == 0 (gate/up: N % 64 == 0), K % 128 == 0.  Errors: MOE_E_INVAL,
 * MOE_E_UNSUPPORTED, MOE_E_DEVICE.  Asynchronous on `stream`.
 * ------------------------------------------------------------------- */
moe_status moe_w4_prepack(const uint8_t* codes, int bits, int N, int K, int gate_up,
                          uint8_t* dst, void* stream);

/* ---------------------------------------------------------------------
 * moe_w4_prepack_scales -- the fp16 group scales of one matrix re-tiled for
 * the matrix-core path next to moe_w4_prepack's codes (same build log and
 * section): a wave then reads the scales of its 32 row pairs for one group
 * as one 128-byte run instead of 64 rows' scattered 2-byte values.
 *   scales  canonical scales [N][K/group] (moe_qmat layout), device
 *   group   32, 64, 128 or 256 (K % group == 0)
 *   gate_up 1 for a gate/up matrix [2I][H], 0 for a down matrix [H][I]
 *   dst     device, N*(K/group)*2 bytes (the same size), 16-byte aligned,
 *           not overlapping scales
 * Layout of dst: 4-byte words ((b * ng + g) * 32 + c), ng = K/group, each
 * the scale of group g of row r0 (low half) and of row r1 (high half):
 * gate/up r0 = 32b + c (gate), r1 = N/2 + 32b + c (up); down r0 = 64b + c,
 * r1 = 64b + 32 + c.
 * The matrix-core kernel copies a wave's block of words into LDS once per
 * tile, so a prepacked matrix has at most 64 groups per row.
 * Limits: N % 64 == 0, K / group <= 64.  Errors: MOE_E_INVAL,
 * MOE_E_UNSUPPORTED, MOE_E_DEVICE.  Asynchronous on `stream`.
 * ------------------------------------------------------------------- */
moe_status moe_w4_prepack_scales(const uint16_t* scales, int N, int K, int group, int gate_up,
                                 uint16_t* dst, void* stream);

/* ---------------------------------------------------------------------
 * moe_w4_gateup_silu -- grouped gate/up projection of every routed pair
 * and every shared-expert token, fused with SiLU(g) * u.
 * Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", section "Keep
 * low-bit weights packed, do the work on the NPU" (grouped expert
 * projections on packed weights with fused gate/up handling, blocked
 * reduction, routing and tile reuse, W4A8 execution) and section "GLM is
 * my next, harder model" (a blocked-dequant matrix kernel over mixed
 * int2/int4 experts).
 *   x          bf16 [T][H]
 *   w13        device table of E moe_qmat, each [2I][H] (gate rows 0..I-1,
 *              up rows I..2I-1)
 *   w13_shared device table of n_shared moe_qmat, each [2*I_shared][H]
 *              (may be null when n_shared = 0)
 *   offsets, sorted_pair, tiles, n_tiles: from moe_permute (same tile_m)
 *   h          (out) rows R = T*k + n_shared*T, row stride ld_h =
 *              max(I, I_shared); row r < T*k is sorted row r, row T*k +
 *              s*T + t is shared expert s and token t.
 *              A16: bf16 [R][ld_h] (h rounded to bf16).
 *              A8 : fp32 [R][ld_h].
 * Precision of the matrix-core path (MOE_PATH_MFMA, chosen automatically
 * for prefill shapes): x enters the MFMAs as fp16 (bf16 -> fp16 rounding
 * toward zero: exact for |x| in [2^-14, 65504], saturating above 65504,
 * losing low bits below 2^-14) against code * scale rounded once to fp16;
 * fp32 accumulation.  Inputs with |x| or |h| above 65504 need
 * MOE_PATH_GEMV or MOE_PATH_MFMA16.
 * ------------------------------------------------------------------- */
moe_status moe_w4_gateup_silu(int act, const uint16_t* x, int T, int H,
                              int I, int E, int k, const moe_qmat* w13,
                              const moe_qmat* w13_shared, int n_shared,
                              int I_shared, const int32_t* offsets,
                              const int32_t* sorted_pair,
                              const int32_t* tiles, const int32_t* n_tiles,
                              int tile_m, void* h, void* workspace,
                              size_t ws_bytes, int flags, void* stream);

/* ---------------------------------------------------------------------
 * moe_w4_route_gateup_silu -- moe_route_permute followed by
 * moe_w4_gateup_silu, with the outputs of both (same argument meanings).
 * Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", section
 * "Remove sync and launch overhead from the token loop": a decode step is
 * dominated by launches and round trips, so for bf16 activations with
 * T*k <= 64, E <= 512, H <= 2048 and tiles of at most 16 rows (the split-K
 * path) this is ONE launch in which every workgroup routes and sorts the
 * batch itself before its share of the gate/up work; other shapes issue
 * the routing call and the gate/up call.  For W4A8 with T <= 64 and H a
 * multiple of 8 (16-byte aligned x) the routing launch also quantizes x
 * (one extra workgroup per token, the row rule of moe_quant_a8_rows) into
 * the workspace, and the gate/up call reads those rows (MOE_X_PREPARED),
 * so no quantizing launch or in-kernel quantization follows.  (moe_w4_layer
 * does the same with the fp16 copy of x on the matrix-core path.)  Errors:
 * those of the two calls.
 * ------------------------------------------------------------------- */
moe_status moe_w4_route_gateup_silu(int act, const float* logits,
                                    const uint16_t* x, int T, int H, int I,
                                    int E, int k, int renormalize,
                                    const moe_qmat* w13,
                                    const moe_qmat* w13_shared, int n_shared,
                                    int I_shared, int tile_m,
                                    int32_t* topk_ids, float* topk_w,
                                    int32_t* counts, int32_t* offsets,
                                    int32_t* sorted_pair, int32_t* pair_pos,
                                    int32_t* tiles, int32_t* n_tiles, void* h,
                                    void* workspace, size_t ws_bytes,
                                    int flags, void* stream);

/* ---------------------------------------------------------------------
 * moe_w4_down_combine -- grouped down projection of every h row and the
 * weighted combine into the token outputs.
 * Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", section "Keep
 * low-bit weights packed, do the work on the NPU" (grouped expert
 * projections straight from packed weights, blocked reduction, W4A8
 * execution; the routed experts' outputs are joined by their gate
 * weights).
 *   h          as written by moe_w4_gateup_silu (same act); A8 rows are
 *              quantized to int8 per row inside this call
 *   w2         device table of E moe_qmat, each [H][I]
 *   w2_shared  device table of n_shared moe_qmat, each [H][I_shared]
 *   shared_gate fp32 [T][n_shared] gate logits of the shared experts, or
 *              null: shared expert s joins token t with weight
 *              sigmoid(shared_gate[t][s]) = 1 / (1 + exp(-l)) (fp32), or
 *              with weight 1.0 when null
 *   topk_w     fp32 [T][k] from moe_route_topk
 *   pair_pos   from moe_permute
 *   out        bf16 [T][H] (out): out[t] = sum_j topk_w[t][j] * y(pair
 *              t*k+j) + sum_s g(t, s) * y(shared s, t), summed in fp32 in
 *              that order (g = the shared gate weight above)
 *              and rounded to bf16; with MOE_OUT_F32 in flags, fp32 [T][H]
 *              holding that sum unrounded
 * Decode batches with bf16 activations (tiles of at most 16 rows, I <= 1024,
 * every h row of the layer fitting in 64 KB of LDS) combine inside the
 * down kernel: a workgroup owns a range of output columns of every token.
 * Otherwise y goes through the workspace (fp32 [R][H]) to a combine kernel.
 * Calls sharing a workspace must be ordered on one stream.
 * ------------------------------------------------------------------- */
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
                               size_t ws_bytes, int flags, void* stream);

/* ---------------------------------------------------------------------
 * moe_w4_layer -- the whole layer: moe_w4_route_gateup_silu followed by
 * moe_w4_down_combine, with the outputs of both (same argument meanings;
 * topk_w and pair_pos are outputs here).
 * Build log "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", sections
 * "Remove sync and launch overhead from the token loop" (fewer launches,
 * no host round trips in a decode step) and "Keep low-bit weights packed,
 * do the work on the NPU" (the layer's projections straight from packed
 * weights).  By default it issues the two calls.  With
 * MOE_LAYER_ONE_LAUNCH, for bf16 activations with T*k <= 64, E <= 128,
 * H <= 2048, I and I_shared <= 1024 and tiles of at most 16 rows, it is
 * ONE launch: every workgroup routes the batch itself, the gate/up and
 * down weight streams are issued together, and the workgroups meet at a
 * grid-wide barrier once h is complete (taken only when the device can
 * hold every workgroup of the grid at once; the wait is bounded, see the
 * error word).  On MI355X the two calls are the faster form at the decode
 * shapes measured (the shared weight stream and the barrier's round trips
 * cost more than the second launch), so the single launch is opt-in.
 * Calls sharing a workspace must be ordered on one stream.
 * Errors: those of the two calls.
 * ------------------------------------------------------------------- */
moe_status moe_w4_layer(int act, const float* logits, const uint16_t* x,
                        int T, int H, int I, int E, int k, int renormalize,
                        const moe_qmat* w13, const moe_qmat* w2,
                        const moe_qmat* w13_shared, const moe_qmat* w2_shared,
                        int n_shared, int I_shared, const float* shared_gate,
                        int tile_m,
                        int32_t* topk_ids, float* topk_w, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_pair,
                        int32_t* pair_pos, int32_t* tiles, int32_t* n_tiles,
                        void* h, void* out, void* workspace,
                        size_t ws_bytes, int flags, void* stream);

/* ---------------------------------------------------------------------
 * moe_w4_layer_noalloc -- moe_w4_layer with no workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace is a library-owned device array of MOE_NOALLOC_SCRATCH_BYTES
 * (32 MiB) per GPU, held from the first call on that GPU until the process
 * ends; the call itself allocates nothing and frees nothing.
 *   arguments  as moe_w4_layer (same meanings, flags included)
 *   err_out    int32 [1] device pointer or null: when given, the call
 *              clears the array's error word first and copies it here at
 *              the end (bits as in the workspace error word above)
 * Shapes whose workspace (moe_workspace_bytes) exceeds the array return
 * MOE_E_WORKSPACE before anything is launched: decode batches fit (the
 * 64-token W4A8 layer needs about 5 MB), a 4096-token prefill chunk does
 * not and needs moe_w4_layer with a caller workspace.
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents: calls that overlap in time on one GPU (other streams,
 * other threads) race on it and must be ordered by the caller.
 * ------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_w4_layer_noalloc(int act, const float* logits, const uint16_t* x,
                                int T, int H, int I, int E, int k,
                                int renormalize, const moe_qmat* w13,
                                const moe_qmat* w2, const moe_qmat* w13_shared,
                                const moe_qmat* w2_shared, int n_shared,
                                int I_shared, const float* shared_gate,
                                int tile_m, int32_t* topk_ids,
                                float* topk_w, int32_t* counts,
                                int32_t* offsets, int32_t* sorted_pair,
                                int32_t* pair_pos, int32_t* tiles,
                                int32_t* n_tiles, void* h, void* out,
                                int32_t* err_out, int flags, void* stream);

/* 1 when moe_w4_layer with these arguments (flags included) issues one
 * launch on the current device, 0 when it issues the two calls, a
 * negative moe_status for arguments it would reject (or no usable
 * device). */
int moe_w4_layer_one_launch(int act, int T, int H, int I, int E, int k,
                            int n_shared, int I_shared, int tile_m, int flags);

/* ---------------------------------------------------------------------
 * moe_read_stream -- measurement aid: one plain streaming read of `bytes`
 * bytes of device memory at `src` (16-byte aligned, bytes % 16 == 0) by
 * n_blocks workgroups of 256 threads, 16-byte loads.  `sink` (device,
 * n_blocks words) is written only in a case that does not occur, so the
 * call moves `bytes` from HBM and writes nothing.  The decode layers'
 * packed-weight bandwidth is reported against this measured ceiling as
 * well as against the published HBM peak (decode is bound by streaming
 * the packed expert weights: build log "Two 96 GB Ascend cards run
 * Qwen3.8 Flash-Next", section "Keep low-bit weights packed, do the work
 * on the NPU").  Errors: MOE_E_INVAL, MOE_E_DEVICE.
 * ------------------------------------------------------------------- */
moe_status moe_read_stream(const void* src, size_t bytes, uint32_t* sink, int n_blocks,
                           void* stream);

/* ---------------------------------------------------------------------
 * Test hooks of the A8 mode (build log "Two 96 GB Ascend cards run Qwen3.8
 * Flash-Next", section "Keep low-bit weights packed, do the work on the
 * NPU": dedicated W4A8 execution).  They take the path that
 * moe_w4_gateup_silu / moe_w4_down_combine take for the same shape and
 * flags (MOE_PATH_AUTO: the product's choice, e.g. the 16-row matrix
 * tiles with int8 rows made in the kernel; MOE_PATH_GEMV or
 * MOE_PATH_MFMA16 to force one; MOE_PATH_MFMA is A16 only and returns
 * MOE_E_UNSUPPORTED) and run those kernels, compiled with the store of
 * the exact int32 per-group partial sums they accumulate added before
 * the sums are scaled:
 *   gate/up: partials [R][2*ld_h][ng_ld], entry (r, n, c) = sum over the
 *            K indices of group c of qx[t][K] * code[n][K]
 *   down   : partials [R][H][ng_ld], from this call's own int8 h codes
 * ng_ld >= K / group of every expert used; entries past an expert's
 * group count are left untouched.  h and out are written as by the
 * product calls.
 * ------------------------------------------------------------------- */
moe_status moe_dbg_w4a8_gateup_partials(
    const uint16_t* x, int T, int H, int I, int E, int k,
    const moe_qmat* w13, const moe_qmat* w13_shared, int n_shared,
    int I_shared, const int32_t* offsets, const int32_t* sorted_pair,
    const int32_t* tiles, const int32_t* n_tiles, int tile_m, void* h,
    void* workspace, size_t ws_bytes, int flags, int32_t* partials, int ng_ld,
    void* stream);

moe_status moe_dbg_w4a8_down_partials(
    const void* h, int T, int H, int I, int E, int k, const moe_qmat* w2,
    const moe_qmat* w2_shared, int n_shared, int I_shared,
    const float* shared_gate, const float* topk_w, const int32_t* offsets, const int32_t* sorted_pair,
    const int32_t* pair_pos, const int32_t* tiles, const int32_t* n_tiles,
    int tile_m, void* out, void* workspace, size_t ws_bytes, int flags,
    int32_t* partials, int ng_ld, void* stream);

/* ---------------------------------------------------------------------
 * moe_dbg_dec_stamps -- measurement aid for the decode timeline (build log
 * "Two 96 GB Ascend cards run Qwen3.8 Flash-Next", section "Remove sync
 * and launch overhead from the token loop": where the time of a decode
 * step goes).  In a library built with MOE_DEC_STAMPS
 * (`python -m packed_bit_grouped_amd.build --stamps OUT.so`) it names the
 * device buffer (unsigned 64-bit [grid][8], caller-owned, zeroed by the
 * caller) into which the decode kernels' workgroups write the 100 MHz
 * realtime counter at each phase end: dec_route_gateup_kernel slots 0
 * entry, 1 routed, 2 sorted, 3 weights issued, 4 activations staged, 5
 * products done; dec_down_combine_kernel 0 entry, 1 tables in, 2 weights
 * issued, 3 h staged, 4 products done, 5 outputs stored.  Null stops the
 * stamps.  It applies to launches that follow it on any stream.  Errors:
 * MOE_E_UNSUPPORTED in the regular library (nothing is touched),
 * MOE_E_DEVICE.
 * ------------------------------------------------------------------- */
moe_status moe_dbg_dec_stamps(unsigned long long* stamps);

#ifdef __cplusplus
}
#endif
#endif /* MOE_W4_H */
